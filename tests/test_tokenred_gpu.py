"""Token reduction on the GPU (through the C ABI) vs the oracle
(oracle/tokenred.py, oracle/stack.py).

Merge and restore compute in fp32 and round once to bf16; the oracle works in
fp64.  A pair's sum of two bf16 values is exact in fp32 unless their
exponents differ by more than 16 bits, so merged rows are compared within one
rounding and counted for bit equality; restored rows likewise.  The reduced
stack uses the stack test's tolerance (tests/test_stack_gpu.py).
"""
import numpy as np
import pytest

import oracle
from oracle import stack as ostack
from oracle import tokenred as otr
from packed_masked_attention_amd import synth
from tests.helpers import bf16_to_np, one_rounding, say, to_dev_bf16
from tests.test_block_gpu import _block_close
from tests.test_stack_gpu import Weights, _WKEYS

pytestmark = pytest.mark.gpu


def _i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("name,hidden", [("tiny_L256", 256), ("block_L8192", 5376)])
def test_merge_and_restore_match_oracle(name, hidden):
    import torch
    from packed_masked_attention_amd import binding as B
    lay = synth.make_layout(synth.workload(name))
    plan = synth.token_reduction_plan(lay)
    L, n = lay["L"], plan["src0"].size
    rng = np.random.default_rng(80)
    x_bits = synth.normal_bf16(rng, (L, hidden))
    after_bits = synth.normal_bf16(rng, (n, hidden))
    say(f"token merge/restore {name}: L={L} -> {n} rows, hidden={hidden}")
    s0, s1 = _i32(plan["src0"]), _i32(plan["src1"])
    x = to_dev_bf16(x_bits)
    xr = torch.full((n, hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.pma_token_merge(hidden, L, s0, s1, x, xr)
    after = to_dev_bf16(after_bits)
    out = torch.full_like(x, float("nan"))
    B.pma_token_restore(hidden, L, s0, s1, x, xr, after, out)
    inplace = x.clone()
    B.pma_token_restore(hidden, L, s0, s1, inplace, xr, after, inplace)
    torch.cuda.synchronize()
    got_bits = xr.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_bits = otr.merge(x_bits, plan["src0"], plan["src1"])
    got, ref = oracle.bf16_to_f64(got_bits), oracle.bf16_to_f64(ref_bits)
    xv = oracle.bf16_to_f64(x_bits)
    exact = (xv[plan["src0"]] + np.where((plan["src1"] >= 0)[:, None], xv[plan["src1"]], xv[plan["src0"]])) / 2
    assert not (np.abs(got - exact) > one_rounding(exact)).any(), "merge"
    same = np.mean(got_bits == ref_bits)
    say(f"  merge bit-equal {same:.6f}")
    assert same > 0.9999
    # restore against the oracle fed the GPU's own merged rows (an input here)
    rref_bits = otr.unmerge(x_bits, got_bits, after_bits, plan["src0"], plan["src1"])
    rgot_bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    rexact = oracle.bf16_to_f64(rref_bits)
    assert not (np.abs(oracle.bf16_to_f64(rgot_bits) - rexact) > 2 * one_rounding(rexact)).any()
    say(f"  restore bit-equal {np.mean(rgot_bits == rref_bits):.6f}")
    assert np.mean(rgot_bits == rref_bits) > 0.999
    assert torch.equal(inplace.view(torch.int16), out.view(torch.int16)), "in-place restore"


def test_reduced_stack_matches_oracle():
    """Blocks [0, 1) full, merge, block 1 on the reduced rows (half-unit
    positions, position scale 1/2), restore, block 2 full -- against the
    oracle's reduced stack."""
    import torch
    from packed_masked_attention_amd import binding as B
    hid, H, ffn, E, T = 256, 2, 512, 64, 1
    lay = synth.layout_from_counts(16, (2, 4, 8), 16, 8, T=T)
    L = lay["L"]
    plan = synth.token_reduction_plan(lay)
    n = plan["src0"].size
    sets = []
    for i in range(3):
        inp = synth.make_block_inputs(L, hid, H, 128, ffn, E, T=T, seed=90 + i, layout=lay,
                                      weight_std=0.05)
        sets.append({k: inp[k] for k in _WKEYS})
        if i == 0:
            x_bits, temb_bits = inp["x"], inp["temb"]
    say(f"reduced stack: L={L} -> {n} rows, hidden={hid}")
    p = B.block_params(hid, ffn, E, H)
    pr = B.block_params(hid, ffn, E, H, pos_scale=plan["pos_scale"])
    dl = B.pma_layout_build(lay)
    dlr = B.pma_layout_build(plan["layout"])
    bits, _ = B.pma_layout_read_status(dlr)
    assert bits == 0, f"reduced layout status {bits:#x}"
    w = Weights(sets)
    temb = to_dev_bf16(temb_bits)
    x = to_dev_bf16(x_bits)
    x1 = torch.empty_like(x)
    B.pma_stack_forward(p, dl, w.structs[:1], temb, x, x1)
    s0, s1 = _i32(plan["src0"]), _i32(plan["src1"])
    xr0 = torch.empty(n, hid, dtype=torch.bfloat16, device="cuda")
    B.pma_token_merge(hid, L, s0, s1, x1, xr0)
    xr1 = torch.empty_like(xr0)
    B.pma_stack_forward(pr, dlr, w.structs[1:2], temb, xr0, xr1)
    B.pma_token_restore(hid, L, s0, s1, x1, xr0, xr1, x1)
    out = torch.empty_like(x)
    B.pma_stack_forward(p, dl, w.structs[2:], temb, x1, out)
    torch.cuda.synchronize()
    dims = {"L": L, "hidden": hid, "heads": H, "head_dim": 128, "ffn": ffn}
    ref = oracle.bf16_to_f64(ostack.reduced_stack_forward(x_bits, temb_bits, sets, lay, plan, 1, 2,
                                                          dims))
    _block_close(bf16_to_np(out), ref, "reduced stack x3", mean_rel=6e-3, max_rel=1.8e-1)
    # the reduction changes the result (the merged rows really are merged)
    plain = oracle.bf16_to_f64(ostack.stack_forward(x_bits, temb_bits, sets, lay, dims))
    assert np.abs(plain - ref).mean() > 1e-3


def test_token_plan_check_flags_bad_plans():
    """pma_token_plan_check on the device: the plan builder's plans pass; a
    src0 outside the sequence, a src1 outside it (other than -1), a row named
    twice and a row named by no entry each set their bit and name the first
    offending entry or row."""
    import torch
    from packed_masked_attention_amd import binding as B
    lay = synth.layout_from_counts(8, (2, 3, 4), 5, 3, T=1)
    plan = synth.token_reduction_plan(lay)
    L = int(lay["L"])
    src0 = torch.from_numpy(plan["src0"]).cuda()
    src1 = torch.from_numpy(plan["src1"]).cuda()
    say(f"token plan check: L={L}, {src0.numel()} reduced rows")
    assert B.pma_token_plan_check(L, src0, src1) == (0, -1, -1)
    pair = int(np.flatnonzero(plan["src1"] >= 0)[0])
    cases = []
    s0 = src0.clone(); s0[3] = L                       # src0 outside the sequence
    cases.append(("src0 out of range", s0, src1, 1, 3))
    s1 = src1.clone(); s1[pair] = -2                   # src1 neither a row nor -1
    cases.append(("src1 out of range", src0, s1, 1, pair))
    s1 = src1.clone(); s1[pair] = int(plan["src0"][0])  # row src0[0] named twice, src1[pair] never
    cases.append(("row named twice", src0, s1, 2 | 4, -1))
    for name, a, b, bits, entry in cases:
        got = B.pma_token_plan_check(L, a, b)
        say(f"  {name}: {got}")
        assert got[0] & bits == bits, name
        if bits & 1:
            assert got[1] == entry, name
        else:
            assert got[1] == -1 and got[2] >= 0, name
    # merge writes zeros for a reduced row whose src0 lies outside the sequence
    x = torch.randn(L, 64, device="cuda").to(torch.bfloat16)
    xr = torch.full((src0.numel(), 64), 7.0, device="cuda", dtype=torch.bfloat16)
    bad = src0.clone(); bad[3] = L
    B.pma_token_merge(64, L, bad, src1, x, xr)
    torch.cuda.synchronize()
    assert torch.all(xr[3] == 0)
