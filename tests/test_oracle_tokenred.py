"""Pins of the token-reduction oracle (oracle/tokenred.py, and the reduced
stack in oracle/stack.py), CPU only: pure-Python brute force, exact special
cases (identical rows, unchanged reduced rows), the merged positions against
the half-unit layout the plan builder hands both sides, and zero-gate blocks
leaving the whole reduced stack the identity.
"""
import numpy as np

import oracle
from oracle import block as oblock
from oracle import stack as ostack
from oracle import tokenred as otr
from packed_masked_attention_amd import synth
from tests.test_oracle_inout import _py_bf16
from tests.test_oracle_pins import _tiny_block

_WKEYS = ("w_ada", "w_qkv", "w_o", "w_fc1", "w_fc2")


def _plan_case(seed=1):
    lay = synth.layout_from_counts(8, (2, 3, 4), 5, 3, T=1)
    plan = synth.token_reduction_plan(lay)
    rng = np.random.default_rng(seed)
    x = synth.normal_bf16(rng, (lay["L"], 6))
    return lay, plan, x


def test_plan_pairs_adjacent_horizontal_video_rows():
    lay, plan, _ = _plan_case()
    src0, src1 = plan["src0"], plan["src1"]
    covered = np.concatenate([src0, src1[src1 >= 0]])
    assert np.array_equal(np.sort(covered), np.arange(lay["L"]))       # every row exactly once
    pos, tags = lay["pos"], lay["tags"]
    for a, b in zip(src0, src1):
        if b >= 0:
            assert tags[a] == tags[b] == synth.TAG_VIDEO
            assert tuple(pos[a, :2]) == tuple(pos[b, :2]) and pos[a, 2] % 2 == 0
            assert pos[b, 2] == pos[a, 2] + 1
    assert (src1 >= 0).sum() == 2 * 3 * 2                     # (2, 3, 4) grid -> 12 pairs
    # the plan's half-unit positions are the oracle's mean positions
    got = plan["layout"]["pos"].astype(np.float64) * np.asarray(plan["pos_scale"])
    assert np.array_equal(got, otr.merged_positions(pos, src0, src1))


def test_merge_brute_force_and_identical_rows():
    lay, plan, x = _plan_case(2)
    got = oracle.bf16_to_f64(otr.merge(x, plan["src0"], plan["src1"]))
    xv = oracle.bf16_to_f64(x)
    for i, (a, b) in enumerate(zip(plan["src0"], plan["src1"])):
        for c in range(x.shape[1]):
            want = xv[a, c] if b < 0 else _py_bf16((float(xv[a, c]) + float(xv[b, c])) / 2.0)
            assert got[i, c] == want
    twin = x.copy()
    twin[plan["src1"][plan["src1"] >= 0]] = twin[plan["src0"][plan["src1"] >= 0]]
    assert np.array_equal(otr.merge(twin, plan["src0"], plan["src1"]), twin[plan["src0"]])


def test_unmerge_brute_force_and_unchanged_rows():
    lay, plan, x = _plan_case(3)
    rng = np.random.default_rng(4)
    xr0 = otr.merge(x, plan["src0"], plan["src1"])
    assert np.array_equal(otr.unmerge(x, xr0, xr0, plan["src0"], plan["src1"]), x)
    xr1 = synth.normal_bf16(rng, xr0.shape)
    got = oracle.bf16_to_f64(otr.unmerge(x, xr0, xr1, plan["src0"], plan["src1"]))
    xv, a0, a1 = (oracle.bf16_to_f64(t) for t in (x, xr0, xr1))
    for i, (a, b) in enumerate(zip(plan["src0"], plan["src1"])):
        for r in (a, b):
            if r < 0:
                continue
            for c in range(x.shape[1]):
                want = _py_bf16(float(xv[r, c]) + (float(a1[i, c]) - float(a0[i, c])))
                assert got[r, c] == want


def test_reduced_stack_with_zero_gates_is_identity():
    inps = [_tiny_block(seed=70 + i, L=96, pad=0) for i in range(3)]
    base = inps[0]
    lay = synth.layout_from_counts(16, (2, 4, 8), 16, 0, T=base["layout"]["T"])
    rng = np.random.default_rng(5)
    x = synth.normal_bf16(rng, (lay["L"], base["hidden"]))
    blocks = []
    hid = base["hidden"]
    for i in inps:
        wa = i["w_ada"].copy().reshape(3, 6, hid, -1)
        wa[:, oblock.GATE_A] = 0
        wa[:, oblock.GATE_F] = 0
        blocks.append({"w_ada": wa.reshape(3, 6 * hid, -1), **{k: i[k] for k in _WKEYS[1:]}})
    plan = synth.token_reduction_plan(lay)
    dims = {"L": lay["L"], "hidden": hid, "heads": base["heads"], "head_dim": 128, "ffn": base["ffn"]}
    got = ostack.reduced_stack_forward(x, base["temb"], blocks, lay, plan, 1, 2, dims)
    assert np.array_equal(got, x)


def _reduced_case(seed0=80):
    """Three weight sets (non-zero gates) on a small video-heavy layout."""
    inps = [_tiny_block(seed=seed0 + i, L=96, pad=0) for i in range(3)]
    base = inps[0]
    lay = synth.layout_from_counts(16, (2, 4, 8), 16, 0, T=base["layout"]["T"])
    rng = np.random.default_rng(seed0)
    x = synth.normal_bf16(rng, (lay["L"], base["hidden"]))
    blocks = [{k: i[k] for k in _WKEYS} for i in inps]
    dims = {"L": lay["L"], "hidden": base["hidden"], "heads": base["heads"], "head_dim": 128,
            "ffn": base["ffn"]}
    return lay, x, base["temb"], blocks, dims


def test_reduced_stack_with_empty_reduced_range_is_the_plain_stack():
    # merge directly followed by restore: the bypass comes back unchanged
    # (x + (y - y) is exact), so every block runs at full resolution in order
    lay, x, temb, blocks, dims = _reduced_case(80)
    plan = synth.token_reduction_plan(lay)
    assert (plan["src1"] >= 0).any()
    full = ostack.stack_forward(x, temb, blocks, lay, dims)
    for m in (0, 1, 2, 3):
        got = ostack.reduced_stack_forward(x, temb, blocks, lay, plan, m, m, dims)
        assert np.array_equal(got, full), m
    # a non-empty reduced range changes the result (the pin above is not vacuous)
    red = ostack.reduced_stack_forward(x, temb, blocks, lay, plan, 1, 2, dims)
    assert not np.array_equal(red, full)


def test_reduced_stack_without_pairs_is_the_plain_stack():
    # a plan that pairs no row (no video row has the target timestep index):
    # the reduced rows are the full rows, at doubled positions read with
    # scale 1/2 (exactly the same angles), so the reduced segment is the
    # plain stack's middle blocks and the restore hands their result back
    lay, x, temb, blocks, dims = _reduced_case(90)
    plan = synth.token_reduction_plan(lay, target_ts=lay["T"] + 7)
    assert (plan["src1"] < 0).all() and np.array_equal(plan["src0"], np.arange(lay["L"]))
    assert np.array_equal(plan["layout"]["pos"], 2 * lay["pos"])
    full = ostack.stack_forward(x, temb, blocks, lay, dims)
    for m, r in ((0, 3), (1, 2), (1, 3), (0, 1)):
        got = ostack.reduced_stack_forward(x, temb, blocks, lay, plan, m, r, dims)
        assert np.array_equal(got, full), (m, r)
    # an off-by-one in the block ranges would run a block twice or skip one
    assert not np.array_equal(ostack.stack_forward(x, temb, blocks[:2], lay, dims), full)
