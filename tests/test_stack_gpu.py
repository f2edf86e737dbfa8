"""The block stack and the token refiner on the GPU (through the C ABI).

Against the oracle (oracle/stack.py, storage mode with the fused QKV
projection) on small shapes that span several tiles and a ragged tail; the
tolerance is the single block's (tests/test_block_gpu.py) widened for the
number of blocks the error passes through: each block's bf16 storage adds
its rounding flips, and the next block's SwiGLU spreads them.  At the full
shapes the stack is checked bit for bit against the same blocks run one by
one through pma_adaln_table + pma_block_forward, and a HIP graph of the stack
is replayed several times, each replay compared with the eager result.
"""
import numpy as np
import pytest

from oracle import stack as ostack
from packed_masked_attention_amd import synth
from tests.helpers import bf16_to_np, say, to_dev_bf16
from tests.test_block_gpu import _block_close, _small_inputs

pytestmark = pytest.mark.gpu

_WKEYS = ("w_ada", "w_qkv", "w_o", "w_fc1", "w_fc2")


class Weights:
    """Device copies of block weight sets plus their BlockWeights structs."""

    def __init__(self, sets, device="cuda"):
        import torch
        from packed_masked_attention_amd import binding as B
        self.t = []
        self.structs = []
        self.ones = torch.ones(128, dtype=torch.float32, device=device)
        for s in sets:
            d = {k: (to_dev_bf16(s[k], device) if isinstance(s[k], np.ndarray) else s[k])
                 for k in _WKEYS}
            self.t.append(d)
            self.structs.append(B.BlockWeights(*(d[k].data_ptr() for k in _WKEYS),
                                               self.ones.data_ptr(), self.ones.data_ptr()))


def _dims(inp):
    return {k: inp[k] for k in ("L", "hidden", "heads", "head_dim", "ffn")}


def _small_stack(n_blocks, seed=50, **kw):
    base = _small_inputs(seed=seed, **kw)
    sets = [{k: base[k] for k in _WKEYS}]
    for i in range(1, n_blocks):
        other = synth.make_block_inputs(base["L"], base["hidden"], base["heads"], 128, base["ffn"],
                                        base["temb_dim"], T=base["layout"]["T"], seed=seed + 100 * i,
                                        layout=base["layout"], weight_std=0.05)
        sets.append({k: other[k] for k in _WKEYS})
    return base, sets


@pytest.mark.parametrize("n_blocks", [1, 2, 3])
def test_stack_matches_oracle(n_blocks):
    import torch
    from packed_masked_attention_amd import binding as B
    base, sets = _small_stack(n_blocks)
    L, hid, H, ffn, E = base["L"], base["hidden"], base["heads"], base["ffn"], base["temb_dim"]
    say(f"stack of {n_blocks}: L={L} hidden={hid} H={H} ffn={ffn} E={E} T={base['layout']['T']}")
    p = B.block_params(hid, ffn, E, H)
    dl = B.pma_layout_build(base["layout"])
    w = Weights(sets)
    x = to_dev_bf16(base["x"])
    temb = to_dev_bf16(base["temb"])
    out = torch.full_like(x, float("nan"))
    B.pma_stack_forward(p, dl, w.structs, temb, x, out)
    torch.cuda.synchronize()
    got = bf16_to_np(out)
    ref_bits = ostack.stack_forward(base["x"], base["temb"], sets, base["layout"], _dims(base))
    import oracle
    ref = oracle.bf16_to_f64(ref_bits)
    _block_close(got, ref, f"stack x{n_blocks}", mean_rel=2e-3 * n_blocks, max_rel=6e-2 * n_blocks)


def test_text_refiner_matches_oracle():
    import torch
    import oracle
    from packed_masked_attention_amd import binding as B
    rng = np.random.default_rng(60)
    n, hid, H, ffn, E, T, text_dim = 200, 256, 2, 512, 64, 2, 320
    tags = np.full(n, synth.TAG_TEXT, np.int32)
    pos = np.zeros((n, 3), np.int32)
    pos[:, 0] = np.arange(n)
    ts = rng.integers(0, T, n).astype(np.int32)
    lay = synth.layout_from_tags(tags, pos, ts, T)
    sets, temb = [], None
    for i in range(2):
        inp = synth.make_block_inputs(n, hid, H, 128, ffn, E, T=T, seed=61 + i, layout=lay,
                                      weight_std=0.05)
        sets.append({k: inp[k] for k in _WKEYS})
        temb = inp["temb"] if temb is None else temb
    text = synth.normal_bf16(rng, (n, text_dim))
    w_text = synth.normal_bf16(rng, (hid, text_dim), text_dim ** -0.5)
    say(f"refiner: n={n} hidden={hid} text_dim={text_dim} blocks=2")
    p = B.block_params(hid, ffn, E, H)
    dl = B.pma_layout_build(lay)
    w = Weights(sets)
    out = torch.full((n, hid), float("nan"), dtype=torch.bfloat16, device="cuda")
    dims = {"L": n, "hidden": hid, "heads": H, "head_dim": 128, "ffn": ffn}
    for nb in (0, 2):
        B.pma_text_refiner(p, dl, w.structs[:nb], to_dev_bf16(temb), to_dev_bf16(text), text_dim,
                           text_dim, to_dev_bf16(w_text), 1e-5, out)
        torch.cuda.synchronize()
        got = bf16_to_np(out)
        ref = oracle.bf16_to_f64(ostack.text_refiner(text, w_text, temb, sets[:nb], lay, dims,
                                                     final_eps=1e-5))
        if nb == 0:
            # projection + norm only: one GEMM rounding and one norm rounding apart
            err = np.abs(got - ref)
            assert err.max() <= 2.0 ** -6 * np.abs(ref).max(), err.max()
        else:
            _block_close(got, ref, "refiner x2", mean_rel=4e-3, max_rel=1.2e-1)


def test_stack_full_size_equals_blocks_one_by_one_and_graph_replays():
    """Three blocks at the block workload's full shapes (L=8192, hidden 5376,
    56 heads, ffn 14336): the stack's output is bit-identical to the blocks
    run one at a time, and every replay of a HIP graph of the stack equals
    the eager result."""
    import torch
    from packed_masked_attention_amd import binding as B
    wl = synth.workload("block_L8192")
    lay = synth.make_layout(wl)
    L, hid, H, ffn, E = wl.L, wl.hidden, wl.H, wl.ffn, wl.temb_dim
    T = lay["T"]
    say(f"stack x3 full size L={L}")
    g = torch.Generator(device="cuda").manual_seed(70)
    rnd = lambda *shape, std=0.02: (torch.randn(*shape, generator=g, device="cuda") * std).to(
        torch.bfloat16)
    sets = [{"w_ada": rnd(3, 6 * hid, E), "w_qkv": rnd(3 * H * 128, hid), "w_o": rnd(hid, H * 128),
             "w_fc1": rnd(2 * ffn, hid), "w_fc2": rnd(hid, ffn)} for _ in range(3)]
    w = Weights(sets)
    x = rnd(L, hid, std=1.0)
    temb = rnd(T, E, std=1.0)
    p = B.block_params(hid, ffn, E, H)
    dl = B.pma_layout_build(lay)
    out = torch.empty_like(x)
    ws = torch.empty(B.pma_stack_workspace_size(p, L, T), dtype=torch.uint8, device="cuda")
    B.pma_stack_forward(p, dl, w.structs, temb, x, out, ws)
    # the same blocks one by one
    table = torch.empty(3, T, 6, hid, dtype=torch.float32, device="cuda")
    bws = torch.empty(B.pma_block_workspace_size(p, L), dtype=torch.uint8, device="cuda")
    cur = x
    for i in range(3):
        nxt = torch.empty_like(x)
        B.pma_adaln_table(p, T, temb, sets[i]["w_ada"], table)
        B.pma_block_forward(p, dl, w.structs[i], table, cur, nxt, bws)
        cur = nxt
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), cur.view(torch.int16))
    assert torch.isfinite(out.float()).all()
    # a graph of the stack, replayed with eager work and synchronisations between
    gout = torch.empty_like(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.pma_stack_forward(p, dl, w.structs, temb, x, gout, ws, stream=s)   # warm-up on s
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.pma_stack_forward(p, dl, w.structs, temb, x, gout, ws)
    for rep in range(3):
        gout.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gout.view(torch.int16), out.view(torch.int16)), f"replay {rep}"
        # eager work between replays
        B.pma_stack_forward(p, dl, w.structs[:1], temb, x, cur, ws)
        torch.cuda.synchronize()
