"""The attention path on the GPU (through the C ABI) vs the CPU oracle."""
import numpy as np
import pytest

import oracle
from packed_masked_attention_amd import synth
from tests.helpers import (Q_OPERAND_SCALE, AttentionRun, assert_close, bf16_to_np,
                           sample_rows, say)

pytestmark = pytest.mark.gpu


def _random_inputs(seed, L, H, pad_frac, scattered=True, scale=1.0):
    rng = np.random.default_rng(seed)
    lay = synth.random_layout(rng, L, pad_frac=pad_frac, scattered=scattered, max_pos=300)
    q, k, v = (synth.normal_bf16(rng, (L, H, 128), scale) for _ in range(3))
    return {"q": q, "k": k, "v": v, "layout": lay, "H": H, "D": 128}


# ------------------------------------------------------------ norm + RoPE

def _within_rounding(got, ref, name):
    bound = np.abs(ref) * 2.0 ** -8 * (1 + 2.0 ** -6) + 2.0 ** -20
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} values beyond one rounding; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r}")


@pytest.mark.parametrize("case", ["tiny", "random", "random_F8"])
def test_qk_norm_rope_matches_oracle(case):
    """F = 16 (the model's rope_freq_dim) and F = 8, where the rotated channels
    end at 48 and a channel's RoPE partner sits in the neighbouring lane."""
    F = 8 if case == "random_F8" else 16
    if case == "tiny":
        inp = synth.make_attention_inputs(synth.workload("tiny_L256"))
        w = None
    else:
        inp = _random_inputs(5 if F == 16 else 7, 777, 3, 0.1)
        w = np.random.default_rng(6).uniform(0.5, 2.0, 128)
    say(f"qk_norm_rope {case}")
    r = AttentionRun(inp, wq=w, wk=w, F=F)
    r.prep()
    L, H = r.L, r.H
    lay = inp["layout"]
    wv = 1.0 if w is None else w.astype(np.float32).astype(np.float64)
    for name, dev, src in (("Q", r.qh, inp["q"]), ("K", r.kh, inp["k"])):
        # the stored Q' carries the logit factor
        c = Q_OPERAND_SCALE if name == "Q" else 1.0
        got = bf16_to_np(dev)                       # [H, Lp, D]
        ref = oracle.qk_norm_rope(src, H, 128, wv, lay["pos"], F=F) * c   # [L, H, D]
        if w is None:   # unit weights: unit-variance outputs, the absolute bound applies
            assert_close(got[:, :L].transpose(1, 0, 2) / c, ref / c, f"{name}' (tol)")
        # within one bf16 rounding (half an ulp, <= |x| 2^-8) of the fp64 value,
        # plus fp32 slack for cancellation in the rotation
        g = got[:, :L].transpose(1, 0, 2)
        _within_rounding(g, ref, name)
        # unrotated channels 6F..127 are the rounded RMSNorm
        nrm = oracle.qk_norm_rope(src, H, 128, wv, np.zeros((L, 3), np.int32), F=F) * c
        _within_rounding(g[..., 6 * F:], nrm[..., 6 * F:], name + " passthrough")
        assert np.all(got[:, L:] == 0)
    vt = bf16_to_np(r.vt)                           # [H, D, Lp]
    v = oracle.bf16_to_f64(inp["v"])                # [L, H, D]
    assert np.array_equal(vt[:, :, :L], v.transpose(1, 2, 0))
    assert np.all(vt[:, :, L:] == 0)


# -------------------------------------------------------------- attention

def _oracle_o(inp, rows=None, w=1.0, store_qk_bf16=False):
    lay = inp["layout"]
    return oracle.attention_path(inp["q"], inp["k"], inp["v"], lay, inp["H"], rows=rows, wq=w, wk=w,
                                 store_qk_bf16=store_qk_bf16)


@pytest.mark.parametrize("case", [
    ("tiny_L256", None),
    ("random_L1000_scattered", (11, 1000, 4, 0.2, True)),
    ("random_L777_tail", (12, 777, 3, 0.1, False)),
    ("random_L64_allpad", (13, 64, 2, 1.0, True)),
    ("random_L1", (14, 1, 2, 0.0, True)),
    ("random_L2500_nopad", (15, 2500, 2, 0.0, True)),
])
def test_attention_full_parity(case):
    name, args = case
    inp = synth.make_attention_inputs(synth.workload(name)) if args is None else _random_inputs(*args)
    say(f"attention full parity {name}")
    r = AttentionRun(inp).run()
    ref, lse = _oracle_o(inp)
    assert_close(r.out(), ref, name)
    assert np.allclose(r.lse_np(), lse, atol=2e-2, rtol=0), "lse"


def test_attention_rope_freq_dim_8():
    """The whole path with F = 8 frequencies per axis (48 rotated channels)
    against the oracle with the same F; F must change the result."""
    inp = _random_inputs(16, 1000, 2, 0.1)
    say("attention rope_freq_dim 8")
    r = AttentionRun(inp, F=8).run()
    ref, lse = oracle.attention_path(inp["q"], inp["k"], inp["v"], inp["layout"], 2, F=8)
    assert_close(r.out(), ref, "F=8")
    assert np.allclose(r.lse_np(), lse, atol=2e-2, rtol=0), "lse"
    plain, _ = _oracle_o(inp)
    assert np.abs(plain - ref).max() > 0.05


def test_attention_preview_grid_halved_spatial_rope():
    """The engine page's 256x256 preview: an 8x8 spatial token grid whose h and
    w RoPE coordinates are halved (pos_scale 1, 1/2, 1/2: half-integer
    positions), through the whole attention path, against the oracle with the
    same scale; the scale must change the result."""
    rng = np.random.default_rng(40)
    lay = synth.layout_from_counts(64, (9, 8, 8), 32, 40, T=1)
    L, H = lay["L"], 4
    q, k, v = (synth.normal_bf16(rng, (L, H, 128)) for _ in range(3))
    inp = {"q": q, "k": k, "v": v, "layout": lay, "H": H, "D": 128}
    sc = (1.0, 0.5, 0.5)
    say(f"attention preview grid L={L} pos_scale={sc}")
    r = AttentionRun(inp, pos_scale=sc).run()
    ref, lse = oracle.attention_path(q, k, v, lay, H, pos_scale=sc)
    assert_close(r.out(), ref, "preview halved")
    assert np.allclose(r.lse_np(), lse, atol=2e-2, rtol=0), "lse"
    plain, _ = oracle.attention_path(q, k, v, lay, H)
    assert np.abs(plain - ref).max() > 0.05   # halving is visible in the output


@pytest.mark.parametrize("name", ["nopad_L4096", "masked_L16384", "long_L32768"])
def test_attention_workload_sampled_rows(name):
    wl = synth.workload(name)
    inp = synth.make_attention_inputs(wl)
    rows = sample_rows(inp["layout"], 160, seed=wl.seed)
    if name == "long_L32768":
        rows = rows[np.random.default_rng(0).permutation(rows.size)[:240]]
        rows.sort()
    say(f"attention sampled parity {name}: {rows.size} rows")
    r = AttentionRun(inp).run()
    got = r.out()[rows]
    ref, lse = _oracle_o(inp, rows=rows)
    st = assert_close(got, ref, name)
    assert np.allclose(r.lse_np()[rows], lse, atol=2e-2, rtol=0)
    say(f"  {name} sampled rows ok: {st}")


def test_attention_sharpened_logits():
    """QK-norm weights 4 scale the logits by 16 (std ~16), so the online max
    changes often and the softmax is peaked.  At that scale one bf16 rounding
    of the stored Q' and K' moves a logit by ~0.1, so the oracle stores Q' and
    K' in bf16 exactly as the GPU path does.  Residual differences: where the
    fp64 and the fp32 value of a Q'/K' element round to neighbouring bf16
    values, a logit moves by up to 16 * 2^-8 * |k_c| ~ 0.06 and a peaked row
    follows it; bf16 P adds 2^-9 relative per weight.  Bound: max 6e-2, mean
    and relative as for unit logits."""
    inp = _random_inputs(21, 1500, 2, 0.1)
    w = np.full(128, 4.0)
    say("attention sharpened logits (QK-norm weights 4)")
    r = AttentionRun(inp, wq=w, wk=w).run()
    ref, _ = _oracle_o(inp, w=4.0, store_qk_bf16=True)
    assert_close(r.out(), ref, "sharpened", max_abs=6e-2)


@pytest.mark.parametrize("case", [("L3000_static", 3000, False), ("L12400_queue_split", 12400, True)])
def test_attention_rising_logits_move_the_reference(case):
    """Keys turn towards a fixed direction u along the sequence, so the logits
    of rows aligned with u rise tile by tile: their softmax reference has to
    move after earlier tiles were accumulated (O and the row sum rescaled
    mid-sequence), at different tiles for different rows of one wave, while
    rows orthogonal to u never move it.  u lives in channels 96..127, which
    RoPE leaves unrotated, so the rise does not depend on positions.  The
    premise (a rise of more than 8 in log2 units past the first 64 keys of the
    row's document) is checked on the oracle's Q', K'; the output against the
    oracle on sampled rows (Q', K' stored in bf16 as the GPU path does), with
    one item per workgroup and with the work queue and its key-range split."""
    name, L, split = case
    rng = np.random.default_rng(70)
    H = 2
    lay = synth.random_layout(rng, L, pad_frac=0.05, scattered=False, max_pos=300)
    u = np.zeros(128)
    u[96:] = 1.0 / np.sqrt(32.0)
    a = rng.uniform(0.0, 4.0, size=(L, H, 1))            # a row's alignment with u
    b = 8.0 * (np.arange(L) / L)[:, None, None]          # keys turn towards u
    big = np.sqrt(128.0) * u
    q = synth.f32_to_bf16_bits((rng.standard_normal((L, H, 128)) + a * big).astype(np.float32))
    k = synth.f32_to_bf16_bits((rng.standard_normal((L, H, 128)) + b * big).astype(np.float32))
    v = synth.normal_bf16(rng, (L, H, 128))
    inp = {"q": q, "k": k, "v": v, "layout": lay, "H": H, "D": 128}
    rows = sample_rows(lay, 160, seed=70)
    qn = oracle.qk_norm_rope(q[rows], H, 128, 1.0, lay["pos"][rows])
    kn = oracle.qk_norm_rope(k, H, 128, 1.0, lay["pos"])
    pad = lay["tags"] == -1
    c2 = np.log2(np.e) / np.sqrt(128.0)
    rise = []
    for i, r in enumerate(rows):
        keys = np.flatnonzero(pad == pad[r])
        for h in range(H):
            sc = (kn[keys, h] @ qn[i, h]) * c2
            rise.append(sc.max() - sc[:64].max())
    rise = np.array(rise)
    say(f"attention rising logits {name}: {np.mean(rise > 8):.2f} of sampled (row, head) rise > 8")
    assert np.mean(rise > 8) > 0.15 and np.mean(rise < 8) > 0.05
    r = AttentionRun(inp, split=split).run()
    ref, lse = _oracle_o(inp, rows=rows, store_qk_bf16=True)
    assert_close(r.out()[rows], ref, name)
    assert np.allclose(r.lse_np()[rows], lse, atol=2e-2, rtol=0), "lse"


def test_attention_structural():
    import torch
    inp = _random_inputs(31, 900, 2, 0.15)
    L, H = 900, 2
    say("attention structural: V=1, determinism, document isolation")
    ones = dict(inp)
    ones["v"] = np.full_like(inp["v"], 0x3F80)      # bf16 1.0
    r = AttentionRun(ones).run()
    assert np.abs(r.out() - 1.0).max() <= 2 ** -7
    r = AttentionRun(inp).run()
    o1 = r.o.clone()
    r.flash()
    torch.cuda.synchronize()
    assert torch.equal(r.o.view(torch.int16), o1.view(torch.int16)), "not deterministic"
    # changing the padding rows' K/V leaves every real row bit-identical, and back
    pad = inp["layout"]["tags"] == -1
    for which in (pad, ~pad):
        mod = dict(inp)
        rng = np.random.default_rng(32)
        k2, v2 = inp["k"].copy(), inp["v"].copy()
        k2[which] = synth.normal_bf16(rng, k2[which].shape, 3.0)
        v2[which] = synth.normal_bf16(rng, v2[which].shape, 3.0)
        mod["k"], mod["v"] = k2, v2
        r2 = AttentionRun(mod).run()
        keep = ~which
        assert np.array_equal(r2.out()[keep], bf16_to_np(o1).reshape(L, H, 128)[keep])


def test_attention_timestep_indices_have_no_effect():
    inp = _random_inputs(41, 600, 2, 0.1)
    say("attention: timestep indices do not change O")
    a = AttentionRun(inp).run().out()
    lay = dict(inp["layout"])
    lay["T"] = 5
    lay["ts_idx"] = np.random.default_rng(42).integers(0, 5, 600).astype(np.int32)
    lay["ts_idx"][lay["tags"] == -1] = 0
    b = AttentionRun(dict(inp, layout=lay)).run().out()
    assert np.array_equal(a, b)


def test_attention_one_call_entry_point():
    import torch
    from packed_masked_attention_amd import binding as B
    inp = _random_inputs(51, 700, 3, 0.1)
    say("attention: pma_attention (prep + flash in one call)")
    r = AttentionRun(inp).run()
    o2 = torch.empty_like(r.o)
    HD = r.H * 128
    B.pma_attention(r.p, r.dl, r.q, HD, r.k, HD, r.v, HD, r.wq, r.wk, o2, HD)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), r.o.view(torch.int16))


def test_attention_call_options():
    """lse = NULL leaves O unchanged; an output row stride wider than H*128
    writes the same rows and leaves the extra columns alone; an explicit
    softmax scale s matches the oracle with QK-norm weights w, w^2 = s*sqrt(128)
    (the logit is (w q_n).(w k_n)/sqrt(128) = s q_n.k_n either way)."""
    import torch
    from packed_masked_attention_amd import binding as B
    inp = _random_inputs(55, 1100, 2, 0.1)
    L, H = 1100, 2
    HD = H * 128
    say("attention call options: lse NULL, wide output stride, explicit scale")
    r = AttentionRun(inp).run()
    o_nolse = torch.full_like(r.o, float("nan"))
    B.pma_flash_attention(r.p, r.dl, r.qh, r.kh, r.vt, o_nolse, HD, None, workspace=r.ws)
    wide = torch.full((L, HD + 72), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.pma_flash_attention(r.p, r.dl, r.qh, r.kh, r.vt, wide, HD + 72, None, workspace=r.ws)
    torch.cuda.synchronize()
    assert torch.equal(o_nolse.view(torch.int16), r.o.view(torch.int16)), "lse NULL"
    assert torch.equal(wide[:, :HD].contiguous().view(torch.int16), r.o.view(torch.int16)), "stride"
    assert torch.isnan(wide[:, HD:].float()).all(), "columns past H*128 written"
    sc = 0.05
    rs = AttentionRun(inp)
    rs.p = B.attn_params(H, scale=sc)
    rs.run()
    w = float(np.sqrt(sc * np.sqrt(128.0)))
    ref, lse = _oracle_o(inp, w=w)
    assert_close(rs.out(), ref, "explicit scale")
    assert np.allclose(rs.lse_np(), lse, atol=2e-2, rtol=0), "lse"
    assert np.abs(ref - r.out()).max() > 0.05   # the scale changes the result


@pytest.mark.parametrize("case", [
    ("L12300_tail_pad", (61, 12300, 2, 12 / 12300, False)),
    ("L13000_scattered", (62, 13000, 3, 0.15, True)),
    ("L9000_two_parts", (63, 9000, 2, 0.1, True)),
])
def test_attention_key_range_split(case):
    """The work queue with the key-range split (flash workspace given) against
    one item per workgroup (no workspace) and the oracle on sampled rows.
    From 8192 keys the last items of each XCD's share run in 2 parts, from
    12288 keys in 4; with 2 or 3 heads every item is among them.  At L=12300
    the last q-tile holds only the 12 padding rows, whose one k-tile leaves
    three parts empty."""
    import torch
    name, args = case
    inp = _random_inputs(*args)
    lay = inp["layout"]
    rows = sample_rows(lay, 120, seed=args[0], tile=256)
    say(f"attention key-range split {name}: {rows.size} sampled rows")
    split = AttentionRun(inp).run()
    whole = AttentionRun(inp, split=False).run()
    ref, lse = _oracle_o(inp, rows=rows)
    assert_close(split.out()[rows], ref, name + " split")
    assert_close(whole.out()[rows], ref, name + " whole")
    assert np.allclose(split.lse_np()[rows], lse, atol=2e-2, rtol=0), "lse split"
    # the two round p to bf16 against different reference maxima (each part
    # keeps its own) and sum in another order: per element within 2^-7 of
    # the |v| ~ 1 scale plus the output rounding, far below on average
    a, b = split.out(), whole.out()
    assert np.all(np.isfinite(a)), name
    d = np.abs(a - b)
    say(f"  split vs whole: max {d.max():.2e} mean {d.mean():.2e}")
    assert np.all(d <= 2.0 ** -7 + np.abs(b) * 2.0 ** -7), name
    assert d.mean() <= 2.5e-4, name
    assert np.abs(split.lse_np() - whole.lse_np()).max() < 1e-3
    # repeatable: the queue hands out units in a different order each run,
    # but every unit computes the same thing
    o1 = split.o.clone()
    split.flash()
    torch.cuda.synchronize()
    assert torch.equal(split.o.view(torch.int16), o1.view(torch.int16))


def test_attention_work_queue_graph_replays():
    """The work-queue path (counters cleared by a kernel, parts merged) inside
    a HIP graph: every replay, with eager work and synchronisations between,
    equals the eager call bit for bit."""
    import torch
    inp = _random_inputs(63, 12500, 2, 0.05, False)
    say("attention work queue in a HIP graph, L=12500 H=2")
    r = AttentionRun(inp).run()
    ref = r.o.clone()
    other = AttentionRun(_random_inputs(64, 12400, 2, 0.1, True))
    other.prep()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        r.flash()                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        r.flash()
    for rep in range(3):
        r.o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(r.o.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        other.flash()                   # eager work on another workspace between replays
        torch.cuda.synchronize()


# ------------------------------------------- positions over the whole range

_PMAX = (1 << 24) - 1      # the layout accepts |p| < 2^24


def _big_position_inputs(seed, L, H, pad_frac=0.1):
    """Random layout whose positions span the accepted range: uniform over
    [-(2^24 - 1), 2^24 - 1] plus rows at both extremes and near zero."""
    rng = np.random.default_rng(seed)
    lay = synth.random_layout(rng, L, pad_frac=pad_frac, scattered=True, max_pos=2)
    pos = rng.integers(-_PMAX, _PMAX + 1, size=(L, 3)).astype(np.int32)
    pos[:6] = [[_PMAX, _PMAX, _PMAX], [-_PMAX, -_PMAX, -_PMAX], [_PMAX, -_PMAX, 0],
               [0, 1, -1], [_PMAX - 1, 3, -_PMAX + 1], [1 << 23, -(1 << 23), 12345]]
    lay = synth.layout_from_tags(lay["tags"], pos, lay["ts_idx"], lay["T"])
    q, k, v = (synth.normal_bf16(rng, (L, H, 128)) for _ in range(3))
    return {"q": q, "k": k, "v": v, "layout": lay, "H": H, "D": 128}


def test_qk_norm_rope_large_positions():
    """Angles up to (2^24 - 1) rad: the prep kernel's fp64 angles and cos/sin
    keep every Q', K' element within one bf16 rounding of the fp64 oracle."""
    inp = _big_position_inputs(70, 650, 3)
    w = np.random.default_rng(71).uniform(0.5, 2.0, 128)
    say("qk_norm_rope at positions up to +-(2^24-1)")
    r = AttentionRun(inp, wq=w, wk=w)
    r.prep()
    lay = inp["layout"]
    wv = w.astype(np.float32).astype(np.float64)
    for name, dev, src in (("Q", r.qh, inp["q"]), ("K", r.kh, inp["k"])):
        c = Q_OPERAND_SCALE if name == "Q" else 1.0
        got = bf16_to_np(dev)[:, :r.L].transpose(1, 0, 2)
        ref = oracle.qk_norm_rope(src, r.H, 128, wv, lay["pos"]) * c
        _within_rounding(got, ref, name + " large positions")


@pytest.mark.parametrize("pad_frac", [0.0, 0.15])
def test_attention_large_positions(pad_frac):
    inp = _big_position_inputs(72 + int(pad_frac * 100), 1100, 3, pad_frac)
    say(f"attention at positions up to +-(2^24-1), padding {pad_frac}")
    r = AttentionRun(inp).run()
    ref, lse = _oracle_o(inp)
    assert_close(r.out(), ref, "large positions")
    assert np.allclose(r.lse_np(), lse, atol=2e-2, rtol=0), "lse"


def _gpu_pair_close(a, b, what):
    """Two GPU results of the same mathematical O (other row order or
    positions, so other tile maps, summation orders and Q'/K' roundings): per
    element within 2^-7 of the |v| ~ 1 scale plus the output rounding, far
    below on average."""
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b)), what
    d = np.abs(a - b)
    say(f"  {what}: max {d.max():.2e} mean {d.mean():.2e}")
    assert np.all(d <= 2.0 ** -7 + np.abs(b) * 2.0 ** -7), what
    assert d.mean() <= 2.5e-4, what


@pytest.mark.parametrize("L", [1500, 12400])
def test_attention_permutation_equivariance(L):
    """Permuting the rows together with their tags, positions and timestep
    indices permutes O (the mask is defined by tag, not by position in the
    sequence).  At 12400 rows the work queue and key-range split run."""
    H = 2
    inp = _random_inputs(80 + L % 7, L, H, 0.12, scattered=False)
    lay = inp["layout"]
    perm = np.random.default_rng(81).permutation(L)
    lay_p = synth.layout_from_tags(lay["tags"][perm], lay["pos"][perm], lay["ts_idx"][perm],
                                   lay["T"])
    inp_p = {"q": inp["q"][perm], "k": inp["k"][perm], "v": inp["v"][perm], "layout": lay_p,
             "H": H, "D": 128}
    say(f"attention permutation equivariance L={L}")
    a = AttentionRun(inp).run()
    b = AttentionRun(inp_p).run()
    rows = sample_rows(lay, 150, seed=82, tile=256)
    ref, _ = _oracle_o(inp, rows=rows)
    assert_close(a.out()[rows], ref, "original order")
    inv = np.argsort(perm)
    assert_close(b.out()[inv][rows], ref, "permuted, mapped back")
    _gpu_pair_close(b.out()[inv], a.out(), "permuted vs original")
    assert np.abs(b.lse_np()[inv] - a.lse_np()).max() < 1e-3


@pytest.mark.parametrize("delta", [(1000, -7, 33), (1 << 23, -(1 << 22), 777777)])
def test_attention_global_position_shift(delta):
    """Shifting every position by one offset leaves O unchanged (the rotation
    makes q'.k' depend only on the offset between positions); Q' and K'
    themselves change, so the GPU results agree within rounding, not bit for
    bit."""
    H = 3
    inp = _random_inputs(90, 1300, H, 0.1)
    lay = inp["layout"]
    pos = lay["pos"].astype(np.int64) + np.asarray(delta, np.int64)
    assert np.abs(pos).max() < (1 << 24)
    lay_s = synth.layout_from_tags(lay["tags"], pos.astype(np.int32), lay["ts_idx"], lay["T"])
    say(f"attention global position shift {delta}")
    a = AttentionRun(inp).run()
    b = AttentionRun(dict(inp, layout=lay_s)).run()
    ref, _ = _oracle_o(inp)
    assert_close(a.out(), ref, "unshifted")
    assert_close(b.out(), ref, "shifted vs unshifted oracle")
    _gpu_pair_close(b.out(), a.out(), "shifted vs unshifted")
    # the Q' of a shifted row does change: the test is not vacuous
    assert not np.array_equal(bf16_to_np(a.qh), bf16_to_np(b.qh))


@pytest.mark.parametrize("pad", [1016, 1004])
def test_attention_maximum_length(pad):
    """The longest sequence the kernel's LDS tile list holds: 6908 k-tiles of
    64 keys (442,112 rows; with pad=1004 the last k-tile is ragged, 52 rows).
    The pages' packed structure at that length: 4096 text rows, a (27, 80, 200)
    video grid, 5000 audio rows and the padding document at the tail; one head
    keeps the run short.  Sampled rows against the fp64 oracle: rows of the
    padding document, the first and last k-tile, the document boundaries and
    random rows."""
    H = 1
    lay = synth.layout_from_counts(4096, (27, 80, 200), 5000, pad)
    L = lay["L"]
    assert -(-L // 64) == 6908
    rng = np.random.default_rng(95 + pad)
    q, k, v = (synth.normal_bf16(rng, (L, H, 128)) for _ in range(3))
    inp = {"q": q, "k": k, "v": v, "layout": lay, "H": H, "D": 128}
    tags = lay["tags"]
    first_pad = int(np.flatnonzero(tags == -1)[0])
    rows = {0, 1, 63, 64, 4095, 4096, first_pad - 1, first_pad, L - 64, L - 2, L - 1}
    rows.update(range(L - 70, L - 60))
    rows.update(rng.integers(first_pad, L, 12).tolist())
    rows.update(rng.integers(0, first_pad, 40).tolist())
    rows = np.array(sorted(rows), dtype=np.int32)
    say(f"attention at the maximum length L={L}: {rows.size} sampled rows")
    r = AttentionRun(inp).run()
    got = r.out()
    assert np.all(np.isfinite(got)), "every row written"
    ref, lse = _oracle_o(inp, rows=rows)
    st = assert_close(got[rows], ref, f"L={L}")
    assert np.allclose(r.lse_np()[rows], lse, atol=2e-2, rtol=0), "lse"
    say(f"  L={L} sampled rows ok: {st}")
