"""Pins of the CPU oracle to things other than itself (CPU only).

Every oracle function is checked against a library routine computing the same
definition (torch fp64 SDPA / layer_norm / rms_norm / silu), a closed form, an
invariant the pages' definitions imply, or hand-derived values stored under
tests/golden/ with their derivation.  Sizes are tiny so the file runs in
seconds.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
from oracle import block as oblock
from packed_masked_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ----------------------------------------------------------------- bf16 ----

def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-30, 30, 20000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert oracle.bf16_round(np.array([1 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert oracle.bf16_round(np.array([1 + 3 * 2.0 ** -8]))[0] == 0x3F82
    # just above a tie rounds up
    assert oracle.bf16_round(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 0x3F81
    assert oracle.bf16_to_f64(np.array([0x3F81], np.uint16))[0] == 1 + 2.0 ** -7


# ------------------------------------------------------------ inv_freq ----

def test_inv_freq_closed_form():
    f = oracle.inv_freq(16, 10000.0)
    assert f[0] == 1.0
    assert math.isclose(f[15], 10.0 ** -3.75, rel_tol=1e-15)
    ratios = f[1:] / f[:-1]
    assert np.allclose(ratios, 10000.0 ** (-1 / 16), rtol=1e-14, atol=0)


# ------------------------------------------------------ QK-RMSNorm/RoPE ----

def _rand_qk(L=40, H=3, D=128, seed=1, scale=1.0):
    rng = np.random.default_rng(seed)
    return _bits(rng.standard_normal((L, H, D)) * scale)


def test_rmsnorm_matches_torch_at_zero_position():
    x = _rand_qk()
    L, H, D = x.shape
    w = np.random.default_rng(2).uniform(0.5, 2.0, D)
    y = oracle.qk_norm_rope(x, H, D, w, np.zeros((L, 3), np.int32))
    ref = Fn.rms_norm(torch.from_numpy(oracle.bf16_to_f64(x)), (D,),
                      torch.from_numpy(w), eps=1e-5).numpy()
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-14)


def test_rmsnorm_constant_vector_closed_form():
    D, c, eps = 128, -0.375, 1e-5
    x = _bits(np.full((1, 1, D), c))
    y = oracle.qk_norm_rope(x, 1, D, 1.0, np.zeros((1, 3), np.int32), eps=eps)
    assert np.allclose(y, math.copysign(1.0, c) / math.sqrt(1 + eps / c ** 2), rtol=1e-15)
    z = oracle.qk_norm_rope(np.zeros((1, 1, D), np.uint16), 1, D, 1.0, np.zeros((1, 3), np.int32))
    assert np.all(z == 0)


def _complex_rope_reference(n, pos, F=16, theta=10000.0):
    """Textbook complex-number RoPE on three sections of 2F channels: channel
    pair (2aF+f, 2aF+f+F) is the complex number re + i*im, multiplied by
    exp(i * pos[a] * theta^(-f/F)); channels >= 6F untouched."""
    out = n.copy()
    for a in range(3):
        base = 2 * a * F
        z = n[..., base:base + F] + 1j * n[..., base + F:base + 2 * F]
        ang = pos[:, a][:, None, None] * (theta ** (-np.arange(F) / F))[None, None, :]
        z = z * np.exp(1j * ang)
        out[..., base:base + F] = z.real
        out[..., base + F:base + 2 * F] = z.imag
    return out


def _rotate_half_1d(x, t, dim=32, theta=10000.0):
    """HF-style 1-D RoPE of width dim: x*cos + rotate_half(x)*sin."""
    half = dim // 2
    freqs = t[:, None] * theta ** (-np.arange(half) / half)[None, :]
    emb = np.concatenate([freqs, freqs], axis=-1)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:dim]
    rot = np.concatenate([-x2, x1], axis=-1)
    return x[..., :dim] * np.cos(emb) + rot * np.sin(emb)


def test_rope_matches_complex_rotation():
    x = _rand_qk(L=50, H=2)
    L, H, D = x.shape
    pos = np.random.default_rng(3).integers(0, 1024, (L, 3)).astype(np.int32)
    n = oracle.qk_norm_rope(x, H, D, 1.0, np.zeros((L, 3), np.int32))
    y = oracle.qk_norm_rope(x, H, D, 1.0, pos)
    assert np.allclose(y, _complex_rope_reference(n, pos), rtol=1e-12, atol=1e-12)


def test_rope_scaled_coordinates():
    """The engine page's 256x256 preview halves the spatial coordinates: with
    scale (1, 1/2, 1/2), doubled spatial positions give exactly the unscaled
    result, and odd ones land halfway (fractional positions), matching the
    complex rotation at those fractional positions."""
    x = _rand_qk(L=40, H=2)
    L, H, D = x.shape
    rng = np.random.default_rng(8)
    pos = rng.integers(0, 300, (L, 3)).astype(np.int32)
    sc = (1.0, 0.5, 0.5)
    doubled = pos.copy()
    doubled[:, 1:] *= 2
    assert np.array_equal(oracle.qk_norm_rope(x, H, D, 1.0, doubled, pos_scale=sc),
                          oracle.qk_norm_rope(x, H, D, 1.0, pos))
    odd = pos.copy()
    odd[:, 1:] = 2 * odd[:, 1:] + 1
    n = oracle.qk_norm_rope(x, H, D, 1.0, np.zeros((L, 3), np.int32))
    y = oracle.qk_norm_rope(x, H, D, 1.0, odd, pos_scale=sc)
    frac = pos.astype(np.float64)
    frac[:, 1:] += 0.5
    assert np.allclose(y, _complex_rope_reference(n, frac), rtol=1e-12, atol=1e-12)
    # the temporal axis keeps its integer positions
    assert np.array_equal(oracle.qk_norm_rope(x, H, D, 1.0, odd, pos_scale=sc)[..., :32],
                          oracle.qk_norm_rope(x, H, D, 1.0, odd)[..., :32])


def test_rope_temporal_only_is_textbook_1d_rope():
    x = _rand_qk(L=30, H=2)
    L, H, D = x.shape
    t = np.arange(L) * 37 % 1000
    pos = np.stack([t, np.zeros(L), np.zeros(L)], axis=1).astype(np.int32)
    n = oracle.qk_norm_rope(x, H, D, 1.0, np.zeros((L, 3), np.int32))
    y = oracle.qk_norm_rope(x, H, D, 1.0, pos)
    assert np.allclose(y[..., :32], _rotate_half_1d(n, t.astype(np.float64)), atol=1e-12)
    assert np.array_equal(y[..., 32:], n[..., 32:])


def test_rope_invariants_norm_offset_passthrough():
    x = _rand_qk(L=64, H=2)
    L, H, D = x.shape
    rng = np.random.default_rng(4)
    pos = rng.integers(0, 500, (L, 3)).astype(np.int32)
    n = oracle.qk_norm_rope(x, H, D, 1.0, np.zeros((L, 3), np.int32))
    y = oracle.qk_norm_rope(x, H, D, 1.0, pos)
    # (i) every rotated pair keeps its norm, so each head keeps its norm
    for a in range(3):
        for f in range(16):
            c0, c1 = 32 * a + f, 32 * a + f + 16
            assert np.allclose(y[..., c0] ** 2 + y[..., c1] ** 2,
                               n[..., c0] ** 2 + n[..., c1] ** 2, rtol=1e-12)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(n, axis=-1), rtol=1e-13)
    # (ii) channels 96..127 pass through bit for bit
    assert np.array_equal(y[..., 96:], n[..., 96:])
    # (iii) q.k depends only on the (t, h, w) offset: shift every position by delta
    delta = np.array([[17, -5, 9]], np.int32)
    y2 = oracle.qk_norm_rope(x, H, D, 1.0, pos + delta)
    dots = np.einsum("ihc,jhc->hij", y[..., :96], y[..., :96])
    dots2 = np.einsum("ihc,jhc->hij", y2[..., :96], y2[..., :96])
    assert np.allclose(dots, dots2, atol=1e-11)


# --------------------------------------------------------------- layout ----

def _dense_mask(tags):
    pad = np.asarray(tags) == -1
    return pad[:, None] == pad[None, :]


def _brute_tiles(tags, bm, bn):
    m = _dense_mask(tags)
    L = len(tags)
    nqt, nkt = -(-L // bm), -(-L // bn)
    cls = np.zeros((nqt, nkt), np.uint8)
    for i in range(nqt):
        for j in range(nkt):
            blk = m[i * bm:(i + 1) * bm, j * bn:(j + 1) * bn]
            cls[i, j] = 0 if not blk.any() else (2 if blk.all() else 1)
    return cls


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("bm,bn", [(64, 64), (128, 64), (128, 128), (256, 64)])
def test_layout_tiles_match_dense_mask(seed, bm, bn):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 700))
    lay = synth.random_layout(rng, L, pad_frac=[0.0, 0.05, 0.3, 1.0, 0.5, 0.1][seed],
                              scattered=seed % 2 == 0)
    cls, count, lst, order = oracle.layout_tiles(lay["tags"], bm, bn)
    want = _brute_tiles(lay["tags"], bm, bn)
    assert np.array_equal(cls, want)
    for qt in range(cls.shape[0]):
        nz = np.flatnonzero(want[qt])
        assert count[qt] == nz.size
        assert np.array_equal(lst[qt, :nz.size], nz)
        assert np.all(lst[qt, nz.size:] == -1)
    # order: a permutation sorted by (count desc, index asc)
    assert sorted(order.tolist()) == list(range(cls.shape[0]))
    keys = [(-count[q], q) for q in order]
    assert keys == sorted(keys)
    assert oracle.allowed_pairs(lay["tags"]) == int(_dense_mask(lay["tags"]).sum())


def test_layout_golden_tile_counts():
    with open(os.path.join(GOLDEN, "layout_tiles.json")) as fh:
        gold = json.load(fh)
    for case in gold["cases"]:
        lay = synth.make_layout(synth.workload(case["workload"]))
        cls, count, lst, order = oracle.layout_tiles(lay["tags"], case["bm"], case["bn"])
        if "classes" in case:
            assert cls.tolist() == case["classes"]
        if "counts" in case:
            got = {"EMPTY": int((cls == 0).sum()), "PARTIAL": int((cls == 1).sum()),
                   "FULL": int((cls == 2).sum())}
            assert got == case["counts"]
        assert oracle.allowed_pairs(lay["tags"]) == case["allowed_pairs"]
        doc = oracle.layout_doc(lay["tags"])
        assert np.array_equal(doc, (lay["tags"] == -1).astype(np.int32))


def test_layout_status_bits():
    base = synth.layout_from_counts(4, (1, 2, 2), 3, 2, T=2)
    assert oracle.layout_status(base) == (0, -1)

    def mutate(fn):
        lay = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in base.items()}
        fn(lay)
        return oracle.layout_status(lay)

    def bad_tag(l): l["tags"][5] = 7
    assert mutate(bad_tag)[0] & 1 and mutate(bad_tag)[1] == 5

    def bad_ts(l): l["ts_idx"][3] = 2
    assert mutate(bad_ts) == (2, 3)

    def pad_ts_ignored(l): l["ts_idx"][12] = 99    # row 12 is padding
    assert mutate(pad_ts_ignored) == (0, -1)

    def bad_pos(l): l["pos"][9, 2] = 1 << 24
    assert mutate(bad_pos) == (4, 9)

    def oob_index(l): l["video_idx"] = np.array([4, 5, 6, 99], np.int32)
    assert mutate(oob_index)[0] & 8

    def unsorted(l): l["video_idx"] = l["video_idx"][::-1].copy()
    assert mutate(unsorted)[0] == 16

    def wrong_tag(l): l["text_idx"] = np.array([0, 1, 2, 4], np.int32)
    assert mutate(wrong_tag)[0] == 32

    def short(l): l["audio_idx"] = l["audio_idx"][:2].copy()
    assert mutate(short)[0] == 64


# ------------------------------------------------------------ attention ----

def _sdpa_reference(q, k, v, tags):
    """torch fp64 scaled_dot_product_attention with a boolean document mask."""
    m = torch.from_numpy(_dense_mask(tags))
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2)
    vt = torch.from_numpy(v).permute(1, 0, 2)
    o = Fn.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
    s = (qt @ kt.transpose(1, 2)) / math.sqrt(q.shape[-1])
    s = s.masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


@pytest.mark.parametrize("seed", range(5))
def test_attention_matches_torch_sdpa(seed):
    rng = np.random.default_rng(seed)
    L, H, D = int(rng.integers(2, 200)), 2, 128
    lay = synth.random_layout(rng, L, pad_frac=[0.0, 0.1, 0.5, 0.9, 0.2][seed])
    q, k, v = (rng.standard_normal((L, H, D)) * 1.5 for _ in range(3))
    o, lse = oracle.attention(q, k, v, lay["tags"])
    ro, rlse = _sdpa_reference(q, k, v, lay["tags"])
    assert np.allclose(o, ro, rtol=1e-11, atol=1e-12)
    assert np.allclose(lse, rlse, rtol=1e-12, atol=1e-12)
    rows = np.array(sorted(set(rng.integers(0, L, 7).tolist())), np.int32)
    o2, _ = oracle.attention(q, k, v, lay["tags"], rows=rows)
    assert np.array_equal(o2, o[rows])


def test_attention_path_tiny_workload_matches_torch():
    inp = synth.make_attention_inputs(synth.workload("tiny_L256"))
    lay, H = inp["layout"], inp["H"]
    o, _ = oracle.attention_path(inp["q"], inp["k"], inp["v"], lay, H)
    qn = oracle.qk_norm_rope(inp["q"], H, 128, 1.0, lay["pos"])
    kn = oracle.qk_norm_rope(inp["k"], H, 128, 1.0, lay["pos"])
    ro, _ = _sdpa_reference(qn, kn, oracle.bf16_to_f64(inp["v"]), lay["tags"])
    assert np.allclose(o, ro, rtol=1e-11, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(7)
    L, H, D = 96, 2, 128
    lay = synth.random_layout(rng, L, pad_frac=0.25)
    tags = lay["tags"]
    q, k = rng.standard_normal((2, L, H, D))
    # V == 1 -> O == 1
    o, _ = oracle.attention(q, k, np.ones((L, H, D)), tags)
    assert np.allclose(o, 1.0, rtol=0, atol=1e-14)
    # Q == 0 -> uniform weights over the row's document -> document mean of V
    v = rng.standard_normal((L, H, D))
    o, lse = oracle.attention(np.zeros((L, H, D)), k, v, tags)
    pad = tags == -1
    for i in range(L):
        same = pad == pad[i]
        assert np.allclose(o[i], v[same].mean(axis=0), atol=1e-13)
        assert np.allclose(lse[i], math.log(same.sum()), atol=1e-13)
    # V one-hot per key (L <= D): O row = attention probabilities, which sum to 1
    v1 = np.zeros((L, H, D))
    v1[np.arange(L), :, np.arange(L)] = 1.0
    o, _ = oracle.attention(q, k, v1, tags)
    assert np.allclose(o.sum(axis=-1), 1.0, atol=1e-13)
    assert np.all(o[..., :L][:, :, ~pad][pad] == 0)     # padding rows ignore real keys
    assert np.all(o[..., :L][:, :, pad][~pad] == 0)     # real rows ignore padding keys


def test_attention_single_row_document_and_isolation():
    rng = np.random.default_rng(8)
    L, H, D = 40, 1, 128
    tags = np.zeros(L, np.int32)
    tags[17] = -1                       # a one-row padding document
    q, k, v = rng.standard_normal((3, L, H, D))
    o, _ = oracle.attention(q, k, v, tags)
    assert np.array_equal(o[17], v[17])
    # changing the other document's K/V leaves a document's output bit-identical
    k2, v2 = k.copy(), v.copy()
    k2[17] += 5.0
    v2[17] -= 3.0
    o2, _ = oracle.attention(q, k2, v2, tags)
    real = np.arange(L) != 17
    assert np.array_equal(o2[real], o[real])


def test_attention_permutation_equivariance():
    rng = np.random.default_rng(9)
    L, H, D = 80, 2, 128
    lay = synth.random_layout(rng, L, pad_frac=0.2)
    q, k, v = rng.standard_normal((3, L, H, D))
    perm = rng.permutation(L)
    o, _ = oracle.attention(q, k, v, lay["tags"])
    op, _ = oracle.attention(q[perm], k[perm], v[perm], lay["tags"][perm])
    assert np.allclose(op, o[perm], atol=1e-13)


def test_attention_f32_twin_agrees():
    rng = np.random.default_rng(10)
    L, H, D = 150, 2, 128
    lay = synth.random_layout(rng, L, pad_frac=0.1)
    q, k, v = rng.standard_normal((3, L, H, D))
    o64, _ = oracle.attention(q, k, v, lay["tags"])
    o32, _ = oracle.attention(q, k, v, lay["tags"], precision="f32")
    assert np.allclose(o32, o64, atol=2e-5)


# ---------------------------------------------------------------- block ----

def _tiny_block(seed=11, L=96, hidden=64, H=2, D=128, ffn=96, E=48, pad=8, T=2):
    rng = np.random.default_rng(seed)
    tags = rng.integers(0, 3, L).astype(np.int32)
    tags[L - pad:] = -1
    pos = rng.integers(0, 40, (L, 3)).astype(np.int32)
    ts = rng.integers(0, T, L).astype(np.int32)
    lay = synth.layout_from_tags(tags, pos, ts, T)
    return synth.make_block_inputs(L, hidden, H, D, ffn, E, T=T, seed=seed, layout=lay,
                                   weight_std=0.1)


def _torch_block(inp, eps=1e-5):
    """The block composed from torch fp64 functional ops (no storage rounding)."""
    f = lambda b: torch.from_numpy(oracle.bf16_to_f64(b))
    lay = inp["layout"]
    L, hid, H, D, ffn = inp["L"], inp["hidden"], inp["heads"], inp["head_dim"], inp["ffn"]
    HD = H * D
    tags = torch.from_numpy(lay["tags"]).long()
    ts = torch.from_numpy(lay["ts_idx"]).long()
    temb, w_ada = f(inp["temb"]), f(inp["w_ada"])
    mods = torch.stack([Fn.linear(temb, w_ada[g]) for g in range(3)])   # [3, T, 6*hid]
    row = mods[tags.clamp(min=0), ts].reshape(L, 6, hid)
    row[tags < 0] = 0
    sh_a, sc_a, g_a, sh_f, sc_f, g_f = row.unbind(1)
    x = f(inp["x"])
    a = Fn.layer_norm(x, (hid,), eps=eps) * (1 + sc_a) + sh_a
    qkv = Fn.linear(a, f(inp["w_qkv"]))
    q, k, v = qkv.split(HD, dim=-1)

    def norm_rope(t):
        t = Fn.rms_norm(t.reshape(L, H, D), (D,), eps=1e-5)
        out = t.clone()
        pos = torch.from_numpy(lay["pos"]).double()
        inv = 10000.0 ** (-torch.arange(16, dtype=torch.float64) / 16)
        for ax in range(3):
            b0 = 32 * ax
            z = torch.complex(t[..., b0:b0 + 16], t[..., b0 + 16:b0 + 32])
            z = z * torch.polar(torch.ones(L, 1, 16, dtype=torch.float64),
                                pos[:, ax, None, None] * inv)
            out[..., b0:b0 + 16], out[..., b0 + 16:b0 + 32] = z.real, z.imag
        return out.permute(1, 0, 2)

    m = (tags < 0)[:, None] == (tags < 0)[None, :]
    o = Fn.scaled_dot_product_attention(norm_rope(q), norm_rope(k),
                                        v.reshape(L, H, D).permute(1, 0, 2), attn_mask=m)
    o = o.permute(1, 0, 2).reshape(L, HD)
    x1 = x + g_a * Fn.linear(o, f(inp["w_o"]))
    b = Fn.layer_norm(x1, (hid,), eps=eps) * (1 + sc_f) + sh_f
    gu = Fn.linear(b, f(inp["w_fc1"]))
    h = Fn.silu(gu[:, :ffn]) * gu[:, ffn:]
    return (x1 + g_f * Fn.linear(h, f(inp["w_fc2"]))).numpy()


def test_block_matches_torch_composition():
    inp = _tiny_block()
    x2 = oblock.block_forward(inp, store_bf16=False)
    ref = _torch_block(inp)
    assert np.allclose(x2, ref, rtol=1e-10, atol=1e-10)
    rows = np.array([0, 5, 50, 90, 95])
    assert np.allclose(oblock.block_forward(inp, rows=rows, store_bf16=False), ref[rows],
                       rtol=1e-10, atol=1e-10)


def test_block_fused_qkv_only_moves_rounding():
    """The fused-projection option drops the bf16 storage of Q and K: in fp64
    mode it is the same composition (pinned to torch above); in storage mode
    its intermediate Q' differs from the unfused one by at most one rounding of
    the pre-norm Q, and V is untouched."""
    inp = _tiny_block(seed=14)
    a64 = oblock.block_forward(inp, store_bf16=False)
    f64 = oblock.block_forward(inp, store_bf16=False, fused_qkv=True)
    assert np.array_equal(a64, f64)
    _, ia = oblock.block_forward(inp, return_intermediates=True)
    _, ib = oblock.block_forward(inp, return_intermediates=True, fused_qkv=True)
    HD = inp["heads"] * inp["head_dim"]
    assert np.array_equal(ia["kv"][:, HD:], ib["kv"][:, HD:])          # V still stored bf16
    assert not np.array_equal(ia["kv"][:, :HD], ib["kv"][:, :HD])      # K no longer rounded
    assert np.array_equal(oracle.bf16_storage(ib["kv"][:, :HD]), ia["kv"][:, :HD])
    rel = np.abs(ia["qn"] - ib["qn"]).max() / np.abs(ib["qn"]).max()
    assert 0 < rel < 2.0 ** -6


def test_block_zero_gates_is_identity():
    inp = _tiny_block(seed=12)
    hid = inp["hidden"]
    mod = oblock.adaln_table(inp["temb"], inp["w_ada"])
    mod[:, :, oblock.GATE_A] = 0
    mod[:, :, oblock.GATE_F] = 0
    x2 = oblock.block_forward(inp, mod=mod)
    assert np.array_equal(x2, oracle.bf16_to_f64(inp["x"]))


def test_block_ln_modulate_pieces():
    inp = _tiny_block(seed=13)
    lay = inp["layout"]
    mod = oblock.adaln_table(inp["temb"], inp["w_ada"])
    x = oracle.bf16_to_f64(inp["x"])
    got = oblock.ln_modulate(x, mod, lay["tags"], lay["ts_idx"], "a", 1e-5)
    ln = Fn.layer_norm(torch.from_numpy(x), (inp["hidden"],), eps=1e-5).numpy()
    sh = oblock.row_modulation(mod, lay["tags"], lay["ts_idx"], 0)
    sc = oblock.row_modulation(mod, lay["tags"], lay["ts_idx"], 1)
    assert np.allclose(got, ln * (1 + sc) + sh, atol=1e-12)
    # x == 0 -> LN is 0 -> output is exactly the gathered shift
    z = oblock.ln_modulate(np.zeros_like(x), mod, lay["tags"], lay["ts_idx"], "a", 1e-5)
    assert np.array_equal(z, sh)
    assert np.all(sh[lay["tags"] == -1] == 0)
    # silu closed forms
    assert oblock.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(oblock.silu(np.array([40.0])), 40.0, rtol=1e-15)
    zz = np.linspace(-8, 8, 101)
    assert np.allclose(oblock.silu(zz), Fn.silu(torch.from_numpy(zz)).numpy(), atol=1e-15)
