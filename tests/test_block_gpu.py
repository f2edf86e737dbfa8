"""The DiT block on the GPU (through the C ABI) vs the CPU oracle.

Tolerances.  Every GPU stage stores bf16 and accumulates in fp32; the oracle
in storage mode rounds the same tensors to bf16 and computes the rest in
fp64.  Stage by stage (test_block_stages_full_size) each GPU stage is within
one bf16 rounding of the oracle's stage applied to the GPU's own input.
End to end the two chains drift: the attention's bf16 probabilities move the
pre-rounding x1 by ~1e-4, flipping about 1% of x1 elements by one ulp, and
the SwiGLU feed-forward's Jacobian (gain ~15 per unit of its input) spreads
each flip over every output.  Block outputs are therefore compared on
(gpu - ref) / rms(ref): mean <= 2e-3 (the target's mean bound, relative to
the output scale) and max <= 6e-2 or one bf16 ulp of ref (at L=8192 the
largest outputs exceed 64, where one ulp is 0.5 = 4.2% of rms).
"""
import numpy as np
import pytest

import oracle
from oracle import block as oblock
from packed_masked_attention_amd import synth
from tests.helpers import Q_OPERAND_SCALE, bf16_to_np, one_rounding, say, to_dev_bf16

pytestmark = pytest.mark.gpu


def _small_inputs(seed=3, L=300, hidden=256, H=2, ffn=512, E=64, pad=20, T=2, std=0.05):
    rng = np.random.default_rng(seed)
    tags = rng.integers(0, 3, L).astype(np.int32)
    tags[L - pad:] = -1
    pos = rng.integers(0, 50, (L, 3)).astype(np.int32)
    pos[tags == -1] = 0
    ts = rng.integers(0, T, L).astype(np.int32)
    ts[tags == -1] = 0
    lay = synth.layout_from_tags(tags, pos, ts, T)
    return synth.make_block_inputs(L, hidden, H, 128, ffn, E, T=T, seed=seed, layout=lay,
                                   weight_std=std)


class BlockRun:
    def __init__(self, inp, device="cuda"):
        import torch
        from packed_masked_attention_amd import binding as B
        self.B, self.inp = B, inp
        L, hid, H, ffn, E = inp["L"], inp["hidden"], inp["heads"], inp["ffn"], inp["temb_dim"]
        self.L, self.hid, self.H, self.ffn, self.E = L, hid, H, ffn, E
        self.T = inp["layout"]["T"]
        self.p = B.block_params(hid, ffn, E, H)
        self.dl = B.pma_layout_build(inp["layout"], device=device)
        d = lambda k: to_dev_bf16(inp[k], device)
        self.x, self.temb = d("x"), d("temb")
        self.w_ada, self.w_qkv, self.w_o = d("w_ada"), d("w_qkv"), d("w_o")
        self.w_fc1, self.w_fc2 = d("w_fc1"), d("w_fc2")
        self.qn = torch.ones(128, dtype=torch.float32, device=device)
        self.kn = torch.ones(128, dtype=torch.float32, device=device)
        self.table = torch.empty(3, self.T, 6, hid, dtype=torch.float32, device=device)
        self.w = B.BlockWeights(self.w_ada.data_ptr(), self.w_qkv.data_ptr(), self.w_o.data_ptr(),
                                self.w_fc1.data_ptr(), self.w_fc2.data_ptr(),
                                self.qn.data_ptr(), self.kn.data_ptr())
        self.out = torch.full_like(self.x, float("nan"))

    def adaln(self):
        self.B.pma_adaln_table(self.p, self.T, self.temb, self.w_ada, self.table)

    def forward(self):
        import torch
        self.B.pma_block_forward(self.p, self.dl, self.w, self.table, self.x, self.out)
        torch.cuda.synchronize()
        return bf16_to_np(self.out)


def _block_close(got, ref, what, mean_rel=2e-3, max_rel=6e-2):
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(got - ref)
    ulp = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -7
    over = err > np.maximum(max_rel * rms, ulp)
    st = {"rms": rms, "max_rel": float(err.max() / rms), "mean_rel": float(err.mean() / rms),
          "n_over": int(over.sum())}
    say(f"  {what}: {st}")
    assert np.all(np.isfinite(got)), what
    assert st["mean_rel"] <= mean_rel, (what, st)
    assert not over.any(), (what, st)


def test_adaln_table_matches_oracle():
    inp = _small_inputs()
    say("adaln table")
    r = BlockRun(inp)
    r.adaln()
    got = r.table.cpu().numpy()
    ref = oblock.adaln_table(inp["temb"], inp["w_ada"])
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())


def test_ln_modulate_matches_oracle():
    import torch
    inp = _small_inputs(seed=4)
    say("ln modulate")
    r = BlockRun(inp)
    r.adaln()
    lay = inp["layout"]
    mod = r.table.cpu().numpy().astype(np.float64)
    x = oracle.bf16_to_f64(inp["x"])
    for which, name in ((0, "a"), (1, "f")):
        out = torch.empty_like(r.x)
        r.B.pma_ln_modulate(r.p, r.dl, r.table, which, r.x, out)
        torch.cuda.synchronize()
        got = bf16_to_np(out)
        ref = oblock.ln_modulate(x, mod, lay["tags"], lay["ts_idx"], name, 1e-5)
        bound = np.abs(ref) * 2.0 ** -8 * 1.02 + 1e-5 * np.abs(ref).max()
        assert np.all(np.abs(got - ref) <= bound), name
    # x == 0: LN is 0, so the output is the gathered shift exactly (rounded to bf16)
    zeros = torch.zeros_like(r.x)
    out = torch.empty_like(r.x)
    r.B.pma_ln_modulate(r.p, r.dl, r.table, 0, zeros, out)
    torch.cuda.synchronize()
    shift = oblock.row_modulation(mod, lay["tags"], lay["ts_idx"], 0)
    assert np.array_equal(bf16_to_np(out), oracle.bf16_storage(shift))


@pytest.mark.parametrize("epi", [0, 1, 2])
@pytest.mark.parametrize("M", [1, 257, 300, 512])
@pytest.mark.parametrize("N,K", [(512, 320), (1792, 64), (1792, 192), (1792, 256), (1792, 448)])
def test_linear_epilogues_match_numpy(epi, M, N, K):
    """N = 1792 with the store and gated-residual epilogues runs the 224-wide
    tiles (one round of tiles either way, the narrower one shorter); K spans
    every stage count mod 5 (K/64 = 5, 1, 3, 4, 7); M = 1 and 257 leave a
    tile with one real row."""
    import torch
    from packed_masked_attention_amd import binding as B
    rng = np.random.default_rng(10 + epi + K)
    T = 2
    say(f"linear epi={epi} M={M} N={N} K={K}")
    A = synth.normal_bf16(rng, (M, K))
    W = synth.normal_bf16(rng, (2 * N if epi == 2 else N, K), 0.05)
    Rr = synth.normal_bf16(rng, (M, N))
    table = rng.standard_normal((3, T, 6, N)).astype(np.float32)
    tags = rng.integers(-1, 3, M).astype(np.int32)
    ts = rng.integers(0, T, M).astype(np.int32)
    dA, dW, dR = to_dev_bf16(A), to_dev_bf16(W), to_dev_bf16(Rr)
    dC = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dt = torch.from_numpy(table).cuda()
    dtags, dts = torch.from_numpy(tags).cuda(), torch.from_numpy(ts).cuda()
    B.pma_linear(M, N, K, dA, K, dW, K, dC, N, epi, R=dR, ldr=N, table=dt, num_timesteps=T,
                 gate_chunk=2, tags=dtags, ts_idx=dts)
    torch.cuda.synchronize()
    got = bf16_to_np(dC)
    acc = oracle.bf16_to_f64(A) @ oracle.bf16_to_f64(W).T
    if epi == 0:
        ref = acc
    elif epi == 1:
        gate = np.zeros((M, N))
        real = tags >= 0
        gate[real] = table[tags[real], ts[real], 2].astype(np.float64)
        ref = oracle.bf16_to_f64(Rr) + gate * acc
    else:
        ref = oblock.silu(acc[:, :N]) * acc[:, N:]
    err = np.abs(got - ref)
    bound = np.abs(ref) * 2.0 ** -8 * 1.02 + 2e-3 * np.sqrt(np.mean(ref ** 2))
    bad = err > bound
    assert not bad.any(), f"{int(bad.sum())} values off; worst {err.max()}"


@pytest.mark.parametrize("M,N,K,offset", [(1, 256, 64, 0.0), (257, 512, 448, 0.0),
                                            (300, 1792, 192, 0.0), (300, 1792, 320, 100.0),
                                            (1000, 5376, 256, 0.0)])
def test_gate_residual_ln_modulate_fused(M, N, K, offset):
    """The gated residual with the row statistics in its epilogue, then the
    norm from those statistics: x1 bit-equal to pma_linear's GATE_RESIDUAL,
    b within one bf16 rounding of the fp64 LN-modulate of that x1 (and of
    the unfused pma_ln_modulate).  N = 1792 and 5376 run 224-wide tiles
    (groups of 224 columns), 256 and 512 the 256-wide ones (groups of 128);
    the residual offset of 100 makes the mean dominate the variance; the
    gate and the modulation come from different tables and chunks (a
    block's fc2 feeding the next block's first norm) in half the cases."""
    import torch
    from packed_masked_attention_amd import binding as B
    rng = np.random.default_rng(20 + M + K)
    T = 2
    say(f"gate residual + ln modulate M={M} N={N} K={K} offset={offset}")
    tags = rng.integers(0, 3, M).astype(np.int32)
    tags[M - M // 10:] = -1
    ts = rng.integers(0, T, M).astype(np.int32)
    ts[tags == -1] = 0
    lay = synth.layout_from_tags(tags, np.zeros((M, 3), np.int32), ts, T)
    p = B.block_params(N, 512, 64, 2)
    dl = B.pma_layout_build(lay)
    A = synth.normal_bf16(rng, (M, K))
    W = synth.normal_bf16(rng, (N, K), 0.05)
    xr = synth.f32_to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32) + np.float32(offset))
    t1 = rng.standard_normal((3, T, 6, N)).astype(np.float32)
    t2 = rng.standard_normal((3, T, 6, N)).astype(np.float32)
    cross = K % 128 == 64   # fc2 -> the next block's first norm
    gate_chunk, which = (5, 0) if cross else (2, 1)
    dA, dW, dx = to_dev_bf16(A), to_dev_bf16(W), to_dev_bf16(xr)
    dt1 = torch.from_numpy(t1).cuda()
    dt2 = torch.from_numpy(t2).cuda() if cross else dt1
    dtags, dts = torch.from_numpy(tags).cuda(), torch.from_numpy(ts).cuda()
    nan = lambda: torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    x1, b, x1_ref, b_ref = nan(), nan(), nan(), nan()
    B.pma_gate_residual_ln_modulate(p, dl, dA, K, K, dW, dt1, gate_chunk, dx, x1, dt2, which, b)
    B.pma_linear(M, N, K, dA, K, dW, K, x1_ref, N, 1, R=dx, ldr=N, table=dt1, num_timesteps=T,
                 gate_chunk=gate_chunk, tags=dtags, ts_idx=dts)
    B.pma_ln_modulate(p, dl, dt2, which, x1_ref, b_ref)
    torch.cuda.synchronize()
    assert torch.equal(x1.view(torch.int16), x1_ref.view(torch.int16)), "x1 differs"
    x1_64 = bf16_to_np(x1)
    mod = (t2 if cross else t1).astype(np.float64)
    ref = oblock.ln_modulate(x1_64, mod, tags, ts, "a" if which == 0 else "f", 1e-5)
    got = bf16_to_np(b)
    bound = np.abs(ref) * 2.0 ** -8 * 1.02 + 1e-5 * np.abs(ref).max()
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{int(bad.sum())} values beyond one rounding of the oracle"
    # the unfused norm meets the same bound; the two differ only where their
    # fp32 statistics round differently (outputs near zero, where the
    # bound's floor dominates, can then differ by a few ulps)
    plain = bf16_to_np(b_ref)
    assert not (np.abs(plain - ref) > bound).any(), "unfused norm beyond one rounding"
    diff = got != plain
    say(f"  b: {int(diff.sum())} of {diff.size} differ from the unfused norm")
    assert diff.mean() < 0.01


@pytest.mark.parametrize("epi", [0, 1])
def test_linear_tile_shapes_agree(epi):
    """The O-projection shape (N = 5376, K = 7168) at M = 8192 runs 224-wide
    tiles (768 tiles, three full rounds on 256 CUs, against 2.625 rounds of
    256-wide ones) and at M = 6144 256-wide tiles (two rounds).  An output row
    depends only on its A row and is summed over K in the same order by both
    shapes, so the first 6144 rows agree bit for bit; a sample of rows is
    checked against fp64."""
    import torch
    from packed_masked_attention_amd import binding as B
    assert torch.cuda.get_device_properties(0).multi_processor_count == 256
    N, K, T = 5376, 7168, 3
    g = torch.Generator(device="cuda").manual_seed(20 + epi)
    A = torch.randn(8192, K, device="cuda", generator=g).to(torch.bfloat16)
    W = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    Rr = torch.randn(8192, N, device="cuda", generator=g).to(torch.bfloat16)
    table = torch.randn(3, T, 6, N, device="cuda", generator=g)
    tags = torch.randint(-1, 3, (8192,), device="cuda", generator=g, dtype=torch.int32)
    ts = torch.randint(0, T, (8192,), device="cuda", generator=g, dtype=torch.int32)
    outs = {}
    for M in (8192, 6144):
        say(f"linear epi={epi} M={M} N={N} K={K}")
        C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        B.pma_linear(M, N, K, A, K, W, K, C, N, epi, R=Rr, ldr=N, table=table, num_timesteps=T,
                     gate_chunk=2, tags=tags, ts_idx=ts)
        torch.cuda.synchronize()
        outs[M] = C
    assert torch.equal(outs[8192][:6144].view(torch.int16), outs[6144].view(torch.int16))
    rows = np.random.default_rng(epi).choice(8192, 48, replace=False)
    got = bf16_to_np(outs[8192][rows].contiguous())
    a64 = bf16_to_np(A[rows].contiguous())
    acc = a64 @ bf16_to_np(W).T
    if epi == 0:
        ref = acc
    else:
        tg, tsn = tags[rows].cpu().numpy(), ts[rows].cpu().numpy()
        tab = table.cpu().numpy().astype(np.float64)
        gate = np.zeros((rows.size, N))
        real = tg >= 0
        gate[real] = tab[tg[real], tsn[real], 2]
        ref = bf16_to_np(Rr[rows].contiguous()) + gate * acc
    err = np.abs(got - ref)
    bound = np.abs(ref) * 2.0 ** -8 * 1.02 + 2e-3 * np.sqrt(np.mean(ref ** 2))
    assert not (err > bound).any(), f"worst {err.max()}"


def test_qkv_projection_column_split_agrees():
    """At L = 8192, H = 56, hidden = 5376 the fused QKV projection runs its
    last 1024 output columns (V heads 48..55) as 128-wide tiles in a second
    launch (2688 wide tiles are 10.5 rounds on 256 CUs; 2560 wide + 256
    narrow ones are 10 rounds and one narrow round); at L = 6144 every column
    runs on 256-wide tiles.  A row's Q', K' and V^T depend only on its own A
    row and position, and both tile shapes sum over K in the same order, so
    the first 6144 rows agree bit for bit; V of sampled rows in the narrow
    columns is checked against fp64."""
    import torch
    from packed_masked_attention_amd import binding as B
    assert torch.cuda.get_device_properties(0).multi_processor_count == 256
    L, H, hidden, F = 8192, 56, 5376, 16
    HD = H * 128
    rng = np.random.default_rng(31)
    tags = rng.integers(0, 3, L).astype(np.int32)
    tags[rng.random(L) < 0.05] = -1
    pos = rng.integers(0, 300, (L, 3)).astype(np.int32)
    pos[tags == -1] = 0
    g = torch.Generator(device="cuda").manual_seed(31)
    a = torch.randn(L, hidden, device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn(3 * HD, hidden, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    wq = torch.rand(128, device="cuda", generator=g) + 0.5
    wk = torch.rand(128, device="cuda", generator=g) + 0.5
    p = B.attn_params(H, F=F)
    out = {}
    for n in (L, 6144):
        say(f"qkv projection L={n} H={H} hidden={hidden}")
        dl = B.pma_layout_build(synth.layout_from_tags(tags[:n], pos[:n], np.zeros(n, np.int32), 1))
        Lp = B.pma_attention_padded_len(n)
        rope = torch.empty(n, 3 * F, 2, dtype=torch.float32, device="cuda")
        qh = torch.full((H, Lp, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        kh = torch.full_like(qh, float("nan"))
        vt = torch.full((H, 128, Lp), float("nan"), dtype=torch.bfloat16, device="cuda")
        B.pma_rope_table(p, dl, rope)
        B.pma_qkv_projection(p, dl, a, hidden, hidden, w, wq, wk, rope, qh, kh, vt)
        torch.cuda.synchronize()
        out[n] = (qh, kh, vt)
    i16 = lambda t: t.contiguous().view(torch.int16)
    assert torch.equal(i16(out[L][0][:, :6144]), i16(out[6144][0][:, :6144]))
    assert torch.equal(i16(out[L][1][:, :6144]), i16(out[6144][1][:, :6144]))
    assert torch.equal(i16(out[L][2][:, :, :6144]), i16(out[6144][2][:, :, :6144]))
    # V of the narrow columns (heads 48..55) on sampled rows, among them rows past 6144
    rows = np.sort(rng.choice(L, 40, replace=False))
    v_ref = bf16_to_np(a[rows].contiguous()) @ bf16_to_np(w[2 * HD + 48 * 128:].contiguous()).T
    got = bf16_to_np(out[L][2][48:, :, rows].permute(2, 0, 1).reshape(rows.size, 8 * 128).contiguous())
    assert np.all(np.abs(got - v_ref) <= one_rounding(v_ref))


_one_rounding = one_rounding


@pytest.mark.parametrize("F,L,H,hidden,sc,pmax", [(16, 700, 4, 512, (1.0, 1.0, 1.0), 300),
                                                  (8, 300, 2, 256, (1.0, 1.0, 1.0), 300),
                                                  (16, 500, 2, 256, (1.0, 0.5, 0.5), 300),
                                                  (16, 600, 2, 256, (1.0, 1.0, 1.0), 1 << 24)])
def test_qkv_projection_matches_oracle(F, L, H, hidden, sc, pmax):
    """pma_qkv_projection (QKV GEMM with the QK-norm + RoPE epilogue) against
    the oracle's norm and rotation of the fp64 product, and against the
    unfused GPU path (pma_linear + pma_qk_norm_rope) on the same inputs.
    pmax = 2^24: positions over the whole accepted range |p| < 2^24 (angles
    up to 2^24 - 1 rad), extremes included."""
    import torch
    from packed_masked_attention_amd import binding as B
    rng = np.random.default_rng(21 + F + (pmax > 300))
    tags = rng.integers(0, 3, L).astype(np.int32)
    tags[rng.random(L) < 0.1] = -1
    if pmax > 300:
        pos = rng.integers(-(pmax - 1), pmax, (L, 3)).astype(np.int32)
        pos[:3] = [[pmax - 1] * 3, [-(pmax - 1)] * 3, [pmax - 1, -(pmax - 1), 1]]
        tags[:3] = 0
    else:
        pos = rng.integers(0, 300, (L, 3)).astype(np.int32)
        pos[tags == -1] = 0
    lay = synth.layout_from_tags(tags, pos, np.zeros(L, np.int32), 1)
    HD = H * 128
    a_bits = synth.normal_bf16(rng, (L, hidden))
    w_bits = synth.normal_bf16(rng, (3 * HD, hidden), 0.05)
    wq = rng.uniform(0.5, 2.0, 128).astype(np.float32)
    wk = rng.uniform(0.5, 2.0, 128).astype(np.float32)
    say(f"qkv projection F={F} L={L} H={H} hidden={hidden}")
    dl = B.pma_layout_build(lay)
    p = B.attn_params(H, F=F, pos_scale=sc)
    Lp = B.pma_attention_padded_len(L)
    a, w = to_dev_bf16(a_bits), to_dev_bf16(w_bits)
    wq_d, wk_d = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()
    rope = torch.empty(L, 3 * F, 2, dtype=torch.float32, device="cuda")
    qh = torch.full((H, Lp, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    kh, vt = torch.full_like(qh, float("nan")), torch.full((H, 128, Lp), float("nan"),
                                                            dtype=torch.bfloat16, device="cuda")
    B.pma_rope_table(p, dl, rope)
    B.pma_qkv_projection(p, dl, a, hidden, hidden, w, wq_d, wk_d, rope, qh, kh, vt)
    # the unfused path on the same inputs
    qkv = torch.empty(L, 3 * HD, dtype=torch.bfloat16, device="cuda")
    B.pma_linear(L, 3 * HD, hidden, a, hidden, w, hidden, qkv, 3 * HD, 0)
    qh2, kh2, vt2 = torch.empty_like(qh), torch.empty_like(kh), torch.empty_like(vt)
    B.pma_qk_norm_rope(p, dl, qkv, 3 * HD, qkv[:, HD:], 3 * HD, qkv[:, 2 * HD:], 3 * HD, wq_d, wk_d,
                       qh2, kh2, vt2)
    torch.cuda.synchronize()

    # rope table: fp32 rounding of the fp64 cos/sin of pos[i][a] * theta^(-f/F)
    inv = oracle.inv_freq(F, 10000.0)
    phi = (pos.astype(np.float64) * np.asarray(sc))[:, :, None] * inv[None, None, :]   # [L, 3, F]
    tab = rope.cpu().numpy().reshape(L, 3, F, 2)
    assert np.abs(tab[..., 0] - np.cos(phi)).max() <= 2.0 ** -24
    assert np.abs(tab[..., 1] - np.sin(phi)).max() <= 2.0 ** -24

    A64, W64 = oracle.bf16_to_f64(a_bits), oracle.bf16_to_f64(w_bits)
    q, k, v = (A64 @ W64[i * HD:(i + 1) * HD].T for i in range(3))
    for name, got_t, x, wv in (("q'", qh, q, wq), ("k'", kh, k, wk)):
        c = Q_OPERAND_SCALE if name == "q'" else 1.0   # the stored Q' carries the logit factor
        ref = oracle.qk_norm_rope(x, H, 128, wv.astype(np.float64), pos, F=F,
                                  pos_scale=sc).transpose(1, 0, 2) * c
        got = bf16_to_np(got_t)
        err = np.abs(got[:, :L] - ref)
        bad = err > _one_rounding(ref)
        say(f"  {name}: max err {err.max():.3e}, {int(bad.sum())} over one rounding")
        assert not bad.any()
        assert np.all(got[:, L:] == 0), f"{name} padding rows"
    vref = v.reshape(L, H, 128).transpose(1, 2, 0)
    vg = bf16_to_np(vt)
    assert not (np.abs(vg[:, :, :L] - vref) > _one_rounding(vref)).any(), "v^T"
    assert np.all(vg[:, :, L:] == 0), "v^T padding columns"
    # V^T is the same bf16 product both ways; Q', K' differ only by the
    # unfused path's extra rounding of Q and K before the norm
    assert torch.equal(vt.view(torch.int16), vt2.view(torch.int16))
    for got_t, ref_t in ((qh, qh2), (kh, kh2)):
        g, r2 = bf16_to_np(got_t), bf16_to_np(ref_t)
        rel = np.abs(g - r2).max() / np.abs(r2).max()
        assert rel < 2.0 ** -6, rel


def test_block_small_matches_oracle():
    inp = _small_inputs(seed=5)
    say("block small: L=300 hidden=256 H=2 ffn=512, 20 padding rows, T=2")
    r = BlockRun(inp)
    r.adaln()
    got = r.forward()
    # the oracle's own AdaLN table (the GPU's is checked on its own below)
    mod = oblock.adaln_table(inp["temb"], inp["w_ada"])
    gmod = r.table.cpu().numpy().astype(np.float64)
    assert np.allclose(gmod, mod, rtol=1e-5, atol=1e-5 * np.abs(mod).max())
    # an even head count takes the fused QKV projection (Q, K not stored)
    ref = oblock.block_forward(inp, mod=mod, fused_qkv=inp["heads"] % 2 == 0)
    _block_close(got, ref, "block small")


def test_block_zero_gates_identity():
    import torch
    inp = _small_inputs(seed=6)
    say("block with zero gates is the identity, bit for bit")
    r = BlockRun(inp)
    r.adaln()
    r.table[:, :, 2] = 0
    r.table[:, :, 5] = 0
    got = r.forward()
    assert np.array_equal(got, oracle.bf16_to_f64(inp["x"]))
    out1 = r.out.clone()
    r.forward()
    assert torch.equal(out1.view(torch.int16), r.out.view(torch.int16)), "not deterministic"


def test_block_full_size_sampled_rows():
    wl = synth.workload("block_L8192")
    say("block L=8192 hidden=5376 H=56 ffn=14336: generating inputs")
    inp = synth.make_block_workload(wl)
    r = BlockRun(inp)
    r.adaln()
    got = r.forward()
    rows = np.sort(np.random.default_rng(7).choice(wl.L, 24, replace=False))
    say(f"  oracle on {rows.size} sampled rows")
    gmod = r.table.cpu().numpy().astype(np.float64)
    ref_mod = oblock.adaln_table(inp["temb"], inp["w_ada"])
    assert np.allclose(gmod, ref_mod, rtol=1e-4, atol=1e-4 * np.abs(ref_mod).max())
    # the end-to-end reference uses the oracle's own table
    ref = oblock.block_forward(inp, rows=rows, mod=ref_mod, fused_qkv=True)
    _block_close(got[rows], ref, "block L8192 sampled rows")


def test_block_stages_full_size():
    """Each stage of the L=8192 block, run through the C ABI, against the
    oracle's same stage fed with the GPU's own input to that stage (sampled
    rows), so an error is attributed to the stage that makes it."""
    import torch
    from packed_masked_attention_amd import binding as B
    wl = synth.workload("block_L8192")
    say("block stages L=8192: generating inputs")
    inp = synth.make_block_workload(wl)
    r = BlockRun(inp)
    r.adaln()
    L, hid, H, ffn = wl.L, wl.hidden, wl.H, wl.ffn
    HD = H * 128
    lay = inp["layout"]
    tags, ts = lay["tags"], lay["ts_idx"]
    mod = r.table.cpu().numpy().astype(np.float64)
    rows = np.sort(np.random.default_rng(8).choice(L, 16, replace=False))
    dev = lambda shape: torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    f64 = lambda t: bf16_to_np(t)
    stats = {}

    def stage(name, got, ref, rel=2.0 ** -8 * 1.02, floor=2e-3):
        err = np.abs(got - ref)
        rms = float(np.sqrt(np.mean(ref ** 2)))
        bound = np.abs(ref) * rel + floor * rms
        stats[name] = {"max_rel": float(err.max() / rms), "mean_rel": float(err.mean() / rms),
                       "n_over": int((err > bound).sum())}
        say(f"  {name}: {stats[name]}")

    a = dev((L, hid))
    B.pma_ln_modulate(r.p, r.dl, r.table, 0, r.x, a)
    qkv = dev((L, 3 * HD))
    B.pma_linear(L, 3 * HD, hid, a, hid, r.w_qkv, hid, qkv, 3 * HD, 0)
    o = dev((L, HD))
    B.pma_attention(r.p.attn, r.dl, qkv, 3 * HD, qkv[:, HD:], 3 * HD, qkv[:, 2 * HD:], 3 * HD,
                    r.qn, r.kn, o, HD)
    x1 = dev((L, hid))
    B.pma_linear(L, hid, HD, o, HD, r.w_o, HD, x1, hid, 1, R=r.x, ldr=hid, table=r.table,
                 num_timesteps=1, gate_chunk=2, tags=r.dl.arrays["tags"],
                 ts_idx=r.dl.arrays["ts_idx"])
    b = dev((L, hid))
    B.pma_ln_modulate(r.p, r.dl, r.table, 1, x1, b)
    h = dev((L, ffn))
    B.pma_linear(L, ffn, hid, b, hid, r.w_fc1, hid, h, ffn, 2)
    x2 = dev((L, hid))
    B.pma_linear(L, hid, ffn, h, ffn, r.w_fc2, ffn, x2, hid, 1, R=x1, ldr=hid, table=r.table,
                 num_timesteps=1, gate_chunk=5, tags=r.dl.arrays["tags"],
                 ts_idx=r.dl.arrays["ts_idx"])
    # a7 + a8 through the fused entry point (row statistics in the projection's
    # epilogue) on the same O: x1 bit for bit, b against the oracle below
    x1f, bf = dev((L, hid)), dev((L, hid))
    B.pma_gate_residual_ln_modulate(r.p, r.dl, o, HD, HD, r.w_o, r.table, 2, r.x, x1f, r.table, 1,
                                    bf)
    torch.cuda.synchronize()
    assert torch.equal(x1f.view(torch.int16), x1.view(torch.int16)), "fused x1 differs"
    x = oracle.bf16_to_f64(inp["x"])
    a_g, qkv_g, o_g, x1_g, b_g, h_g, x2_g = (f64(t) for t in (a, qkv, o, x1, b, h, x2))
    bf_g = f64(bf)
    stage("a", a_g[rows], oblock.ln_modulate(x[rows], mod, tags[rows], ts[rows], "a", 1e-5))
    wq = oracle.bf16_to_f64(inp["w_qkv"])
    stage("qkv", qkv_g[rows], a_g[rows] @ wq.T)
    q_bits = oracle.bf16_round(qkv_g[:, :HD])
    k_bits = oracle.bf16_round(qkv_g[:, HD:2 * HD])
    v_bits = oracle.bf16_round(qkv_g[:, 2 * HD:])
    o_ref, _ = oracle.attention_path(q_bits, k_bits, v_bits, lay, H, rows=rows,
                                     store_qk_bf16=True)
    stage("o", o_g[rows], o_ref.reshape(rows.size, HD), floor=1e-2)
    gate_a = oblock.row_modulation(mod, tags, ts, oblock.GATE_A)[rows]
    stage("x1", x1_g[rows], x[rows] + gate_a * (o_g[rows] @ oracle.bf16_to_f64(inp["w_o"]).T))
    b_ref = oblock.ln_modulate(x1_g[rows], mod, tags[rows], ts[rows], "f", 1e-5)
    stage("b", b_g[rows], b_ref)
    stage("b (fused gate + norm)", bf_g[rows], b_ref)
    w1 = oracle.bf16_to_f64(inp["w_fc1"])
    g_ = b_g[rows] @ w1[:ffn].T
    u_ = b_g[rows] @ w1[ffn:].T
    stage("h", h_g[rows], oblock.silu(g_) * u_)
    gate_f = oblock.row_modulation(mod, tags, ts, oblock.GATE_F)[rows]
    stage("x2", x2_g[rows], x1_g[rows] + gate_f * (h_g[rows] @ oracle.bf16_to_f64(inp["w_fc2"]).T))
    bad = {k: v for k, v in stats.items() if v["n_over"]}
    assert not bad, bad
