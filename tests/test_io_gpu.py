"""The input/output path on the GPU (through the C ABI) vs the CPU oracle.

Tolerances.  The GPU computes in fp32 (the pages keep the timestep MLP, the
patch projections and the output heads in fp32); the oracle in fp64.
  * fp32 results (temb, head table, velocities) are compared element by
    element against eps_rel * S, where S = sum_k |a_k w_k| is the magnitude of
    the terms of that output's dot product (computed in fp64 beside the
    oracle).  An fp32 dot product of K terms is off by at most K * 2^-24 * S
    (2^-11.6 S at K = 5376); with random signs the partial sums stay near
    sqrt(K) terms in size and the error is ~2^-24 S, as measured.
    eps_rel = 2^-18 keeps a 64x margin over that while a dropped or wrong
    term (~S / K = 2^-12.4 S at K = 5376, more at smaller K) still fails.
  * bf16 results (the packed rows) must be within one rounding of the fp64
    value: half an ulp plus the fp32 error (helpers.one_rounding); text rows
    and untouched rows are compared bit for bit.
"""
import numpy as np
import pytest

import oracle
from oracle import inout
from packed_masked_attention_amd import synth
from tests.helpers import bf16_to_np, one_rounding, say, to_dev_bf16

pytestmark = pytest.mark.gpu

EPS_REL = 2.0 ** -18
SENTINEL = 0x7FC1          # a NaN bf16 pattern the projections never produce


def _dev():
    import torch
    from packed_masked_attention_amd import binding as B
    B.check(B.lib().pma_device_check())
    return torch.device("cuda", 0)


def _f32(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def _check_fp32(got, ref, terms, name):
    err = np.abs(np.asarray(got, np.float64) - ref)
    bound = EPS_REL * terms + 1e-30
    ratio = float((err / bound).max()) if err.size else 0.0
    say(f"  {name}: max |err| {err.max() if err.size else 0:.3e}, worst err/bound {ratio:.3f}")
    assert ratio <= 1.0, name


def _layouts():
    """(name, layout): packed layouts with contiguous and scattered rows."""
    rng = np.random.default_rng(11)
    return {
        "tiny_L256": synth.make_layout(synth.workload("tiny_L256")),
        "random_L700_T3": synth.random_layout(rng, 700, pad_frac=0.15, T=3),
        "block_L8192": synth.make_layout(synth.workload("block_L8192")),
    }


# ------------------------------------------------------- timestep MLP ----

@pytest.mark.parametrize("T,fd,inner,E", [(3, 256, 5376, 2688), (8, 16, 4100, 36), (1, 4, 4, 4)])
def test_timestep_embed_matches_oracle(T, fd, inner, E):
    import torch
    from packed_masked_attention_amd import binding as B
    dev = _dev()
    lay = synth.layout_from_counts(0, (1, 1, T), 0, 0, T)
    t = np.linspace(0.0, 1.0, T) if T > 1 else np.array([0.37])
    d = synth.make_io_inputs(lay, hidden=128, freq_dim=fd, inner_dim=inner, temb_dim=E, seed=7,
                             timesteps=t)
    say(f"timestep MLP T={T} freq={fd} inner={inner} E={E}")
    p = B.temb_params(fd, inner, E)
    inner_t = torch.empty(T, inner, dtype=torch.float32, device=dev)
    temb = torch.empty(T, E, dtype=torch.float32, device=dev)
    temb_b = torch.empty(T, E, dtype=torch.bfloat16, device=dev)
    B.pma_timestep_embed(p, T, _f32(d["t"], dev), _f32(d["w1"], dev), _f32(d["b1"], dev),
                         _f32(d["w2"], dev), _f32(d["b2"], dev), inner_t, temb, temb_b)
    torch.cuda.synchronize()
    ts = d["t"].astype(np.float64)
    ref, h_ref = inout.timestep_mlp(ts, d["w1"], d["b1"], d["w2"], d["b2"], freq_dim=fd)
    e = inout.timestep_sinusoid(ts, fd)
    s1 = np.abs(e) @ np.abs(d["w1"].astype(np.float64)).T + np.abs(d["b1"])
    _check_fp32(inner_t.cpu().numpy(), h_ref, s1, "inner")
    w2a = np.abs(d["w2"].astype(np.float64))
    # layer 2's own terms, plus layer 1's error carried through silu (slope <= 1.1) and |w2|
    s2 = np.abs(h_ref) @ w2a.T + np.abs(d["b2"]) + 1.1 * (s1 @ w2a.T)
    got = temb.cpu().numpy()
    _check_fp32(got, ref, s2, "temb")
    # the bf16 copy is the fp32 result rounded once, nearest-even
    want_bits = synth.f32_to_bf16_bits(got)
    assert np.array_equal(temb_b.view(torch.int16).cpu().numpy().view(np.uint16), want_bits)


# ------------------------------------------------------------- packing ----

def _pack(d, lay, dev, hidden, x0=None):
    import torch
    from packed_masked_attention_amd import binding as B
    p = B.io_params(hidden, d["video_channels"], d["audio_channels"], d["video_out"],
                    d["audio_out"], d["temb_dim"])
    dl = B.pma_layout_build(lay, device=dev)
    L = lay["L"]
    if x0 is None:
        x = torch.full((L, hidden), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    else:
        x = to_dev_bf16(x0, dev)
    text = to_dev_bf16(d["text"], dev) if d["text"].size else None
    B.pma_pack_rows(p, dl, _f32(d["video"], dev), _f32(d["w_video"], dev), _f32(d["b_video"], dev),
                    _f32(d["audio"], dev), _f32(d["w_audio"], dev), _f32(d["b_audio"], dev),
                    text, hidden, x)
    torch.cuda.synchronize()
    return x, p, dl


@pytest.mark.parametrize("name,hidden", [("tiny_L256", 256), ("random_L700_T3", 384),
                                         ("block_L8192", 5376)])
def test_pack_rows_matches_oracle(name, hidden):
    import torch
    dev = _dev()
    lay = _layouts()[name]
    d = synth.make_io_inputs(lay, hidden=hidden, inner_dim=64, temb_dim=64, seed=8)
    say(f"pack {name} hidden={hidden}: video {lay['video_idx'].size}, audio "
        f"{lay['audio_idx'].size}, text {lay['text_idx'].size}")
    x, _, _ = _pack(d, lay, dev, hidden)
    got_bits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    L = lay["L"]
    ref_bits = inout.pack_rows(np.full((L, hidden), SENTINEL, np.uint16), d["video"], d["w_video"],
                               d["b_video"], lay["video_idx"], d["audio"], d["w_audio"],
                               d["b_audio"], lay["audio_idx"], d["text"], lay["text_idx"])
    # text rows and untouched rows bit for bit
    keep = np.ones(L, bool)
    keep[lay["video_idx"]] = False
    keep[lay["audio_idx"]] = False
    assert np.array_equal(got_bits[keep], ref_bits[keep])
    for rows, w, b, idx, nm in ((d["video"], d["w_video"], d["b_video"], lay["video_idx"], "video"),
                                (d["audio"], d["w_audio"], d["b_audio"], lay["audio_idx"], "audio")):
        if idx.size == 0:
            continue
        ref = rows.astype(np.float64) @ w.astype(np.float64).T + b
        got = oracle.bf16_to_f64(got_bits[idx])
        err = np.abs(got - ref)
        bad = err > one_rounding(ref)
        same = np.mean(got_bits[idx] == oracle.bf16_round(ref))
        say(f"  {nm}: max |err| {err.max():.3e}, bit-equal to rounded fp64 {same:.5f}, "
            f"{int(bad.sum())} over one rounding")
        assert not bad.any(), nm


def test_pack_rows_skips_out_of_range_and_empty_modalities():
    import torch
    dev = _dev()
    rng = np.random.default_rng(12)
    lay = synth.random_layout(rng, 300, pad_frac=0.1, T=2)
    # no audio rows: retag them as text
    tags = lay["tags"].copy()
    tags[tags == synth.TAG_AUDIO] = synth.TAG_TEXT
    lay = synth.layout_from_tags(tags, lay["pos"], lay["ts_idx"], 2)
    d = synth.make_io_inputs(lay, hidden=256, inner_dim=64, temb_dim=64, seed=9)
    bad_lay = dict(lay)
    vid = lay["video_idx"].copy()
    vid[5] = lay["L"] + 7               # out of range: skipped by the kernel
    bad_lay["video_idx"] = vid
    x, _, _ = _pack(d, bad_lay, dev, 256)
    got = x.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = inout.pack_rows(np.full((lay["L"], 256), SENTINEL, np.uint16), d["video"][np.arange(vid.size) != 5],
                          d["w_video"], d["b_video"], np.delete(vid, 5), d["audio"], d["w_audio"],
                          d["b_audio"], lay["audio_idx"], d["text"], lay["text_idx"])
    untouched = np.all(ref == SENTINEL, axis=1)
    assert np.array_equal(got[untouched], ref[untouched])
    assert np.all(got[lay["video_idx"][5]] == SENTINEL)
    diff = np.abs(oracle.bf16_to_f64(got[~untouched]) - oracle.bf16_to_f64(ref[~untouched]))
    assert diff.max() <= 2.0 ** -7 * np.abs(oracle.bf16_to_f64(ref[~untouched])).max()


# -------------------------------------------------------- output heads ----

def _head_table_dev(d, T, temb, dev, p):
    import torch
    from packed_masked_attention_amd import binding as B
    hidden = d["hidden"]
    table = torch.empty(2, T, 2, hidden, dtype=torch.float32, device=dev)
    B.pma_head_table(p, T, _f32(temb, dev), _f32(d["w_mod"], dev), table)
    torch.cuda.synchronize()
    return table


@pytest.mark.parametrize("T", [1, 3])
def test_head_table_matches_oracle(T):
    from packed_masked_attention_amd import binding as B
    dev = _dev()
    hidden, E = 5376, 2688
    lay = synth.layout_from_counts(0, (1, 1, 4), 0, 0, T)
    d = synth.make_io_inputs(lay, hidden=hidden, inner_dim=64, temb_dim=E, seed=10)
    temb = synth.normal_f32(np.random.Generator(np.random.PCG64(20 + T)), (T, E))
    say(f"head table T={T} hidden={hidden} E={E}")
    p = B.io_params(hidden, time_embed_dim=E)
    got = _head_table_dev(d, T, temb, dev, p).cpu().numpy()
    ref = inout.head_table(temb, d["w_mod"])
    terms = np.stack([(np.abs(temb.astype(np.float64)) @ np.abs(d["w_mod"][g].astype(np.float64)).T)
                      .reshape(T, 2, hidden) for g in range(2)])
    _check_fp32(got, ref, terms, "table")


def _head_terms(x_bits, idx, ts_idx, table, head, w, eps):
    """S[i, j] = sum_k |a'_ik w_jk| of each head output (fp64)."""
    x = oracle.bf16_to_f64(np.asarray(x_bits)[idx])
    ts = np.asarray(ts_idx)[idx]
    a = np.abs(inout.layer_norm(x, eps) * (1.0 + table[head, ts, 1]) + table[head, ts, 0])
    return a @ np.abs(np.asarray(w, np.float64)).T


@pytest.mark.parametrize("name,hidden", [("tiny_L256", 256), ("random_L700_T3", 384),
                                         ("block_L8192", 5376)])
def test_unpack_rows_matches_oracle(name, hidden):
    import torch
    from packed_masked_attention_amd import binding as B
    dev = _dev()
    lay = _layouts()[name]
    T = lay["T"]
    E = 64
    d = synth.make_io_inputs(lay, hidden=hidden, inner_dim=64, temb_dim=E, seed=13)
    say(f"unpack {name} hidden={hidden} T={T}: video {lay['video_idx'].size}, "
        f"audio {lay['audio_idx'].size}")
    # the modulation table is an oracle value handed to both sides (fp32)
    temb = synth.normal_f32(np.random.Generator(np.random.PCG64(30)), (T, E))
    table = inout.head_table(temb, d["w_mod"]).astype(np.float32)
    p = B.io_params(hidden, time_embed_dim=E)
    dl = B.pma_layout_build(lay, device=dev)
    x = to_dev_bf16(d["x"], dev)
    nv, na = lay["video_idx"].size, lay["audio_idx"].size
    vout = torch.full((max(nv, 1), 96), float("nan"), dtype=torch.float32, device=dev)
    aout = torch.full((max(na, 1), 32), float("nan"), dtype=torch.float32, device=dev)
    B.pma_unpack_rows(p, dl, x, _f32(table, dev), _f32(d["w_vout"], dev), _f32(d["b_vout"], dev),
                      _f32(d["w_aout"], dev), _f32(d["b_aout"], dev), vout, aout)
    torch.cuda.synchronize()
    tab64 = table.astype(np.float64)
    for head, idx, w, b, out, nm in ((0, lay["video_idx"], d["w_vout"], d["b_vout"], vout, "video"),
                                     (1, lay["audio_idx"], d["w_aout"], d["b_aout"], aout, "audio")):
        if idx.size == 0:
            continue
        ref = inout.output_head(d["x"], idx, lay["ts_idx"], tab64, head, w, b, eps=1e-5)
        terms = _head_terms(d["x"], idx, lay["ts_idx"], tab64, head, w, 1e-5) + np.abs(b)
        _check_fp32(out[:idx.size].cpu().numpy(), ref, terms, nm)


def test_input_output_path_end_to_end():
    """timestep MLP -> head table, and pack -> unpack on the packed stream
    (no blocks in between), against the oracle's composition."""
    import torch
    from packed_masked_attention_amd import binding as B
    dev = _dev()
    rng = np.random.default_rng(14)
    lay = synth.random_layout(rng, 1500, pad_frac=0.05, T=2)
    hidden, inner, E = 512, 768, 256
    d = synth.make_io_inputs(lay, hidden=hidden, inner_dim=inner, temb_dim=E, seed=15,
                             timesteps=[0.0, 0.85])
    T = 2
    say(f"end to end L={lay['L']} hidden={hidden} inner={inner} E={E}")
    tp = B.temb_params(256, inner, E)
    inner_t = torch.empty(T, inner, dtype=torch.float32, device=dev)
    temb = torch.empty(T, E, dtype=torch.float32, device=dev)
    B.pma_timestep_embed(tp, T, _f32(d["t"], dev), _f32(d["w1"], dev), _f32(d["b1"], dev),
                         _f32(d["w2"], dev), _f32(d["b2"], dev), inner_t, temb, None)
    p = B.io_params(hidden, time_embed_dim=E)
    table = torch.empty(2, T, 2, hidden, dtype=torch.float32, device=dev)
    B.pma_head_table(p, T, temb, _f32(d["w_mod"], dev), table)
    x, _, dl = _pack(d, lay, dev, hidden, x0=d["x"])
    nv, na = lay["video_idx"].size, lay["audio_idx"].size
    vout = torch.empty(nv, 96, dtype=torch.float32, device=dev)
    aout = torch.empty(na, 32, dtype=torch.float32, device=dev)
    B.pma_unpack_rows(p, dl, x, table, _f32(d["w_vout"], dev), _f32(d["b_vout"], dev),
                      _f32(d["w_aout"], dev), _f32(d["b_aout"], dev), vout, aout)
    torch.cuda.synchronize()
    temb_ref, _ = inout.timestep_mlp(d["t"].astype(np.float64), d["w1"], d["b1"], d["w2"], d["b2"])
    tab_ref = inout.head_table(temb_ref, d["w_mod"])
    x_ref = inout.pack_rows(d["x"], d["video"], d["w_video"], d["b_video"], lay["video_idx"],
                            d["audio"], d["w_audio"], d["b_audio"], lay["audio_idx"], d["text"],
                            lay["text_idx"])
    for head, idx, w, b, out, nm in ((0, lay["video_idx"], d["w_vout"], d["b_vout"], vout, "video"),
                                     (1, lay["audio_idx"], d["w_aout"], d["b_aout"], aout, "audio")):
        ref = inout.output_head(x_ref, idx, lay["ts_idx"], tab_ref, head, w, b, eps=1e-5)
        got = out.cpu().numpy().astype(np.float64)
        # packed rows may differ from the oracle's by one bf16 rounding, which
        # the normalised head passes on at ~2^-9 of its output scale
        rel = np.abs(got - ref).max() / np.sqrt(np.mean(ref ** 2))
        say(f"  {nm}: max |err| / rms {rel:.3e}")
        assert rel < 2.0 ** -6, nm
