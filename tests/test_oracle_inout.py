"""Pins of the input/output-path oracle (oracle/inout.py) to things other than
itself (CPU only): closed forms of the sinusoid, torch's own Linear / SiLU /
layer_norm as library routines for special cases, pure-Python brute force on
tiny inputs, and invariants of the gather/scatter by index tensors.
"""
import math

import numpy as np
import torch
import torch.nn.functional as Fn

import oracle
from oracle import inout
from packed_masked_attention_amd import synth


def _py_bf16(v: float) -> float:
    """Round a float to the nearest bf16 value, ties to even (pure Python, normal range)."""
    if v == 0.0:
        return 0.0
    m, e = math.frexp(v)          # v = m * 2^e, 0.5 <= |m| < 1
    q = round(m * 256.0)          # 8 significant bits; Python rounds halves to even
    return math.ldexp(q / 256.0, e)


# -------------------------------------------------------------- sinusoid ----

def test_sinusoid_at_zero_is_cosines_one_sines_zero():
    e = inout.timestep_sinusoid([0.0], 256)
    assert e.shape == (1, 256)
    assert np.array_equal(e[0, :128], np.ones(128))
    assert np.array_equal(e[0, 128:], np.zeros(128))


def test_sinusoid_frequencies_are_geometric_from_one():
    # timesteps stay in [0, 1], so every angle t*w_j <= 1 rad and atan2 recovers it
    t = 0.75
    e = inout.timestep_sinusoid([t], 256)[0]
    ang = np.arctan2(e[128:], e[:128]) / t
    assert abs(ang[0] - 1.0) < 1e-15                        # the first frequency is 1
    ratio = ang[1:] / ang[:-1]
    assert np.allclose(ratio, 10000.0 ** (-1.0 / 128), rtol=1e-9, atol=0)
    assert abs(ang[-1] - 10000.0 ** (-127.0 / 128)) < 1e-12  # last = max_period^(-(half-1)/half)
    assert np.allclose(e[:128] ** 2 + e[128:] ** 2, 1.0, atol=1e-15)


def test_sinusoid_small_t_is_linear_in_sines():
    t = 1e-6
    e = inout.timestep_sinusoid([t], 16)[0]
    w = np.array([10000.0 ** (-j / 8) for j in range(8)])
    assert np.allclose(e[8:], t * w, rtol=1e-10, atol=0)


# ------------------------------------------------------------------- MLP ----

def test_timestep_mlp_matches_torch_linear_silu_linear():
    rng = np.random.default_rng(1)
    fd, inner, E = 16, 24, 12
    t = np.array([0.0, 0.3, 1.0])
    w1, b1 = rng.standard_normal((inner, fd)), rng.standard_normal(inner)
    w2, b2 = rng.standard_normal((E, inner)), rng.standard_normal(E)
    got, h = inout.timestep_mlp(t, w1, b1, w2, b2, freq_dim=fd)
    # torch modules on the sinusoid written from its closed form above
    half = fd // 2
    freqs = torch.tensor([10000.0 ** (-j / half) for j in range(half)], dtype=torch.float64)
    ang = torch.tensor(t, dtype=torch.float64)[:, None] * freqs[None]
    emb = torch.cat([torch.cos(ang), torch.sin(ang)], dim=1)
    lin1 = torch.nn.Linear(fd, inner, dtype=torch.float64)
    lin2 = torch.nn.Linear(inner, E, dtype=torch.float64)
    with torch.no_grad():
        lin1.weight.copy_(torch.from_numpy(w1)); lin1.bias.copy_(torch.from_numpy(b1))
        lin2.weight.copy_(torch.from_numpy(w2)); lin2.bias.copy_(torch.from_numpy(b2))
        hh = torch.nn.SiLU()(lin1(emb))
        want = lin2(hh).numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    assert np.allclose(h, hh.numpy(), rtol=1e-12, atol=1e-12)


def test_timestep_mlp_identity_weights_give_silu_of_embedding():
    fd = 8
    t = [0.5]
    got, _ = inout.timestep_mlp(t, np.eye(fd), np.zeros(fd), np.eye(fd), np.zeros(fd), freq_dim=fd)
    e = torch.tensor(inout.timestep_sinusoid(t, fd))
    assert np.allclose(got, Fn.silu(e).numpy(), rtol=1e-14, atol=0)


# ------------------------------------------------------------------ pack ----

def _tiny_io(seed=0):
    lay = synth.random_layout(np.random.default_rng(seed), 40, pad_frac=0.2, T=2)
    return lay, synth.make_io_inputs(lay, hidden=8, video_channels=4, audio_channels=3,
                                     video_out=2, audio_out=2, freq_dim=4, inner_dim=8,
                                     temb_dim=4, seed=seed)


def test_pack_rows_brute_force_and_untouched_rows():
    lay, d = _tiny_io(3)
    L, hid = lay["L"], 8
    sentinel = np.full((L, hid), 0x7fc1, dtype=np.uint16)   # a NaN pattern no row can produce
    got = inout.pack_rows(sentinel, d["video"], d["w_video"], d["b_video"], lay["video_idx"],
                          d["audio"], d["w_audio"], d["b_audio"], lay["audio_idx"], d["text"],
                          lay["text_idx"])
    val = oracle.bf16_to_f64(got)
    for rows, w, b, idx in ((d["video"], d["w_video"], d["b_video"], lay["video_idx"]),
                            (d["audio"], d["w_audio"], d["b_audio"], lay["audio_idx"])):
        for i, r in enumerate(idx):
            for c in range(hid):
                s = float(b[c]) + sum(float(rows[i][k]) * float(w[c][k]) for k in range(rows.shape[1]))
                assert val[r, c] == _py_bf16(s), (r, c)
    for i, r in enumerate(lay["text_idx"]):
        assert np.array_equal(got[r], d["text"][i])
    pad = np.flatnonzero(lay["tags"] < 0)
    assert pad.size > 0 and np.all(got[pad] == 0x7fc1)


# ------------------------------------------------------------------ head ----

def test_head_table_brute_force():
    rng = np.random.default_rng(4)
    T, E, hid = 2, 3, 4
    temb = rng.standard_normal((T, E))
    w = rng.standard_normal((2, 2 * hid, E))
    tab = inout.head_table(temb, w)
    assert tab.shape == (2, T, 2, hid)
    for m in range(2):
        for t in range(T):
            for k in range(2):
                for c in range(hid):
                    s = sum(temb[t][e] * w[m][k * hid + c][e] for e in range(E))
                    assert abs(tab[m, t, k, c] - s) < 1e-12


def test_output_head_identity_projection_is_torch_layer_norm():
    lay, d = _tiny_io(5)
    hid = 8
    idx = lay["video_idx"]
    table = np.zeros((2, lay["T"], 2, hid))
    out = inout.output_head(d["x"], idx, lay["ts_idx"], table, 0, np.eye(hid), np.zeros(hid),
                            eps=1e-5)
    x = torch.from_numpy(oracle.bf16_to_f64(d["x"][idx]))
    want = Fn.layer_norm(x, (hid,), eps=1e-5).numpy()
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)


def test_output_head_gathers_modulation_by_row_timestep():
    lay, d = _tiny_io(6)
    hid = 8
    T = lay["T"]
    table = np.zeros((2, T, 2, hid))
    for t in range(T):
        table[1, t, 0, :] = 10.0 * (t + 1)        # shift = 10 (t+1) on the audio head
        table[1, t, 1, :] = -1.0                  # scale = -1 removes the normalised part
    idx = lay["audio_idx"]
    out = inout.output_head(d["x"], idx, lay["ts_idx"], table, 1, np.eye(hid), np.zeros(hid))
    want = 10.0 * (lay["ts_idx"][idx] + 1.0)
    assert np.allclose(out, want[:, None], rtol=0, atol=1e-12)
    # a non-identity projection is linear in the modulated row and adds the bias
    w = np.arange(2 * hid, dtype=np.float64).reshape(2, hid)
    out2 = inout.output_head(d["x"], idx, lay["ts_idx"], table, 1, w, np.array([1.0, -2.0]))
    assert np.allclose(out2, want[:, None] * w.sum(axis=1)[None] + np.array([1.0, -2.0]),
                       rtol=1e-12, atol=1e-9)
