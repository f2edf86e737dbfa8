"""The steps either side of the block stack, in numpy fp64 (test infrastructure
only; see __init__).

Pages: "MiniMaxH3Transformer3DModel" (diffusers API page) -- constructor
parameters freq_dim (sinusoidal embedding of the timestep, timesteps taken
unscaled in [0, 1]), time_embed_hidden_dim and time_embed_dim (inner and
output widths of the timestep MLP), in_channels x prod(patch_size) and
audio_in_channels (widths of the latent rows), final_norm_eps (epsilon of
norm_out); forward parameters (hidden_states, audio_hidden_states and
encoder_hidden_states are ordered as video_indices, audio_indices and
text_indices; timestep holds the distinct values and timestep_indices points
each row into it); returns (the video and audio velocities in the row order of
their index tensors); intro (the patch projections, the timestep MLP and the
two output heads are float32, the block stack bfloat16).  "MiniMax H3
Inference Engine voor Mac computers" -- implementation notes: the fp32 patch
projections round straight to bf16 into the packed hidden stream; the final
audio/video AdaLN reads its rows at their offsets in the residual stream and
the heads apply the modulation while loading their projection tiles.

Readings (listed in the design doc):
  * sinusoid: half = freq_dim / 2 frequencies w_j = max_period^(-j / half),
    j = 0..half-1, max_period = 10000; embedding = [cos(t w) | sin(t w)].
  * timestep MLP: Linear(freq_dim -> inner, bias) -> SiLU -> Linear(inner ->
    time_embed_dim, bias), fp32 weights.
  * patch projections: Linear(channels -> hidden, bias) per modality, fp32,
    result rounded once to bf16 into row idx[i] of the packed stream; text
    rows arrive already projected (bf16) and are copied to their rows; rows
    named by no index tensor are left untouched.
  * output head m (0 video, 1 audio): (shift, scale) = temb[ts] @ W_mod[m]^T
    (two chunks of hidden, no bias, like the block's AdaLN), then
    out = (LN(x) * (1 + scale) + shift) @ W_out[m]^T + b_out[m] in fp32, with
    LN without affine, population variance and eps = final_norm_eps; ts is the
    timestep index of the gathered row.
Weights are [out, in]: y = u @ W.T.
"""
from __future__ import annotations

import numpy as np

from . import bf16_round, bf16_to_f64


def timestep_sinusoid(t, freq_dim: int = 256, max_period: float = 10000.0) -> np.ndarray:
    """[T, freq_dim] embedding of unscaled timesteps: cosines, then sines."""
    t = np.asarray(t, dtype=np.float64).reshape(-1)
    half = freq_dim // 2
    w = np.array([max_period ** (-j / half) for j in range(half)])
    ang = t[:, None] * w[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def silu(z):
    return z / (1.0 + np.exp(-z))


def timestep_mlp(t, w1, b1, w2, b2, freq_dim: int = 256, max_period: float = 10000.0):
    """temb [T, E] and the inner activation [T, inner] of the timestep MLP."""
    e = timestep_sinusoid(t, freq_dim, max_period)
    h = silu(e @ np.asarray(w1, np.float64).T + np.asarray(b1, np.float64))
    temb = h @ np.asarray(w2, np.float64).T + np.asarray(b2, np.float64)
    return temb, h


def pack_rows(x_bits: np.ndarray, video, w_video, b_video, video_idx, audio, w_audio, b_audio,
              audio_idx, text_bits, text_idx) -> np.ndarray:
    """Packed stream after the input projections: a copy of x_bits ([L, hidden]
    bf16 bits) with the video, audio and text rows written at their indices."""
    out = np.array(x_bits, dtype=np.uint16, copy=True)
    for rows, w, b, idx in ((video, w_video, b_video, video_idx),
                            (audio, w_audio, b_audio, audio_idx)):
        idx = np.asarray(idx, dtype=np.int64)
        if idx.size:
            y = np.asarray(rows, np.float64) @ np.asarray(w, np.float64).T + np.asarray(b, np.float64)
            out[idx] = bf16_round(y)
    tidx = np.asarray(text_idx, dtype=np.int64)
    if tidx.size:
        out[tidx] = np.asarray(text_bits, dtype=np.uint16)[:, :out.shape[1]]
    return out


def head_table(temb, w_mod) -> np.ndarray:
    """[2, T, 2, hidden]: (shift, scale) of each output head per timestep."""
    temb = np.asarray(temb, np.float64)
    w = np.asarray(w_mod, np.float64)                  # [2, 2*hidden, E]
    G, two_h, _ = w.shape
    return np.stack([(temb @ w[g].T).reshape(temb.shape[0], 2, two_h // 2) for g in range(G)])


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def output_head(x_bits, idx, ts_idx, table, head: int, w_out, b_out, eps: float = 1e-5):
    """Velocity rows [len(idx), out_channels] of head ``head`` (0 video, 1 audio)."""
    idx = np.asarray(idx, dtype=np.int64)
    x = bf16_to_f64(np.asarray(x_bits, dtype=np.uint16)[idx])
    ts = np.asarray(ts_idx, dtype=np.int64)[idx]
    shift = table[head, ts, 0]
    scale = table[head, ts, 1]
    y = layer_norm(x, eps) * (1.0 + scale) + shift
    return y @ np.asarray(w_out, np.float64).T + np.asarray(b_out, np.float64)
