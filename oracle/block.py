"""DiT block forward in numpy fp64 (test infrastructure only; see __init__).

Pages: "MiniMaxH3Transformer3DModel" (diffusers API page) -- intro (one block
stack over the packed sequence; the per-row modality tag selects the AdaLN
modulation parameters), constructor parameters (hidden_size, ffn_dim with a
SwiGLU feed-forward, time_embed_dim as the input of every AdaLN projection,
norm_eps of the pre-attention and pre-feed-forward norms, qk_norm_eps), intro
(block stack stored in bfloat16).  "MiniMax H3 Inference Engine voor Mac
computers" -- implementation notes: fc1 -> SwiGLU -> fc2 as the feed-forward,
the bf16 residual written exactly after each gated residual add.

Readings (listed in the design doc):
  * AdaLN: per tag g a linear map W_ada[g]: time_embed_dim -> 6*hidden, no
    bias and no activation; chunks in the order shift_a, scale_a, gate_a,
    shift_f, scale_f, gate_f; padding rows get all-zero modulation.
  * modulate(u) = u * (1 + scale) + shift; the gate scales the sublayer output
    before the residual add.
  * pre-norms: LayerNorm without affine, population variance, eps = norm_eps.
  * W_fc1 rows = [gate | up]; silu on the gate half; no biases anywhere.
  * QKV rows = [Q heads | K heads | V heads], head-contiguous.
Weights are [out, in]: y = u @ W.T.

``store_bf16=True`` rounds to bf16 exactly the tensors the GPU path stores
(a, Q, K, V, normalised Q and K, O, x1, b, h, x2; the normalised Q is stored
times log2(e)/sqrt(D), see stored_query); every other value is fp64.
"""
from __future__ import annotations

import numpy as np

from . import attention, bf16_storage, bf16_to_f64, qk_norm_rope, stored_query

SHIFT_A, SCALE_A, GATE_A, SHIFT_F, SCALE_F, GATE_F = range(6)


def adaln_table(temb_bits, w_ada_bits) -> np.ndarray:
    """mod[g, t, k, c] = sum_e temb[t, e] * W_ada[g][k*hidden + c, e]."""
    temb = bf16_to_f64(temb_bits)                    # [T, E]
    w = bf16_to_f64(w_ada_bits)                      # [3, 6*hidden, E]
    G, six_h, E = w.shape
    hidden = six_h // 6
    out = np.empty((G, temb.shape[0], 6, hidden))
    for g in range(G):
        out[g] = (temb @ w[g].T).reshape(temb.shape[0], 6, hidden)
    return out


def row_modulation(mod: np.ndarray, tags, ts_idx, chunk: int) -> np.ndarray:
    """Per-row [L, hidden] slice of the table selected by (tag, timestep index);
    zero for padding rows."""
    tags = np.asarray(tags)
    ts = np.asarray(ts_idx)
    out = np.zeros((tags.size, mod.shape[-1]))
    real = tags >= 0
    out[real] = mod[tags[real], ts[real], chunk]
    return out


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def ln_modulate(x: np.ndarray, mod: np.ndarray, tags, ts_idx, which: str, eps: float):
    """LN(x) * (1 + scale) + shift with (shift, scale) of the attention ('a') or
    feed-forward ('f') half, gathered per row by (tag, timestep index)."""
    sh, sc = (SHIFT_A, SCALE_A) if which == "a" else (SHIFT_F, SCALE_F)
    shift = row_modulation(mod, tags, ts_idx, sh)
    scale = row_modulation(mod, tags, ts_idx, sc)
    return layer_norm(x, eps) * (1.0 + scale) + shift


def silu(z):
    return z / (1.0 + np.exp(-z))


def block_forward(inp: dict, rows=None, store_bf16: bool = True, eps: float = 1e-5,
                  qk_eps: float = 1e-5, F: int = 16, theta: float = 10000.0,
                  wq=1.0, wk=1.0, mod: np.ndarray | None = None,
                  return_intermediates: bool = False, fused_qkv: bool = False,
                  pos_scale=None):
    """x2 for the listed rows (all rows when ``rows`` is None).

    ``fused_qkv``: the QKV projection hands its Q and K columns straight to
    the QK-norm + RoPE (the engine page's fused QK normalisation/RoPE kernel)
    without storing them, so in storage mode Q and K are not rounded to bf16
    before the norm (V, Q' and K' still are)."""
    lay = inp["layout"]
    tags, ts = lay["tags"], lay["ts_idx"]
    L, hidden, H, D, ffn = inp["L"], inp["hidden"], inp["heads"], inp["head_dim"], inp["ffn"]
    HD = H * D
    rows = np.arange(L) if rows is None else np.asarray(rows)
    st = bf16_storage if store_bf16 else (lambda z: z)

    if mod is None:
        mod = adaln_table(inp["temb"], inp["w_ada"])
    x = bf16_to_f64(inp["x"])                                        # [L, hidden]
    a = st(ln_modulate(x, mod, tags, ts, "a", eps))                  # all rows (K, V)
    w_qkv = bf16_to_f64(inp["w_qkv"])
    st_qk = (lambda z: z) if fused_qkv else st
    kv = a @ w_qkv[HD:].T                                            # [L, 2*HD]
    kv = np.concatenate([st_qk(kv[:, :HD]), st(kv[:, HD:])], axis=1)
    qr = st_qk(a[rows] @ w_qkv[:HD].T)                               # [n, HD]

    # the attention path on stored bf16 Q, K, V
    q_all = np.zeros((L, HD))
    q_all[rows] = qr
    qn = qk_norm_rope(q_all, H, D, wq, lay["pos"], F, theta, qk_eps, pos_scale)
    kn = qk_norm_rope(kv[:, :HD], H, D, wk, lay["pos"], F, theta, qk_eps, pos_scale)
    if store_bf16:
        qn, kn = stored_query(qn, D), bf16_storage(kn)
    v = kv[:, HD:].reshape(L, H, D)
    o, _ = attention(qn, kn, v, tags, rows=rows)
    o = st(o.reshape(rows.size, HD))

    gate_a = row_modulation(mod, tags, ts, GATE_A)[rows]
    gate_f = row_modulation(mod, tags, ts, GATE_F)[rows]
    x1 = st(x[rows] + gate_a * (o @ bf16_to_f64(inp["w_o"]).T))
    b = st(ln_modulate(x1, mod, tags[rows], ts[rows], "f", eps))
    w_fc1 = bf16_to_f64(inp["w_fc1"])
    g = b @ w_fc1[:ffn].T
    u = b @ w_fc1[ffn:].T
    h = st(silu(g) * u)
    x2 = st(x1 + gate_f * (h @ bf16_to_f64(inp["w_fc2"]).T))
    if return_intermediates:
        return x2, {"mod": mod, "a": a, "q": qr, "kv": kv, "qn": qn, "kn": kn, "o": o,
                    "x1": x1, "b": b, "h": h}
    return x2
