"""Seeded synthetic inputs for the packed masked attention path.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle.  It draws random numbers and lays out the packed sequence; it holds
none of the method's arithmetic (no norm, rotation, softmax or projection).

Packed layout (pages: "MiniMaxH3Transformer3DModel", intro and forward
parameters): one 1-D sequence of rows, each row tagged 0 video, 1 text,
2 audio, or -1 for padding; per-row (t, h, w) rotary coordinates; per-row
timestep indices; three ascending index tensors naming the video, audio and
text rows.

Row order used here: text rows, then video rows in (t, h, w) row-major order,
then audio rows, then padding rows at the tail (the tail split into its own
document follows the class description of the same page).  Positions: video
rows carry their grid coordinate; text and audio rows carry (i, 0, 0) with i
their index inside their own run; padding rows carry (0, 0, 0).

Random numbers: numpy Generator(PCG64(seed)); floats drawn with
standard_normal(dtype=float32) in C order, scaled, then rounded to bf16 with
round-to-nearest-even on the float32 bit pattern.  Draw order: Q, K, V, then
random timestep indices, then (block inputs) x, temb, W_ada, W_qkv, W_o,
W_fc1, W_fc2.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TAG_VIDEO, TAG_TEXT, TAG_AUDIO, TAG_PAD = 0, 1, 2, -1


@dataclass(frozen=True)
class Workload:
    name: str
    L: int
    text: int
    video: tuple  # (t, h, w) grid
    audio: int
    pad: int
    H: int = 56
    D: int = 128
    T: int = 1
    random_ts: bool = False
    seed: int = 0
    block: bool = False
    hidden: int = 5376
    ffn: int = 14336
    temb_dim: int = 2688
    weight_std: float = 0.02
    extra: dict = field(default_factory=dict)

    @property
    def n_video(self) -> int:
        t, h, w = self.video
        return t * h * w


# The five workloads: tiny CPU-checkable, mask-free 4k, masked 16k (the
# headline), full block at 8k, long 32k.
WORKLOADS = {
    "tiny_L256": Workload("tiny_L256", 256, 32, (3, 8, 8), 16, 16, H=4, seed=0),
    "nopad_L4096": Workload("nopad_L4096", 4096, 256, (6, 20, 30), 240, 0, seed=1),
    "masked_L16384": Workload("masked_L16384", 16384, 512, (9, 40, 40), 656, 816, seed=2),
    "block_L8192": Workload("block_L8192", 8192, 512, (12, 20, 30), 480, 0, seed=3,
                            block=True),
    "long_L32768": Workload("long_L32768", 32768, 1024, (12, 40, 64), 1024, 0, T=2,
                            random_ts=True, seed=4),
}
WORKLOAD_ORDER = ["tiny_L256", "nopad_L4096", "masked_L16384", "block_L8192", "long_L32768"]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[WORKLOAD_ORDER[name_or_index]]
    return WORKLOADS[name_or_index]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns (nearest, ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def layout_from_counts(text: int, video: tuple, audio: int, pad: int, T: int = 1,
                       ts_idx=None) -> dict:
    """Build the packed layout (text, video grid, audio, padding tail)."""
    t, h, w = video
    nv = t * h * w
    L = text + nv + audio + pad
    tags = np.empty(L, dtype=np.int32)
    pos = np.zeros((L, 3), dtype=np.int32)
    o = 0
    tags[o:o + text] = TAG_TEXT
    pos[o:o + text, 0] = np.arange(text)
    o += text
    tags[o:o + nv] = TAG_VIDEO
    tt, hh, ww = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")
    pos[o:o + nv, 0] = tt.ravel()
    pos[o:o + nv, 1] = hh.ravel()
    pos[o:o + nv, 2] = ww.ravel()
    o += nv
    tags[o:o + audio] = TAG_AUDIO
    pos[o:o + audio, 0] = np.arange(audio)
    o += audio
    tags[o:o + pad] = TAG_PAD
    if ts_idx is None:
        ts_idx = np.zeros(L, dtype=np.int32)
    ts_idx = np.asarray(ts_idx, dtype=np.int32).copy()
    ts_idx[tags == TAG_PAD] = 0
    return layout_from_tags(tags, pos, ts_idx, T)


def layout_from_tags(tags, pos, ts_idx, T: int) -> dict:
    tags = np.ascontiguousarray(tags, dtype=np.int32)
    return {
        "L": int(tags.size),
        "T": int(T),
        "tags": tags,
        "pos": np.ascontiguousarray(pos, dtype=np.int32).reshape(-1, 3),
        "ts_idx": np.ascontiguousarray(ts_idx, dtype=np.int32),
        "video_idx": np.flatnonzero(tags == TAG_VIDEO).astype(np.int32),
        "audio_idx": np.flatnonzero(tags == TAG_AUDIO).astype(np.int32),
        "text_idx": np.flatnonzero(tags == TAG_TEXT).astype(np.int32),
    }


def random_layout(rng: np.random.Generator, L: int, pad_frac: float = 0.1,
                  T: int = 1, scattered: bool = True, max_pos: int = 64) -> dict:
    """A random layout with random tags (padding scattered or at the tail)."""
    u = rng.random(L)
    tags = rng.integers(0, 3, size=L).astype(np.int32)
    if scattered:
        tags[u < pad_frac] = TAG_PAD
    else:
        npad = int(round(pad_frac * L))
        if npad:
            tags[L - npad:] = TAG_PAD
    pos = rng.integers(0, max_pos, size=(L, 3)).astype(np.int32)
    pos[tags == TAG_PAD] = 0
    ts = rng.integers(0, T, size=L).astype(np.int32)
    ts[tags == TAG_PAD] = 0
    return layout_from_tags(tags, pos, ts, T)


def make_attention_inputs(wl: Workload) -> dict:
    """Q, K, V as bf16 bits [L, H, D] ~ N(0, 1), plus the layout."""
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    shape = (wl.L, wl.H, wl.D)
    q = normal_bf16(rng, shape)
    k = normal_bf16(rng, shape)
    v = normal_bf16(rng, shape)
    ts = rng.integers(0, wl.T, size=wl.L).astype(np.int32) if wl.random_ts else None
    lay = layout_from_counts(wl.text, wl.video, wl.audio, wl.pad, wl.T, ts)
    assert lay["L"] == wl.L
    return {"q": q, "k": k, "v": v, "layout": lay, "H": wl.H, "D": wl.D}


def make_layout(wl: Workload) -> dict:
    """The workload's layout alone (replays the stream when timestep indices
    are drawn after Q, K and V)."""
    if wl.random_ts:
        return make_attention_inputs(wl)["layout"]
    return layout_from_counts(wl.text, wl.video, wl.audio, wl.pad, wl.T)


def make_block_inputs(L: int, hidden: int, heads: int, head_dim: int, ffn: int,
                      temb_dim: int, T: int = 1, seed: int = 3, weight_std: float = 0.02,
                      layout: dict | None = None, text=None, video=None, audio=None,
                      pad: int = 0) -> dict:
    """Residual rows x ~ N(0,1), timestep embedding ~ N(0,1), weights ~ N(0, std).

    Weights are stored [out, in] (row j holds the input weights of output j):
      w_ada [3, 6*hidden, temb_dim]  (one projection per modality tag)
      w_qkv [3*heads*head_dim, hidden]  rows: Q heads | K heads | V heads
      w_o   [hidden, heads*head_dim]
      w_fc1 [2*ffn, hidden]  rows: gate half | up half
      w_fc2 [hidden, ffn]
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    hd = heads * head_dim
    x = normal_bf16(rng, (L, hidden))
    temb = normal_bf16(rng, (T, temb_dim))
    w_ada = normal_bf16(rng, (3, 6 * hidden, temb_dim), weight_std)
    w_qkv = normal_bf16(rng, (3 * hd, hidden), weight_std)
    w_o = normal_bf16(rng, (hidden, hd), weight_std)
    w_fc1 = normal_bf16(rng, (2 * ffn, hidden), weight_std)
    w_fc2 = normal_bf16(rng, (hidden, ffn), weight_std)
    if layout is None:
        layout = layout_from_counts(text, video, audio, pad, T)
    assert layout["L"] == L
    return {"x": x, "temb": temb, "w_ada": w_ada, "w_qkv": w_qkv, "w_o": w_o,
            "w_fc1": w_fc1, "w_fc2": w_fc2, "layout": layout, "L": L, "hidden": hidden,
            "heads": heads, "head_dim": head_dim, "ffn": ffn, "temb_dim": temb_dim}


def token_reduction_plan(layout: dict, target_ts=None) -> dict:
    """Pair horizontally adjacent target-video rows of a packed layout.

    Layout construction only (the caller's job): rows are taken in sequence
    order; a video row at (t, h, 2j) whose next row is the video row at
    (t, h, 2j + 1) forms a pair when both are target rows (timestep index
    == target_ts, or every video row when target_ts is None).  Every other
    row stays on its own.  Returns src0/src1 ([n_reduced], src1 = -1 for an
    unpaired row) and the reduced layout, whose positions are in half units
    (every coordinate doubled; a pair sits at w = 4j + 1, i.e. 2j + 1/2 in
    full units), to be used with a position scale of 1/2 on every axis."""
    tags, pos, ts = layout["tags"], layout["pos"], layout["ts_idx"]
    L = tags.size
    target = (tags == TAG_VIDEO) & ((ts == target_ts) if target_ts is not None else True)
    src0, src1 = [], []
    i = 0
    while i < L:
        if (i + 1 < L and target[i] and target[i + 1] and pos[i, 2] % 2 == 0
                and pos[i + 1, 0] == pos[i, 0] and pos[i + 1, 1] == pos[i, 1]
                and pos[i + 1, 2] == pos[i, 2] + 1):
            src0.append(i)
            src1.append(i + 1)
            i += 2
        else:
            src0.append(i)
            src1.append(-1)
            i += 1
    src0 = np.asarray(src0, np.int32)
    src1 = np.asarray(src1, np.int32)
    rpos = 2 * pos[src0].astype(np.int64)
    paired = src1 >= 0
    rpos[paired, 2] += 1
    red = layout_from_tags(tags[src0], rpos.astype(np.int32), ts[src0], layout["T"])
    return {"src0": src0, "src1": src1, "layout": red, "pos_scale": (0.5, 0.5, 0.5)}


def normal_f32(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def make_io_inputs(layout: dict, hidden: int = 5376, video_channels: int = 96,
                   audio_channels: int = 32, video_out: int = 96, audio_out: int = 32,
                   freq_dim: int = 256, inner_dim: int = 5376, temb_dim: int = 2688,
                   seed: int = 5, timesteps=None) -> dict:
    """Inputs of the steps either side of the block stack.

    Draw order (fp32 unless noted): timesteps ~ U[0, 1) [T] (unless given),
    w1 [inner, freq] ~ N(0, 1/freq), b1 [inner] ~ N(0, 0.02^2),
    w2 [temb, inner] ~ N(0, 1/inner), b2 [temb] ~ N(0, 0.02^2),
    video rows [num_video, video_channels] ~ N(0, 1),
    w_video [hidden, video_channels] ~ N(0, 1/video_channels), b_video ~ N(0, 0.02^2),
    audio rows / w_audio / b_audio likewise, text rows bf16 [num_text, hidden] ~ N(0, 1),
    w_mod [2, 2*hidden, temb] ~ N(0, 0.02^2), w_vout [video_out, hidden] ~ N(0, 1/hidden),
    b_vout ~ N(0, 0.02^2), w_aout / b_aout likewise, x bf16 [L, hidden] ~ N(0, 1).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    T = int(layout["T"])
    nv, na, nt = (int(np.asarray(layout[k]).size) for k in ("video_idx", "audio_idx", "text_idx"))
    if timesteps is None:
        t = rng.random(T, dtype=np.float32)
    else:
        t = np.asarray(timesteps, dtype=np.float32).reshape(T)
    out = {"t": t}
    out["w1"] = normal_f32(rng, (inner_dim, freq_dim), freq_dim ** -0.5)
    out["b1"] = normal_f32(rng, (inner_dim,), 0.02)
    out["w2"] = normal_f32(rng, (temb_dim, inner_dim), inner_dim ** -0.5)
    out["b2"] = normal_f32(rng, (temb_dim,), 0.02)
    out["video"] = normal_f32(rng, (nv, video_channels))
    out["w_video"] = normal_f32(rng, (hidden, video_channels), video_channels ** -0.5)
    out["b_video"] = normal_f32(rng, (hidden,), 0.02)
    out["audio"] = normal_f32(rng, (na, audio_channels))
    out["w_audio"] = normal_f32(rng, (hidden, audio_channels), audio_channels ** -0.5)
    out["b_audio"] = normal_f32(rng, (hidden,), 0.02)
    out["text"] = normal_bf16(rng, (nt, hidden))
    out["w_mod"] = normal_f32(rng, (2, 2 * hidden, temb_dim), 0.02)
    out["w_vout"] = normal_f32(rng, (video_out, hidden), hidden ** -0.5)
    out["b_vout"] = normal_f32(rng, (video_out,), 0.02)
    out["w_aout"] = normal_f32(rng, (audio_out, hidden), hidden ** -0.5)
    out["b_aout"] = normal_f32(rng, (audio_out,), 0.02)
    out["x"] = normal_bf16(rng, (int(layout["L"]), hidden))
    out.update(layout=layout, hidden=hidden, video_channels=video_channels,
               audio_channels=audio_channels, video_out=video_out, audio_out=audio_out,
               freq_dim=freq_dim, inner_dim=inner_dim, temb_dim=temb_dim)
    return out


def make_block_workload(wl: Workload) -> dict:
    return make_block_inputs(wl.L, wl.hidden, wl.H, wl.D, wl.ffn, wl.temb_dim, wl.T,
                             wl.seed, wl.weight_std, text=wl.text, video=wl.video,
                             audio=wl.audio, pad=wl.pad)
