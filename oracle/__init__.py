"""CPU oracle for the packed masked attention path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``packed_masked_attention_amd`` and never imports it; the only code both
sides use is the seeded input generator ``packed_masked_attention_amd.synth``,
which holds none of the method's arithmetic.

The arithmetic lives in ``oracle.c`` (fp64 definition, plus an fp32 twin of
the attention loop used only for CPU timing) and ``block.py`` (the DiT block
composed in numpy fp64).  Pages are cited by title and section in those files.

Parity pins (tests/test_oracle_*.py) tie every function here to something
other than itself: library routines (torch fp64 SDPA, layer_norm, rms_norm,
silu, numpy matmul), closed forms, invariants and hand-derived tile counts.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build (tests/run_sanitizers.py)
_SAN_PATH = os.path.join(_HERE, "liboracle_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g"]
_lock = threading.Lock()
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_f32p = ctypes.POINTER(ctypes.c_float)


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math); with
    sanitize, into liboracle_san.so under ASan + UBSan (loaded instead when
    ORACLE_SANITIZED=1, with gcc's ASan runtime preloaded)."""
    out = _SAN_PATH if sanitize else _LIB_PATH
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(_SRC):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", *(SAN_FLAGS if sanitize else []),
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def lib():
    global _lib
    with _lock:
        if _lib is None:
            san = os.environ.get("ORACLE_SANITIZED") == "1"
            L = ctypes.CDLL(build(force=False, sanitize=san))
            L.oracle_bf16_value.restype = ctypes.c_double
            L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
            L.oracle_bf16_round.restype = ctypes.c_uint16
            L.oracle_bf16_round.argtypes = [ctypes.c_double]
            L.oracle_bf16_to_f64.argtypes = [_u16p, _f64p, ctypes.c_int64]
            L.oracle_bf16_round_array.argtypes = [_f64p, _u16p, ctypes.c_int64]
            L.oracle_layout_status.restype = ctypes.c_int32
            L.oracle_layout_status.argtypes = [
                ctypes.c_int32, ctypes.c_int32, _i32p, _i32p, _i32p,
                _i32p, ctypes.c_int32, _i32p, ctypes.c_int32, _i32p, ctypes.c_int32,
                _i32p]
            L.oracle_layout_doc.argtypes = [ctypes.c_int32, _i32p, _i32p]
            L.oracle_layout_tiles.argtypes = [ctypes.c_int32, _i32p, ctypes.c_int32,
                                              ctypes.c_int32, _u8p, _i32p, _i32p, _i32p]
            L.oracle_allowed_pairs.restype = ctypes.c_int64
            L.oracle_allowed_pairs.argtypes = [ctypes.c_int32, _i32p]
            L.oracle_inv_freq.argtypes = [ctypes.c_int32, ctypes.c_double, _f64p]
            L.oracle_qk_norm_rope.argtypes = [
                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                ctypes.c_double, ctypes.c_double, _f64p, ctypes.c_int64, _f64p,
                _i32p, _f64p, _f64p]
            for name, p in (("oracle_attention_f64", _f64p), ("oracle_attention_f32", _f32p)):
                fn = getattr(L, name)
                fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, p, p, p,
                               _i32p, ctypes.c_double, _i32p, ctypes.c_int32, p, p]
            L.oracle_num_threads.restype = ctypes.c_int32
            _lib = L
    return _lib


def _ptr(a: np.ndarray, t):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(t)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


# ---------------------------------------------------------------- bf16 ----

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    lib().oracle_bf16_to_f64(_ptr(bits, _u16p), _ptr(out, _f64p), bits.size)
    return out


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 bit patterns, nearest with ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_bf16_round_array(_ptr(x, _f64p), _ptr(out, _u16p), x.size)
    return out


def bf16_storage(x: np.ndarray) -> np.ndarray:
    """Value a tensor holds after being stored as bf16 (fp64 result)."""
    return bf16_to_f64(bf16_round(x))


def stored_query(qn: np.ndarray, D: int = 128) -> np.ndarray:
    """Normalised, rotated queries as the GPU path stores them: rounded to bf16
    after multiplication by log2(e)/sqrt(D) (its attention kernel takes exp2 of
    the raw product), returned with that factor divided out in fp64."""
    c = np.log2(np.e) / np.sqrt(D)
    return bf16_storage(qn * c) / c


# -------------------------------------------------------------- layout ----

def layout_status(layout: dict) -> tuple[int, int]:
    tags = _i32(layout["tags"])
    L = tags.shape[0]
    pos = _i32(layout["pos"]).reshape(L, 3)
    ts = _i32(layout["ts_idx"])
    vid, aud, txt = (_i32(layout[k]) for k in ("video_idx", "audio_idx", "text_idx"))
    err = np.zeros(1, dtype=np.int32)
    st = lib().oracle_layout_status(
        L, int(layout["T"]), _ptr(tags, _i32p), _ptr(pos, _i32p), _ptr(ts, _i32p),
        _ptr(vid, _i32p), vid.size, _ptr(aud, _i32p), aud.size, _ptr(txt, _i32p),
        txt.size, _ptr(err, _i32p))
    return int(st), int(err[0])


def layout_doc(tags) -> np.ndarray:
    tags = _i32(tags)
    doc = np.empty_like(tags)
    lib().oracle_layout_doc(tags.size, _ptr(tags, _i32p), _ptr(doc, _i32p))
    return doc


def layout_tiles(tags, bm: int, bn: int):
    """Return (cls[nqt,nkt] uint8, count[nqt], list[nqt,nkt] (-1 padded), order[nqt])."""
    tags = _i32(tags)
    L = tags.size
    nqt, nkt = -(-L // bm), -(-L // bn)
    cls = np.empty((nqt, nkt), dtype=np.uint8)
    count = np.empty(nqt, dtype=np.int32)
    lst = np.empty((nqt, nkt), dtype=np.int32)
    order = np.empty(nqt, dtype=np.int32)
    lib().oracle_layout_tiles(L, _ptr(tags, _i32p), bm, bn, _ptr(cls, _u8p),
                              _ptr(count, _i32p), _ptr(lst, _i32p), _ptr(order, _i32p))
    return cls, count, lst, order


def allowed_pairs(tags) -> int:
    tags = _i32(tags)
    return int(lib().oracle_allowed_pairs(tags.size, _ptr(tags, _i32p)))


# --------------------------------------------------------- norm + RoPE ----

def inv_freq(F: int, theta: float) -> np.ndarray:
    out = np.empty(F, dtype=np.float64)
    lib().oracle_inv_freq(F, theta, _ptr(out, _f64p))
    return out


def qk_norm_rope(x: np.ndarray, H: int, D: int, weight, pos, F: int = 16,
                 theta: float = 10000.0, eps: float = 1e-5, pos_scale=None) -> np.ndarray:
    """x: bf16 bits (uint16) or real values, [L, ld] (ld >= H*D) or [L, H, D].
    pos_scale: per-axis scale of the (t, h, w) coordinates (None = 1, 1, 1).
    Returns fp64 [L, H, D]."""
    x = np.asarray(x)
    x = bf16_to_f64(x) if x.dtype == np.uint16 else np.ascontiguousarray(x, np.float64)
    L = x.shape[0]
    x2 = np.ascontiguousarray(x.reshape(L, -1))
    ld = x2.shape[1]
    assert ld >= H * D and 6 * F <= D
    w = np.ascontiguousarray(np.broadcast_to(np.asarray(weight, np.float64), (D,)))
    p = _i32(pos).reshape(L, 3)
    y = np.empty((L, H, D), dtype=np.float64)
    sc = None if pos_scale is None else np.ascontiguousarray(pos_scale, dtype=np.float64).reshape(3)
    lib().oracle_qk_norm_rope(L, H, D, F, float(theta), float(eps), _ptr(x2, _f64p), ld,
                              _ptr(w, _f64p), _ptr(p, _i32p),
                              None if sc is None else _ptr(sc, _f64p), _ptr(y, _f64p))
    return y


# ----------------------------------------------------------- attention ----

def attention(q, k, v, tags, rows=None, scale=None, precision="f64"):
    """q, k, v: [L, H, D] real arrays. Returns (o [n, H, D], lse [n, H])."""
    dt = np.float64 if precision == "f64" else np.float32
    fn = lib().oracle_attention_f64 if precision == "f64" else lib().oracle_attention_f32
    pt = _f64p if precision == "f64" else _f32p
    q = np.ascontiguousarray(q, dtype=dt)
    k = np.ascontiguousarray(k, dtype=dt)
    v = np.ascontiguousarray(v, dtype=dt)
    L, H, D = q.shape
    tags = _i32(tags)
    rows = np.arange(L, dtype=np.int32) if rows is None else _i32(rows)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.empty((rows.size, H, D), dtype=dt)
    lse = np.empty((rows.size, H), dtype=dt)
    fn(L, H, D, _ptr(q, pt), _ptr(k, pt), _ptr(v, pt), _ptr(tags, _i32p), float(scale),
       _ptr(rows, _i32p), rows.size, _ptr(o, pt), _ptr(lse, pt))
    return o, lse


def attention_path(q_bits, k_bits, v_bits, layout: dict, H: int, D: int = 128,
                   rows=None, wq=1.0, wk=1.0, F: int = 16, theta: float = 10000.0,
                   eps: float = 1e-5, store_qk_bf16: bool = False, precision="f64",
                   pos_scale=None):
    """QK-RMSNorm + 3-axis RoPE on Q and K, then masked attention.

    Inputs are bf16 bit arrays [L, H, D] (or [L, ld] with head h at column h*D).
    ``store_qk_bf16`` rounds the normalised, rotated Q and K to bf16 as the
    GPU path stores them between its two kernels: K as it is, Q multiplied by
    the logit factor log2(e)/sqrt(D) (the stored query operand carries the
    softmax scale and the base change to exp2), the factor then divided out
    in fp64.  Otherwise the path stays in fp64 end to end.
    """
    L = np.asarray(q_bits).shape[0]
    pos = layout["pos"]
    qn = qk_norm_rope(q_bits, H, D, wq, pos, F, theta, eps, pos_scale)
    kn = qk_norm_rope(k_bits, H, D, wk, pos, F, theta, eps, pos_scale)
    if store_qk_bf16:
        qn = stored_query(qn, D)
        kn = bf16_storage(kn)
    vv = bf16_to_f64(np.ascontiguousarray(v_bits).reshape(L, -1)[:, :H * D]).reshape(L, H, D)
    return attention(qn, kn, vv, layout["tags"], rows=rows, precision=precision)


def num_threads() -> int:
    return int(lib().oracle_num_threads())
