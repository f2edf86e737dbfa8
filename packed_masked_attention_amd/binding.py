"""ctypes binding of libpma (the C ABI in include/pma.h).

Argument marshalling only: every function here forwards to the C entry point
of the same name; all arithmetic runs in libpma's HIP kernels.  Device
buffers are torch CUDA tensors (PyTorch provides memory and streams only) and
are passed as raw pointers.  Loading fails loudly when libpma.so is missing:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpma.so")
if os.environ.get("PMA_SANITIZED") == "1":
    # the host-sanitized build (tests/run_sanitizers.py); needs clang's ASan
    # runtime preloaded
    LIB_PATH = os.path.join(_HERE, "libpma_san.so")

PMA_OK = 0
PMA_ERR_LAYOUT = 5
STATUS_NAMES = ["PMA_OK", "PMA_ERR_NULL", "PMA_ERR_SHAPE", "PMA_ERR_ALIGN", "PMA_ERR_WORKSPACE",
                "PMA_ERR_LAYOUT", "PMA_ERR_DEVICE", "PMA_ERR_UNSUPPORTED"]
TILE_EMPTY, TILE_PARTIAL, TILE_FULL = 0, 1, 2

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class PmaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{name}: {detail}")


class LayoutDesc(ctypes.Structure):
    _fields_ = [("seq_len", _i32), ("num_timesteps", _i32),
                ("token_tags", _vp), ("position_ids", _vp), ("timestep_indices", _vp),
                ("video_indices", _vp), ("audio_indices", _vp), ("text_indices", _vp),
                ("num_video", _i32), ("num_audio", _i32), ("num_text", _i32)]


class Layout(ctypes.Structure):
    _fields_ = [("seq_len", _i32), ("num_timesteps", _i32), ("tile_m", _i32), ("tile_n", _i32),
                ("num_q_tiles", _i32), ("num_k_tiles", _i32),
                ("token_tags", _vp), ("position_ids", _vp), ("timestep_indices", _vp),
                ("doc", _vp), ("tile_class", _vp), ("tile_count", _vp), ("tile_list", _vp),
                ("tile_order", _vp), ("status", _vp), ("scratch", _vp)]


class AttnParams(ctypes.Structure):
    _fields_ = [("num_heads", _i32), ("head_dim", _i32), ("rope_freq_dim", _i32),
                ("rope_theta", ctypes.c_float), ("qk_norm_eps", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("pos_scale", ctypes.c_float * 3)]


class BlockParams(ctypes.Structure):
    _fields_ = [("hidden", _i32), ("ffn_dim", _i32), ("time_embed_dim", _i32),
                ("norm_eps", ctypes.c_float), ("attn", AttnParams)]


class BlockWeights(ctypes.Structure):
    _fields_ = [("w_ada", _vp), ("w_qkv", _vp), ("w_o", _vp), ("w_fc1", _vp), ("w_fc2", _vp),
                ("q_norm_weight", _vp), ("k_norm_weight", _vp)]


class LinearArgs(ctypes.Structure):
    _fields_ = [("M", _i32), ("N", _i32), ("K", _i32), ("A", _vp), ("lda", _i64), ("W", _vp),
                ("ldw", _i64), ("C", _vp), ("ldc", _i64), ("epilogue", _i32), ("R", _vp),
                ("ldr", _i64), ("table", _vp), ("num_timesteps", _i32), ("gate_chunk", _i32),
                ("token_tags", _vp), ("timestep_indices", _vp)]


EPI_STORE, EPI_GATE_RESIDUAL, EPI_SWIGLU = 0, 1, 2


class TembParams(ctypes.Structure):
    _fields_ = [("freq_dim", _i32), ("inner_dim", _i32), ("embed_dim", _i32),
                ("max_period", ctypes.c_float)]


class IoParams(ctypes.Structure):
    _fields_ = [("hidden", _i32), ("video_channels", _i32), ("audio_channels", _i32),
                ("video_out", _i32), ("audio_out", _i32), ("time_embed_dim", _i32),
                ("final_norm_eps", ctypes.c_float)]

_SIGS = {
    "pma_status_string": (ctypes.c_char_p, [_i32]),
    "pma_last_error": (ctypes.c_char_p, []),
    "pma_device_check": (_i32, []),
    "pma_layout_workspace_size": (_i32, [_i32, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)]),
    "pma_layout_build": (_i32, [ctypes.POINTER(LayoutDesc), _i32, _i32, _vp, ctypes.c_size_t, _vp,
                                ctypes.POINTER(Layout)]),
    "pma_layout_read_status": (_i32, [ctypes.POINTER(Layout), _vp, ctypes.POINTER(_i32),
                                      ctypes.POINTER(_i32)]),
    "pma_attention_tiles": (_i32, [ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "pma_attention_padded_len": (_i32, [_i32, ctypes.POINTER(_i32)]),
    "pma_qk_norm_rope": (_i32, [ctypes.POINTER(AttnParams), ctypes.POINTER(Layout), _vp, _i64, _vp,
                                _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pma_flash_workspace_size": (_i32, [ctypes.POINTER(AttnParams), _i32,
                                        ctypes.POINTER(ctypes.c_size_t)]),
    "pma_flash_attention": (_i32, [ctypes.POINTER(AttnParams), ctypes.POINTER(Layout), _vp, _vp,
                                   _vp, _vp, _i64, _vp, _vp, ctypes.c_size_t, _vp]),
    "pma_flash_attention_static": (_i32, [ctypes.POINTER(AttnParams), ctypes.POINTER(Layout), _vp,
                                          _vp, _vp, _vp, _i64, _vp, _vp]),
    "pma_attention_workspace_size": (_i32, [ctypes.POINTER(AttnParams), _i32,
                                            ctypes.POINTER(ctypes.c_size_t)]),
    "pma_attention": (_i32, [ctypes.POINTER(AttnParams), ctypes.POINTER(Layout), _vp, _i64, _vp,
                             _i64, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp, ctypes.c_size_t,
                             _vp]),
    "pma_adaln_table": (_i32, [ctypes.POINTER(BlockParams), _i32, _vp, _vp, _vp, _vp]),
    "pma_ln_modulate": (_i32, [ctypes.POINTER(BlockParams), ctypes.POINTER(Layout), _vp, _i32,
                               _vp, _vp, _vp]),
    "pma_linear": (_i32, [ctypes.POINTER(LinearArgs), _vp]),
    "pma_gate_ln_workspace_size": (_i32, [ctypes.POINTER(BlockParams), _i32,
                                          ctypes.POINTER(ctypes.c_size_t)]),
    "pma_gate_residual_ln_modulate": (_i32, [ctypes.POINTER(BlockParams), ctypes.POINTER(Layout),
                                             _vp, _i64, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i32,
                                             _vp, _vp, ctypes.c_size_t, _vp]),
    "pma_rope_table": (_i32, [ctypes.POINTER(AttnParams), ctypes.POINTER(Layout), _vp, _vp]),
    "pma_qkv_projection": (_i32, [ctypes.POINTER(AttnParams), ctypes.POINTER(Layout), _vp, _i64,
                                  _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pma_block_workspace_size": (_i32, [ctypes.POINTER(BlockParams), _i32,
                                        ctypes.POINTER(ctypes.c_size_t)]),
    "pma_block_forward": (_i32, [ctypes.POINTER(BlockParams), ctypes.POINTER(Layout),
                                 ctypes.POINTER(BlockWeights), _vp, _vp, _vp, _vp,
                                 ctypes.c_size_t, _vp]),
    "pma_stack_workspace_size": (_i32, [ctypes.POINTER(BlockParams), _i32, _i32,
                                        ctypes.POINTER(ctypes.c_size_t)]),
    "pma_stack_forward": (_i32, [ctypes.POINTER(BlockParams), ctypes.POINTER(Layout), _i32,
                                 ctypes.POINTER(BlockWeights), _vp, _vp, _vp, _vp,
                                 ctypes.c_size_t, _vp]),
    "pma_refiner_workspace_size": (_i32, [ctypes.POINTER(BlockParams), _i32, _i32,
                                          ctypes.POINTER(ctypes.c_size_t)]),
    "pma_text_refiner": (_i32, [ctypes.POINTER(BlockParams), ctypes.POINTER(Layout), _i32,
                                ctypes.POINTER(BlockWeights), _vp, _vp, _i64, _i32, _vp,
                                ctypes.c_float, _vp, _vp, ctypes.c_size_t, _vp]),
    "pma_token_merge": (_i32, [_i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "pma_token_restore": (_i32, [_i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pma_token_plan_check": (_i32, [_i32, _i32, _vp, _vp, _vp, _vp, ctypes.POINTER(_i32),
                                    ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "pma_timestep_embed": (_i32, [ctypes.POINTER(TembParams), _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp]),
    "pma_pack_rows": (_i32, [ctypes.POINTER(IoParams), ctypes.POINTER(LayoutDesc), _vp, _vp, _vp,
                             _vp, _vp, _vp, _vp, _i64, _vp, _vp]),
    "pma_head_table": (_i32, [ctypes.POINTER(IoParams), _i32, _vp, _vp, _vp, _vp]),
    "pma_unpack_workspace_size": (_i32, [ctypes.POINTER(IoParams), _i32, _i32,
                                         ctypes.POINTER(ctypes.c_size_t)]),
    "pma_unpack_rows": (_i32, [ctypes.POINTER(IoParams), ctypes.POINTER(LayoutDesc), _vp, _vp,
                               _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
}

_lib = None


def lib():
    """Load libpma.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m packed_masked_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def check(status: int) -> None:
    if status != PMA_OK:
        raise PmaError(status, lib().pma_last_error().decode())


def ptr(t) -> int | None:
    """Device pointer of a torch tensor (None for None)."""
    return None if t is None else t.data_ptr()


def stream_ptr(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# ------------------------------------------------------------------ layout

def pma_layout_workspace_size(seq_len: int, tile_m: int = 0, tile_n: int = 0) -> int:
    n = ctypes.c_size_t()
    check(lib().pma_layout_workspace_size(seq_len, tile_m, tile_n, ctypes.byref(n)))
    return n.value


class DeviceLayout:
    """A built layout: the device arrays of the packed layout, the workspace
    the builder wrote into, and the pma_layout struct."""

    def __init__(self, arrays: dict, workspace, layout: Layout, desc: LayoutDesc):
        self.arrays = arrays
        self.workspace = workspace
        self.struct = layout
        self.desc = desc

    @property
    def seq_len(self) -> int:
        return self.struct.seq_len


def pma_layout_build(layout, device="cuda", tile_m: int = 0, tile_n: int = 0,
                     stream=None) -> DeviceLayout:
    """Build a layout.  ``layout`` is either a host layout dict (see
    synth.layout_from_tags), copied to the device first, or a DeviceLayout,
    rebuilt in place from its device-resident arrays and workspace."""
    import torch
    if isinstance(layout, DeviceLayout):
        dl = layout
        out = Layout()
        check(lib().pma_layout_build(ctypes.byref(dl.desc), dl.struct.tile_m, dl.struct.tile_n,
                                     ptr(dl.workspace), dl.workspace.numel(), stream_ptr(stream),
                                     ctypes.byref(out)))
        dl.struct = out
        return dl
    arr = {}
    for k in ("tags", "pos", "ts_idx", "video_idx", "audio_idx", "text_idx"):
        a = np.ascontiguousarray(np.asarray(layout[k], dtype=np.int32))
        arr[k] = torch.from_numpy(a).to(device) if a.size else None
    L = int(np.asarray(layout["tags"]).size)
    desc = LayoutDesc(L, int(layout["T"]), ptr(arr["tags"]), ptr(arr["pos"]), ptr(arr["ts_idx"]),
                      ptr(arr["video_idx"]), ptr(arr["audio_idx"]), ptr(arr["text_idx"]),
                      int(np.asarray(layout["video_idx"]).size),
                      int(np.asarray(layout["audio_idx"]).size),
                      int(np.asarray(layout["text_idx"]).size))
    nbytes = pma_layout_workspace_size(L, tile_m, tile_n)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    out = Layout()
    check(lib().pma_layout_build(ctypes.byref(desc), tile_m, tile_n, ptr(ws), nbytes,
                                 stream_ptr(stream), ctypes.byref(out)))
    return DeviceLayout(arr, ws, out, desc)


def pma_layout_read_status(dl: DeviceLayout, stream=None) -> tuple[int, int]:
    """(status bits, first bad row); does not raise on a non-zero status."""
    bits, row = _i32(), _i32()
    st = lib().pma_layout_read_status(ctypes.byref(dl.struct), stream_ptr(stream),
                                      ctypes.byref(bits), ctypes.byref(row))
    if st not in (PMA_OK, 5):
        check(st)
    return bits.value, row.value


def layout_arrays(dl: DeviceLayout) -> dict:
    """Copy the built layout's device arrays to host numpy arrays."""
    import torch
    s = dl.struct
    nqt, nkt, L = s.num_q_tiles, s.num_k_tiles, s.seq_len
    ws = dl.workspace
    base = ws.data_ptr()

    def view(p, n, dtype):
        off = p - base
        esz = torch.tensor([], dtype=dtype).element_size()
        return ws[off:off + n * esz].view(dtype).cpu().numpy()

    return {"doc": view(s.doc, L, torch.int32),
            "cls": view(s.tile_class, nqt * nkt, torch.uint8).reshape(nqt, nkt),
            "count": view(s.tile_count, nqt, torch.int32),
            "list": view(s.tile_list, nqt * nkt, torch.int32).reshape(nqt, nkt),
            "order": view(s.tile_order, nqt, torch.int32)}


# --------------------------------------------------------------- attention

def attn_params(H: int, D: int = 128, F: int = 16, theta: float = 10000.0, eps: float = 1e-5,
                scale: float = 0.0, pos_scale=(1.0, 1.0, 1.0)) -> AttnParams:
    return AttnParams(H, D, F, theta, eps, scale, (ctypes.c_float * 3)(*pos_scale))


def pma_attention_tiles() -> tuple[int, int]:
    m, n = _i32(), _i32()
    check(lib().pma_attention_tiles(ctypes.byref(m), ctypes.byref(n)))
    return m.value, n.value


def pma_attention_padded_len(seq_len: int) -> int:
    out = _i32()
    check(lib().pma_attention_padded_len(seq_len, ctypes.byref(out)))
    return out.value


def pma_qk_norm_rope(p: AttnParams, dl: DeviceLayout, q, q_ld, k, k_ld, v, v_ld, wq, wk,
                     qh, kh, vt, stream=None) -> None:
    check(lib().pma_qk_norm_rope(ctypes.byref(p), ctypes.byref(dl.struct), ptr(q), q_ld, ptr(k),
                                 k_ld, ptr(v), v_ld, ptr(wq), ptr(wk), ptr(qh), ptr(kh), ptr(vt),
                                 stream_ptr(stream)))


def pma_rope_table(p: AttnParams, dl: DeviceLayout, table, stream=None) -> None:
    check(lib().pma_rope_table(ctypes.byref(p), ctypes.byref(dl.struct), ptr(table),
                               stream_ptr(stream)))


def pma_qkv_projection(p: AttnParams, dl: DeviceLayout, a, lda, hidden, w_qkv, wq, wk, rope,
                       qh, kh, vt, stream=None) -> None:
    check(lib().pma_qkv_projection(ctypes.byref(p), ctypes.byref(dl.struct), ptr(a), lda, hidden,
                                   ptr(w_qkv), ptr(wq), ptr(wk), ptr(rope), ptr(qh), ptr(kh),
                                   ptr(vt), stream_ptr(stream)))


def pma_flash_workspace_size(p: AttnParams, seq_len: int) -> int:
    n = ctypes.c_size_t()
    check(lib().pma_flash_workspace_size(ctypes.byref(p), seq_len, ctypes.byref(n)))
    return n.value


def pma_flash_attention(p: AttnParams, dl: DeviceLayout, qh, kh, vt, o, o_ld, lse=None,
                        workspace=None, stream=None) -> None:
    """workspace: None (every item whole) or a device buffer of at least
    pma_flash_workspace_size bytes (the last items split over their keys)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().pma_flash_attention(ctypes.byref(p), ctypes.byref(dl.struct), ptr(qh), ptr(kh),
                                    ptr(vt), ptr(o), o_ld, ptr(lse), ptr(workspace), nbytes,
                                    stream_ptr(stream)))


def pma_flash_attention_static(p: AttnParams, dl: DeviceLayout, qh, kh, vt, o, o_ld, lse=None,
                               stream=None) -> None:
    """pma_flash_attention without a workspace: its scratch is the library's
    static device array (allocates nothing; overlapping calls on one GPU race)."""
    check(lib().pma_flash_attention_static(ctypes.byref(p), ctypes.byref(dl.struct), ptr(qh),
                                           ptr(kh), ptr(vt), ptr(o), o_ld, ptr(lse),
                                           stream_ptr(stream)))


def pma_attention_workspace_size(p: AttnParams, seq_len: int) -> int:
    n = ctypes.c_size_t()
    check(lib().pma_attention_workspace_size(ctypes.byref(p), seq_len, ctypes.byref(n)))
    return n.value


def pma_attention(p: AttnParams, dl: DeviceLayout, q, q_ld, k, k_ld, v, v_ld, wq, wk, o, o_ld,
                  lse=None, workspace=None, stream=None) -> None:
    import torch
    nbytes = pma_attention_workspace_size(p, dl.seq_len)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    check(lib().pma_attention(ctypes.byref(p), ctypes.byref(dl.struct), ptr(q), q_ld, ptr(k),
                              k_ld, ptr(v), v_ld, ptr(wq), ptr(wk), ptr(o), o_ld, ptr(lse),
                              ptr(workspace), workspace.numel(), stream_ptr(stream)))


# ------------------------------------------------------------------- block

def block_params(hidden: int, ffn: int, temb_dim: int, H: int, eps: float = 1e-5,
                 **attn) -> BlockParams:
    return BlockParams(hidden, ffn, temb_dim, eps, attn_params(H, **attn))


def pma_adaln_table(p: BlockParams, num_timesteps: int, temb, w_ada, table, stream=None) -> None:
    check(lib().pma_adaln_table(ctypes.byref(p), num_timesteps, ptr(temb), ptr(w_ada), ptr(table),
                                stream_ptr(stream)))


def pma_ln_modulate(p: BlockParams, dl: DeviceLayout, table, which: int, x, out,
                    stream=None) -> None:
    check(lib().pma_ln_modulate(ctypes.byref(p), ctypes.byref(dl.struct), ptr(table), which,
                                ptr(x), ptr(out), stream_ptr(stream)))


def pma_linear(M, N, K, A, lda, W, ldw, C, ldc, epilogue=EPI_STORE, R=None, ldr=0, table=None,
               num_timesteps=1, gate_chunk=0, tags=None, ts_idx=None, stream=None) -> None:
    args = LinearArgs(M, N, K, ptr(A), lda, ptr(W), ldw, ptr(C), ldc, epilogue, ptr(R), ldr,
                      ptr(table), num_timesteps, gate_chunk, ptr(tags), ptr(ts_idx))
    check(lib().pma_linear(ctypes.byref(args), stream_ptr(stream)))


def pma_gate_ln_workspace_size(p: BlockParams, seq_len: int) -> int:
    n = ctypes.c_size_t()
    check(lib().pma_gate_ln_workspace_size(ctypes.byref(p), seq_len, ctypes.byref(n)))
    return n.value


def pma_gate_residual_ln_modulate(p: BlockParams, dl: DeviceLayout, a, lda: int, K: int, w,
                                  gate_table, gate_chunk: int, x, x1, mod_table, which: int, b,
                                  workspace=None, stream=None) -> None:
    import torch
    if workspace is None:
        workspace = torch.empty(pma_gate_ln_workspace_size(p, dl.seq_len), dtype=torch.uint8,
                                device=x.device)
    check(lib().pma_gate_residual_ln_modulate(
        ctypes.byref(p), ctypes.byref(dl.struct), ptr(a), lda, K, ptr(w), ptr(gate_table),
        gate_chunk, ptr(x), ptr(x1), ptr(mod_table), which, ptr(b), ptr(workspace),
        workspace.numel(), stream_ptr(stream)))


def pma_block_workspace_size(p: BlockParams, seq_len: int) -> int:
    n = ctypes.c_size_t()
    check(lib().pma_block_workspace_size(ctypes.byref(p), seq_len, ctypes.byref(n)))
    return n.value


def pma_block_forward(p: BlockParams, dl: DeviceLayout, w: BlockWeights, table, x_in, x_out,
                      workspace=None, stream=None) -> None:
    import torch
    nbytes = pma_block_workspace_size(p, dl.seq_len)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x_in.device)
    check(lib().pma_block_forward(ctypes.byref(p), ctypes.byref(dl.struct), ctypes.byref(w),
                                  ptr(table), ptr(x_in), ptr(x_out), ptr(workspace),
                                  workspace.numel(), stream_ptr(stream)))


def block_weights_array(ws) -> ctypes.Array:
    """A C array of BlockWeights from a list of them."""
    arr = (BlockWeights * len(ws))()
    for i, w in enumerate(ws):
        arr[i] = w
    return arr


def pma_stack_workspace_size(p: BlockParams, seq_len: int, num_timesteps: int) -> int:
    n = ctypes.c_size_t()
    check(lib().pma_stack_workspace_size(ctypes.byref(p), seq_len, num_timesteps, ctypes.byref(n)))
    return n.value


def pma_stack_forward(p: BlockParams, dl: DeviceLayout, weights, temb, x_in, x_out,
                      workspace=None, stream=None) -> None:
    """weights: list of BlockWeights (or a ctypes array of them), one per block."""
    import torch
    arr = weights if isinstance(weights, ctypes.Array) else block_weights_array(weights)
    nbytes = pma_stack_workspace_size(p, dl.seq_len, dl.struct.num_timesteps)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x_in.device)
    check(lib().pma_stack_forward(ctypes.byref(p), ctypes.byref(dl.struct), len(arr), arr,
                                  ptr(temb), ptr(x_in), ptr(x_out), ptr(workspace),
                                  workspace.numel(), stream_ptr(stream)))


def pma_refiner_workspace_size(p: BlockParams, n_text: int, num_timesteps: int) -> int:
    n = ctypes.c_size_t()
    check(lib().pma_refiner_workspace_size(ctypes.byref(p), n_text, num_timesteps,
                                           ctypes.byref(n)))
    return n.value


def pma_text_refiner(p: BlockParams, dl_text: DeviceLayout, weights, temb, text, text_ld,
                     text_dim, w_text, final_norm_eps, out, workspace=None, stream=None) -> None:
    import torch
    arr = weights if isinstance(weights, ctypes.Array) else block_weights_array(weights)
    nbytes = pma_refiner_workspace_size(p, dl_text.seq_len, dl_text.struct.num_timesteps)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=text.device)
    check(lib().pma_text_refiner(ctypes.byref(p), ctypes.byref(dl_text.struct), len(arr),
                                 arr if len(arr) else None, ptr(temb), ptr(text), text_ld,
                                 text_dim, ptr(w_text), final_norm_eps, ptr(out), ptr(workspace),
                                 workspace.numel(), stream_ptr(stream)))


def pma_token_merge(hidden: int, seq_len: int, src0, src1, x, xr, stream=None) -> None:
    check(lib().pma_token_merge(hidden, seq_len, src0.numel(), ptr(src0), ptr(src1), ptr(x),
                                ptr(xr), stream_ptr(stream)))


def pma_token_restore(hidden: int, seq_len: int, src0, src1, bypass, xr_before, xr_after, x_out,
                      stream=None) -> None:
    check(lib().pma_token_restore(hidden, seq_len, src0.numel(), ptr(src0), ptr(src1),
                                  ptr(bypass), ptr(xr_before), ptr(xr_after), ptr(x_out),
                                  stream_ptr(stream)))


def pma_token_plan_check(seq_len: int, src0, src1, workspace=None, stream=None):
    """(bits, first_bad_entry, first_bad_row) of a token-reduction plan; bits 0 =
    valid.  Synchronises the stream.  workspace: int32 device tensor of at least
    seq_len + 3 entries (allocated here when None)."""
    import torch
    if workspace is None:
        workspace = torch.empty(seq_len + 3, dtype=torch.int32, device=src0.device)
    bits, fe, fr = _i32(), _i32(), _i32()
    st = lib().pma_token_plan_check(seq_len, src0.numel(), ptr(src0), ptr(src1), ptr(workspace),
                                    stream_ptr(stream), ctypes.byref(bits), ctypes.byref(fe),
                                    ctypes.byref(fr))
    if st not in (PMA_OK, PMA_ERR_LAYOUT):
        check(st)
    return bits.value, fe.value, fr.value


# ------------------------------------------------------- input / output path

def temb_params(freq_dim: int = 256, inner_dim: int = 5376, embed_dim: int = 2688,
                max_period: float = 10000.0) -> TembParams:
    return TembParams(freq_dim, inner_dim, embed_dim, max_period)


def io_params(hidden: int = 5376, video_channels: int = 96, audio_channels: int = 32,
              video_out: int = 96, audio_out: int = 32, time_embed_dim: int = 2688,
              final_norm_eps: float = 1e-5) -> IoParams:
    return IoParams(hidden, video_channels, audio_channels, video_out, audio_out, time_embed_dim,
                    final_norm_eps)


def pma_timestep_embed(p: TembParams, num_timesteps: int, timestep, w1, b1, w2, b2, inner, temb,
                       temb_bf16=None, stream=None) -> None:
    check(lib().pma_timestep_embed(ctypes.byref(p), num_timesteps, ptr(timestep), ptr(w1),
                                   ptr(b1), ptr(w2), ptr(b2), ptr(inner), ptr(temb),
                                   ptr(temb_bf16), stream_ptr(stream)))


def pma_pack_rows(p: IoParams, dl: DeviceLayout, video, w_video, b_video, audio, w_audio,
                  b_audio, text, text_ld, x, stream=None) -> None:
    check(lib().pma_pack_rows(ctypes.byref(p), ctypes.byref(dl.desc), ptr(video), ptr(w_video),
                              ptr(b_video), ptr(audio), ptr(w_audio), ptr(b_audio), ptr(text),
                              text_ld, ptr(x), stream_ptr(stream)))


def pma_head_table(p: IoParams, num_timesteps: int, temb, w_mod, table, stream=None) -> None:
    check(lib().pma_head_table(ctypes.byref(p), num_timesteps, ptr(temb), ptr(w_mod), ptr(table),
                               stream_ptr(stream)))


def pma_unpack_workspace_size(p: IoParams, num_video: int, num_audio: int) -> int:
    n = ctypes.c_size_t()
    check(lib().pma_unpack_workspace_size(ctypes.byref(p), num_video, num_audio, ctypes.byref(n)))
    return n.value


def pma_unpack_rows(p: IoParams, dl: DeviceLayout, x, table, w_video_out, b_video_out,
                    w_audio_out, b_audio_out, video_out, audio_out, workspace=None,
                    stream=None) -> None:
    import torch
    d = dl.desc
    nbytes = pma_unpack_workspace_size(p, d.num_video, d.num_audio)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    check(lib().pma_unpack_rows(ctypes.byref(p), ctypes.byref(d), ptr(x), ptr(table),
                                ptr(w_video_out), ptr(b_video_out), ptr(w_audio_out),
                                ptr(b_audio_out), ptr(video_out), ptr(audio_out), ptr(workspace),
                                workspace.numel(), stream_ptr(stream)))
