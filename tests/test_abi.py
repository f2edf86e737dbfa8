"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

from packed_masked_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "pma.h")) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pma_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libpma.so not built")
    return B.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(B.exported_symbols()) | set(names)
    assert set(B.exported_symbols()) <= set(names)


def test_status_strings(lib):
    for code, name in enumerate(B.STATUS_NAMES):
        assert lib.pma_status_string(code).decode() == name


def test_host_side_argument_errors(lib):
    n = ctypes.c_size_t()
    assert lib.pma_layout_workspace_size(0, 128, 64, ctypes.byref(n)) == 2
    assert lib.pma_layout_workspace_size(100, 96, 64, ctypes.byref(n)) == 2
    assert lib.pma_layout_workspace_size(100, 128, 64, None) == 1
    assert lib.pma_layout_workspace_size(1000, 128, 64, ctypes.byref(n)) == 0 and n.value > 0
    m, k = ctypes.c_int32(), ctypes.c_int32()
    assert lib.pma_attention_tiles(ctypes.byref(m), ctypes.byref(k)) == 0
    assert (m.value, k.value) in {(128, 64), (256, 64)}
    out = B.Layout()
    assert lib.pma_layout_build(None, 0, 0, None, 0, None, ctypes.byref(out)) == 1
    d = B.LayoutDesc(100, 1, None, None, None, None, None, None, 0, 0, 0)
    assert lib.pma_layout_build(ctypes.byref(d), 0, 0, None, 0, None, ctypes.byref(out)) == 1
    d = B.LayoutDesc(100, 0, 8, 8, 8, None, None, None, 0, 0, 0)
    assert lib.pma_layout_build(ctypes.byref(d), 0, 0, 256, 1 << 20, None, ctypes.byref(out)) == 2
    d = B.LayoutDesc(100, 1, 256, 256, 256, None, None, None, 0, 0, 0)
    assert lib.pma_layout_build(ctypes.byref(d), 0, 0, 256, 16, None, ctypes.byref(out)) == 4
    assert lib.pma_layout_build(ctypes.byref(d), 0, 0, 264, 1 << 20, None, ctypes.byref(out)) == 3
    assert "aligned" in lib.pma_last_error().decode()
    p = B.attn_params(4, D=64)
    assert lib.pma_attention_workspace_size(ctypes.byref(p), 100, ctypes.byref(n)) == 7
    p = B.attn_params(4, F=12)
    assert lib.pma_attention_workspace_size(ctypes.byref(p), 100, ctypes.byref(n)) == 7
    p = B.attn_params(56)
    fw = ctypes.c_size_t()
    assert lib.pma_flash_workspace_size(ctypes.byref(p), 16384, ctypes.byref(fw)) == 0
    # 256 B of work-queue counters, then 16 split items per XCD (of 56 x 64 / 8
    # = 448) x 4 parts, each 256 rows x (128 channels + max + row sum) fp32,
    # then 1024 workgroups x 4 clock stamps of 8 bytes
    stamps = 1024 * 4 * 8
    assert fw.value == 256 + 8 * 16 * 4 * 256 * 130 * 4 + stamps
    # below 128 k-tiles (8192 keys) nothing is split: the counters alone
    assert lib.pma_flash_workspace_size(ctypes.byref(B.attn_params(2)), 100, ctypes.byref(n)) == 0
    assert n.value == 256
    assert lib.pma_flash_workspace_size(ctypes.byref(B.attn_params(2)), 8128, ctypes.byref(n)) == 0
    assert n.value == 256
    # from 128 k-tiles on: 2 heads x 32 q-tiles, 8 items per XCD, all split;
    # four part slots per item (two used below 12288 keys)
    assert lib.pma_flash_workspace_size(ctypes.byref(B.attn_params(2)), 8192, ctypes.byref(n)) == 0
    assert n.value == 256 + 8 * 8 * 4 * 256 * 130 * 4 + stamps
    assert lib.pma_flash_workspace_size(ctypes.byref(B.attn_params(2)), 12288, ctypes.byref(n)) == 0
    # 2 heads x 48 q-tiles: 12 items per XCD, all 12 split
    assert n.value == 256 + 8 * 12 * 4 * 256 * 130 * 4 + stamps
    assert lib.pma_flash_workspace_size(ctypes.byref(p), 0, ctypes.byref(n)) == 2
    assert lib.pma_attention_workspace_size(ctypes.byref(p), 16384, ctypes.byref(n)) == 0
    assert n.value == 3 * 56 * 16384 * 128 * 2 + fw.value
    lp = ctypes.c_int32()
    assert lib.pma_attention_padded_len(16385, ctypes.byref(lp)) == 0 and lp.value == 16640
    lay = B.Layout()
    assert lib.pma_flash_attention(ctypes.byref(p), ctypes.byref(lay), None, None, None, None, 0,
                                   None, None, 0, None) == 1
    # a layout past the kernel's LDS tile-list capacity is refused on the host
    tm, tn = ctypes.c_int32(), ctypes.c_int32()
    lib.pma_attention_tiles(ctypes.byref(tm), ctypes.byref(tn))
    fake = ctypes.c_void_p(256)
    nk = 6909   # one more than the LDS tile list holds
    big = B.Layout(nk * tn.value, 1, tm.value, tn.value, (nk * tn.value + tm.value - 1) // tm.value,
                   nk, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake)
    assert lib.pma_flash_attention(ctypes.byref(p), ctypes.byref(big), fake, fake, fake, fake,
                                   56 * 128, None, None, 0, None) == 2
    assert "k-tiles" in lib.pma_last_error().decode()
    # a flash workspace that is misaligned or too small
    ok = B.Layout(8192, 1, tm.value, tn.value, 8192 // tm.value, 8192 // tn.value, fake, fake, fake,
                  fake, fake, fake, fake, fake, fake, fake)
    assert lib.pma_flash_workspace_size(ctypes.byref(p), 8192, ctypes.byref(fw)) == 0
    assert lib.pma_flash_attention(ctypes.byref(p), ctypes.byref(ok), fake, fake, fake, fake,
                                   56 * 128, None, ctypes.c_void_p(256 + 64), fw.value, None) == 3
    assert lib.pma_flash_attention(ctypes.byref(p), ctypes.byref(ok), fake, fake, fake, fake,
                                   56 * 128, None, fake, fw.value - 1, None) == 4
    assert "flash workspace" in lib.pma_last_error().decode()


def test_io_path_host_side_argument_errors(lib):
    n = ctypes.c_size_t()
    fake = ctypes.c_void_p(256)
    p = B.io_params()
    assert lib.pma_unpack_workspace_size(ctypes.byref(p), 7200, 480, ctypes.byref(n)) == 0
    # stats (8 B per row) and the K-range partials of every output, each part
    # 256-byte aligned; 7200 rows use 12 ranges of 448 columns, 480 rows 84 of 64
    want = sum((s + 255) // 256 * 256 for s in (8 * 7200, 4 * 12 * 7200 * 96, 8 * 480,
                                                 4 * 84 * 480 * 32))
    assert n.value == want
    for bad in (B.io_params(hidden=100), B.io_params(video_channels=48), B.io_params(audio_out=160),
                B.io_params(time_embed_dim=6), B.io_params(final_norm_eps=-1.0)):
        assert lib.pma_unpack_workspace_size(ctypes.byref(bad), 1, 1, ctypes.byref(n)) == 2
    d = B.LayoutDesc(100, 1, fake, fake, fake, fake, None, None, 10, 0, 0)
    # workspace too small, then misaligned
    assert lib.pma_unpack_rows(ctypes.byref(p), ctypes.byref(d), fake, fake, fake, fake, fake,
                               fake, fake, fake, fake, 16, None) == 4
    assert lib.pma_unpack_rows(ctypes.byref(p), ctypes.byref(d), fake, fake, fake, fake, fake,
                               fake, fake, fake, ctypes.c_void_p(264), 1 << 24, None) == 3
    d9 = B.LayoutDesc(100, 9, fake, fake, fake, fake, None, None, 10, 0, 0)
    assert lib.pma_unpack_rows(ctypes.byref(p), ctypes.byref(d9), fake, fake, fake, fake, fake,
                               fake, fake, fake, fake, 1 << 24, None) == 2
    # counts beyond seq_len; an index array missing for a non-zero count
    d2 = B.LayoutDesc(100, 1, fake, fake, fake, fake, fake, fake, 60, 30, 20)
    assert lib.pma_pack_rows(ctypes.byref(p), ctypes.byref(d2), fake, fake, fake, fake, fake, fake,
                             fake, 5376, fake, None) == 2
    d3 = B.LayoutDesc(100, 1, fake, fake, fake, None, fake, fake, 10, 0, 0)
    assert lib.pma_pack_rows(ctypes.byref(p), ctypes.byref(d3), fake, fake, fake, fake, fake, fake,
                             fake, 5376, fake, None) == 1
    d4 = B.LayoutDesc(100, 1, fake, fake, fake, fake, fake, fake, 10, 0, 5)
    assert lib.pma_pack_rows(ctypes.byref(p), ctypes.byref(d4), fake, fake, fake, fake, fake, fake,
                             fake, 5370, fake, None) == 2
    assert "text_ld" in lib.pma_last_error().decode()
    tp = B.temb_params()
    assert lib.pma_timestep_embed(ctypes.byref(tp), 9, fake, fake, fake, fake, fake, fake, fake,
                                  None, None) == 2
    tp_bad = B.temb_params(freq_dim=254)
    assert lib.pma_timestep_embed(ctypes.byref(tp_bad), 1, fake, fake, fake, fake, fake, fake,
                                  fake, None, None) == 2
    assert lib.pma_head_table(ctypes.byref(p), 0, fake, fake, fake, None) == 2
    assert lib.pma_head_table(ctypes.byref(p), 1, ctypes.c_void_p(260), fake, fake, None) == 3


def test_stack_and_refiner_host_side_argument_errors(lib):
    n = ctypes.c_size_t()
    fake = ctypes.c_void_p(256)
    p = B.block_params(5376, 14336, 2688, 56)
    blk = ctypes.c_size_t()
    assert lib.pma_block_workspace_size(ctypes.byref(p), 8192, ctypes.byref(blk)) == 0
    assert lib.pma_stack_workspace_size(ctypes.byref(p), 8192, 1, ctypes.byref(n)) == 0
    # block workspace + AdaLN table [3][1][6][5376] fp32 + one residual buffer
    assert n.value == blk.value + 3 * 6 * 5376 * 4 + 8192 * 5376 * 2
    assert lib.pma_stack_workspace_size(ctypes.byref(p), 8192, 0, ctypes.byref(n)) == 2
    lay = B.Layout(8192, 1, 256, 64, 32, 128, fake, fake, fake, fake, fake, fake, fake, fake,
                   fake, fake)
    w = B.block_weights_array([B.BlockWeights(256, 256, 256, 256, 256, 256, 256)])
    assert lib.pma_stack_forward(ctypes.byref(p), ctypes.byref(lay), 0, w, fake, fake,
                                 ctypes.c_void_p(512), fake, 1 << 40, None) == 2
    assert lib.pma_stack_forward(ctypes.byref(p), ctypes.byref(lay), 1, w, fake, fake, fake,
                                 fake, 1 << 40, None) == 2          # x_out aliases x_in
    w0 = B.block_weights_array([B.BlockWeights(256, 256, None, 256, 256, 256, 256)])
    assert lib.pma_stack_forward(ctypes.byref(p), ctypes.byref(lay), 1, w0, fake, fake,
                                 ctypes.c_void_p(512), fake, 1 << 40, None) == 1
    assert lib.pma_stack_forward(ctypes.byref(p), ctypes.byref(lay), 1, w, fake, fake,
                                 ctypes.c_void_p(512), fake, 1024, None) == 4
    assert lib.pma_refiner_workspace_size(ctypes.byref(p), 512, 1, ctypes.byref(n)) == 0
    assert lib.pma_text_refiner(ctypes.byref(p), ctypes.byref(lay), 2, w, fake, fake, 5120, 5000,
                                fake, ctypes.c_float(1e-5), fake, fake, 1 << 40, None) == 2
    assert lib.pma_text_refiner(ctypes.byref(p), ctypes.byref(lay), 2, w, fake, fake, 5120, 5120,
                                fake, ctypes.c_float(-1.0), fake, fake, 1 << 40, None) == 2


def test_token_reduction_host_side_argument_errors(lib):
    fake = ctypes.c_void_p(256)
    out = ctypes.c_int32()
    # merge / restore: hidden not a multiple of 8, more reduced rows than rows, NULLs
    assert lib.pma_token_merge(60, 100, 50, fake, fake, fake, fake, None) == 2
    assert lib.pma_token_merge(64, 100, 101, fake, fake, fake, fake, None) == 2
    assert lib.pma_token_merge(64, 100, 50, None, fake, fake, fake, None) == 1
    assert lib.pma_token_merge(64, 100, 50, fake, fake, ctypes.c_void_p(264), fake, None) == 3
    assert lib.pma_token_restore(64, 100, 50, fake, fake, fake, fake, None, fake, None) == 1
    # plan check: shape and NULL workspace before any device work
    assert lib.pma_token_plan_check(0, 0, fake, fake, fake, None, ctypes.byref(out), None,
                                    None) == 2
    assert lib.pma_token_plan_check(100, 101, fake, fake, fake, None, None, None, None) == 2
    assert lib.pma_token_plan_check(100, 50, fake, fake, None, None, None, None, None) == 1
    assert lib.pma_token_plan_check(100, 50, fake, fake, ctypes.c_void_p(258), None, None, None,
                                    None) == 3


def test_gate_ln_host_side_argument_errors(lib):
    n = ctypes.c_size_t()
    fake = ctypes.c_void_p(256)
    p = B.block_params(5376, 14336, 2688, 56)
    # at most hidden / 128 = 42 (mean, M2) fp32 pairs per row
    assert lib.pma_gate_ln_workspace_size(ctypes.byref(p), 8192, ctypes.byref(n)) == 0
    assert n.value == 8192 * 42 * 8
    assert lib.pma_gate_ln_workspace_size(ctypes.byref(p), 0, ctypes.byref(n)) == 2
    assert lib.pma_gate_ln_workspace_size(ctypes.byref(p), 100, None) == 1
    lay = B.Layout(8192, 1, 256, 64, 32, 128, fake, fake, fake, fake, fake, fake, fake, fake,
                   fake, fake)
    f = lib.pma_gate_residual_ln_modulate

    def call(gate_chunk=2, which=1, b=fake, ws=fake, ws_bytes=1 << 40, K=7168):
        return f(ctypes.byref(p), ctypes.byref(lay), fake, 7168, K, fake, fake, gate_chunk, fake,
                 fake, fake, which, b, ws, ws_bytes, None)

    assert call(which=2) == 2
    assert call(gate_chunk=3) == 2
    assert call(b=None) == 1
    assert call(ws=None) == 1
    assert call(ws=ctypes.c_void_p(128)) == 3
    assert call(ws_bytes=8192 * 42 * 8 - 1) == 4
    assert call(K=100) == 2          # K % 64 != 0, caught by the projection's checks
