#!/usr/bin/env python3
"""Packed masked attention on one MI355X: TFLOP/s and fraction of bf16 MFMA peak.

A step is one pass of the attention hot path over the masked L=16384 packed
sequence (512 text rows, 14400 video rows on a (9,40,40) grid, 656 audio
rows, 816 padding rows in their own document; 56 heads x 128 channels, bf16
Q/K/V ~ N(0,1), seeded): layout build -> QK-RMSNorm + 3-axis RoPE -> masked
flash attention, all through the libpma C ABI with inputs resident in HBM.

value = algorithmic FLOPs / step time, algorithmic FLOPs = 4*H*D*sum_d n_d^2
(only the (query, key) pairs the document mask allows).  The roofline object
is the flash attention kernel alone, timed with HIP events on the stream it is
launched on; the cpu_baseline object is the CPU oracle's fp32 attention loop
timed on a bounded sample of query rows on the host cores.

With --workload block_L8192 the step is instead one DiT block forward
(AdaLN table + LN/modulate + QKV + attention path + O-projection + FFN) at
L=8192, hidden 5376, ffn 14336; value is the block's algorithmic TFLOP/s and
the roofline object is the fc1+SwiGLU GEMM (the block's largest kernel) timed
in its own launches.

With --workload io_L8192 (or io_L16384) the step is the input/output path on
that packed layout: timestep MLP, output-head table, patch projections into
the packed stream, output heads; value is its fp32 TFLOP/s and the roofline
object is the video patch projection against the fp32 MFMA peak.

With --workload forward_L8192 the step is the whole transformer forward at
L=8192: timestep MLP, head table, token refiner (2 blocks on the 512 text
rows), pack, the 50-block stack and the output heads; value is its
algorithmic TFLOP/s, and a HIP graph of the same step is timed beside it.

With --workload gate_ln_L8192 the block's O-projection + gated residual and
the pre-FFN LN-modulate are timed two ways, interleaved: as the block runs
them (two launches) and as pma_gate_residual_ln_modulate (the norm
statistics taken in the projection's epilogue); value is the first, in us.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--copy-probe BYTES]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6          # 256 CU x 4096 flop/clk x 2.4 GHz, dense
HBM_PEAK_GBS = 8000.0
METRIC = "packed masked attention TFLOP/s + % bf16 MFMA peak at L=16384,H=56,D=128"
COUNTERS = os.path.join(ROOT, "profiles", "flash_fwd_masked_L16384_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(path: str) -> str:
    """16 hex digits of the sha256 of a kernel source plus the extra compiler
    options the build gives that file, so counters taken on other code (a
    different source or different code generation) do not apply."""
    from packed_masked_attention_amd.build import EXTRA
    h = hashlib.sha256()
    with open(path, "rb") as fh:
        h.update(fh.read())
    opts = EXTRA.get(os.path.basename(path))
    if opts:
        h.update(" ".join(opts).encode())
    return h.hexdigest()[:16]


def gpu_state():
    """Current sclk/mclk DPM levels and average power of the first amdgpu card,
    read from sysfs (no child process: the GPU is initialised by then), or
    None where unavailable.  Read outside the timed region."""
    import glob
    import re
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for key, name in (("sclk_mhz", "pp_dpm_sclk"), ("mclk_mhz", "pp_dpm_mclk")):
            try:
                with open(os.path.join(dev, name)) as fh:
                    for line in fh:
                        m = re.search(r"([0-9]+)\s*mhz\s*\*", line, re.IGNORECASE)
                        if m:
                            out[key] = float(m.group(1))
            except OSError:
                pass
        for f in glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_average")) + \
                glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_input")):
            try:
                with open(f) as fh:
                    out.setdefault("power_w", int(fh.read().strip()) / 1e6)
            except (OSError, ValueError):
                pass
        if out:
            return out
    return None


class ClockSampler:
    """Samples the card's current sclk level and power from sysfs in a
    background thread while the timed loop runs (sysfs reads only, no GPU
    call), so the fraction of peak can also be stated at the clock the card
    actually ran at.  Every sample is kept; the median is reported."""

    def __init__(self, period_s: float = 0.01):
        import threading
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._th = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            st = gpu_state()
            if st:
                self.samples.append(st)
            self._stop.wait(self.period)

    def __enter__(self):
        self._th.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._th.join()

    def summary(self):
        import numpy as np
        sc = [s["sclk_mhz"] for s in self.samples if "sclk_mhz" in s]
        pw = [s["power_w"] for s in self.samples if "power_w" in s]
        if not sc:
            return None
        return {"samples": len(sc), "sclk_mhz_median": float(np.median(sc)),
                "sclk_mhz_range": [float(min(sc)), float(max(sc))],
                "power_w_median": float(np.median(pw)) if pw else None}


STAMP_BYTES = 1024 * 4 * 8      # the flash workspace's clock-stamp area (its last bytes)


def flash_clock(fws, n_groups: int):
    """Effective shader clock of the last persistent flash launch, from the
    clock stamps its workgroups leave at the end of the flash workspace: per
    workgroup the shader-clock counter and the 100 MHz real-time counter at
    its start and its end.  MHz = sum of shader cycles / sum of real time."""
    import numpy as np
    st = fws[-STAMP_BYTES:].cpu().numpy().view(np.uint64).reshape(-1, 4)[:n_groups].astype(np.float64)
    cyc = (st[:, 2] - st[:, 0]).sum()
    rt = (st[:, 3] - st[:, 1]).sum()
    if not (rt > 0 and cyc > 0):
        return None
    mhz = cyc / rt * 100.0
    return mhz if 50.0 < mhz < 5000.0 else None


def cpu_model() -> str | None:
    """The host CPU's model name from /proc/cpuinfo (no child process)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


NOMINAL_SCLK_MHZ = 2400.0


def at_clock(achieved: float, mhz) -> dict | None:
    """Fraction of the bf16 peak scaled to a measured shader clock (MHz)."""
    if not mhz:
        return None
    peak = BF16_PEAK_TFLOPS * mhz / NOMINAL_SCLK_MHZ
    return {"sclk_mhz": round(mhz, 1), "peak": round(peak, 1), "frac": round(achieved / peak, 4),
            "source": "shader-clock / real-time counters stamped by the flash kernel's "
                      "workgroups in the last timed launch"}


def attention_flops(tags, H: int, D: int) -> int:
    import numpy as np
    tags = np.asarray(tags)
    npad = int((tags == -1).sum())
    nreal = tags.size - npad
    return 4 * H * D * (npad * npad + nreal * nreal)


def traffic_from_profiles(path: str = COUNTERS, source: str = "flash_fwd.hip",
                          key: str = "flash_fwd_sha256_16"):
    """HBM bytes per launch of a kernel from committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size), if they were
    taken on the current kernel source; else None."""
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        c = json.load(fh)
    src = os.path.join(ROOT, "packed_masked_attention_amd", "csrc", source)
    if c.get(key) != source_hash(src):
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_baseline(inp: dict, target_s: float = 12.0) -> dict:
    """The oracle's fp32 two-pass attention on a random sample of query rows
    (all heads), sized to roughly target_s seconds of CPU work."""
    import numpy as np
    import oracle
    lay, H, D = inp["layout"], inp["H"], inp["D"]
    L = lay["L"]
    t0 = time.perf_counter()
    qn = oracle.qk_norm_rope(inp["q"], H, D, 1.0, lay["pos"]).astype(np.float32)
    kn = oracle.qk_norm_rope(inp["k"], H, D, 1.0, lay["pos"]).astype(np.float32)
    v = oracle.bf16_to_f64(inp["v"]).astype(np.float32)
    t_prep = time.perf_counter() - t0
    tags = lay["tags"]
    pad = tags == -1
    n_doc = np.where(pad, pad.sum(), (~pad).sum())
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(L, size=16, replace=False)).astype(np.int32)
    t0 = time.perf_counter()
    oracle.attention(qn, kn, v, tags, rows=rows, precision="f32")
    t_probe = time.perf_counter() - t0
    n = int(min(L, max(16, 16 * target_s / max(t_probe, 1e-3))))
    rows = np.sort(rng.choice(L, size=n, replace=False)).astype(np.int32)
    t0 = time.perf_counter()
    oracle.attention(qn, kn, v, tags, rows=rows, precision="f32")
    t_attn = time.perf_counter() - t0
    flops = 4 * H * D * int(n_doc[rows].sum())
    return {"value": flops / t_attn / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"fp32 two-pass attention for {n} random query rows x {H} heads of "
                      f"the L={L} workload ({t_attn:.1f} s); QK-norm+RoPE of all rows "
                      f"took {t_prep:.1f} s and is not in the rate"}


def block_cpu_baseline(inp: dict, target_s: float = 12.0) -> dict:
    """The oracle's DiT block (numpy fp64 with bf16 storage, the fused-QKV
    rounding) for a random sample of query rows.  It always projects K and V
    of every row (attention needs them); the counted FLOPs are the work it
    does: the K/V projection of all rows plus, per sampled row, the Q
    projection, attention over the row's document, O-projection and FFN."""
    import numpy as np
    import oracle
    from oracle import block as oblock
    lay = inp["layout"]
    L, hid, H, D, ffn = inp["L"], inp["hidden"], inp["heads"], inp["head_dim"], inp["ffn"]
    HD = H * D
    tags = np.asarray(lay["tags"])
    pad = tags == -1
    n_doc = np.where(pad, pad.sum(), (~pad).sum())
    rng = np.random.default_rng(0)

    def run(n):
        rows = np.sort(rng.choice(L, size=n, replace=False))
        t0 = time.perf_counter()
        oblock.block_forward(inp, rows=rows, fused_qkv=True)
        dt = time.perf_counter() - t0
        fl = 2 * L * hid * 2 * HD + sum(2 * hid * HD + 4 * HD * int(n_doc[r]) + 2 * HD * hid
                                         + 2 * hid * 2 * ffn + 2 * ffn * hid for r in rows)
        return rows.size, dt, fl

    n, dt, fl = run(16)
    if dt < target_s / 2:
        n, dt, fl = run(int(min(L, 16 * max(1.0, target_s / max(dt, 1e-3)))))
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"fp64 block for {n} random query rows of the L={L} workload ({dt:.1f} s), "
                      f"including the K/V projection of all {L} rows the attention needs"}


def io_cpu_baseline(d: dict, lay: dict, target_s: float = 10.0) -> dict:
    """The oracle's input/output path (numpy fp64): timestep MLP and head table
    in full, the video patch projection and video output head on a random
    sample of video rows."""
    import numpy as np
    import oracle
    from oracle import inout
    t0 = time.perf_counter()
    temb, _ = inout.timestep_mlp(d["t"].astype(np.float64), d["w1"], d["b1"], d["w2"], d["b2"],
                                 freq_dim=d["freq_dim"])
    table = inout.head_table(temb, d["w_mod"])
    dt0 = time.perf_counter() - t0
    T, hid, E, inner, fd = temb.shape[0], d["hidden"], d["temb_dim"], d["inner_dim"], d["freq_dim"]
    fl0 = 2 * T * (fd * inner + inner * E) + 2 * T * E * 4 * hid
    vidx = np.asarray(lay["video_idx"])
    rng = np.random.default_rng(0)

    def run(n):
        pick = np.sort(rng.choice(vidx.size, size=min(n, vidx.size), replace=False))
        t1 = time.perf_counter()
        _ = d["video"][pick].astype(np.float64) @ d["w_video"].astype(np.float64).T + d["b_video"]
        inout.output_head(d["x"], vidx[pick], lay["ts_idx"], table, 0, d["w_vout"], d["b_vout"])
        return pick.size, time.perf_counter() - t1, 2 * pick.size * 96 * hid * 2

    n, dt, fl = run(256)
    if dt < target_s / 2:
        n, dt, fl = run(int(256 * max(1.0, (target_s - dt0) / max(dt, 1e-3))))
    return {"value": (fl0 + fl) / (dt0 + dt) / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"fp64 timestep MLP + head table ({dt0:.1f} s) and the video projection + "
                      f"video head for {n} random video rows ({dt:.1f} s)"}


def copy_probe(nbytes: int) -> None:
    """A plain device copy of known size, for scaling rocprofv3 HBM counters."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes}))


def block_bench(args) -> int:
    import numpy as np
    import torch
    from packed_masked_attention_amd import binding as B
    from packed_masked_attention_amd import synth

    torch.cuda.set_device(0)
    wl = synth.workload(args.workload)
    log(f"[bench] generating {wl.name} inputs")
    inp = synth.make_block_workload(wl)
    L, hid, H, ffn, E = wl.L, wl.hidden, wl.H, wl.ffn, wl.temb_dim
    HD = H * wl.D
    dev = torch.device("cuda", 0)
    to_dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev) \
        .view(torch.bfloat16)
    x, temb = to_dev(inp["x"]), to_dev(inp["temb"])
    w_ada, w_qkv, w_o = to_dev(inp["w_ada"]), to_dev(inp["w_qkv"]), to_dev(inp["w_o"])
    w_fc1, w_fc2 = to_dev(inp["w_fc1"]), to_dev(inp["w_fc2"])
    ones = torch.ones(wl.D, dtype=torch.float32, device=dev)
    p = B.block_params(hid, ffn, E, H)
    dl = B.pma_layout_build(inp["layout"], device=dev)
    T = inp["layout"]["T"]
    table = torch.empty(3, T, 6, hid, dtype=torch.float32, device=dev)
    w = B.BlockWeights(w_ada.data_ptr(), w_qkv.data_ptr(), w_o.data_ptr(), w_fc1.data_ptr(),
                       w_fc2.data_ptr(), ones.data_ptr(), ones.data_ptr())
    out = torch.empty_like(x)
    ws = torch.empty(B.pma_block_workspace_size(p, L), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        B.pma_adaln_table(p, T, temb, w_ada, table)
        B.pma_block_forward(p, dl, w, table, x, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    attn = attention_flops(inp["layout"]["tags"], H, wl.D)
    gemm = 2 * L * hid * (3 * HD) + 2 * L * HD * hid + 2 * L * hid * (2 * ffn) + 2 * L * ffn * hid
    ada = 2 * 3 * 6 * hid * E * T
    flops = attn + gemm + ada
    # dominant kernel: fc1 + SwiGLU, in its own launches on this stream
    bb = torch.empty(L, hid, dtype=torch.bfloat16, device=dev).normal_()
    hh = torch.empty(L, ffn, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        B.pma_linear(L, ffn, hid, bb, hid, w_fc1, hid, hh, ffn, B.EPI_SWIGLU)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        B.pma_linear(L, ffn, hid, bb, hid, w_fc1, hid, hh, ffn, B.EPI_SWIGLU)
    e1.record(stream)
    torch.cuda.synchronize()
    fc1_ms = e0.elapsed_time(e1) / args.steps
    fc1_flops = 2 * L * (2 * ffn) * hid
    achieved = fc1_flops / (fc1_ms * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12
    outj = {
        "metric": "DiT block forward TFLOP/s at L=8192, hidden 5376, 56x128 heads, ffn 14336",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "seq_len": L, "hidden": hid, "heads": H,
                   "head_dim": wl.D, "ffn_dim": ffn, "time_embed_dim": E,
                   "algorithmic_flops": flops,
                   "step": "AdaLN table + one DiT block forward",
                   "pct_bf16_peak_step": round(100 * value / BF16_PEAK_TFLOPS, 2)},
        "roofline": {"kernel": "gemm_kernel<SWIGLU> (fc1)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profiles(
                         os.path.join(ROOT, "profiles", "gemm_fc1_block_L8192_counters.json"),
                         "gemm.hip", "source_sha256_16"),
                     "avg_ms": round(fc1_ms, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        outj["cpu_baseline"] = block_cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(outj), flush=True)
    return 0


FP32_PEAK_TFLOPS = 157.3          # dense fp32 MFMA


def io_bench(args) -> int:
    """The steps either side of the block stack on one packed layout: timestep
    MLP (T distinct timesteps), output-head modulation table, input
    projections + text scatter into the packed stream, and the two output
    heads.  value = fp32 TFLOP/s of the whole step; roofline = the video
    patch projection (the largest single-launch contraction), fp32 MFMA."""
    import numpy as np
    import torch
    from packed_masked_attention_amd import binding as B
    from packed_masked_attention_amd import synth

    torch.cuda.set_device(0)
    base = {"io_L8192": "block_L8192", "io_L16384": "masked_L16384"}.get(args.workload)
    if base is None:
        log(f"unknown workload {args.workload}")
        return 2
    lay = synth.make_layout(synth.workload(base))
    hidden, fd, inner, E = 5376, 256, 5376, 2688
    log(f"[bench] generating {args.workload} inputs")
    d = synth.make_io_inputs(lay, hidden=hidden, freq_dim=fd, inner_dim=inner, temb_dim=E)
    dev = torch.device("cuda", 0)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    T = lay["T"]
    nv, na, nt = (int(lay[k].size) for k in ("video_idx", "audio_idx", "text_idx"))
    tp, p = B.temb_params(fd, inner, E), B.io_params(hidden, time_embed_dim=E)
    t, w1, b1, w2, b2 = (f(d[k]) for k in ("t", "w1", "b1", "w2", "b2"))
    inner_t = torch.empty(T, inner, device=dev)
    temb = torch.empty(T, E, device=dev)
    temb_b = torch.empty(T, E, dtype=torch.bfloat16, device=dev)
    w_mod = f(d["w_mod"])
    table = torch.empty(2, T, 2, hidden, device=dev)
    dl = B.pma_layout_build(lay, device=dev)
    x = torch.empty(lay["L"], hidden, dtype=torch.bfloat16, device=dev).normal_()
    video, wv, bv = f(d["video"]), f(d["w_video"]), f(d["b_video"])
    audio, wa, ba = f(d["audio"]), f(d["w_audio"]), f(d["b_audio"])
    text = torch.from_numpy(d["text"].view(np.int16)).to(dev).view(torch.bfloat16)
    hw = [f(d[k]) for k in ("w_vout", "b_vout", "w_aout", "b_aout")]
    vout = torch.empty(nv, 96, device=dev)
    aout = torch.empty(na, 32, device=dev)
    ws = torch.empty(B.pma_unpack_workspace_size(p, nv, na), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        B.pma_timestep_embed(tp, T, t, w1, b1, w2, b2, inner_t, temb, temb_b)
        B.pma_head_table(p, T, temb, w_mod, table)
        B.pma_pack_rows(p, dl, video, wv, bv, audio, wa, ba, text, hidden, x)
        B.pma_unpack_rows(p, dl, x, table, *hw, vout, aout, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    rows_f = nv * 96 + na * 32
    flops = (2 * T * (fd * inner + inner * E) + 2 * T * E * 4 * hidden
             + 2 * rows_f * hidden * 2)
    # the video projection alone: a descriptor naming only the video rows
    desc_v = B.LayoutDesc(lay["L"], T, dl.desc.token_tags, dl.desc.position_ids,
                          dl.desc.timestep_indices, dl.desc.video_indices, None, None, nv, 0, 0)
    dlv = B.DeviceLayout(dl.arrays, dl.workspace, dl.struct, desc_v)
    for _ in range(3):
        B.pma_pack_rows(p, dlv, video, wv, bv, None, None, None, None, hidden, x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        B.pma_pack_rows(p, dlv, video, wv, bv, None, None, None, None, hidden, x)
    e1.record(stream)
    torch.cuda.synchronize()
    proj_ms = e0.elapsed_time(e1) / args.steps
    proj_flops = 2 * nv * 96 * hidden
    achieved = proj_flops / (proj_ms * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12
    outj = {
        "metric": "input/output path fp32 TFLOP/s (timestep MLP, head table, patch projections, "
                  "output heads)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "seq_len": int(lay["L"]), "hidden": hidden,
                   "rows": {"video": nv, "audio": na, "text": nt}, "num_timesteps": T,
                   "freq_dim": fd, "time_embed_hidden_dim": inner, "time_embed_dim": E,
                   "algorithmic_flops": flops,
                   "step": "timestep MLP + head table + pack (projections, text scatter) + "
                           "unpack (output heads)"},
        "roofline": {"kernel": "proj_scatter_kernel (video patch projection)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": FP32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / FP32_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profiles(
                         os.path.join(ROOT, "profiles", "proj_scatter_video_io_L8192_counters.json"),
                         "inout.hip", "source_sha256_16"),
                     "avg_ms": round(proj_ms, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        outj["cpu_baseline"] = io_cpu_baseline(d, lay, args.cpu_seconds)
    print(json.dumps(outj), flush=True)
    return 0


def forward_bench(args) -> int:
    """The whole transformer forward on the L=8192 packed layout: timestep MLP,
    head table, token refiner (2 blocks over the 512 text rows), pack, 50 DiT
    blocks, output heads.  Weights are seeded N(0, 0.02^2) bf16 generated on
    the device (about 67 GB); the fp32 input/output weights come from
    synth.make_io_inputs.  value = algorithmic TFLOP/s of the whole step;
    roofline = the fc1 + SwiGLU GEMM (the largest kernel) in its own launches.
    The step is also captured in a HIP graph and its replays timed."""
    import numpy as np
    import torch
    from packed_masked_attention_amd import binding as B
    from packed_masked_attention_amd import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    wl = synth.workload("block_L8192")
    lay = synth.make_layout(wl)
    L, hid, H, ffn, E, D = wl.L, wl.hidden, wl.H, wl.ffn, wl.temb_dim, wl.D
    HD = H * D
    T = lay["T"]
    n_blocks, n_ref, text_dim = args.blocks, 2, 5120
    tidx = lay["text_idx"]
    nt = int(tidx.size)
    text_lay = synth.layout_from_tags(np.full(nt, synth.TAG_TEXT, np.int32), lay["pos"][tidx],
                                      lay["ts_idx"][tidx], T)
    log(f"[bench] generating forward_L8192 weights ({n_blocks} + {n_ref} blocks)")
    g = torch.Generator(device=dev).manual_seed(8)

    def rnd(*shape, std=0.02):
        return (torch.randn(*shape, generator=g, device=dev) * std).to(torch.bfloat16)

    ones = torch.ones(D, dtype=torch.float32, device=dev)
    keep = []

    def weight_set():
        t = [rnd(3, 6 * hid, E), rnd(3 * HD, hid), rnd(hid, HD), rnd(2 * ffn, hid), rnd(hid, ffn)]
        keep.append(t)
        return B.BlockWeights(*(x.data_ptr() for x in t), ones.data_ptr(), ones.data_ptr())

    blocks = B.block_weights_array([weight_set() for _ in range(n_blocks)])
    refiner = B.block_weights_array([weight_set() for _ in range(n_ref)])
    w_text = rnd(hid, text_dim, std=text_dim ** -0.5)
    d = synth.make_io_inputs(lay, hidden=hid, inner_dim=5376, temb_dim=E)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    t, w1, b1, w2, b2 = (f(d[k]) for k in ("t", "w1", "b1", "w2", "b2"))
    w_mod = f(d["w_mod"])
    video, wv, bv = f(d["video"]), f(d["w_video"]), f(d["b_video"])
    audio, wa, ba = f(d["audio"]), f(d["w_audio"]), f(d["b_audio"])
    hw = [f(d[k]) for k in ("w_vout", "b_vout", "w_aout", "b_aout")]
    text = rnd(nt, text_dim, std=1.0)
    nv, na = int(lay["video_idx"].size), int(lay["audio_idx"].size)
    tp, io = B.temb_params(256, 5376, E), B.io_params(hid, time_embed_dim=E)
    p = B.block_params(hid, ffn, E, H)
    dl = B.pma_layout_build(lay, device=dev)
    dlt = B.pma_layout_build(text_lay, device=dev)
    inner_t = torch.empty(T, 5376, device=dev)
    temb = torch.empty(T, E, device=dev)
    temb_b = torch.empty(T, E, dtype=torch.bfloat16, device=dev)
    table = torch.empty(2, T, 2, hid, device=dev)
    text_out = torch.empty(nt, hid, dtype=torch.bfloat16, device=dev)
    x = torch.empty(L, hid, dtype=torch.bfloat16, device=dev).normal_()
    x2 = torch.empty_like(x)
    vout = torch.empty(nv, 96, device=dev)
    aout = torch.empty(na, 32, device=dev)
    ws_ref = torch.empty(B.pma_refiner_workspace_size(p, nt, T), dtype=torch.uint8, device=dev)
    ws_stack = torch.empty(B.pma_stack_workspace_size(p, L, T), dtype=torch.uint8, device=dev)
    ws_io = torch.empty(B.pma_unpack_workspace_size(io, nv, na), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    # token reduction (engine page): blocks 1-3 at full resolution, the target
    # video rows paired for blocks 4-39, restored from the bypass before block 40
    red = None
    if args.token_reduction and n_blocks < 40:
        log("--token-reduction restores before block 40: it needs --blocks 40 or more")
        return 2
    if args.token_reduction:
        plan = synth.token_reduction_plan(lay)
        s0 = torch.from_numpy(plan["src0"]).to(dev)
        s1 = torch.from_numpy(plan["src1"]).to(dev)
        nr = int(plan["src0"].size)
        red = {"plan": plan, "s0": s0, "s1": s1, "n": nr, "a": 3, "b": min(39, n_blocks),
               "dl": B.pma_layout_build(plan["layout"], device=dev),
               "p": B.block_params(hid, ffn, E, H, pos_scale=plan["pos_scale"]),
               "xr0": torch.empty(nr, hid, dtype=torch.bfloat16, device=dev),
               "xr1": torch.empty(nr, hid, dtype=torch.bfloat16, device=dev),
               "x1": torch.empty_like(x)}
        blist = list(blocks)

    def run_stack():
        if red is None:
            B.pma_stack_forward(p, dl, blocks, temb_b, x, x2, ws_stack)
            return
        r = red
        B.pma_stack_forward(p, dl, blist[:r["a"]], temb_b, x, r["x1"], ws_stack)
        B.pma_token_merge(hid, L, r["s0"], r["s1"], r["x1"], r["xr0"])
        B.pma_stack_forward(r["p"], r["dl"], blist[r["a"]:r["b"]], temb_b, r["xr0"], r["xr1"],
                            ws_stack)
        B.pma_token_restore(hid, L, r["s0"], r["s1"], r["x1"], r["xr0"], r["xr1"], r["x1"])
        B.pma_stack_forward(p, dl, blist[r["b"]:], temb_b, r["x1"], x2, ws_stack)

    def step():
        B.pma_timestep_embed(tp, T, t, w1, b1, w2, b2, inner_t, temb, temb_b)
        B.pma_head_table(io, T, temb, w_mod, table)
        B.pma_text_refiner(p, dlt, refiner, temb_b, text, text_dim, text_dim, w_text, 1e-5,
                           text_out, ws_ref)
        B.pma_pack_rows(io, dl, video, wv, bv, audio, wa, ba, text_out, hid, x)
        run_stack()
        B.pma_unpack_rows(io, dl, x2, table, *hw, vout, aout, ws_io)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ref_v = vout.clone()
    # the same step as one HIP graph
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    graph_same = bool(torch.equal(vout, ref_v))
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms_graph = (time.perf_counter() - t0) * 1e3 / args.steps

    def block_flops(n, tags):
        attn = attention_flops(tags, H, D)
        gemm = 2 * n * hid * (3 * HD) + 2 * n * HD * hid + 2 * n * hid * (2 * ffn) + 2 * n * ffn * hid
        return attn + gemm + 2 * 3 * 6 * hid * E * T
    io_flops = (2 * T * (256 * 5376 + 5376 * E) + 2 * T * E * 4 * hid
                + 2 * (nv * 96 + na * 32) * hid * 2)
    if red is None:
        stack_flops = n_blocks * block_flops(L, lay["tags"])
    else:
        n_red = red["b"] - red["a"]
        stack_flops = ((n_blocks - n_red) * block_flops(L, lay["tags"])
                       + n_red * block_flops(red["n"], red["plan"]["layout"]["tags"]))
    flops = (stack_flops + n_ref * block_flops(nt, text_lay["tags"])
             + 2 * nt * text_dim * hid + io_flops)
    # dominant kernel: fc1 + SwiGLU at L rows, in its own launches on this stream
    bb = torch.empty(L, hid, dtype=torch.bfloat16, device=dev).normal_()
    hh = torch.empty(L, ffn, dtype=torch.bfloat16, device=dev)
    w_fc1 = keep[0][3]
    for _ in range(3):
        B.pma_linear(L, ffn, hid, bb, hid, w_fc1, hid, hh, ffn, B.EPI_SWIGLU)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        B.pma_linear(L, ffn, hid, bb, hid, w_fc1, hid, hh, ffn, B.EPI_SWIGLU)
    e1.record(stream)
    torch.cuda.synchronize()
    fc1_ms = e0.elapsed_time(e1) / 10
    achieved = 2 * L * (2 * ffn) * hid / (fc1_ms * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12
    outj = {
        "metric": f"MiniMax-H3 transformer forward TFLOP/s at L=8192 ({n_blocks} blocks + "
                  f"{n_ref} refiner blocks + input/output path"
                  + (", token reduction)" if red else ")"),
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "forward_L8192", "seq_len": L, "hidden": hid, "heads": H,
                   "head_dim": D, "ffn_dim": ffn, "blocks": n_blocks, "refiner_blocks": n_ref,
                   "text_rows": nt, "text_dim": text_dim, "algorithmic_flops": flops,
                   "token_reduction": None if red is None else {
                       "reduced_rows": red["n"], "full_blocks_before": red["a"],
                       "reduced_blocks": red["b"] - red["a"], "restored_before_block": red["b"] + 1},
                   "ms_per_step_hip_graph": round(ms_graph, 3),
                   "hip_graph_output_equal": graph_same,
                   "pct_bf16_peak_step": round(100 * value / BF16_PEAK_TFLOPS, 2)},
        "roofline": {"kernel": "gemm_kernel<SWIGLU> (fc1)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "avg_ms": round(fc1_ms, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(outj), flush=True)
    return 0


def gate_ln_bench(args) -> int:
    """The block's a7 + a8 pair at L=8192 two ways, interleaved on one GPU:
    the O-projection with the gated residual, then the LN-modulate pass (the
    block's path), against pma_gate_residual_ln_modulate (the same
    projection also taking each rounded row's norm statistics in its
    epilogue, the norm pass reading them instead of reducing the row)."""
    import numpy as np
    import torch
    from packed_masked_attention_amd import binding as B
    from packed_masked_attention_amd import synth

    torch.cuda.set_device(0)
    wl = synth.workload("block_L8192")
    lay = synth.layout_from_counts(wl.text, wl.video, wl.audio, wl.pad, wl.T)
    L, N, K, T = wl.L, wl.hidden, wl.H * wl.D, lay["T"]
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed)
    rnd = lambda *shape, std=1.0: (std * torch.randn(*shape, device=dev, generator=g)).to(torch.bfloat16)
    A, W, x = rnd(L, K), rnd(N, K, std=wl.weight_std), rnd(L, N)
    table = torch.randn(3, T, 6, N, device=dev, generator=g)
    p = B.block_params(N, wl.ffn, wl.temb_dim, wl.H)
    dl = B.pma_layout_build(lay, device=dev)
    tags = torch.from_numpy(lay["tags"]).to(dev)
    ts = torch.from_numpy(lay["ts_idx"]).to(dev)
    x1, b = torch.empty_like(x), torch.empty_like(x)
    ws = torch.empty(B.pma_gate_ln_workspace_size(p, L), dtype=torch.uint8, device=dev)

    def unfused():
        B.pma_linear(L, N, K, A, K, W, K, x1, N, B.EPI_GATE_RESIDUAL, R=x, ldr=N, table=table,
                     num_timesteps=T, gate_chunk=2, tags=tags, ts_idx=ts)
        B.pma_ln_modulate(p, dl, table, 1, x1, b)

    def fused():
        B.pma_gate_residual_ln_modulate(p, dl, A, K, K, W, table, 2, x, x1, table, 1, b, ws)

    def norm_only():
        B.pma_ln_modulate(p, dl, table, 1, x1, b)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    cases = {"unfused": unfused, "fused": fused, "norm_only": norm_only}
    for fn in cases.values():
        for _ in range(args.warmup):
            fn()
    torch.cuda.synchronize()
    reps = 5
    us = {k: [] for k in cases}
    t0 = time.perf_counter()
    for r in range(reps):
        for k, fn in cases.items():
            us[k].append(timed(fn, args.steps))
        log(f"[bench] rep {r}: " + ", ".join(f"{k} {v[-1]:.1f} us" for k, v in us.items()))
    wall = time.perf_counter() - t0
    med = {k: float(np.median(v)) for k, v in us.items()}
    flops = 2.0 * L * N * K
    out = {
        "metric": "O-projection + gated residual + pre-FFN LN-modulate time at L=8192",
        "value": round(med["unfused"], 1), "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(med["unfused"] / 1e3, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gate_ln_L8192", "seq_len": L, "hidden": N, "K": K,
                   "step": "x1 = x + gate_a (O W_o^T); b = LN(x1)(1 + scale_f) + shift_f",
                   "reps": reps, "wall_s": round(wall, 2)},
        "median_us": {k: round(v, 1) for k, v in med.items()},
        "fused_minus_unfused_us": round(med["fused"] - med["unfused"], 1),
        "projection_tflops_unfused_pair": round(flops / (med["unfused"] * 1e-6) / 1e12, 1),
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="masked_L16384")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--blocks", type=int, default=50, help="DiT blocks of forward_L8192")
    ap.add_argument("--token-reduction", action="store_true",
                    help="forward_L8192 with the engine's token reduction (blocks 4-39 paired)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe", type=int, default=0, help=argparse.SUPPRESS)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the path is built and measured on a single MI355X.", file=sys.stderr)
        return 2
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return 0
    if args.workload.startswith("block"):
        return block_bench(args)
    if args.workload.startswith("io_"):
        return io_bench(args)
    if args.workload == "forward_L8192":
        return forward_bench(args)
    if args.workload == "gate_ln_L8192":
        return gate_ln_bench(args)

    import numpy as np
    import torch
    from packed_masked_attention_amd import binding as B
    from packed_masked_attention_amd import synth

    torch.cuda.set_device(0)
    wl = synth.workload(args.workload)
    log(f"[bench] generating {wl.name} inputs")
    inp = synth.make_attention_inputs(wl)
    lay = inp["layout"]
    L, H, D = wl.L, wl.H, wl.D
    flops = attention_flops(lay["tags"], H, D)

    dev = torch.device("cuda", 0)
    to_dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev) \
        .view(torch.bfloat16)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    wq = torch.ones(D, dtype=torch.float32, device=dev)
    wk = torch.ones(D, dtype=torch.float32, device=dev)
    dl = B.pma_layout_build(lay, device=dev)
    bits, row = B.pma_layout_read_status(dl)
    if bits:
        raise RuntimeError(f"layout status {bits:#x} row {row}")
    p = B.attn_params(H)
    Lp = B.pma_attention_padded_len(L)
    qh = torch.empty(H, Lp, D, dtype=torch.bfloat16, device=dev)
    kh = torch.empty_like(qh)
    vt = torch.empty(H, D, Lp, dtype=torch.bfloat16, device=dev)
    o = torch.empty(L, H * D, dtype=torch.bfloat16, device=dev)
    # partial results of the key-range split of the last work items
    fws = torch.empty(B.pma_flash_workspace_size(p, L), dtype=torch.uint8, device=dev)
    HD = H * D
    stream = torch.cuda.current_stream()

    def step(ev=None):
        B.pma_layout_build(dl)
        B.pma_qk_norm_rope(p, dl, q, HD, k, HD, v, HD, wq, wk, qh, kh, vt)
        if ev is not None:
            ev[0].record(stream)
        B.pma_flash_attention(p, dl, qh, kh, vt, o, HD, workspace=fws)
        if ev is not None:
            ev[1].record(stream)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    state_before = gpu_state()
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    state_after = gpu_state()
    clock = clk.summary()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    flash_mhz = flash_clock(fws, n_cu)
    ms_step = wall * 1e3 / args.steps
    per_launch = np.array([a.elapsed_time(b) for a, b in evs])
    flash_ms = float(per_launch.mean())
    q25, q50, q75 = (float(x) for x in np.percentile(per_launch, [25, 50, 75]))
    log(f"[bench] flash per launch: median {q50:.4f} ms, IQR {q25:.4f}-{q75:.4f} ms; "
        f"gpu before {state_before}, after {state_after}, during {clock}; flash kernel "
        f"clock {flash_mhz} MHz")
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (flash_ms * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(inp, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "seq_len": L, "heads": H, "head_dim": D,
                   "rows": {"text": wl.text, "video": wl.n_video, "audio": wl.audio,
                            "padding": wl.pad},
                   "video_grid": list(wl.video), "documents": sorted(
                       {int((lay["tags"] == -1).sum()), int((lay["tags"] != -1).sum())} - {0},
                       reverse=True),
                   "algorithmic_flops": flops,
                   "step": "layout build + QK-RMSNorm/RoPE + masked flash attention",
                   "pct_bf16_peak_step": round(100 * value / BF16_PEAK_TFLOPS, 2)},
        "roofline": {"kernel": "flash_fwd_kernel (events around the call: it and the "
                               "flash_merge_kernel of its split items)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profiles(), "avg_ms": round(flash_ms, 4),
                     "median_ms": round(q50, 4), "iqr_ms": [round(q25, 4), round(q75, 4)],
                     "at_measured_clock": at_clock(achieved, flash_mhz)},
        "cpu_baseline": cpu,
        "gpu_state": {"before": state_before, "after": state_after, "during": clock},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
