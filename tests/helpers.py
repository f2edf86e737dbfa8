"""Shared helpers for the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from packed_masked_attention_amd import synth

# Tolerances: max |err| <= 1.5e-2 and mean |err| <= 2e-3 on unit-variance
# inputs with fp32 accumulation (the target's literal bound), plus a relative
# gate mean|err| / rms(ref) <= 1e-2 that stays meaningful when outputs are
# small (long sequences average many values, so |O| shrinks like 1/sqrt(n)).
MAX_ABS = 1.5e-2
MEAN_ABS = 2e-3
MEAN_REL = 1e-2

# The stored query operand Q' is the normalised, rotated query times the
# logit factor softmax_scale * log2(e) (default softmax_scale 1/sqrt(128)).
Q_OPERAND_SCALE = np.log2(np.e) / np.sqrt(128.0)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_np(t) -> np.ndarray:
    """bf16 torch tensor -> fp64 numpy (exact)."""
    import torch
    return oracle.bf16_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def to_dev_bf16(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def err_stats(got: np.ndarray, ref: np.ndarray) -> dict:
    e = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) or 1.0
    return {"max_abs": float(e.max()), "mean_abs": float(e.mean()),
            "mean_rel": float(e.mean() / rms), "rms_ref": rms}


def assert_close(got, ref, what="", max_abs=MAX_ABS, mean_abs=MEAN_ABS, mean_rel=MEAN_REL):
    st = err_stats(np.asarray(got, np.float64), np.asarray(ref, np.float64))
    say(f"  {what}: {st}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert st["max_abs"] <= max_abs, (what, st)
    assert st["mean_abs"] <= mean_abs, (what, st)
    assert st["mean_rel"] <= mean_rel, (what, st)
    return st


def sample_rows(layout: dict, n_other: int, seed: int, tile: int = 128) -> np.ndarray:
    """Every padding row, rows at each tile and document boundary, and n_other
    random rows."""
    tags = np.asarray(layout["tags"])
    L = tags.size
    rng = np.random.default_rng(seed)
    rows = set(np.flatnonzero(tags == -1).tolist())
    for b in range(0, L + 1, tile):
        for r in (b - 1, b):
            if 0 <= r < L:
                rows.add(r)
    change = np.flatnonzero(np.diff((tags == -1).astype(np.int8)) != 0)
    for c in change:
        rows.update([int(c), int(c) + 1])
    rows.update(rng.integers(0, L, n_other).tolist())
    rows.update([0, L - 1])
    return np.array(sorted(rows), dtype=np.int32)


class AttentionRun:
    """Run the attention path through the C ABI on one layout + Q/K/V."""

    def __init__(self, inp: dict, wq=None, wk=None, device="cuda", pos_scale=(1.0, 1.0, 1.0),
                 split=True, F=16):
        import torch
        from packed_masked_attention_amd import binding as B
        self.B = B
        self.inp = inp
        lay = inp["layout"]
        self.L = lay["L"]
        self.H = inp["H"]
        self.D = inp.get("D", 128)
        self.dl = B.pma_layout_build(lay, device=device)
        self.p = B.attn_params(self.H, F=F, pos_scale=pos_scale)
        self.q = to_dev_bf16(inp["q"], device)
        self.k = to_dev_bf16(inp["k"], device)
        self.v = to_dev_bf16(inp["v"], device)
        D = self.D
        self.wq = torch.ones(D, dtype=torch.float32, device=device) if wq is None else \
            torch.as_tensor(np.broadcast_to(wq, (D,)).astype(np.float32)).to(device)
        self.wk = torch.ones(D, dtype=torch.float32, device=device) if wk is None else \
            torch.as_tensor(np.broadcast_to(wk, (D,)).astype(np.float32)).to(device)
        self.Lp = B.pma_attention_padded_len(self.L)
        self.qh = torch.empty(self.H, self.Lp, D, dtype=torch.bfloat16, device=device)
        self.kh = torch.empty_like(self.qh)
        self.vt = torch.empty(self.H, D, self.Lp, dtype=torch.bfloat16, device=device)
        self.o = torch.full((self.L, self.H * D), float("nan"), dtype=torch.bfloat16, device=device)
        self.lse = torch.full((self.H, self.L), float("nan"), dtype=torch.float32, device=device)
        # the flash workspace turns on the key-range split of the last items
        self.ws = torch.empty(B.pma_flash_workspace_size(self.p, self.L), dtype=torch.uint8,
                              device=device) if split else None

    def prep(self):
        HD = self.H * self.D
        self.B.pma_qk_norm_rope(self.p, self.dl, self.q, HD, self.k, HD, self.v, HD, self.wq,
                                self.wk, self.qh, self.kh, self.vt)

    def flash(self):
        self.B.pma_flash_attention(self.p, self.dl, self.qh, self.kh, self.vt, self.o,
                                   self.H * self.D, self.lse, workspace=self.ws)

    def run(self):
        import torch
        self.prep()
        self.flash()
        torch.cuda.synchronize()
        return self

    def out(self) -> np.ndarray:
        return bf16_to_np(self.o).reshape(self.L, self.H, self.D)

    def lse_np(self) -> np.ndarray:
        return self.lse.cpu().numpy().T  # [L, H]


def one_rounding(ref, rel=2.0 ** -16):
    """|gpu - ref| allowed for a bf16 value rounded once from an fp32
    computation of the fp64 reference: half an ulp of ref plus the fp32
    computation's error.  That error is absolute on the scale of the
    operands (an fp32 dot product's rounding does not shrink with its
    result), so it is taken relative to |ref| + rms(ref): a few hundred
    fp32 terms, a fp32 norm and rotation stay well below 2^-16 of it."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return 2.0 ** (e - 8) + rel * (a + rms) + 1e-30
