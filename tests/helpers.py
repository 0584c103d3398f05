"""Test-side helpers: device upload of stored inputs, guard-banded outputs and the
comparison rules (tolerances stated once, here).

Tolerances (per output kind):
* bf16 / fp16:  |y - ref| <= 2e-2 + 2e-2 |ref|, element by element.
* fp32:         |y - ref| <= 1e-4 * max(|ref|, rho), rho = RMS of the reference tensor.
  "1e-4 relative" needs a floor where the reference crosses zero (GELU at 0), where fp32
  accumulation error does not vanish; the RMS floor never binds for positive outputs
  such as row partials and RMSNorm scales.
* E4M3 codes:   with the GPU's own row scale s, q_ref = E4M3_RNE(clamp(v_ref / s, +-448));
  the ordinal distance between q_gpu and q_ref is at most 1 (+0 and -0 coincide).
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O
from gelu_bf16_gemm_amd import inputs as I

TORCH_DT = {I.F32: torch.float32, I.BF16: torch.bfloat16, I.F16: torch.float16, I.F8E4M3: torch.uint8}
SENTINEL = 0x5A


def note(msg: str) -> None:
    """Name the case before a GPU step (visible even if the step never returns)."""
    print(msg, file=sys.stderr, flush=True)


def dev(stored: np.ndarray, dtype: int) -> torch.Tensor:
    a = np.ascontiguousarray(stored)
    t = torch.from_numpy(a)
    if dtype == I.BF16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def host64(t: torch.Tensor) -> np.ndarray:
    """Stored values of a GPU tensor as float64 (bf16/fp16 widen exactly)."""
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    return t.float().cpu().numpy().astype(np.float64)


class Guarded:
    """An output of rows x cols (leading dimension ld >= cols) inside a buffer with guard rows
    above and below and guard columns to the right, all filled with a sentinel byte."""

    def __init__(self, rows: int, cols: int, dtype: int, ld: int | None = None, guard_rows: int = 3):
        es = torch.empty(0, dtype=TORCH_DT[dtype]).element_size()
        if ld is None:
            step = 16 // es                    # keep rows 16-byte aligned, leave a column guard
            ld = -(-(cols + step) // step) * step
        self.rows, self.cols, self.ld, self.g = rows, cols, ld, guard_rows
        self.buf = torch.empty((rows + 2 * guard_rows) * ld, dtype=TORCH_DT[dtype], device="cuda")
        self.buf.view(torch.uint8).fill_(SENTINEL)
        self.view = self.buf.view(rows + 2 * guard_rows, ld)[guard_rows:guard_rows + rows, :cols]

    def intact(self) -> bool:
        full = self.buf.view(torch.uint8).view(self.rows + 2 * self.g, -1).cpu().numpy()
        es = self.buf.element_size()
        mask = np.ones(full.shape, dtype=bool)
        mask[self.g:self.g + self.rows, :self.cols * es] = False
        return bool((full[mask] == SENTINEL).all())


def check_lowp(y: np.ndarray, ref: np.ndarray, what: str) -> None:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (what, y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = np.abs(y - ref)
    bound = 2e-2 + 2e-2 * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside 2e-2+2e-2|ref|; "
                           f"worst err {err.max():.3g} at {np.unravel_index(np.argmax(err - bound), err.shape)}")


def check_f32(y: np.ndarray, ref: np.ndarray, what: str, rel: float = 1e-4) -> None:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (what, y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    rho = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = rel * np.maximum(np.abs(ref), rho)
    err = np.abs(y - ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside {rel}*max(|ref|, rms); "
                           f"worst rel {(err / np.maximum(np.abs(ref), rho)).max():.3g}")


def check_f32_e4m3_acc(y: np.ndarray, ref: np.ndarray, mag: np.ndarray, what: str) -> None:
    """fp32 outputs of E4M3 inputs. The E4M3 MFMA sums each block of 64 products with its own
    internal alignment rather than exact fp32 additions (an in-bounds probe of one instruction
    measured errors up to 2.1e-4 of the block's sum of |products| on random codes, exact sums
    when the terms align), so the bound scales with mag = sum_k |x_k w_k| |sa sw| and an
    epilogue amplification of at most 2: 1e-3 * mag + 1e-4 * max(|ref|, rms)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (what, y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    rho = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = 1e-3 * mag + 1e-4 * np.maximum(np.abs(ref), rho)
    err = np.abs(y - ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside 1e-3 mag + 1e-4 max(|ref|, rms)"


def check_out(y: np.ndarray, ref: np.ndarray, dtype: int, what: str) -> None:
    if dtype == I.F32:
        check_f32(y, ref, what)
    else:
        check_lowp(y, ref, what)


def check_fp8(codes: np.ndarray, scales: np.ndarray, vref: np.ndarray, what: str) -> None:
    codes = np.asarray(codes, np.uint8)
    q_ref = O.quantize_fp8_rows(vref, scales)
    d = np.abs(O.e4m3_ordinal(codes) - O.e4m3_ordinal(q_ref))
    assert (d <= 1).all(), f"{what}: {int((d > 1).sum())} codes more than 1 ulp away (max {d.max()})"


def workspace_ok(ws) -> bool:
    """The FP8 workspace after a call: no rendezvous gave up waiting (error word 0) and the
    tile ticket counter is back at zero (the rest of the workspace is the library's state)."""
    w = ws[:2].cpu().numpy()
    return int(w[0]) == 0 and int(w[1]) == 0
