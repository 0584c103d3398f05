"""Test-side helpers: device upload of stored inputs and guard-banded outputs. The comparison
rules (tolerances, stated once) live in oracle/parity.py and are re-exported here.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O  # noqa: F401
from gelu_bf16_gemm_amd import inputs as I
from oracle.parity import (F32_TINY, U32, check_f32, check_f32_e4m3_acc, check_fp8, check_lowp,  # noqa: F401
                           check_out, gemm_floor)

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


def workspace_ok(ws) -> bool:
    """The FP8 workspace after a call: no rendezvous gave up waiting (error word 0) and the
    tile ticket counter is back at zero (the rest of the workspace is the library's state)."""
    w = ws[:2].cpu().numpy()
    return int(w[0]) == 0 and int(w[1]) == 0
