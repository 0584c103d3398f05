"""How the E4M3 matrix instruction accumulates, measured through the C ABI.

fp32 outputs of E4M3 inputs are held to 1e-3 of sum_k |x_k w_k| (plus 1e-4 |ref|) instead of the
fp32-input 1e-4 |ref|, on the reading that the E4M3 MFMA does not add its 64 products per block with
exact fp32 roundings. This test measures that error on the library's own E4M3 path: codes drawn
over every finite exponent (subnormals and 448 included), no scales, fp32 output, so the exact
result is the fp64 sum of the decoded products (E4M3 products carry at most 8 significant bits and
span 2^-18 .. 2^18, so K of them sum exactly in fp64). It records the worst error relative to
sum |products| and checks that it stays inside the bound the parity tests use.
"""
import numpy as np
import pytest
import torch

from gelu_bf16_gemm_amd import binding as B
from gelu_bf16_gemm_amd import inputs as I
from helpers import Guarded, dev, host64, note
from oracle import fusedops_oracle as O

pytestmark = pytest.mark.gpu


def _codes(rng, shape):
    c = I.random_e4m3_codes(rng, shape, e_lo=0, e_hi=15)
    nan = (c & 0x7F) == 0x7F
    return np.where(nan, c - 1, c).astype(np.uint8)  # the all-ones pattern is NaN: use 448


@pytest.mark.parametrize("K", [64, 128, 2048])
def test_e4m3_block_sums_within_the_tolerance_bound(K):
    M, N = 256, 256
    rng = np.random.default_rng([404, K])
    X, W = _codes(rng, (M, K)), _codes(rng, (N, K))
    note(f"e4m3 accumulation M={M} N={N} K={K}")
    y = Guarded(M, N, I.F32)
    st = B.fusedops_linear_epilogue(dev(X, I.F8E4M3), dev(W, I.F8E4M3), y.view, ops=[], out_dtype=I.F32)
    assert st == B.OK, B.status_string(st)
    torch.cuda.synchronize()
    xv, wv = O.e4m3_decode(X), O.e4m3_decode(W)
    exact = xv @ wv.T
    mag = np.abs(xv) @ np.abs(wv).T
    got = host64(y.view)
    rel = np.abs(got - exact) / np.where(mag > 0, mag, 1.0)
    worst = float(rel.max())
    note(f"  worst |y - exact| / sum|x w| = {worst:.3e}; median {float(np.median(rel)):.3e}")
    assert y.intact()
    assert np.all(np.isfinite(got))
    # the parity tests' bound for fp32 outputs of E4M3 inputs
    assert worst <= 1e-3, worst
