"""The GELU-erf approximation the kernels use for 16-bit and E4M3 outputs, checked on the CPU
against the function it stands for.

The kernels compute v Phi(v) as max(v, 0) - |v| h with h = 0.5 erfc(|v| / sqrt 2), and h as
2^p(min(|v|, 6)) for a degree-7 polynomial p fitted to log2 h. The coefficients are read from
the kernel source and evaluated the way the kernel does (fp32 Horner with fused multiply-adds,
exact powers of two), then compared with scipy's erfc in fp64. The kernel source states the
bounds checked here: relative error of h at most 9.1e-6 on [0, 6], absolute error of the GELU
value at most 4.6e-7 for |v| <= 6, and beyond, where h(6) stands for h(|v|), an error of at most
9.9e-10 |v|. A wrong coefficient, a dropped term or a sign error in any of them breaks the first
bound by orders of magnitude.
"""
import os
import re

import numpy as np
from scipy.special import erfc

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gelu_bf16_gemm_amd", "csrc",
                   "common.h")


# the kernels' two forms of h: degree 7 for any 16-bit or E4M3 output, degree 6 for bf16 outputs
FORMS = {"gelu_erf_h": 8, "gelu_erf_h_bf16": 7}  # function -> number of coefficients


def _coefficients(name="gelu_erf_h"):
    text = open(SRC).read()
    body = text[text.index(f"float {name}(float x)"):]
    body = body[:body.index("}")]
    found = dict(re.findall(r"\b(C\d)\s*=\s*([-+0-9.eE]+)f", body))
    n = FORMS[name]
    assert sorted(found) == [f"C{i}" for i in range(n)], found
    return [np.float32(float(found[f"C{i}"])) for i in range(n)]


def _h_kernel(x32, name="gelu_erf_h"):
    """2^p(x) with p evaluated as the kernel does: fp32, one rounding per fused multiply-add."""
    c = _coefficients(name)
    p = np.full_like(x32, c[-1])
    for k in range(len(c) - 2, -1, -1):
        # fma(p, x, c_k) rounded once: exact in fp64 for fp32 operands, then rounded to fp32
        p = (p.astype(np.float64) * x32.astype(np.float64) + np.float64(c[k])).astype(np.float32)
    return np.exp2(p.astype(np.float64))  # the hardware exp2 is within an ulp; exact here


def _gelu_kernel(v, name="gelu_erf_h"):
    v = np.asarray(v, np.float64)
    a = np.abs(v).astype(np.float32)
    x = np.minimum(a, np.float32(6.0))
    return np.maximum(v, 0.0) - a.astype(np.float64) * _h_kernel(x, name)


def test_h_relative_error_on_the_fitted_range():
    x = np.linspace(0.0, 6.0, 600001).astype(np.float32)
    h = 0.5 * erfc(x.astype(np.float64) / np.sqrt(2.0))
    rel = np.abs(_h_kernel(x) / h - 1.0)
    assert rel.max() <= 9.1e-6, rel.max()


def test_gelu_absolute_error():
    v = np.concatenate([np.linspace(-6.0, 6.0, 600001), [-5.999999, 0.0, 5.999999]])
    exact = v * 0.5 * erfc(-v / np.sqrt(2.0))
    err = np.abs(_gelu_kernel(v) - exact)
    assert err.max() <= 4.6e-7, (err.max(), v[np.argmax(err)])
    # past |v| = 6 the clamped h(6) = 9.9e-10 stands for h(|v|)
    v = np.concatenate([np.linspace(-40.0, -6.0, 100001), np.linspace(6.0, 40.0, 100001), [-1e4, 1e4]])
    exact = v * 0.5 * erfc(-v / np.sqrt(2.0))
    err = np.abs(_gelu_kernel(v) - exact)
    assert (err <= 9.9e-10 * np.abs(v)).all(), (err / np.abs(v)).max()


def test_gelu_special_values():
    # v Phi(v): 0 at 0, v for large positive v, a vanishing negative tail
    assert _gelu_kernel(0.0) == 0.0
    assert abs(_gelu_kernel(10.0) - 10.0) < 1e-8
    assert -1e-8 < _gelu_kernel(-10.0) <= 0.0
    # Phi(1) = 0.841344746..., so GELU(1) = 0.841344746 and GELU(-1) = -0.158655254
    assert abs(_gelu_kernel(1.0) - 0.8413447460685429) < 1e-6
    assert abs(_gelu_kernel(-1.0) + 0.15865525393145707) < 1e-6


def test_bf16_form_bounds():
    # degree 6 for bf16 outputs: h within 4.9e-5, the GELU value within 6.6e-6 for |v| <= 6 and
    # within 9.9e-10 |v| beyond (h(6) clamped), all far below half a bf16 ulp (2^-9 of the value)
    x = np.linspace(0.0, 6.0, 600001).astype(np.float32)
    h = 0.5 * erfc(x.astype(np.float64) / np.sqrt(2.0))
    rel = np.abs(_h_kernel(x, "gelu_erf_h_bf16") / h - 1.0)
    assert rel.max() <= 4.9e-5, rel.max()
    v = np.linspace(-6.0, 6.0, 600001)
    err = np.abs(_gelu_kernel(v, "gelu_erf_h_bf16") - v * 0.5 * erfc(-v / np.sqrt(2.0)))
    assert err.max() <= 6.6e-6, err.max()
    v = np.concatenate([np.linspace(-40.0, -6.0, 100001), np.linspace(6.0, 40.0, 100001)])
    err = np.abs(_gelu_kernel(v, "gelu_erf_h_bf16") - v * 0.5 * erfc(-v / np.sqrt(2.0)))
    assert (err <= 9.9e-10 * np.abs(v)).all()
