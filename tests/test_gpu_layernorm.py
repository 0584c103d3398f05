"""Parity of the LayerNorm+GELU row kernel (HIP path through the C ABI) with the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle as O
from gelu_bf16_gemm_amd import inputs as I

from helpers import Guarded, check_f32, check_out, dev, host64, note

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gelu_bf16_gemm_amd import binding as B  # noqa: E402

FORM = {"tanh": B.GELU_TANH, "erf": B.GELU_ERF, "none": B.GELU_NONE}


def run_ln(rows, cols, io=I.F16, out=I.F16, pd=I.F16, form="tanh", eps=1e-5, seed=0, gamma=True,
           beta=True, inplace=False, mean=0.0, std=1.0):
    rng = np.random.default_rng([202, rows, cols, seed])
    x = I.random_stored(rng, (rows, cols), io, mean=mean, std=std)
    g = I.random_stored(rng, (cols,), pd, mean=1.0, std=0.1) if gamma else None
    b = I.random_stored(rng, (cols,), pd, std=0.1) if beta else None
    note(f"layernorm rows={rows} cols={cols} io={io} out={out} pd={pd} form={form} inplace={inplace}")
    if inplace:
        y = Guarded(rows, cols, io)
        y.view.copy_(dev(x, io))
        xd = y.view
    else:
        y = Guarded(rows, cols, out)
        xd = dev(x, io)
    st = B.fusedops_layernorm_gelu(xd, y.view, None if g is None else dev(g, pd), None if b is None else dev(b, pd),
                                   eps=eps, gelu_form=FORM[form])
    assert st == B.OK, B.status_string(st)
    torch.cuda.synchronize()
    ref = O.layernorm_gelu(I.to_f64(x, io), None if g is None else I.to_f64(g, pd),
                           None if b is None else I.to_f64(b, pd), eps, form)
    got = host64(y.view)
    check_out(got, ref, io if inplace else out, "LN+GELU")
    assert y.intact()
    return got


@pytest.mark.parametrize("rows,cols", [(257, 4096), (257, 3000), (5, 8), (33, 520), (9, 16384), (7, 6000),
                                       (3, 4104)])
def test_ln_gelu_tanh_f16(rows, cols):
    run_ln(rows, cols)


@pytest.mark.parametrize("io,out,pd", [(I.BF16, I.BF16, I.BF16), (I.F32, I.F32, I.F32), (I.F16, I.F32, I.F16),
                                       (I.F32, I.F16, I.BF16)])
def test_ln_dtypes(io, out, pd):
    run_ln(65, 3000 if io != I.F32 else 2996, io=io, out=out, pd=pd)
    run_ln(3, 12000, io=io, out=out, pd=pd, seed=1)


def test_ln_erf_form():
    run_ln(65, 4096, form="erf")


def test_ln_moments_before_affine():
    """gamma = 1, beta = 0, no GELU, fp32 output: each row has mean 0 and variance
    var / (var + eps), the invariants of LayerNorm before the affine step."""
    got = run_ln(64, 3000, io=I.F16, out=I.F32, form="none", gamma=False, beta=False, mean=3.0, std=2.0)
    assert np.abs(got.mean(axis=1)).max() < 1e-5
    assert np.abs(got.var(axis=1) - 1.0).max() < 1e-4


def test_ln_in_place():
    run_ln(40, 4096, inplace=True)


def test_ln_constant_rows():
    """A constant row normalises to 0, so the output is GELU(beta) exactly up to rounding."""
    rows, cols = 4, 1024
    x = np.full((rows, cols), 1.5, np.float16)
    b = I.random_stored(np.random.default_rng(3), (cols,), I.F16, std=0.5)
    y = Guarded(rows, cols, I.F32)
    note("layernorm constant rows")
    assert B.fusedops_layernorm_gelu(dev(x, I.F16), y.view, None, dev(b, I.F16), eps=1e-5) == B.OK
    torch.cuda.synchronize()
    check_f32(host64(y.view), np.tile(O.gelu_tanh(I.to_f64(b, I.F16)), (rows, 1)), "GELU(beta)")
