"""Parity of the LayerNorm+GELU row kernel (HIP path through the C ABI) with the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle as O
from gelu_bf16_gemm_amd import inputs as I

from helpers import U32, Guarded, check_f32, check_out, dev, host64, note

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
    # fp32 floor: the statistics are fp32 sums over the row, so the normalised value carries an
    # error of about (cols + 8) u (|x| + |mu|) rstd; gamma and the activation's slope carry it on
    x64 = I.to_f64(x, io)
    mu, var = O.layernorm_stats(x64)
    rstd = 1.0 / np.sqrt(var + eps)
    dxhat = (cols + 8) * U32 * (np.abs(x64) + np.abs(mu)[:, None]) * rstd[:, None]
    pre = O.layernorm(x64, None if g is None else I.to_f64(g, pd), None if b is None else I.to_f64(b, pd), eps)
    gabs = 1.0 if g is None else np.abs(I.to_f64(g, pd))[None, :]
    f = {"tanh": O.gelu_tanh, "erf": O.gelu_erf, "none": lambda v: v}[form]
    dd = 1e-6 * np.maximum(1.0, np.abs(pre))
    slope = np.abs(f(pre + dd) - f(pre - dd)) / (2 * dd)
    check_out(got, ref, io if inplace else out, "LN+GELU", dxhat * gabs * slope)
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


def test_ln_erf_negative_tail_fp32_output():
    """beta around -5.5 puts most normalised values in [-8, -3]: fp32 outputs keep 1e-4 relative
    accuracy in GELU_erf's negative tail (row kernels for a 2-byte input and fp32 output)."""
    rows, cols = 33, 3000
    rng = np.random.default_rng(405)
    x = I.random_stored(rng, (rows, cols), I.F16)
    b = I.random_stored(rng, (cols,), I.F16, mean=-5.5, std=0.5)
    y = Guarded(rows, cols, I.F32)
    note("layernorm erf negative tail fp32 output")
    assert B.fusedops_layernorm_gelu(dev(x, I.F16), y.view, None, dev(b, I.F16), eps=1e-5,
                                     gelu_form=B.GELU_ERF) == B.OK
    torch.cuda.synchronize()
    pre = O.layernorm(I.to_f64(x, I.F16), None, I.to_f64(b, I.F16), 1e-5)
    ref = O.gelu_erf(pre)
    got = host64(y.view)
    tail = (pre > -8) & (pre < -3)
    assert tail.mean() > 0.8
    # the bound of run_ln: the statistics' fp32 error moves the normalised value by at most
    # about (cols + 8) u (|x| + |mu|) rstd, times GELU's slope
    x64 = I.to_f64(x, I.F16)
    mu, var = O.layernorm_stats(x64)
    rstd = 1.0 / np.sqrt(var + 1e-5)
    dxhat = (cols + 8) * U32 * (np.abs(x64) + np.abs(mu)[:, None]) * rstd[:, None]
    dd = 1e-6 * np.maximum(1.0, np.abs(pre))
    slope = np.abs(O.gelu_erf(pre + dd) - O.gelu_erf(pre - dd)) / (2 * dd)
    check_f32(got, ref, "LN GELU_erf tail", dxhat * slope)
    rel = np.abs(got[tail] - ref[tail]) / np.abs(ref[tail])
    assert np.median(rel) < 1e-4, np.median(rel)
    assert y.intact()


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
