"""Every workload at its full size, in the launch configuration the benchmark times, checked
against the oracle on EVERY output element: the oracle runs on the host in blocks of 1024 rows
(whole rows, so per-row quantities such as RMSNorm partials, FP8 scales and cross-entropy
statistics are checked too). FP8 workloads also pass the tier-2 scale rule at full size: every
scale is bit-exactly fl32(max |y32| / 448) of the same kernel's fp32 values."""

import numpy as np
import pytest
import torch

from gelu_bf16_gemm_amd import inputs as I
from oracle import parity as P

from helpers import note

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gelu_bf16_gemm_amd import binding as B  # noqa: E402
from gelu_bf16_gemm_amd import workloads as WL  # noqa: E402

BLOCK = 1024


def blocks(M):
    for r0 in range(0, M, BLOCK):
        yield np.arange(r0, min(M, r0 + BLOCK))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", [n for n, s in I.WORKLOADS.items() if s["kind"] == "linear"])
def test_linear_workload_full_size(name):
    spec = I.WORKLOADS[name]
    note(f"full-size {name}: drawing inputs")
    inp = I.make_linear_inputs(spec)
    run = WL.LinearRun(spec, inp)
    note(f"full-size {name}: launch")
    run.launch()
    torch.cuda.synchronize()
    y32 = None
    if spec.get("quant_fp8"):
        # tier 2: the same op list without quantisation, fp32 output, from the same kernel's mainloop
        y32 = torch.empty((run.M, run.n_out), dtype=torch.float32, device="cuda")
        ops = [o for o in run.ops_by_copy[0] if o.kind != B.OP_QUANT_FP8_ROW]
        note(f"full-size {name}: fp32 values of the same op list")
        B.check(B.fusedops_linear_epilogue(run.X[0], run.W[0], y32, ops=ops, out_dtype=I.F32))
        torch.cuda.synchronize()
        assert run.workspace_ok()
    W64 = P.decode_weights(spec, inp)
    for rows in blocks(spec["M"]):
        note(f"full-size {name}: rows {rows[0]}..{rows[-1]}")
        out = run.outputs(rows)
        if y32 is not None:
            out["y32"] = y32[rows[0]:rows[-1] + 1].cpu().numpy().astype(np.float64)
        P.check_linear_rows(spec, inp, rows, out, W64=W64, name=name)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", [n for n, s in I.WORKLOADS.items() if s["kind"] == "chain"])
def test_chain_workload_full_size(name):
    spec = I.WORKLOADS[name]
    note(f"full-size {name}: drawing inputs")
    inp = I.make_chain_inputs(spec)
    run = WL.ChainRun(spec, inp)
    note(f"full-size {name}: launch")
    run.launch()
    torch.cuda.synchronize()
    for rows in blocks(spec["M"]):
        note(f"full-size {name}: rows {rows[0]}..{rows[-1]}")
        P.check_chain_rows(spec, inp, rows, run.outputs(rows), name=name)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", [n for n, s in I.WORKLOADS.items() if s["kind"] == "ln"])
def test_layernorm_workload_full_size(name):
    spec = I.WORKLOADS[name]
    note(f"full-size {name}: drawing inputs")
    inp = I.make_ln_inputs(spec)
    run = WL.LnRun(spec, inp)
    note(f"full-size {name}: launch")
    run.launch()
    torch.cuda.synchronize()
    for rows in blocks(spec["rows"]):
        P.check_ln_rows(spec, inp, rows, run.outputs(rows), name=name)
