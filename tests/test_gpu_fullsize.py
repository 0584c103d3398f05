"""Every workload at its full size, in the launch configuration the benchmark times,
checked against the oracle on sampled rows (whole rows, so per-row quantities such as
RMSNorm partials and FP8 scales are checked too)."""

import numpy as np
import pytest
import torch

import oracle as O
from gelu_bf16_gemm_amd import inputs as I

from helpers import check_f32, check_fp8, check_out, dev, host64, note

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gelu_bf16_gemm_amd import binding as B  # noqa: E402
from gelu_bf16_gemm_amd import workloads as WL  # noqa: E402


def sample_rows(M, n=24, seed=0):
    rng = np.random.default_rng([303, M, seed])
    rows = set(range(min(8, M))) | set(range(max(0, M - 8), M)) | set(rng.integers(0, M, n).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", [n for n, s in I.WORKLOADS.items() if s["kind"] == "linear"])
def test_linear_workload_full_size(name):
    spec = I.WORKLOADS[name]
    note(f"full-size {name}: drawing inputs")
    inp = I.make_linear_inputs(spec)
    run = WL.LinearRun(spec, inp)
    note(f"full-size {name}: launch")
    run.launch()
    torch.cuda.synchronize()
    M = spec["M"]
    rows = sample_rows(M)
    dt = spec["in_dtype"]
    fp8 = dt == I.F8E4M3
    X = O.e4m3_decode(inp["X"][rows]) if fp8 else I.to_f64(inp["X"][rows], dt)
    W = O.e4m3_decode(inp["W"]) if fp8 else I.to_f64(inp["W"], dt)
    vec_dt = I.BF16 if fp8 else dt
    ref = O.linear_epilogue(X, W, bias=I.to_f64(inp["b"], vec_dt) if "b" in inp else None,
                            residual=I.to_f64(inp["z"][rows], I.BF16) if "z" in inp else None,
                            col_scale=I.to_f64(inp["gamma"], I.BF16) if "gamma" in inp else None,
                            act=spec.get("act"),
                            x_scale=inp["sa"][rows].astype(np.float64) if "sa" in inp else None,
                            w_scale=inp["sw"].astype(np.float64) if "sw" in inp else None)
    if "rope_cs" in inp:
        N, d = spec["N"], spec["rope"]
        ref["y"] = O.rope_pairs(ref["y"], inp["rope_cs"][rows].astype(np.float64), d,
                                N - N // spec["split"] if spec.get("split") else N)
    out = run.outputs(rows)
    if spec.get("quant_fp8"):
        s = out["scales"].astype(np.float32)
        check_fp8(out["y"], s, ref["y"], f"{name} codes")
        s_ref = O.fp8_row_scale(np.abs(ref["y"]).max(axis=1)).astype(np.float64)
        np.testing.assert_allclose(s.astype(np.float64), s_ref, rtol=2e-4)
        assert run.workspace_ok()
    elif spec.get("xent"):
        lab = inp["labels"][rows]
        m_ref, s_ref = O.xent_chunk_stats(ref["y"], 64)
        check_f32(out["stats"][:, 0::2], m_ref, f"{name} chunk max")
        check_f32(out["stats"][:, 1::2], s_ref, f"{name} chunk sum-exp")
        check_f32(out["target"], ref["y"][np.arange(len(rows)), lab], f"{name} target")
        check_f32(out["loss"], O.cross_entropy(ref["y"], lab), f"{name} loss")
    elif spec.get("split"):
        d = spec["N"] // spec["split"]
        for i, blk in enumerate(out["split"]):
            check_out(blk, ref["y"][:, i * d:(i + 1) * d], spec["out_dtype"], f"{name} block {i}")
    else:
        check_out(out["y"], ref["y"], spec["out_dtype"], f"{name} Y")
    if spec.get("store_aux"):
        check_out(out["aux"], ref["h1"], I.BF16, f"{name} h1")
    if spec.get("rowsumsq"):
        check_f32(out["partials"], ref["partials"], f"{name} partials")
        check_f32(out["r"], O.rmsnorm_finalize(ref["partials"], spec["N"], spec["eps"]), f"{name} r")


@pytest.mark.parametrize("name", [n for n, s in I.WORKLOADS.items() if s["kind"] == "chain"])
def test_chain_workload_full_size(name):
    spec = I.WORKLOADS[name]
    note(f"full-size {name}: drawing inputs")
    inp = I.make_chain_inputs(spec)
    run = WL.ChainRun(spec, inp)
    note(f"full-size {name}: launch")
    run.launch()
    torch.cuda.synchronize()
    rows = sample_rows(spec["M"])
    out = run.outputs(rows)
    ref = O.pattern_a_chain(I.to_f64(inp["X"][rows], I.BF16), I.to_f64(inp["W0"], I.BF16),
                            I.to_f64(inp["z"][rows], I.BF16), I.to_f64(inp["gamma"], I.BF16),
                            I.to_f64(inp["W1"], I.BF16), spec["eps"], act=spec["act"], h2_stored=out["h2"])
    check_out(out["h1"], ref["h1"], I.BF16, f"{name} h1")
    check_f32(out["partials"], ref["partials"], f"{name} partials")
    check_out(out["h2"], ref["h2"], I.BF16, f"{name} h2")
    check_out(out["y"], ref["y"], I.BF16, f"{name} y")


@pytest.mark.parametrize("name", [n for n, s in I.WORKLOADS.items() if s["kind"] == "ln"])
def test_layernorm_workload_full_size(name):
    spec = I.WORKLOADS[name]
    note(f"full-size {name}: drawing inputs")
    inp = I.make_ln_inputs(spec)
    run = WL.LnRun(spec, inp)
    note(f"full-size {name}: launch")
    run.launch()
    torch.cuda.synchronize()
    rows = sample_rows(spec["rows"], n=64)
    ref = O.layernorm_gelu(I.to_f64(inp["x"][rows], I.F16), I.to_f64(inp["gamma"], I.F16),
                           I.to_f64(inp["beta"], I.F16), spec["eps"], spec["form"])
    check_out(run.outputs(rows), ref, I.F16, name)
