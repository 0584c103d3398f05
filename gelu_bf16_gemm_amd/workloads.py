"""Device set-up and launch of the named workloads (inputs from ``inputs.WORKLOADS``).

Plumbing only: torch allocates device memory, the binding launches the HIP kernels.
Each run can hold several copies of its inputs and rotate through them per launch,
so a timed loop does not keep re-reading operands that stay resident in the 256 MB
last-level cache.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from . import inputs as I

_TORCH = {I.F32: torch.float32, I.BF16: torch.bfloat16, I.F16: torch.float16, I.F8E4M3: torch.uint8}


def to_device(stored: np.ndarray, dtype: int) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(stored))
    if dtype == I.BF16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def _host64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    return t.float().cpu().numpy().astype(np.float64)


class LinearRun:
    """One fused-linear workload: Y = epilogue(X W^T + b), plus the RMSNorm finalize when the
    epilogue writes row partials."""

    def __init__(self, spec: dict, inp: dict, copies: int = 1):
        self.spec = spec
        M, N, K = inp["M"], inp["N"], inp["K"]
        self.M, self.N, self.K = M, N, K
        dt = spec["in_dtype"]
        self.copies = copies
        self.X = [to_device(inp["X"], dt) for _ in range(copies)]
        self.W = [to_device(inp["W"], dt) for _ in range(copies)]
        vec_dt = dt if dt == I.F32 else I.BF16
        self.b = to_device(inp["b"], vec_dt) if "b" in inp else None
        self.sa = to_device(inp["sa"], I.F32) if "sa" in inp else None
        self.sw = to_device(inp["sw"], I.F32) if "sw" in inp else None
        self.rope_cs = to_device(inp["rope_cs"], I.F32) if "rope_cs" in inp else None
        self.z = [to_device(inp["z"], I.BF16) for _ in range(copies)] if "z" in inp else None
        self.gamma = to_device(inp["gamma"], I.BF16) if "gamma" in inp else None
        act = spec.get("act")
        self.n_out = N // 2 if act == "swiglu" else N
        quant = spec.get("quant_fp8", False)
        self.out_dtype = I.F8E4M3 if quant else spec["out_dtype"]
        dev = "cuda"
        self.aux = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if spec.get("store_aux") else None
        T = -(-N // 128)
        self.partials = torch.empty((M, T), dtype=torch.float32, device=dev) if spec.get("rowsumsq") else None
        self.r = torch.empty(M, dtype=torch.float32, device=dev) if spec.get("rowsumsq") else None
        self.scales = torch.empty(M, dtype=torch.float32, device=dev) if quant else None
        self.split = None
        self.y = None
        self.xent = None
        if spec.get("xent"):
            T = -(-N // B.XENT_COLS)
            self.xent = {"labels": torch.from_numpy(inp["labels"]).cuda(),
                         "stats": torch.empty((M, 2 * T), dtype=torch.float32, device=dev),
                         "target": torch.empty(M, dtype=torch.float32, device=dev),
                         "loss": torch.empty(M, dtype=torch.float32, device=dev)}
        elif spec.get("split"):
            d = N // spec["split"]
            self.split = [torch.empty((M, d), dtype=_TORCH[self.out_dtype], device=dev) for _ in range(spec["split"])]
        else:
            self.y = torch.empty((M, self.n_out), dtype=_TORCH[self.out_dtype], device=dev)
        self.ops_by_copy = [self._ops(i) for i in range(copies)]
        self._calls, self._calls_stream = None, None
        self.ws = None
        if quant:
            nbytes = B.fusedops_linear_workspace_bytes(M, N, K, self.ops_by_copy[0])
            self.ws = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
        self.eps = spec.get("eps", 1e-6)

    def _ops(self, i: int) -> list:
        s = self.spec
        ops = []
        if self.z is not None:
            ops.append(B.op(B.OP_RESIDUAL_ADD, self.z[i]))
        if self.aux is not None:
            ops.append(B.op(B.OP_STORE_AUX, out=self.aux))
        if self.partials is not None:
            ops.append(B.op(B.OP_ROWSUMSQ_PARTIAL, out=self.partials))
        if self.gamma is not None:
            ops.append(B.op(B.OP_COL_SCALE, self.gamma))
        act = s.get("act")
        if act == "gelu_erf":
            ops.append(B.op(B.OP_GELU_ERF))
        elif act == "gelu_tanh":
            ops.append(B.op(B.OP_GELU_TANH))
        elif act == "swiglu":
            ops.append(B.op(B.OP_SWIGLU))
        if self.scales is not None:
            ops.append(B.op(B.OP_QUANT_FP8_ROW, out=self.scales))
        if self.split is not None:
            ops.append(B.op(B.OP_SPLIT_COLS, split=self.split))
        if self.sa is not None:
            ops.append(B.op(B.OP_DEQUANT_ROW, self.sa))
        if self.sw is not None:
            ops.append(B.op(B.OP_DEQUANT_COL, self.sw))
        if self.rope_cs is not None:
            ops.append(B.op(B.OP_ROPE, self.rope_cs, head_dim=s["rope"]))
        if self.xent is not None:
            x = self.xent
            ops.append(B.xent_op(x["labels"], x["stats"], x["target"]))
        return ops

    def launch(self, i: int = 0, stream=None) -> None:
        """One pass of the workload (input copy i % copies). On the current stream the calls are
        marshalled once per copy, so a launch loop is not bounded by per-call marshalling."""
        i %= self.copies
        if stream is None:
            if self._calls is None or self._calls_stream != torch.cuda.current_stream():
                self._calls_stream = torch.cuda.current_stream()
                self._calls = [B.prepare_linear_epilogue(self.X[c], self.W[c], self.y, bias=self.b,
                                                         ops=self.ops_by_copy[c], workspace=self.ws,
                                                         out_dtype=self.out_dtype) for c in range(self.copies)]
            B.check(self._calls[i]())
        else:
            B.check(B.fusedops_linear_epilogue(self.X[i], self.W[i], self.y, bias=self.b, ops=self.ops_by_copy[i],
                                               workspace=self.ws, out_dtype=self.out_dtype, stream=stream))
        if self.partials is not None:
            B.check(B.fusedops_rmsnorm_finalize(self.partials, self.N, self.eps, self.r, stream=stream))
        if self.xent is not None:
            x = self.xent
            B.check(B.fusedops_cross_entropy_finalize(x["stats"], self.N, x["target"], x["labels"], x["loss"],
                                                      stream=stream))

    def outputs(self, rows) -> dict:
        idx = torch.as_tensor(np.asarray(rows), device="cuda")
        out = {}
        if self.y is not None:
            out["y"] = _host64(self.y.index_select(0, idx))
        if self.split is not None:
            out["split"] = [_host64(s.index_select(0, idx)) for s in self.split]
        if self.aux is not None:
            out["aux"] = _host64(self.aux.index_select(0, idx))
        if self.partials is not None:
            out["partials"] = _host64(self.partials.index_select(0, idx))
            out["r"] = _host64(self.r.index_select(0, idx))
        if self.scales is not None:
            out["scales"] = _host64(self.scales.index_select(0, idx))
        if self.xent is not None:
            for k in ("stats", "target", "loss"):
                out[k] = _host64(self.xent[k].index_select(0, idx))
        return out

    def workspace_ok(self) -> bool:
        """No row rendezvous gave up (error word 0) and the ticket counter is back at zero."""
        if self.ws is None:
            return True
        w = self.ws[:2].cpu().numpy()
        return int(w[0]) == 0 and int(w[1]) == 0

    # algorithmic work of one pass
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    def bytes(self) -> float:
        """HBM bytes the method must move: each input once, each output once."""
        s, M, N, K = self.spec, self.M, self.N, self.K
        es_in = {I.F32: 4, I.BF16: 2, I.F16: 2, I.F8E4M3: 1}[s["in_dtype"]]
        es_out = {I.F32: 4, I.BF16: 2, I.F16: 2, I.F8E4M3: 1}[self.out_dtype]
        b = (M * K + N * K) * es_in + M * self.n_out * es_out
        if self.b is not None:
            b += N * self.b.element_size()
        if self.sa is not None:
            b += M * 4
        if self.sw is not None:
            b += N * 4
        if self.rope_cs is not None:
            b += self.rope_cs.numel() * 4
        if self.xent is not None:
            # labels, statistics written and read back, target, loss; no logits when y is absent
            b += M * 4 + self.xent["stats"].numel() * 4 * 2 + M * 4 * 2 + M * 4
            if self.y is None:
                b -= M * self.n_out * es_out
        if self.z is not None:
            b += M * N * 2
        if self.aux is not None:
            b += M * N * 2
        if self.gamma is not None:
            b += N * 2
        if self.partials is not None:
            b += M * (-(-N // 128)) * 4 * 2 + M * 4        # partials written, read back, r written
        if self.scales is not None:
            b += M * 4
        return float(b)


class ChainRun:
    """Pattern A end to end: GEMM 1 (residual, h1, row partials, gamma) writes h2; GEMM 2 reads
    h2 and applies the deferred RMSNorm row scale from the partials (ROW_RMS) before its
    activation. One pass = both launches."""

    def __init__(self, spec: dict, inp: dict, copies: int = 1):
        self.spec = spec
        M, d, K0, N2 = spec["M"], spec["d"], spec["K0"], spec["N2"]
        self.M, self.d, self.K0, self.N2 = M, d, K0, N2
        self.copies = copies
        dev = "cuda"
        self.X = [to_device(inp["X"], I.BF16) for _ in range(copies)]
        self.W0 = to_device(inp["W0"], I.BF16)
        self.z = [to_device(inp["z"], I.BF16) for _ in range(copies)]
        self.gamma = to_device(inp["gamma"], I.BF16)
        self.W1 = to_device(inp["W1"], I.BF16)
        T = -(-d // 128)
        self.h1 = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
        self.partials = torch.empty((M, T), dtype=torch.float32, device=dev)
        self.h2 = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
        self.n_out = N2 // 2 if spec["act"] == "swiglu" else N2
        self.y = torch.empty((M, self.n_out), dtype=torch.bfloat16, device=dev)
        self.ops1 = [[B.op(B.OP_RESIDUAL_ADD, self.z[i]), B.op(B.OP_STORE_AUX, out=self.h1),
                      B.op(B.OP_ROWSUMSQ_PARTIAL, out=self.partials), B.op(B.OP_COL_SCALE, self.gamma)]
                     for i in range(copies)]
        act = {"swiglu": B.OP_SWIGLU, "gelu_erf": B.OP_GELU_ERF}[spec["act"]]
        self.ops2 = [B.op(act), B.row_rms_op(self.partials, d, spec["eps"])]

    def launch(self, i: int = 0, stream=None) -> None:
        i %= self.copies
        B.check(B.fusedops_linear_epilogue(self.X[i], self.W0, self.h2, ops=self.ops1[i], stream=stream))
        B.check(B.fusedops_linear_epilogue(self.h2, self.W1, self.y, ops=self.ops2, stream=stream))

    def outputs(self, rows) -> dict:
        idx = torch.as_tensor(np.asarray(rows), device="cuda")
        return {k: _host64(getattr(self, k).index_select(0, idx)) for k in ("h1", "partials", "h2", "y")}

    def flops(self) -> float:
        return 2.0 * self.M * self.d * self.K0 + 2.0 * self.M * self.N2 * self.d

    def bytes(self) -> float:
        """HBM bytes the chain must move: inputs once, h1 / h2 / partials written once and h2 and
        the partials read once more by the second GEMM, y written once."""
        M, d, K0, N2 = self.M, self.d, self.K0, self.N2
        T = -(-d // 128)
        return float(2 * (M * K0 + d * K0 + M * d + d + N2 * d) + 2 * M * d * 2 + M * T * 4 * 2
                     + 2 * M * d + 2 * M * self.n_out)


class LnRun:
    """The LayerNorm+GELU row workload."""

    def __init__(self, spec: dict, inp: dict, copies: int = 1):
        self.spec = spec
        self.rows, self.cols = inp["rows"], inp["cols"]
        dt = spec["io_dtype"]
        self.copies = copies
        self.x = [to_device(inp["x"], dt) for _ in range(copies)]
        self.gamma = to_device(inp["gamma"], dt)
        self.beta = to_device(inp["beta"], dt)
        self.y = torch.empty((self.rows, self.cols), dtype=_TORCH[dt], device="cuda")
        self.form = {"tanh": B.GELU_TANH, "erf": B.GELU_ERF, "none": B.GELU_NONE}[spec["form"]]

    def launch(self, i: int = 0, stream=None) -> None:
        B.check(B.fusedops_layernorm_gelu(self.x[i % self.copies], self.y, self.gamma, self.beta,
                                          eps=self.spec["eps"], gelu_form=self.form, stream=stream))

    def outputs(self, rows) -> np.ndarray:
        idx = torch.as_tensor(np.asarray(rows), device="cuda")
        return _host64(self.y.index_select(0, idx))

    def flops(self) -> float:
        return 0.0

    def bytes(self) -> float:
        es = 4 if self.spec["io_dtype"] == I.F32 else 2
        return float(2 * self.rows * self.cols * es + 2 * self.cols * es)
