"""Benchmark of the fused-linear hot path on one MI355X.

One step is one pass of the whole hot path: every workload once, at full size, on
synthetic seeded inputs already resident in HBM (the LayerNorm+GELU rows, the fused
QKV projection with split store, the MLP-up Linear+GELU, the out-projection with
residual + RMSNorm partials + finalize, the gate/up SwiGLU, and the decode / prefill
SwiGLU + FP8 row quantisation, plus the small fp32 Linear+GELU).

`value` is the fused GEMM+epilogue throughput of the step in TFLOP/s: the sum of 2MNK
over the GEMM workloads divided by their summed launch time. Each workload's own TFLOP/s
or GB/s and roofline fraction is reported beside it. A workload's launch time is the median
of 5 repetitions, each the average of `--steps` launches bracketed by HIP events on the
stream the kernels run on; inputs rotate over several copies so operands do not stay
resident in the 256 MB last-level cache between launches.

After each workload's timing, its oracle leg runs the fp64 oracle on sampled rows: the
time it takes is that workload's `cpu_baseline`, and the GPU's outputs for the same rows
are compared with it by the test suite's rules. A workload whose outputs fail reports no
rate and leaves `value`. (`--no-cpu-baseline` skips the oracle legs: "parity": "not
checked".)

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 matrix / vector
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
METRIC = "fused GEMM+epilogue TFLOP/s (%MFMA peak); LN+GELU GB/s (%HBM peak)"

# (workload, bound) in step order; "hbm" workloads are rated in GB/s against the HBM peak
SUITE = [
    ("ln_gelu_f16_32768x4096", "hbm"),
    ("ln_gelu_f16_32768x3000", "hbm"),
    ("qkv_bias_split_bf16_4096x12288x4096", "mfma"),
    ("mlp_up_gelu_bf16_8192x16384x4096", "mfma"),
    ("outproj_residual_rms_bf16_16384x2048x2048", "mfma"),
    ("gateup_swiglu_bf16_16384x16384x2048", "mfma"),
    ("decode_swiglu_fp8_bf16_32x16384x2048", "hbm"),
    ("prefill_swiglu_fp8_bf16_16384x16384x2048", "mfma"),
    ("linear_gelu_f32_64x256x256", "latency"),
]
DOMINANT = "mlp_up_gelu_bf16_8192x16384x4096"
# Widening beyond the suite above (the pattern-A chain, the cross-entropy LM head, RoPE, E4M3
# inputs): timed and reported under "next_workloads",
# each against the fp8 MFMA peak, and not part of `value`.
NEXT = [
    ("chain_outproj_gateup_rms_bf16_16384x2048x16384", "mfma"),
    ("lmhead_xent_bf16_4096x32768x2048", "mfma"),
    ("qkv_bias_rope_split_bf16_4096x12288x4096", "mfma"),
    ("downproj_residual_fp8in_16384x2048x8192", "mfma"),
    ("mlp_up_gelu_fp8in_8192x16384x4096", "mfma"),
]


SETTLE_MS = 100.0
REPS = 5


def time_workload(run, steps: int, warmup: int, settle_ms: float = SETTLE_MS, reps: int = REPS) -> list:
    """Average launch time in ms of each of `reps` repetitions of `steps` launches, after an
    untimed warm-up of at least `warmup` launches and at least `settle_ms` of launches. The GPU
    idles while a workload's inputs are made on the host, and after an idle spell its clock takes
    a few tens of ms of load to settle (measured: the first 50 ms of MLP-up launches run up to
    25 % slower, the first 20 ms of QKV launches up to 3x on the first one); the timed launches
    are the steady state a loop of such layers runs in. Each repetition is bracketed by HIP
    events on the stream the kernels run on (torch's current stream, which the binding passes)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while i < warmup or (time.perf_counter() - t0) * 1e3 < settle_ms:
        run.launch(i)
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()    # the wall clock follows the GPU, not the enqueueing
    out = []
    for _ in range(reps):
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for j in range(steps):
            run.launch(i + j)
        end.record()
        torch.cuda.synchronize()
        i += steps
        out.append(start.elapsed_time(end) / steps)
    return out


def copies_for(spec) -> int:
    """Input copies so that one rotation exceeds the 256 MB last-level cache."""
    from gelu_bf16_gemm_amd import inputs as I
    if spec["kind"] == "ln":
        per = spec["rows"] * spec["cols"] * 2
    elif spec["kind"] == "chain":
        per = (spec["M"] * spec["K0"] + spec["M"] * spec["d"]) * 2
    else:
        es = {I.F32: 4, I.F8E4M3: 1}.get(spec["in_dtype"], 2)
        per = (spec["M"] + spec["N"]) * spec["K"] * es + (spec["M"] * spec["N"] * 2 if spec.get("residual") else 0)
    return max(1, min(8, -(-(300 << 20) // max(per, 1))))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads() -> int:
    from threadpoolctl import threadpool_info
    return int(max([p.get("num_threads", 1) for p in threadpool_info()] + [1]))


def cpu_baseline(seconds_target: float = 10.0, seconds_cap: float = 30.0) -> dict:
    """The oracle (unchanged) on the dominant workload: whole passes over its M rows in
    1024-row blocks until at least `seconds_target` of oracle time (stopping early once
    `seconds_cap` is passed). Input generation is outside the timed region."""
    import oracle as O
    from gelu_bf16_gemm_amd import inputs as I

    spec = I.WORKLOADS[DOMINANT]
    M, N, K = spec["M"], spec["N"], spec["K"]
    block = 1024
    rng = I.rng_for(spec["config_id"], 9)
    W = I.to_f64(I.store(I.normal(rng, (N, K), std=K ** -0.5), I.BF16), I.BF16)
    b = I.to_f64(I.store(I.normal(rng, (N,), std=0.02), I.BF16), I.BF16)
    total_rows, t_total, passes = 0, 0.0, 0
    while t_total < seconds_target:
        for r0 in range(0, M, block):
            X = I.to_f64(I.store(I.normal(rng, (min(block, M - r0), K)), I.BF16), I.BF16)
            t0 = time.perf_counter()
            O.linear_epilogue(X, W, bias=b, act="gelu_erf")
            t_total += time.perf_counter() - t0
            total_rows += X.shape[0]
            if t_total > seconds_cap:
                break
        passes += 1
        if t_total > seconds_cap:
            break
    flops = 2.0 * total_rows * N * K
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": oracle_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "oracle": "numpy float64 with a BLAS matmul for the contraction, scipy's erfc (the oracle as written)",
            "sample": f"{total_rows} rows ({passes} pass(es) over the {M} rows of {DOMINANT} in "
                      f"{block}-row blocks; bias + GELU erf, fp64), {t_total:.1f} s of oracle time"}


def sample_rows(M: int, n: int = 48) -> "np.ndarray":
    """The first and last 8 rows and a seeded spread between them."""
    import numpy as np
    rng = np.random.default_rng([505, M])
    return np.array(sorted(set(range(min(8, M))) | set(range(max(0, M - 8), M)) |
                           set(rng.integers(0, M, n).tolist())))


def oracle_leg(name: str, spec: dict, inp: dict, run) -> dict:
    """The oracle on sampled rows of the workload just timed: its time on those rows (this
    workload's cpu_baseline) and the parity gate of the GPU's outputs for the same rows (every
    output of each sampled row, by the comparison rules of the test suite)."""
    import oracle as O  # noqa: F401  (the oracle leg: the only part of this script that runs it)
    from oracle import parity as P

    from gelu_bf16_gemm_amd import inputs as I

    rows = sample_rows(spec["M"] if "M" in spec else spec["rows"])
    t0 = time.perf_counter()
    if spec["kind"] == "ln":
        dt = spec["io_dtype"]
        ref = O.layernorm_gelu(I.to_f64(inp["x"][rows], dt), I.to_f64(inp["gamma"], dt), I.to_f64(inp["beta"], dt),
                               spec["eps"], spec["form"])
        t = time.perf_counter() - t0
        work, unit = 4.0 * len(rows) * spec["cols"], "GB/s"
        check = lambda: P.check_out(run.outputs(rows), ref, spec["io_dtype"], name)  # noqa: E731
    elif spec["kind"] == "chain":
        out = run.outputs(rows)
        t0 = time.perf_counter()
        try:
            P.check_chain_rows(spec, inp, rows, out, name=name)   # the oracle and the comparison together
            failed = None
        except AssertionError as e:
            failed = e
        t = time.perf_counter() - t0
        work, unit = 2.0 * len(rows) * (spec["d"] * spec["K0"] + spec["N2"] * spec["d"]), "TFLOP/s"

        def check():
            if failed is not None:
                raise failed
    else:
        W64 = P.decode_weights(spec, inp)
        t0 = time.perf_counter()
        P.linear_rows(spec, inp, rows, W64)
        t = time.perf_counter() - t0
        work, unit = 2.0 * len(rows) * spec["N"] * spec["K"], "TFLOP/s"
        check = lambda: P.check_linear_rows(spec, inp, rows, run.outputs(rows), W64=W64, name=name)  # noqa: E731
    parity = "pass"
    try:
        check()
    except AssertionError as e:
        parity = f"FAIL: {str(e)[:300]}"
    rate = work / t / (1e12 if unit == "TFLOP/s" else 1e9)
    return {"parity": parity, "parity_rows": int(len(rows)),
            "cpu_baseline": {"value": round(rate, 4), "unit": unit, "seconds": round(t, 4), "rows": int(len(rows)),
                             "kind": "oracle"}}


def _profile_record(path: str):
    """The machine-readable record of one committed rocprofv3 summary, and whether the sources
    it lists are still the ones the counters were taken on (their sha256 matches)."""
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if m is None:
        return None, False
    rec = json.loads(m.group(1))
    h = hashlib.sha256()
    for p in rec["sources"]:
        h.update(p.encode())
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return rec, h.hexdigest() == rec["sources_sha256"]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from its committed rocprofv3 summary
    (FETCH_SIZE and WRITE_SIZE scaled by the copy calibration), or None when there is no
    summary or the kernel's sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.md")
    if not os.path.exists(path):
        return None
    rec, current = _profile_record(path)
    return rec["traffic_bytes_per_launch"] if rec is not None and current else None


def profile_summary(workload: str) -> dict:
    """Per kernel of `workload`, the figures of its committed rocprofv3 summary (profiles/):
    average duration under the trace, HBM traffic per launch, MFMA busy fraction and the clock
    it held, resident waves per CU and LDS bank conflicts per access. Counter figures of a
    summary whose kernel sources have changed since are withheld (null, "current": false)."""
    out = {}
    pdir = os.path.join(ROOT, "profiles")
    for name in sorted(os.listdir(pdir)) if os.path.isdir(pdir) else []:
        if not name.endswith(f"__{workload}.md"):
            continue
        rec, current = _profile_record(os.path.join(pdir, name))
        if rec is None:
            continue
        keep = ("avg_duration_ns", "traffic_bytes_per_launch", "algorithmic_bytes_per_launch", "mfma_busy_frac",
                "clock_ghz", "waves_per_cu", "lds_bank_conflicts_per_access")
        out[name.split("__", 1)[0]] = {"current": current, "summary": f"profiles/{name}",
                                       **{k: (rec.get(k) if current else None) for k in keep}}
    return out


def copy_calibration(launches: int) -> dict:
    """torch.neg over 1 GiB of fp32 into a second 1 GiB buffer: each launch reads and writes
    exactly 2**30 bytes, the known size a profiler's HBM byte counters are divided by."""
    import torch

    n = 1 << 28
    x = torch.empty(n, dtype=torch.float32, device="cuda").uniform_()
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(launches):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / launches
    del x, y
    torch.cuda.empty_cache()
    return {"kernel": "torch.neg fp32 elementwise", "bytes_read": 1 << 30, "bytes_written": 1 << 30,
            "launches": launches, "ms": round(ms, 4)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default=None, help="comma-separated workload names (default: whole suite)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first stream 1 GiB through a plain elementwise kernel (read once, write once) "
                         "so that HBM byte counters can be scaled against a known size")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(the row-split sharding needs no exchange and is described in the design notes)",
              file=sys.stderr)
        return 2

    import torch

    from gelu_bf16_gemm_amd import inputs as I
    from gelu_bf16_gemm_amd import workloads as WL

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    names = [n for n, _ in SUITE + NEXT] if args.only is None else args.only.split(",")
    bound = dict(SUITE + NEXT)
    suite = {n for n, _ in SUITE}
    results = {}
    calib = copy_calibration(args.steps) if args.copy_calibration else None
    for name in names:
        spec = I.WORKLOADS[name]
        print(f"[bench] {name}: inputs", file=sys.stderr, flush=True)
        if spec["kind"] == "ln":
            inp = I.make_ln_inputs(spec)
            run = WL.LnRun(spec, inp, copies=copies_for(spec))
        elif spec["kind"] == "chain":
            inp = I.make_chain_inputs(spec)
            run = WL.ChainRun(spec, inp, copies=copies_for(spec))
        else:
            inp = I.make_linear_inputs(spec)
            run = WL.LinearRun(spec, inp, copies=copies_for(spec))
        print(f"[bench] {name}: timing", file=sys.stderr, flush=True)
        reps = time_workload(run, args.steps, args.warmup)
        ms = statistics.median(reps)
        fl, by = run.flops(), run.bytes()
        r = {"ms": round(ms, 5), "ms_reps": [round(x, 5) for x in reps], "bound": bound.get(name, "mfma")}
        if fl:
            r["TFLOP/s"] = round(fl / ms / 1e9, 2)
            peak = {I.F32: PEAK_F32_TFLOPS, I.F8E4M3: PEAK_FP8_TFLOPS}.get(spec.get("in_dtype"), PEAK_BF16_TFLOPS)
            r["mfma_frac"] = round(fl / ms / 1e9 / peak, 4)
        r["bytes"] = int(by)
        r["GB/s"] = round(by / ms / 1e6, 1)
        r["hbm_frac"] = round(by / ms / 1e6 / PEAK_HBM_GBPS, 4)
        r["profile"] = profile_summary(name)
        if args.no_cpu_baseline:
            r["parity"] = "not checked"
        else:
            print(f"[bench] {name}: oracle on sampled rows (cpu baseline + parity gate)", file=sys.stderr, flush=True)
            r.update(oracle_leg(name, spec, inp, run))
            if r["parity"] != "pass":
                # a rate is reported only for outputs that match the oracle
                for k in ("TFLOP/s", "mfma_frac", "GB/s", "hbm_frac"):
                    r[k] = None
        results[name] = r
        del run, inp
        torch.cuda.empty_cache()
        print(f"[bench] {name}: {r}", file=sys.stderr, flush=True)

    gemm = [n for n in names if I.WORKLOADS[n]["kind"] == "linear" and n in suite
            and results[n].get("parity") in ("pass", "not checked")]
    gemm_ms = sum(results[n]["ms"] for n in gemm)
    gemm_flops = sum(2.0 * I.WORKLOADS[n]["M"] * I.WORKLOADS[n]["N"] * I.WORKLOADS[n]["K"] for n in gemm)
    value = gemm_flops / gemm_ms / 1e9 if gemm_ms > 0 else 0.0
    step_ms = sum(r["ms"] for n, r in results.items() if n in suite)

    roof = None
    if DOMINANT in results:
        d = results[DOMINANT]
        roof = {"bound": "mfma", "achieved": d["TFLOP/s"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(d["TFLOP/s"] / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic("gemm_bf16_t256_kernel", DOMINANT),
                "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": int(d["bytes"]),
                "kernel": "gemm_bf16_t256_kernel", "workload": DOMINANT}
    ln = results.get("ln_gelu_f16_32768x4096")
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_min_ms": SETTLE_MS, "repetitions": REPS,
        "timing": f"per workload: median of {REPS} repetitions of `steps` launches, each bracketed by HIP events",
        "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "fused-linear hot path suite (one pass of every workload at full size)",
                   "workloads": [n for n in names if n in suite]},
        "roofline": roof,
        "ln_gelu": None if ln is None else {
            "bound": "hbm", "achieved": ln["GB/s"], "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": ln["hbm_frac"],
            "traffic": measured_traffic("ln_gelu_fast_kernel", "ln_gelu_f16_32768x4096"),
            "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": int(ln["bytes"]),
            "kernel": "ln_gelu_fast_kernel", "workload": "ln_gelu_f16_32768x4096"},
        "workloads": {n: r for n, r in results.items() if n in suite},
        "next_workloads": {n: r for n, r in results.items() if n not in suite},
    }
    if calib is not None:
        line["copy_calibration"] = calib
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
