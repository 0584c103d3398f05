"""Register and scratch budget of the GEMM kernels, checked on the CPU by compiling them for
gfx950 (hipcc cross-compiles; no GPU needed).

Every 256 x 256 instance keeps 256 fp32 accumulators per lane in AGPRs and runs one wave per
SIMD; what the compiler cannot keep in the remaining registers it spills to scratch. A spill
reload inside the K loop would stall the matrix cores every step, so the mainloop of every
instance must be free of scratch traffic. Outside the K loop (tile set-up and the epilogue)
some instances still spill; their per-lane scratch sizes are pinned here so that a change
that adds spills fails instead of passing unnoticed.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gelu_bf16_gemm_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "--cuda-device-only", "-S", "-Rpass-analysis=kernel-resource-usage"]

# epilogue configuration ids of the static 256 x 256 instances (epi::config values)
CFG = {0: "generic", 2147833089: "bias+gelu_erf", 2147832961: "bias+split", 2147832862: "residual+aux+rms+gamma",
       2147833600: "swiglu", 2147835712: "swiglu+fp8", 2147833632: "rowscale+swiglu", 2149929984: "xent",
       2148881537: "bias+split+rope"}
# scratch bytes per lane allowed outside the K loop: (LDS-DMA mainloop, register-staged mainloop)
T256_BUDGET = {"generic": (92, 0), "bias+gelu_erf": (0, 36), "bias+split": (0, 60),
               "residual+aux+rms+gamma": (64, 136), "swiglu": (8, 52), "swiglu+fp8": (16, 32),
               "rowscale+swiglu": (12, 36), "xent": (196, 252), "bias+split+rope": (52, 120)}
# the other GEMM kernels, by instance (E4M3 inputs: epilogue configuration id; fp32: token tile)
OTHER_BUDGET = {"gemm_fp8_t256_kernelILj2147833089E": 36, "gemm_fp8_t256_kernelILj2147832834E": 100,
                "gemm_fp8_t256_kernelILj0E": 44, "gemm_bf16_skinny_kernelI": 0,
                "gemm_f32_kernelILi128E": 0, "gemm_f32_kernelILi64E": 0}
# resident waves per SIMD the launch configuration of each kernel relies on
OCCUPANCY = {"gemm_bf16_t256_kernel": 1, "gemm_fp8_t256_kernel": 1, "gemm_bf16_skinny_kernel": 2}

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _compile(name):
    src = os.path.join(CSRC, name)
    out = subprocess.run([HIPCC, *FLAGS, src, "-o", "-"], capture_output=True, text=True, cwd=CSRC,
                         timeout=900)
    assert out.returncode == 0, out.stderr[-2000:]
    return out.stdout, out.stderr


@pytest.fixture(scope="module")
def builds():
    names = ["gemm_bf16.hip", "gemm_fp8.hip", "gemm_bf16_skinny.hip", "gemm_f32.hip"]
    with cf.ThreadPoolExecutor(len(names)) as ex:
        return dict(zip(names, ex.map(_compile, names)))


def _resources(remarks):
    """{mangled kernel name: {"scratch": bytes per lane, "occupancy": waves per SIMD}}"""
    res, cur = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = res.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and cur is not None:
            cur["scratch"] = int(m.group(1))
        m = re.search(r"remark:\s+Occupancy \[waves/SIMD\]: (\d+)", line)
        if m and cur is not None:
            cur["occupancy"] = int(m.group(1))
    return res


def _functions(asm):
    """{mangled name: list of instruction lines} for every kernel in an assembly listing."""
    out = {}
    for part in re.split(r"\n(?=_Z\w+:)", asm):
        m = re.match(r"(_Z\w+):", part)
        if m:
            out[m.group(1)] = [l.strip() for l in part.split("\n")]
    return out


def _mainloop_scratch_ops(lines, min_mfma=16):
    """Scratch loads and stores inside the K loop: the innermost (shortest) loop that holds
    at least `min_mfma` MFMAs (the persistent tile loop around it holds them too)."""
    labels = {}
    best = None
    for i, l in enumerate(lines):
        m = re.match(r"(\.LBB\d+_\d+):", l)
        if m:
            labels[m.group(1)] = i
        m = re.match(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\d+_\d+)", l)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            a = labels[m.group(1)]
            n = sum(1 for x in lines[a:i] if x.startswith("v_mfma"))
            if n >= min_mfma and (best is None or i - a < best[1] - best[0]):
                best = (a, i)
    assert best is not None, "no MFMA loop found"
    a, b = best
    return [x for x in lines[a:b + 1] if x.startswith(("scratch_load", "scratch_store"))]


def test_t256_mainloops_spill_free_and_budgets(builds):
    asm, rem = builds["gemm_bf16.hip"]
    res = _resources(rem)
    fns = _functions(asm)
    seen = set()
    for name, r in res.items():
        m = re.search(r"gemm_bf16_t256_kernelILj(\d+)ELb([01])E", name)
        if not m:
            continue
        cfg, dma = CFG[int(m.group(1))], m.group(2) == "1"
        seen.add((cfg, dma))
        assert r["occupancy"] >= OCCUPANCY["gemm_bf16_t256_kernel"], (cfg, dma, r)
        budget = T256_BUDGET[cfg][0 if dma else 1]
        assert r["scratch"] <= budget, f"{cfg} ({'dma' if dma else 'staged'}): {r['scratch']} B/lane > {budget}"
        assert _mainloop_scratch_ops(fns[name]) == [], f"{cfg} ({'dma' if dma else 'staged'}) spills in its K loop"
    assert len(seen) == 2 * len(CFG)


@pytest.mark.parametrize("src,kernel", [("gemm_fp8.hip", "gemm_fp8_t256_kernel"),
                                        ("gemm_bf16_skinny.hip", "gemm_bf16_skinny_kernel"),
                                        ("gemm_f32.hip", "gemm_f32_kernel")])
def test_other_gemm_budgets(builds, src, kernel):
    asm, rem = builds[src]
    res = {n: r for n, r in _resources(rem).items() if kernel in n}
    fns = _functions(asm)
    assert res, kernel
    for name, r in res.items():
        if kernel in OCCUPANCY:
            assert r["occupancy"] >= OCCUPANCY[kernel], (name, r)
        budget = [b for k, b in OTHER_BUDGET.items() if k in name]
        assert len(budget) == 1, name
        assert r["scratch"] <= budget[0], f"{name}: {r['scratch']} B/lane > {budget[0]}"
        if kernel != "gemm_f32_kernel":
            assert _mainloop_scratch_ops(fns[name], min_mfma=8) == [], f"{name} spills in its K loop"
