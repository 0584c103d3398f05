"""Host-side checks of bench.py's contract (no GPU)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_profile(root, kernel, workload, src_rel, src_text, traffic):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    os.makedirs(os.path.dirname(os.path.join(root, src_rel)), exist_ok=True)
    with open(os.path.join(root, src_rel), "w") as f:
        f.write(src_text)
    import hashlib
    h = hashlib.sha256()
    h.update(src_rel.encode())
    h.update(src_text.encode())
    rec = {"sources": [src_rel], "sources_sha256": h.hexdigest(), "traffic_bytes_per_launch": traffic}
    with open(os.path.join(root, "profiles", f"{kernel}__{workload}.md"), "w") as f:
        f.write("# summary\n\n```json\n" + json.dumps(rec, indent=1) + "\n```\n")


def test_traffic_read_while_sources_unchanged_and_dropped_after(tmp_path, monkeypatch):
    root = str(tmp_path)
    _write_profile(root, "k", "w", "src/k.hip", "kernel v1\n", 123456)
    monkeypatch.setattr(bench, "ROOT", root)
    assert bench.measured_traffic("k", "w") == 123456
    with open(os.path.join(root, "src/k.hip"), "w") as f:
        f.write("kernel v2\n")
    assert bench.measured_traffic("k", "w") is None
    assert bench.measured_traffic("missing", "w") is None


def test_committed_profiles_parse():
    """Every committed summary carries a machine-readable record naming existing sources."""
    pdir = os.path.join(ROOT, "profiles")
    n = 0
    for name in sorted(os.listdir(pdir)):
        if "__" not in name or not name.endswith(".md"):
            continue
        kernel, workload = name[:-3].split("__", 1)
        text = open(os.path.join(pdir, name)).read()
        rec = json.loads(text.split("```json\n", 1)[1].split("\n```", 1)[0])
        assert rec["kernel"] == kernel and rec["workload"] == workload
        for p in rec["sources"]:
            assert os.path.exists(os.path.join(ROOT, p)), p
        assert rec["traffic_bytes_per_launch"] > 0
        n += 1
    assert n >= 1


class _FakeRun:
    """Stands in for a workload runner: returns given outputs for the sampled rows."""

    def __init__(self, fn):
        self.fn = fn

    def outputs(self, rows):
        return self.fn(rows)


def test_oracle_leg_gates_on_parity():
    """The oracle leg passes outputs equal to the oracle's and fails (so the rate is withheld)
    for outputs 1 % off; it reports the oracle's own rate on the sampled rows."""
    import numpy as np

    from gelu_bf16_gemm_amd import inputs as I
    from oracle import parity as P

    name = "linear_gelu_f32_64x256x256"
    spec = I.WORKLOADS[name]
    inp = I.make_linear_inputs(spec)
    good = _FakeRun(lambda rows: {"y": P.linear_rows(spec, inp, rows)["y"]})
    bad = _FakeRun(lambda rows: {"y": P.linear_rows(spec, inp, rows)["y"] * 1.01})
    r = bench.oracle_leg(name, spec, inp, good)
    assert r["parity"] == "pass" and r["parity_rows"] == len(bench.sample_rows(64))
    assert r["cpu_baseline"]["kind"] == "oracle" and r["cpu_baseline"]["value"] > 0
    assert bench.oracle_leg(name, spec, inp, bad)["parity"].startswith("FAIL")
    ln = "ln_gelu_f16_32768x3000"
    lspec = dict(I.WORKLOADS[ln], rows=64)
    linp = I.make_ln_inputs(lspec)
    import oracle as O
    ref = lambda rows: O.layernorm_gelu(I.to_f64(linp["x"][rows], I.F16), I.to_f64(linp["gamma"], I.F16),  # noqa: E731
                                        I.to_f64(linp["beta"], I.F16), 1e-5, "tanh")
    assert bench.oracle_leg(ln, lspec, linp, _FakeRun(ref))["parity"] == "pass"
    assert bench.oracle_leg(ln, lspec, linp, _FakeRun(lambda rows: ref(rows) + 0.1))["parity"].startswith("FAIL")
    rows = bench.sample_rows(16384)
    assert rows[0] == 0 and rows[-1] == 16383 and len(rows) > 50 and np.all(np.diff(rows) > 0)


def test_every_workload_has_a_profile():
    """Each workload bench.py times has a committed rocprofv3 summary of its kernels, and
    bench.py attaches those figures to the workload's result."""
    for name, _ in bench.SUITE + bench.NEXT:
        prof = bench.profile_summary(name)
        assert prof, name
        for k, rec in prof.items():
            assert rec["summary"].startswith("profiles/") and k in rec["summary"]
