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
