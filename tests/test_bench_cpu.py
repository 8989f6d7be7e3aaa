"""bench.py's host-side logic, on the CPU: the one-GPU guard, the source digest
that decides whether a committed counter record still applies, and the mapping
from workloads to their rocprofv3 summaries."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from moe_routed_expert_amd.workloads import (COMBINE_WORKLOADS, DOWN_WORKLOADS, GROUPED_WORKLOADS,  # noqa: E402
                                             HEADLINE, WORKLOADS)


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_code_only_ignores_comments_and_layout_but_not_code():
    a = "int f(int x) {  // doubles x\n    return 2 * x; /* the\n  factor */ }\n"
    b = "/* header */ int f(int x) { return 2 * x; }"
    c = "int f(int x) { return 3 * x; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_every_measured_workload_has_its_summary():
    measured = [WORKLOADS[HEADLINE], WORKLOADS["router_65536x7168"]]
    measured += [GROUPED_WORKLOADS[n] for n in GROUPED_WORKLOADS if n.startswith("grouped_131072")]
    measured += [DOWN_WORKLOADS[n] for n in DOWN_WORKLOADS if n.startswith("down_131072")]
    measured += [COMBINE_WORKLOADS[n] for n in COMBINE_WORKLOADS if n.startswith("combine_131072")]
    assert len(measured) == 6
    for w in measured:
        path = os.path.join(ROOT, "profiles", bench.profile_name(w))
        assert os.path.exists(path), path
        text = open(path).read()
        assert "rocprofv3" in text, path  # the command that made it
        start = text.index("```json") + len("```json")
        rec = json.loads(text[start:text.index("```", start)])
        assert rec["workload"] == w.name
        assert set(rec) >= {"kernel_source_digest", "fetch_scale", "write_scale", "kernels"}
        for k in rec["kernels"].values():
            assert k["hbm_bytes_per_launch"] == pytest.approx(k["read_bytes"] + k["write_bytes"])
            # streaming kernels record their algorithmic bytes, the GEMMs the minimum
            # (every operand read once, every output written once)
            floor = k["algorithmic_bytes"] if "algorithmic_bytes" in k else k["min_bytes"]
            assert k["hbm_bytes_per_launch"] >= 0.99 * floor


def test_traffic_is_used_only_while_the_sources_match(monkeypatch):
    w = WORKLOADS[HEADLINE]
    text = open(os.path.join(ROOT, "profiles", bench.profile_name(w))).read()
    start = text.index("```json") + len("```json")
    rec = json.loads(text[start:text.index("```", start)])
    kernel = "swiglu_clamped_bwd"
    monkeypatch.setattr(bench, "kernel_source_digest", lambda op: rec["kernel_source_digest"])
    assert bench.load_traffic(kernel, w) == rec["kernels"][kernel]["hbm_bytes_per_launch"]
    assert bench.load_traffic("no_such_kernel", w) is None
    monkeypatch.setattr(bench, "kernel_source_digest", lambda op: "0" * 16)
    assert bench.load_traffic(kernel, w) is None


def test_digest_changes_with_the_code_of_its_own_op_only(tmp_path, monkeypatch):
    from moe_routed_expert_amd import build as hip_build
    for name in set(n for names in bench.KERNEL_SOURCES.values() for n in names):
        (tmp_path / name).write_text(open(os.path.join(hip_build.CSRC, name)).read())
    monkeypatch.setattr(hip_build, "CSRC", str(tmp_path))
    before = {op: bench.kernel_source_digest(op) for op in bench.KERNEL_SOURCES}
    src = tmp_path / "moe_combine.hip"
    src.write_text(src.read_text() + "\n// a comment only\n")
    assert {op: bench.kernel_source_digest(op) for op in bench.KERNEL_SOURCES} == before
    src.write_text(src.read_text() + "\nstatic int unused_marker = 1;\n")
    after = {op: bench.kernel_source_digest(op) for op in bench.KERNEL_SOURCES}
    assert after["combine"] != before["combine"]
    assert all(after[op] == before[op] for op in bench.KERNEL_SOURCES if op != "combine")
