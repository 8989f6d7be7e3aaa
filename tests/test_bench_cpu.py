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


def _bf16_bits(values):
    import numpy as np
    f = np.asarray(values, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_same_run_parity_comparison_counts_ulps_zeros_and_nans():
    """The bench's element comparison (its same-run parity check): ulp distances
    across binades, zeros and their signs, NaN positions, fp16 and fp32."""
    import numpy as np
    want = _bf16_bits([[1.0, 2.0, -3.0, 0.0], [0.5, -0.0, 7.0, 1e-38]])
    r = bench.compare_bits(want.copy(), want, "bf16")
    assert r == {"exact_frac": 1.0, "max_ulp": 0, "zeros_and_nans_match": True}
    got = want.copy()
    got[0, 0] += 1                      # one ulp above 1.0
    got[0, 2] -= 1                      # one ulp towards zero from -3.0
    r = bench.compare_bits(got, want, "bf16")
    assert r["max_ulp"] == 1 and r["zeros_and_nans_match"] and r["exact_frac"] == 6 / 8
    got = want.copy()
    got[1, 0] = _bf16_bits([0.5])[0] - 1  # just below 0.5: across a binade, still one ulp
    assert bench.compare_bits(got, want, "bf16")["max_ulp"] == 1
    for i, j, v in ((0, 3, -0.0), (1, 1, 0.0), (0, 1, 0.0)):   # a zero's sign, a zero on one side only
        got = want.copy()
        got[i, j] = _bf16_bits([v])[0]
        assert not bench.compare_bits(got, want, "bf16")["zeros_and_nans_match"], (i, j, v)
    got, w2 = want.copy(), want.copy()
    got[1, 2], w2[1, 2] = 0x7FC1, 0x7FC0  # NaN on both sides with different payloads: same position
    r = bench.compare_bits(got, w2, "bf16")
    assert r["zeros_and_nans_match"] and r["exact_frac"] == 1.0
    got = want.copy()
    got[1, 2] = 0x7FC0                    # NaN on one side only
    assert not bench.compare_bits(got, want, "bf16")["zeros_and_nans_match"]
    h = np.array([[1.0, -2.0]], np.float16).view(np.uint16)
    g = h.copy()
    g[0, 1] += 3
    assert bench.compare_bits(g, h, "f16")["max_ulp"] == 3
    f = np.array([[1.0, -2.0, 0.0]], np.float32).view(np.uint32)
    g = f.copy()
    g[0, 0] += 2
    r = bench.compare_bits(g, f, "f32")
    assert r["max_ulp"] == 2 and r["zeros_and_nans_match"]
    # chunking over rows gives the same answer
    rng = np.random.default_rng(1)
    big = _bf16_bits(rng.standard_normal((50, 64)))
    g = big.copy()
    g[37, 5] += 1
    assert bench.compare_bits(g, big, "bf16", rows_per_chunk=7) == bench.compare_bits(g, big, "bf16")


def test_dprobs_comparison_is_relative_to_the_sum_of_absolute_terms():
    import numpy as np
    r = bench.compare_dprobs(np.array([1.0, 2.0], np.float32), np.array([1.0, 2.0 + 1e-4]), np.array([1.0, 10.0]))
    assert abs(r["max_err_over_sum_abs_terms"] - 1e-5) < 1e-9


def test_same_run_parity_on_oracle_outputs_and_planted_errors():
    """same_run_parity with the oracle's own outputs as the step's outputs is
    bit-exact and within the bar; a 2-ulp or a 1-ulp (router) error is not."""
    import numpy as np
    import oracle
    from moe_routed_expert_amd.workloads import custom
    w = WORKLOADS["swiglu_256x128"]
    d = w.generate()
    y = oracle.swiglu_clamped_fwd(d["x"], d["probs"], w.rows, w.cols, w.limit)
    gx, gp = oracle.swiglu_clamped_bwd(d["x"], d["probs"], d["grad_out"], w.rows, w.cols, w.limit)
    r = bench.same_run_parity(oracle, w, d, "bf16", "bf16", True, y.copy(), gx.copy(), gp.astype(np.float32), 1)
    assert r["within_bar"] is True and r["y"]["exact_frac"] == 1.0 and r["grad_x"]["exact_frac"] == 1.0
    assert r["grad_probs"]["max_err_over_sum_abs_terms"] == 0.0
    nz = np.flatnonzero((y.ravel() & 0x7FFF) != 0)[0]
    y2 = y.copy().ravel()
    y2[nz] += 2
    r = bench.same_run_parity(oracle, w, d, "bf16", "bf16", True, y2.reshape(y.shape), gx.copy(),
                              gp.astype(np.float32), 1)
    assert r["within_bar"] is False and r["y"]["max_ulp"] == 2
    r = bench.same_run_parity(oracle, w, d, "bf16", "bf16", False, y.copy(), gx.copy(), None, 1)
    assert r["within_bar"] is True and r["grad_probs"] is None

    wr = custom("router", 16, 64, x_sigma=1.0, seed=5)
    dr = wr.generate()
    out = oracle.router_weight_mul_fwd(dr["x"], dr["probs"], wr.rows, wr.cols)
    rgx, rgp = oracle.router_weight_mul_bwd(dr["grad_out"], dr["x"], dr["probs"], wr.rows, wr.cols)
    r = bench.same_run_parity(oracle, wr, dr, "bf16", "bf16", True, out.copy(), rgx.copy(), rgp.astype(np.float32), 1)
    assert r["within_bar"] is True
    bad = out.copy()
    bad[3, 3] += 1
    r = bench.same_run_parity(oracle, wr, dr, "bf16", "bf16", True, bad, rgx.copy(), rgp.astype(np.float32), 1)
    assert r["within_bar"] is False
