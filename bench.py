#!/usr/bin/env python3
"""Benchmark of the routed-expert epilogue on one MI355X.

A step is one pass of the whole path over the workload, inputs resident in
HBM: swiglu_clamped_fwd followed by swiglu_clamped_bwd (with the per-row
probability gradient), launched through the C ABI on torch's current stream.
The default workload is the per-GPU share of the pages' large-node shape:
rows = 131072, inter = 2048 (x is 131072 x 4096 bf16, about 1.07 GB), L = 10.

value = algorithmic bytes of one step / wall time of one step, where the
algorithmic bytes are every input read once and every output written once:
  forward  rows * (6*inter + 4)     (x, probs in; y out)
  backward rows * (10*inter + 8)    (x, grad_y, probs in; grad_x, grad_probs out)
Per-kernel times come from HIP events recorded on the launch stream around
every launch inside the timed region.

Prints one JSON line. Options:
  --gpus N           only 1 is measured (the path has no cross-GPU step here)
  --steps K          timed steps (default 100)
  --warmup W         untimed steps first (default 10)
  --workload NAME    swiglu_* or router_65536x7168 (router: fwd + bwd of the
                     fp32 router-weight multiply)
  --dtype D          storage dtype of x / y / gradients: bf16 (default), f16, f32
  --out-dtype D      router output (and grad_out) dtype: the x dtype or f32
  --no-grad-probs    backward without the probability gradient (probabilities
                     that carry no gradient; the router then does not read x)
  --no-cpu-baseline  skip the oracle timing on the host
  --warm             SwiGLU / router / combine: launch each kernel straight
                     after the previous one. The default is a 1 GiB write
                     before every launch, outside its events, which evicts L2
                     and the 256 MB Infinity Cache, so a workload smaller than
                     them is not served from them; the step time is then the
                     sum of the kernels' event times
  --no-copy-ceiling  skip timing the 1 GiB device copy whose bandwidth the
                     SwiGLU / router lines also report a fraction of (it runs
                     after the host-side input generation, before the
                     settling and the warm-up steps)
  --settle-seconds S SwiGLU / router: run the step untimed for S seconds
                     (default 0.1) before the W warm-up steps, so that the
                     timed steps see the GPU's steady state; the line reports
                     how many steps that was (0 turns it off)
  --all              the four SwiGLU workloads and the router workload in
                     turn, one JSON line each (the default is the headline
                     workload alone, one line)
  --workload grouped_* the gate_up grouped GEMM with the clamped SwiGLU
                     epilogue fused into it (one launch per step; x = [gate | up]
                     is written too, as the backward needs it, unless --no-x):
                     value in TFLOP/s of the two products, roofline against
                     the dense bf16 MFMA peak
  --no-x             grouped: write y only
  --workload down_*  the down-projection grouped GEMM with the router-weight
                     multiply fused into it (bf16 or fp32 output, as the
                     workload names): TFLOP/s of the product, MFMA roofline
  --workload combine_* the fp32 combine of routed rows into tokens: HBM GB/s
                     of the local rows read once, row_of read once and the
                     output written once
  --copy-calibration time a 1 GiB device-to-device copy instead (torch's copy_,
                     carried out by the HIP runtime's copy kernel): the plain
                     copy of known size whose FETCH_SIZE / WRITE_SIZE readings
                     scale those counters for the kernels above
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published peak
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published peak (no sparsity)
METRICS = {
    "swiglu": "achieved HBM GB/s (% of MI355X peak), clamped-SwiGLU fwd+bwd at 131072×4096 bf16",
    "swiglu_other": "achieved HBM GB/s (% of MI355X peak), clamped-SwiGLU fwd+bwd",
    "router": "achieved HBM GB/s (% of MI355X peak), fp32 router-weight multiply fwd+bwd",
    "grouped": "achieved TFLOP/s (% of MI355X dense bf16 peak), gate_up grouped GEMM + clamped SwiGLU epilogue",
    "down": "achieved TFLOP/s (% of MI355X dense bf16 peak), down-projection grouped GEMM + router-weight multiply",
    "combine": "achieved HBM GB/s (% of MI355X peak), fp32 combine of routed rows into tokens",
}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--dtype", default="bf16", choices=("bf16", "f16", "f32"))
    ap.add_argument("--out-dtype", default=None, choices=("bf16", "f16", "f32"))
    ap.add_argument("--no-grad-probs", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the oracle baseline: whole-workload passes until it is spent")
    ap.add_argument("--cpu-threads", type=int, default=None)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-x", action="store_true")
    ap.add_argument("--warm", action="store_true",
                    help="SwiGLU / router / combine: no cache flush between launches (default: a 1 GiB write before each)")
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="SwiGLU / router: do not time the 1 GiB device copy (the box's copy ceiling)")
    ap.add_argument("--settle-seconds", type=float, default=0.1,
                    help="SwiGLU / router: run the step untimed for this long before the warm-up steps (0: off)")
    ap.add_argument("--all", action="store_true",
                    help="every SwiGLU and router workload in turn, one JSON line each")
    return ap.parse_args()


# The sources each op's kernels are built from (with the public header and
# the build flags): a counter record stays valid while these are unchanged.
KERNEL_SOURCES = {
    "swiglu": ("swiglu_clamped.hip", "swiglu_math.h", "epi_common.h"),
    "router": ("router_weight_mul.hip", "epi_common.h"),
    "grouped": ("grouped_swiglu.hip", "grouped_map.h", "swiglu_math.h", "epi_common.h"),
    "down": ("grouped_swiglu.hip", "grouped_map.h", "swiglu_math.h", "epi_common.h"),
    "combine": ("moe_combine.hip", "epi_common.h"),
}


def _code_only(text: str) -> str:
    """C/C++ source with comments removed and whitespace collapsed (string
    literals in these sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest(op: str) -> str:
    """Digest of one op's HIP sources (code only, comments ignored) and the
    build flags, to tell whether counter readings taken earlier still describe
    the kernels being timed."""
    from moe_routed_expert_amd import build as hip_build
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[op]:
        with open(os.path.join(hip_build.CSRC, name)) as fh:
            h.update(_code_only(fh.read()).encode())
    with open(os.path.join(ROOT, "include", "moe_epi.h")) as fh:
        h.update(_code_only(fh.read()).encode())
    h.update(" ".join(hip_build.FLAGS).encode())
    return h.hexdigest()[:16]


PROFILE_FOR = {"swiglu": "swiglu_clamped", "router": "router_weight_mul"}

# SwiGLU workloads up to this many rows also report the oracle on one thread
SINGLE_THREAD_ROWS = 8192


def op_of(workload) -> str:
    from moe_routed_expert_amd.workloads import CombineWorkload, DownWorkload, GroupedWorkload
    if isinstance(workload, GroupedWorkload):
        return "grouped"
    if isinstance(workload, DownWorkload):
        return "down"
    if isinstance(workload, CombineWorkload):
        return "combine"
    return workload.op


def profile_name(workload) -> str:
    """The committed rocprofv3 summary that covers a workload's kernels."""
    op = op_of(workload)
    if op == "grouped":
        return "grouped_gate_up_swiglu_" + workload.name[len("grouped_"):] + ".md"
    if op == "down":
        return "grouped_down_router_" + workload.name[len("down_"):] + ".md"
    if op == "combine":
        return "moe_combine_" + workload.name[len("combine_"):] + ".md"
    return f"{PROFILE_FOR[op]}_{workload.rows}x{workload.cols}.md"


def load_traffic(kernel: str, workload) -> float | None:
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profile_name; FETCH_SIZE and WRITE_SIZE, each
    scaled by its reading for a device copy of known size). None if there is
    no summary or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", profile_name(workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    start = text.find("```json")
    if start < 0:
        return None
    block = text[start + len("```json"):text.find("```", start + 7)]
    rec = json.loads(block)
    if rec.get("kernel_source_digest") != kernel_source_digest(op_of(workload)):
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


COPY_CEILING_LAUNCHES = 100


def copy_ceiling(steps: int = COPY_CEILING_LAUNCHES) -> dict:
    """Bandwidth of a plain 1 GiB device-to-device copy on this machine (torch's
    copy_, carried out by the HIP runtime's copy kernel), bytes read plus bytes
    written over the average launch time: what a kernel that only moves data
    sustains here, next to the 8 TB/s peak."""
    import torch
    n = 1 << 29  # 2**29 bf16 = 1 GiB
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    avg = sum(a.elapsed_time(b) for a, b in evs) / steps
    gbs = 2 * n * 2 / (avg * 1e-3) / 1e9
    # The two buffers go back to torch's cache, not to the HIP runtime, so that no
    # release of device memory runs beside the launches timed next.
    del src, dst
    return {"GB/s": gbs, "frac_of_peak": gbs / PEAK_HBM_GBS,
            "how": f"1 GiB device-to-device copy (torch copy_), read + written bytes over the average of {steps} "
                   "launches"}


def copy_calibration(args):
    import torch
    n = 1 << 29  # 2**29 bf16 = 1 GiB
    src = torch.randn(n, device="cuda").to(torch.bfloat16)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    avg = sum(ms) / len(ms)
    nbytes = 2 * n * 2
    print(json.dumps({"calibration": "torch device copy", "bytes_read_per_launch": n * 2,
                      "bytes_written_per_launch": n * 2, "avg_ms": avg, "median_ms": ms[len(ms) // 2],
                      "GB/s": nbytes / (avg * 1e-3) / 1e9}), flush=True)


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}). "
              "Rows are independent and every reduction stays inside a row, so the path shards by rows "
              "with no exchange; per-GPU throughput is the figure. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import moe_routed_expert_amd as epi
    from moe_routed_expert_amd.workloads import HEADLINE, WORKLOADS

    if not os.path.exists(epi.binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    epi.binding.lib()
    if args.copy_calibration:
        return copy_calibration(args)

    from moe_routed_expert_amd.workloads import COMBINE_WORKLOADS, DOWN_WORKLOADS, GROUPED_WORKLOADS
    if args.workload in GROUPED_WORKLOADS:
        return grouped_main(args, GROUPED_WORKLOADS[args.workload])
    if args.workload in DOWN_WORKLOADS:
        return down_main(args, DOWN_WORKLOADS[args.workload])
    if args.workload in COMBINE_WORKLOADS:
        return combine_main(args, COMBINE_WORKLOADS[args.workload])
    if args.all:
        for name in WORKLOADS:  # the five SwiGLU / router workloads, one line each
            epilogue_main(args, WORKLOADS[name])
        return None
    return epilogue_main(args, WORKLOADS[args.workload or HEADLINE])


# Bits of the storage types, for the parity check of the SwiGLU / router lines.
_EXP_FRAC = {"bf16": (16, 0x7F80, 0x007F), "f16": (16, 0x7C00, 0x03FF), "f32": (32, 0x7F800000, 0x007FFFFF)}


def _host_bits(t, dt: str):
    import numpy as np
    import torch
    if dt == "f32":
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _as_bits(a, dt: str):
    import numpy as np
    return np.ascontiguousarray(a).view(np.uint32 if dt == "f32" else np.uint16)


def compare_bits(got, want, dt: str, rows_per_chunk: int = 16384) -> dict:
    """Element-by-element comparison of two arrays of one storage type (bit
    patterns, rows first): the share of elements that are bit-identical (or
    NaN on both sides, whatever the payloads), the largest distance in units
    in the last place among the others, and whether NaN positions, zero
    positions and the signs of zeros all agree. Only the elements whose bits
    differ are examined further."""
    import numpy as np
    nbits, exp, frac = _EXP_FRAC[dt]
    mag_mask = (1 << (nbits - 1)) - 1
    same = n = max_ulp = 0
    specials_match = True
    for r0 in range(0, got.shape[0], rows_per_chunk):
        g = got[r0:r0 + rows_per_chunk].ravel()
        w_ = want[r0:r0 + rows_per_chunk].ravel()
        differ = g != w_
        n += int(g.size)
        same += int(g.size - np.count_nonzero(differ))
        if not differ.any():
            continue
        gd, wd = g[differ].astype(np.int64), w_[differ].astype(np.int64)
        nan_g = ((gd & exp) == exp) & ((gd & frac) != 0)
        nan_w = ((wd & exp) == exp) & ((wd & frac) != 0)
        both_nan = nan_g & nan_w            # NaN on both sides: the same position, payloads aside
        if (nan_g ^ nan_w).any() or ((gd & mag_mask) == 0).any() or ((wd & mag_mask) == 0).any():
            specials_match = False          # a NaN or a zero (or a zero's sign) on one side only
        keep = ~(nan_g | nan_w)
        og = np.where(gd >> (nbits - 1) == 1, -(gd & mag_mask), gd & mag_mask)[keep]
        ow = np.where(wd >> (nbits - 1) == 1, -(wd & mag_mask), wd & mag_mask)[keep]
        if og.size:
            max_ulp = max(max_ulp, int(np.abs(og - ow).max()))
        same += int(both_nan.sum())
    return {"exact_frac": same / n if n else 1.0, "max_ulp": max_ulp, "zeros_and_nans_match": specials_match}


def compare_dprobs(got, want, abs_sum) -> dict:
    """The probability gradient against the oracle's: |difference| over the
    row's sum of |terms| (the bar is 2e-5)."""
    import numpy as np
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    ratio = err / np.maximum(abs_sum, 1e-30)
    return {"max_err_over_sum_abs_terms": float(ratio.max(initial=0.0))}


def same_run_parity(oracle, w, d, dt: str, od: str, want_gp: bool, got_first, got_gx, got_gp, threads) -> dict:
    """The SwiGLU or router outputs of one step (host bit patterns; got_gp
    float32 or None) against one oracle pass over the same inputs d, element
    by element, with the bar the GPU tests use."""
    code = {"bf16": oracle.BF16, "f16": oracle.F16, "f32": oracle.F32}
    rows, cols = w.rows, w.cols
    if w.op == "swiglu":
        want_first = oracle.swiglu_clamped_fwd_typed(d["x"], code[dt], d["probs"], rows, cols, w.limit,
                                                     threads=threads)
        ref_gx, ref_gp, ref_abs = oracle.swiglu_clamped_bwd_typed(d["x"], code[dt], d["probs"], d["grad_out"], rows,
                                                                  cols, w.limit, want_grad_probs=want_gp,
                                                                  threads=threads, with_abs_sum=True)
    else:
        want_first = oracle.router_weight_mul_fwd_typed(d["x"], code[dt], d["probs"], code[od], rows, cols,
                                                        threads=threads)
        ref_gx, ref_gp, ref_abs = oracle.router_weight_mul_bwd_typed(d["grad_out"], code[od], d["x"], code[dt],
                                                                     d["probs"], rows, cols, want_grad_probs=want_gp,
                                                                     threads=threads, with_abs_sum=True)
    c_out = compare_bits(got_first, _as_bits(want_first, od).reshape(got_first.shape), od)
    c_gx = compare_bits(got_gx, _as_bits(ref_gx, dt).reshape(got_gx.shape), dt)
    c_gp = compare_dprobs(got_gp, ref_gp, ref_abs) if got_gp is not None and ref_abs is not None else None
    if w.op == "router":   # one fp32 multiply, one rounding: bit-exact in every dtype
        bar = "out and grad_x bit-exact; d_probs within 2e-5 of the sum of |terms|"
        within = c_out["exact_frac"] == 1.0 and c_gx["exact_frac"] == 1.0
    elif dt != "f32":
        bar = ("y and grad_x within 1 ulp with zeros, their signs and NaNs bit-exact; "
               "d_probs within 2e-5 of the sum of |terms|")
        within = all(c["max_ulp"] <= 1 and c["zeros_and_nans_match"] for c in (c_out, c_gx))
    else:
        bar = ("fp32 storage: reported only. The bound is derived per element in the GPU tests: where sigma "
               "underflows the outputs are tiny and their ulp counts large")
        within = None
    if within is not None and c_gp is not None:
        within = within and c_gp["max_err_over_sum_abs_terms"] <= 2e-5
    return {"rows": rows, "checked": "every element", "bar": bar, "within_bar": within,
            ("y" if w.op == "swiglu" else "out"): c_out, "grad_x": c_gx, "grad_probs": c_gp}


def epilogue_main(args, w):
    """One clamped-SwiGLU or router-weight-multiply workload: forward + backward per step."""
    import numpy as np
    import torch

    import moe_routed_expert_amd as epi
    from moe_routed_expert_amd.workloads import HEADLINE

    dt = args.dtype
    od = (args.out_dtype or dt) if w.op == "router" else dt
    want_gp = not args.no_grad_probs
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {w.name} ({dt}{'' if od == dt else ' -> ' + od})", file=sys.stderr, flush=True)
    d = w.generate(dtype=dt, grad_dtype=od)

    def upload(a, kind):
        if kind == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x = upload(d["x"], dt)
    p = torch.from_numpy(d["probs"]).to(dev)
    gy = upload(d["grad_out"], od)
    rows, cols = w.rows, w.cols
    gp = torch.empty((rows,), dtype=torch.float32, device=dev) if want_gp else None
    if w.op == "swiglu":
        y = torch.empty((rows, cols), dtype=tdt[dt], device=dev)
        gx = torch.empty_like(x)
        names = ("swiglu_clamped_fwd", "swiglu_clamped_bwd")
        first_out = y
        fwd = lambda: epi.swiglu_clamped_fwd(x, p, y, w.limit)
        bwd = lambda: epi.swiglu_clamped_bwd(x, p, gy, gx, gp, w.limit)
    else:
        out = torch.empty((rows, cols), dtype=tdt[od], device=dev)
        gx = torch.empty_like(x)
        names = ("router_weight_mul_fwd", "router_weight_mul_bwd")
        first_out = out
        fwd = lambda: epi.router_weight_mul_fwd(x, p, out)
        bwd = lambda: epi.router_weight_mul_bwd(gy, x if want_gp else None, p, gx, gp)
    fwd_b, bwd_b = w.fwd_bytes(dt, od), w.bwd_bytes(want_gp, dt, od)

    # unless --warm: a 1 GiB write before each launch evicts L2 and the 256 MB
    # Infinity Cache, so that a workload smaller than them is not served from
    # them; the flushes lie outside the kernels' events
    scratch = None if args.warm else torch.empty((1 << 28,), dtype=torch.float32, device=dev)

    # The copy ceiling is timed after the inputs are generated on the host and
    # uploaded, so that the GPU is not idle between it and the steps below.
    ceiling = None
    if not args.no_copy_ceiling:
        print("[bench] timing a 1 GiB device copy (the copy ceiling)", file=sys.stderr, flush=True)
        ceiling = copy_ceiling(COPY_CEILING_LAUNCHES)

    def step(ev=None):  # warm-up and timed steps are the same work
        if scratch is not None:
            scratch.zero_()
        if ev:
            ev[0].record()
        fwd()
        if ev:
            ev[1].record()
        if scratch is not None:
            scratch.zero_()
        if ev:
            ev[2].record()
        bwd()
        if ev:
            ev[3].record()

    # Settling: the same step, untimed, for --settle-seconds before the W
    # warm-up steps. When these kernels start on a GPU that has not run them
    # for a while, launches 2 to ~15 ran up to 17% slower than the steady
    # state and recovered step by step; 1000 back-to-back device copies
    # (0.4 s) beforehand did not prevent it, while a run of the same steps
    # about 10 s earlier did. The line reports the steps this took.
    settle_steps, t = 0, time.perf_counter()
    if args.settle_seconds > 0:
        print(f"[bench] settling for {args.settle_seconds:g} s", file=sys.stderr, flush=True)
    while time.perf_counter() - t < args.settle_seconds:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    E = lambda: torch.cuda.Event(enable_timing=True)
    evs = [(E(), E(), E(), E()) for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = np.array([a.elapsed_time(b) for a, b, _, _ in evs])
    bwd_ms = np.array([c.elapsed_time(d) for _, _, c, d in evs])

    # with flushes in the loop the step time is the two kernels' event time,
    # otherwise the wall time of the whole timed region
    ms_per_step = float((fwd_ms + bwd_ms).mean()) if scratch is not None else wall * 1e3 / args.steps
    value = (fwd_b + bwd_b) / (ms_per_step * 1e-3) / 1e9

    def kstats(name, nbytes, ms):
        avg = float(ms.mean())
        gbs = nbytes / (avg * 1e-3) / 1e9
        k = {"avg_us": avg * 1e3, "median_us": float(np.median(ms)) * 1e3, "min_us": float(ms.min()) * 1e3,
             "algorithmic_bytes": nbytes, "GB/s": gbs, "frac_of_peak": gbs / PEAK_HBM_GBS}
        if ceiling is not None:
            k["frac_of_copy"] = gbs / ceiling["GB/s"]
        return k

    kernels = {names[0]: kstats(names[0], fwd_b, fwd_ms), names[1]: kstats(names[1], bwd_b, bwd_ms)}
    # Counter traffic is taken for the bf16, with-gradient launch only.
    variant = []
    if dt != "bf16" or od != dt:
        variant.append(f"{dt} storage" + ("" if od == dt else f", {od} output"))
    if not want_gp:
        variant.append("no probability gradient")
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
    traffic = load_traffic(dom, w) if not variant else None
    roofline = {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["GB/s"], "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": kernels[dom]["GB/s"] / PEAK_HBM_GBS, "traffic": traffic,
                "algorithmic_bytes_per_launch": kernels[dom]["algorithmic_bytes"]}

    cpu = cpu1 = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        threads = args.cpu_threads or oracle.default_threads()
        code = {"bf16": oracle.BF16, "f16": oracle.F16, "f32": oracle.F32}

        # Parity on the same inputs in the same run: the outputs of the last
        # timed step against one untimed oracle pass, element by element.
        print(f"[bench] parity: the last timed step's outputs against one oracle pass", file=sys.stderr, flush=True)
        parity = same_run_parity(oracle, w, d, dt, od, want_gp, _host_bits(first_out, od), _host_bits(gx, dt),
                                 gp.cpu().numpy() if gp is not None else None, threads)
        print(f"[bench] oracle on the host ({threads} threads): whole-workload passes for >= {args.cpu_seconds:g} s",
              file=sys.stderr, flush=True)

        def oracle_pass():  # reads `threads` when called
            if w.op == "swiglu":
                oracle.swiglu_clamped_fwd_typed(d["x"], code[dt], d["probs"], rows, cols, w.limit, threads=threads)
                oracle.swiglu_clamped_bwd_typed(d["x"], code[dt], d["probs"], d["grad_out"], rows, cols, w.limit,
                                                want_grad_probs=want_gp, threads=threads)
            else:
                oracle.router_weight_mul_fwd_typed(d["x"], code[dt], d["probs"], code[od], rows, cols,
                                                   threads=threads)
                oracle.router_weight_mul_bwd_typed(d["grad_out"], code[od], d["x"], code[dt], d["probs"], rows,
                                                   cols, want_grad_probs=want_gp, threads=threads)

        passes, t = 0, time.perf_counter()
        while True:  # whole passes until the time budget is spent (at least one, at most 100)
            oracle_pass()
            passes += 1
            ct = time.perf_counter() - t
            if ct >= args.cpu_seconds or passes >= 100:
                break
        cpu = {"value": passes * (fwd_b + bwd_b) / ct / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{passes} passes over the whole workload ({rows} rows, forward + backward), {ct:.1f} s"}
        if w.op == "swiglu" and rows <= SINGLE_THREAD_ROWS:
            # the small workloads also on one host thread
            print(f"[bench] oracle on one host thread: whole-workload passes for >= {args.cpu_seconds / 4:g} s",
                  file=sys.stderr, flush=True)
            threads = 1
            passes, ct = oracle_timed(oracle_pass, args.cpu_seconds / 4)
            cpu1 = {"value": passes * (fwd_b + bwd_b) / ct / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                    "sample": f"{passes} passes over the whole workload ({rows} rows, forward + backward), "
                              f"{ct:.1f} s"}

    headline = w.name == HEADLINE and not variant
    line = {
        # the headline string names the 131072 x 4096 shape; other shapes and variants name themselves
        "metric": METRICS[w.op] if headline or (w.op == "router" and not variant) else
        METRICS["swiglu_other" if w.op == "swiglu" else w.op] + f" ({w.name}{', ' if variant else ''}{', '.join(variant)})",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"steps": settle_steps, "seconds": args.settle_seconds,
                   "what": "untimed steps of the same work before the warm-up steps"},
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "op": w.op, "rows": rows,
                   ("inter" if w.op == "swiglu" else "hidden"): cols,
                   "limit": w.limit, "storage": dt, "output": od, "grad_probs": want_gp,
                   "io": f"{dt} tensors, fp32 probs; fp32 arithmetic", "bytes_per_step": fwd_b + bwd_b,
                   "caches": "warm from the previous launch" if args.warm else
                   "flushed before every launch (1 GiB write outside the events)"},
        "frac_of_peak": value / PEAK_HBM_GBS,
        "frac_of_copy": None if ceiling is None else value / ceiling["GB/s"],
        "copy_ceiling": ceiling,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    if cpu1 is not None:
        line["cpu_baseline_1thread"] = cpu1
    if headline and w.op == "swiglu":
        # The pages' one timing, on other hardware and another implementation:
        # context for the backward, never vs_baseline.
        line["context"] = {
            "source": "page nemo_automodel.components.moe.swiglu_triton, module description",
            "figure": "a torch.compile backward of this op (d_gate and d_up concatenated) on GB200: "
                      "about 0.7 ms over about 1.1 GB at the large-node shape, near one quarter of that "
                      "GPU's HBM bandwidth",
            "this_run_backward_ms": kernels[names[1]]["avg_us"] / 1e3,
            "this_run_backward_bytes": bwd_b,
        }
    print(json.dumps(line), flush=True)


def grouped_main(args, w):
    """One step = one fused grouped GEMM + epilogue launch over the whole workload."""
    import numpy as np
    import torch

    import moe_routed_expert_amd as epi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    d = w.generate()
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    a, wg, wu = bf(d["a"]), bf(d["w_gate"]), bf(d["w_up"])
    offs = torch.from_numpy(d["offs"]).to(dev)
    p = torch.from_numpy(d["probs"]).to(dev)
    y = torch.empty((w.tokens, w.inter), dtype=torch.bfloat16, device=dev)
    x = None if args.no_x else torch.empty((w.tokens, 2 * w.inter), dtype=torch.bfloat16, device=dev)
    step = lambda: epi.grouped_gate_up_swiglu_fwd(a, wg, wu, offs, p, y, x, w.limit)

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    flops = w.flops()
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    avg_ms = float(ms.mean())
    achieved = flops / (avg_ms * 1e-3) / 1e12
    name = "grouped_gate_up_swiglu_fwd"
    kernels = {name: {"avg_us": avg_ms * 1e3, "median_us": float(np.median(ms)) * 1e3, "min_us": float(ms.min()) * 1e3,
                      "flops": flops, "TFLOP/s": achieved, "frac_of_peak": achieved / PEAK_BF16_TFLOPS,
                      "min_hbm_bytes": w.min_bytes(not args.no_x)}}
    traffic = None if args.no_x else load_traffic(name, w)
    roofline = {"bound": "mfma", "kernel": name, "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic, "flops_per_launch": flops}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = args.cpu_threads or oracle.default_threads()
        # sample: the first 8 rows of every expert, regrouped with their own counts
        ends = d["offs"].astype(np.int64)
        starts = np.concatenate([[0], ends[:-1]])
        idx = np.concatenate([np.arange(s0, min(s0 + 8, e0)) for s0, e0 in zip(starts, ends)]).astype(np.int64)
        sub_offs = np.cumsum([min(8, max(0, e0 - s0)) for s0, e0 in zip(starts, ends)]).astype(np.int32)
        sa, sp = d["a"][idx], d["probs"][idx]
        print(f"[bench] oracle on the host ({threads} threads): {idx.size} sampled rows per pass for >= "
              f"{args.cpu_seconds:g} s", file=sys.stderr, flush=True)
        passes, t = 0, time.perf_counter()
        while True:
            oracle.grouped_swiglu_fwd(sa, d["w_gate"], d["w_up"], sub_offs, sp, idx.size, w.hidden, w.inter,
                                      w.experts, w.limit, threads=threads)
            passes += 1
            ct = time.perf_counter() - t
            if ct >= args.cpu_seconds or passes >= 100:
                break
        sample_flops = 2 * idx.size * w.hidden * 2 * w.inter
        cpu = {"value": passes * sample_flops / ct / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": f"{passes} passes over {idx.size} rows (the first 8 of each expert), {ct:.1f} s"}

    line = {
        "metric": METRICS["grouped"] + f" ({w.name}{', y only' if args.no_x else ''})",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "op": "grouped", "tokens": w.tokens, "hidden": w.hidden, "inter": w.inter,
                   "experts": w.experts, "limit": w.limit, "write_x": not args.no_x,
                   "io": "bf16 a / weights / y / x, fp32 probs; bf16 MFMA products, fp32 accumulation",
                   "flops_per_step": flops},
        "frac_of_peak": value / PEAK_BF16_TFLOPS,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def time_launches(step, args):
    """Warm up, then time args.steps launches: (per-launch ms from HIP events on the launch
    stream, wall ms per step)."""
    import numpy as np
    import torch
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return np.array([e0.elapsed_time(e1) for e0, e1 in evs]), wall * 1e3 / args.steps


def time_flushed(launch, args, dev):
    """Warm up, then time args.steps launches, each after a 1 GiB write (a fill
    kernel, outside the launch's events): per-launch ms from HIP events."""
    import numpy as np
    import torch
    scratch = torch.empty((1 << 28,), dtype=torch.float32, device=dev)
    print(f"[bench] warmup {args.warmup} steps (caches flushed before every launch)", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        scratch.zero_()
        launch()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    for e0, e1 in evs:
        scratch.zero_()
        e0.record()
        launch()
        e1.record()
    torch.cuda.synchronize()
    return np.array([e0.elapsed_time(e1) for e0, e1 in evs])


def oracle_timed(run, seconds):
    """Whole passes of run() until `seconds` are spent (at least one, at most 100): (passes, s)."""
    passes, t = 0, time.perf_counter()
    while True:
        run()
        passes += 1
        ct = time.perf_counter() - t
        if ct >= seconds or passes >= 100:
            return passes, ct


def down_main(args, w):
    """One step = one fused down-projection grouped GEMM + router multiply launch."""
    import numpy as np
    import torch

    import moe_routed_expert_amd as epi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    d = w.generate()
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    h, wd = bf(d["h"]), bf(d["w_down"])
    offs = torch.from_numpy(d["offs"]).to(dev)
    p = torch.from_numpy(d["probs"]).to(dev)
    out = torch.empty((w.tokens, w.hidden), dtype=torch.float32 if w.out_dtype == "f32" else torch.bfloat16,
                      device=dev)
    ms, ms_per_step = time_launches(lambda: epi.grouped_down_router_fwd(h, wd, offs, p, out), args)
    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    avg_ms = float(ms.mean())
    achieved = flops / (avg_ms * 1e-3) / 1e12
    name = "grouped_down_router_fwd"
    kernels = {name: {"avg_us": avg_ms * 1e3, "median_us": float(np.median(ms)) * 1e3, "min_us": float(ms.min()) * 1e3,
                      "flops": flops, "TFLOP/s": achieved, "frac_of_peak": achieved / PEAK_BF16_TFLOPS,
                      "min_hbm_bytes": w.min_bytes()}}
    roofline = {"bound": "mfma", "kernel": name, "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": load_traffic(name, w), "flops_per_launch": flops}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = args.cpu_threads or oracle.default_threads()
        # sample: the first 8 rows of every expert, regrouped with their own counts
        ends = d["offs"].astype(np.int64)
        starts = np.concatenate([[0], ends[:-1]])
        idx = np.concatenate([np.arange(s0, min(s0 + 8, e0)) for s0, e0 in zip(starts, ends)]).astype(np.int64)
        sub_offs = np.cumsum([min(8, max(0, e0 - s0)) for s0, e0 in zip(starts, ends)]).astype(np.int32)
        sh, sp = d["h"][idx], d["probs"][idx]
        code = oracle.F32 if w.out_dtype == "f32" else oracle.BF16
        print(f"[bench] oracle on the host ({threads} threads): {idx.size} sampled rows per pass for >= "
              f"{args.cpu_seconds:g} s", file=sys.stderr, flush=True)
        passes, ct = oracle_timed(lambda: oracle.grouped_down_router_fwd(
            sh, d["w_down"], sub_offs, sp, idx.size, w.inter, w.hidden, w.experts, out_dtype=code, threads=threads),
            args.cpu_seconds)
        sample_flops = 2 * idx.size * w.inter * w.hidden
        cpu = {"value": passes * sample_flops / ct / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": f"{passes} passes over {idx.size} rows (the first 8 of each expert), {ct:.1f} s"}

    line = {
        "metric": METRICS["down"] + f" ({w.name})",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "op": "down", "tokens": w.tokens, "inter": w.inter, "hidden": w.hidden,
                   "experts": w.experts, "output": w.out_dtype,
                   "io": f"bf16 h / weights, fp32 probs, {w.out_dtype} out; bf16 MFMA products, fp32 accumulation",
                   "flops_per_step": flops},
        "frac_of_peak": value / PEAK_BF16_TFLOPS,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def combine_main(args, w):
    """One step = one combine launch over every token."""
    import numpy as np
    import torch

    import moe_routed_expert_amd as epi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    d = w.generate()
    eo_np, row_of, rows = d["expert_out"], d["row_of"], d["rows"]
    if w.eo_dtype == "f32":
        eo = torch.from_numpy(eo_np).to(dev)
    else:
        eo = torch.from_numpy(eo_np.view(np.int16)).view(
            torch.bfloat16 if w.eo_dtype == "bf16" else torch.float16).to(dev)
    ro = torch.from_numpy(row_of).to(dev)
    out = torch.empty((w.tokens, w.hidden), dtype=torch.float32, device=dev)
    launch = lambda: epi.moe_combine_fwd(eo, ro, out)
    if args.warm:
        ms, ms_per_step = time_launches(launch, args)
    else:  # as the SwiGLU lines: a 1 GiB write before every launch, outside its events
        ms = time_flushed(launch, args, dev)
        ms_per_step = float(ms.mean())
    nbytes = w.min_bytes(row_of, rows)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    avg_ms = float(ms.mean())
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    name = "moe_combine_fwd"
    kernels = {name: {"avg_us": avg_ms * 1e3, "median_us": float(np.median(ms)) * 1e3, "min_us": float(ms.min()) * 1e3,
                      "algorithmic_bytes": nbytes, "GB/s": gbs, "frac_of_peak": gbs / PEAK_HBM_GBS}}
    roofline = {"bound": "hbm", "kernel": name, "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS, "traffic": load_traffic(name, w), "algorithmic_bytes_per_launch": nbytes}

    cpu = parity = None
    if not args.no_cpu_baseline:
        import oracle
        threads = args.cpu_threads or oracle.default_threads()
        sample = w.tokens  # the whole workload: a pass takes a fraction of a second
        code = {"bf16": oracle.BF16, "f16": oracle.F16, "f32": oracle.F32}[w.eo_dtype]
        eo_o = eo_np.view(np.float16) if w.eo_dtype == "f16" else eo_np
        sro = np.ascontiguousarray(row_of[:sample])
        # parity in the same run: the last timed launch's output against one
        # untimed oracle pass, every element, bit-exact (the same binary32
        # additions in the same order)
        print("[bench] parity: the last timed launch's output against one oracle pass", file=sys.stderr, flush=True)
        want = oracle.moe_combine(eo_o, code, sro, rows, sample, w.top_k, w.hidden, threads=threads)
        c = compare_bits(_host_bits(out, "f32"), _as_bits(want, "f32").reshape(w.tokens, w.hidden), "f32")
        parity = {"rows": w.tokens, "checked": "every element", "bar": "bit-exact", "within_bar": c["exact_frac"] == 1.0,
                  "out": c}
        del want
        print(f"[bench] oracle on the host ({threads} threads): {sample} tokens per pass for >= "
              f"{args.cpu_seconds:g} s", file=sys.stderr, flush=True)
        passes, ct = oracle_timed(lambda: oracle.moe_combine(eo_o, code, sro, rows, sample, w.top_k, w.hidden,
                                                             threads=threads), args.cpu_seconds)
        valid = int(((sro >= 0) & (sro < rows)).sum())
        sample_bytes = valid * w.hidden * eo_np.itemsize + sro.size * 4 + sample * w.hidden * 4
        cpu = {"value": passes * sample_bytes / ct / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{passes} passes over all {sample} tokens, {ct:.1f} s"}

    line = {
        "metric": METRICS["combine"] + f" ({w.name})",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "op": "combine", "tokens": w.tokens, "hidden": w.hidden, "top_k": w.top_k,
                   "global_experts": w.global_experts, "local_experts": w.local_experts, "rows": rows,
                   "expert_out": w.eo_dtype, "io": f"{w.eo_dtype} routed rows, int32 row_of, fp32 out; fp32 adds",
                   "bytes_per_step": nbytes,
                   "caches": "warm from the previous launch" if args.warm else
                   "flushed before every launch (1 GiB write outside the events)"},
        "frac_of_peak": value / PEAK_HBM_GBS,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
