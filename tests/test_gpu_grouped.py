"""GPU parity of the fused gate_up grouped GEMM + clamped SwiGLU epilogue
(grouped_gate_up_swiglu_fwd) against the oracle.

Two separate bars (tests/gpu_util.py):
  - x = [gate | up], the grouped-GEMM output in bf16, against the oracle's exact
    sums: within the bound of an fp32 accumulation of `hidden` products plus half
    a bf16 ulp;
  - y against the oracle's clamped SwiGLU forward of the kernel's own x: the
    streaming forward's bar (1 bf16 ulp, zeros bit-exact), since the epilogue
    computes from the bf16 gate and up.
The call without x_out must give bit-identical y, and rows of no expert must be
left untouched.
"""
import sys

import numpy as np
import pytest
import torch

import moe_routed_expert_amd as epi
import oracle
from moe_routed_expert_amd.workloads import GROUPED_WORKLOADS, GroupedWorkload
from tests.gpu_util import assert_bf16_parity, assert_gemm_bf16_within, to_dev_bf16, to_host_bits

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FBF   # a NaN pattern the kernel never writes


def say(msg):
    print(f"\n[gpu-grouped] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    epi.binding.lib()
    yield
    torch.cuda.synchronize()


def run(d, tokens, hidden, inter, experts, L, with_x=True):
    a, wg, wu = to_dev_bf16(d["a"]), to_dev_bf16(d["w_gate"]), to_dev_bf16(d["w_up"])
    offs = torch.from_numpy(d["offs"]).cuda()
    p = torch.from_numpy(d["probs"]).cuda()
    y = torch.full((tokens, inter), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    x = torch.full((tokens, 2 * inter), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16) \
        if with_x else None
    epi.grouped_gate_up_swiglu_fwd(a, wg, wu, offs, p, y, x, L)
    torch.cuda.synchronize()
    return to_host_bits(y), (to_host_bits(x) if with_x else None)


def covered_rows(offs, tokens):
    cov = np.zeros(tokens, bool)
    start = 0
    for c in offs:
        end = min(max(int(c), start), tokens)
        cov[start:end] = True
        start = end
    return cov


def check(d, tokens, hidden, inter, experts, L, what):
    y, x = run(d, tokens, hidden, inter, experts, L)
    cov = covered_rows(d["offs"], tokens)
    assert (y[~cov] == SENTINEL).all() and (x[~cov] == SENTINEL).all(), f"{what}: rows of no expert written"
    s, s_abs = oracle.grouped_gate_up(d["a"], d["w_gate"], d["w_up"], d["offs"], tokens, hidden, inter, experts,
                                      with_abs_sum=True)
    sx = assert_gemm_bf16_within(x[cov], s[cov], s_abs[cov], hidden, f"{what} x")
    y_o = oracle.swiglu_clamped_fwd(x[cov], d["probs"][cov], int(cov.sum()), inter, L)
    sy = assert_bf16_parity(y[cov], y_o, f"{what} y")
    y2, _ = run(d, tokens, hidden, inter, experts, L, with_x=False)
    assert np.array_equal(y2, y), f"{what}: y differs without x_out"
    say(f"{what}: x {sx}, y exact {sy['exact']:.5f}")


def test_epilogue_reads_the_bf16_rounded_sums_not_the_accumulators():
    """Designed inputs (tests/grouped_designed.py): exact binary32 sums that are not bf16 values,
    and per row a probability that puts one column's output on different bf16 values under the
    two readings of the epilogue's input. The kernel must give x = the bf16 roundings and, in
    every target column, the oracle's y (the bf16-rounded reading) bit for bit."""
    from tests import grouped_designed as gd
    d = gd.build()
    y, x = run(d, gd.TOKENS, gd.HIDDEN, gd.INTER, gd.EXPERTS, gd.LIMIT)
    y_o, x_o = oracle.grouped_swiglu_fwd(d["a"], d["w_gate"], d["w_up"], d["offs"], d["probs"], gd.TOKENS,
                                         gd.HIDDEN, gd.INTER, gd.EXPERTS, gd.LIMIT)
    assert np.array_equal(x, x_o) and np.array_equal(x, d["x_bits"])
    rows = np.arange(gd.TOKENS)
    yt = y[rows, d["target"]]
    assert np.array_equal(yt, y_o[rows, d["target"]]) and np.array_equal(yt, d["want_bits"])
    assert (yt != d["other_bits"]).all()
    st = assert_bf16_parity(y, y_o, "designed y")
    y2, _ = run(d, gd.TOKENS, gd.HIDDEN, gd.INTER, gd.EXPERTS, gd.LIMIT, with_x=False)
    assert np.array_equal(y2, y)
    say(f"designed: {gd.TOKENS} target outputs on the bf16-rounded reading, y exact {st['exact']:.5f}")


def test_small_named_workload():
    w = GROUPED_WORKLOADS["grouped_4096x1024x512_e5"]
    check(w.generate(), w.tokens, w.hidden, w.inter, w.experts, w.limit, w.name)


# tails in every dimension: tokens not a multiple of 128 per expert, hidden not a
# multiple of 64 (a partial K step, its valid part shorter than, equal to and
# longer than one 32-wide sub-step, loaded in the prologue or inside the loop),
# inter not a multiple of 128 (a partial column tile), a single expert, many
# small experts, an empty expert
@pytest.mark.parametrize("tokens,hidden,inter,experts,split", [
    (300, 64, 128, 3, "dirichlet"), (257, 200, 136, 4, "one_empty"), (1000, 512, 256, 1, "even"),
    (129, 96, 8, 7, "dirichlet"), (640, 1032, 264, 16, "dirichlet"), (1, 8, 8, 1, "even"),
    (200, 184, 72, 3, "dirichlet"), (333, 232, 40, 5, "dirichlet"),
    # many experts: dozens of partial row tiles, the grid's tile groups span experts
    (3000, 128, 512, 64, "dirichlet"),
])
def test_shapes(tokens, hidden, inter, experts, split):
    w = GroupedWorkload(f"g_{tokens}x{hidden}x{inter}_e{experts}", tokens, hidden, inter, experts, 7.0,
                        seed=tokens + hidden + inter + experts, split=split, gate_up_sigma=5.0)
    check(w.generate(), tokens, hidden, inter, experts, w.limit, w.name)


@pytest.mark.parametrize("offs", [[50, 20, 300, 100], [0, 0, 0, 257], [257, 257, 257, 257], [-5, 10, 10, 200],
                                  [100, 1000, 5, 7]])
def test_counts_that_are_empty_decreasing_or_too_large(offs):
    w = GroupedWorkload("g_offs", 257, 64, 32, 4, 7.0, seed=31)
    d = w.generate()
    d["offs"] = np.array(offs, dtype=np.int32)
    check(d, 257, 64, 32, 4, 7.0, f"offs {offs}")


def test_every_token_in_one_expert_of_sixteen():
    # all other experts empty, before and after it: their row ranges are empty and
    # the grid's worst-case row tiles beyond the real ones exit without writing
    w = GroupedWorkload("g_skew", 2000, 96, 256, 16, 7.0, seed=34)
    d = w.generate()
    d["offs"] = np.array([0] * 7 + [2000] * 9, dtype=np.int32)
    check(d, 2000, 96, 256, 16, 7.0, "one expert holds every token")


def test_full_size_sampled_rows_and_every_epilogue_row():
    w = GROUPED_WORKLOADS["grouped_131072x7168x2048_e8"]
    say(f"{w.name}: generate")
    d = w.generate()
    say(f"{w.name}: gpu (with and without x)")
    y, x = run(d, w.tokens, w.hidden, w.inter, w.experts, w.limit)
    y2, _ = run(d, w.tokens, w.hidden, w.inter, w.experts, w.limit, with_x=False)
    assert np.array_equal(y, y2)
    assert not (y == SENTINEL).any()
    # sampled rows: each expert's first and last rows, rows at 128-row tile edges, random rows
    offs = d["offs"].astype(np.int64)
    starts = np.concatenate([[0], offs[:-1]])
    rng = np.random.default_rng(5)
    pick = set()
    for s0, e0 in zip(starts, offs):
        if e0 > s0:
            pick |= {s0, s0 + 1, e0 - 1, min(s0 + 127, e0 - 1), min(s0 + 128, e0 - 1)}
    pick |= set(rng.integers(0, w.tokens, 200).tolist())
    idx = np.array(sorted(pick))
    # the oracle on the sampled rows: regroup them by expert with their own offs
    expert_of = np.searchsorted(offs, idx, side="right")
    sub_offs = np.array([np.sum(expert_of <= e) for e in range(w.experts)], dtype=np.int32)
    say(f"{w.name}: oracle on {idx.size} sampled rows")
    s, s_abs = oracle.grouped_gate_up(d["a"][idx], d["w_gate"], d["w_up"], sub_offs, idx.size, w.hidden, w.inter,
                                      w.experts, with_abs_sum=True)
    sx = assert_gemm_bf16_within(x[idx], s, s_abs, w.hidden, f"{w.name} x")
    # the epilogue on every row: the oracle's SwiGLU forward of the kernel's own x
    say(f"{w.name}: oracle epilogue on every row")
    y_o = oracle.swiglu_clamped_fwd(x, d["probs"], w.tokens, w.inter, w.limit)
    sy = assert_bf16_parity(y, y_o, f"{w.name} y")
    say(f"{w.name}: x {sx} on {idx.size} sampled rows, y exact {sy['exact']:.5f} on all {w.tokens}")


@pytest.mark.parametrize("k_dim", [4177920, 4178048])
def test_reductions_beside_the_32_bit_load_offset_limit(k_dim):
    """The main loop loads in buffer form (32-bit byte offsets from each tile's base)
    while (BM + 1) * k_dim * 2 bytes stay below 2^31, i.e. k_dim <= 4178003 for 256-row
    tiles, and in global form past that. 257 tokens in two row tiles put the largest
    offsets just below and just above the limit. Inputs are built on the device:
    a[t, h] = 1 where h = t (mod 7), else 0, and all weights 1, so every gate and up
    output is the count of such h, exact in fp32 (below 2^24) and in bf16 after
    rounding; y is checked against the oracle's forward of the kernel's own x."""
    tokens, inter, experts, L = 257, 8, 1, 7.0
    say(f"k_dim {k_dim}: device inputs ({tokens * k_dim * 2 / 2**30:.2f} GiB of activations)")
    h = torch.arange(k_dim, device="cuda") % 7
    a = (h[None, :] == (torch.arange(tokens, device="cuda") % 7)[:, None]).to(torch.bfloat16)
    del h
    w = torch.ones((experts, inter, k_dim), dtype=torch.bfloat16, device="cuda")
    offs = torch.tensor([tokens], dtype=torch.int32, device="cuda")
    p = torch.linspace(0.1, 1.0, tokens, device="cuda")
    y = torch.empty((tokens, inter), dtype=torch.bfloat16, device="cuda")
    x = torch.empty((tokens, 2 * inter), dtype=torch.bfloat16, device="cuda")
    epi.grouped_gate_up_swiglu_fwd(a, w, w, offs, p, y, x, L)
    torch.cuda.synchronize()
    del a, w
    t = np.arange(tokens)
    counts = (k_dim - 1 - t % 7) // 7 + 1  # h in [0, k_dim) with h = t (mod 7)
    want = (counts.astype(np.float32).view(np.uint32) + 0x7FFF + ((counts.astype(np.float32).view(np.uint32) >> 16) & 1)) >> 16
    xb = to_host_bits(x)
    assert np.array_equal(xb[:, :inter], np.repeat(want.astype(np.uint16)[:, None], inter, 1)), "gate sums"
    assert np.array_equal(xb[:, inter:], np.repeat(want.astype(np.uint16)[:, None], inter, 1)), "up sums"
    y_o = oracle.swiglu_clamped_fwd(xb, p.cpu().numpy(), tokens, inter, L)
    assert_bf16_parity(to_host_bits(y), y_o, f"k_dim {k_dim} y")
    say(f"k_dim {k_dim}: exact sums, y within the bar")
