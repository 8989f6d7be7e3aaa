"""GPU parity of the down-projection grouped GEMM with the router-weight multiply
(grouped_down_router_fwd) and of the combine of routed rows into tokens
(moe_combine_fwd), against the oracle.

Bars (tests/gpu_util.py):
  - down: every output is the router multiply (one binary32 product, rounded
    once to the output dtype) of a bf16 value within the fp32-accumulation bound
    of the exact grouped sum; the bf16 output is, bit for bit, the bf16 rounding
    of the float32 output (the same GEMM, one more rounding); rows of no expert
    are left untouched;
  - combine: bit-exact (the same binary32 additions in the same order).
The exact grouped sums and their absolute sums come from the oracle's grouped
product (oracle.grouped_gate_up with the down weights as both operands: the
same grouped definition with the roles of the widths swapped).
"""
import sys

import numpy as np
import pytest
import torch

import moe_routed_expert_amd as epi
import oracle
from moe_routed_expert_amd.workloads import (COMBINE_WORKLOADS, DOWN_WORKLOADS, CombineWorkload, DownWorkload)
from tests.gpu_util import assert_down_router_within, to_dev_bf16, to_host_bits

pytestmark = pytest.mark.gpu
SENTINEL16 = 0x7FBF          # a bf16 NaN pattern the kernel never writes
SENTINEL32 = 0x7FC0DEAD      # a float32 NaN pattern the kernel never writes


def say(msg):
    print(f"\n[gpu-down-combine] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    epi.binding.lib()
    yield
    torch.cuda.synchronize()


def covered_rows(offs, tokens):
    cov = np.zeros(tokens, bool)
    start = 0
    for c in offs:
        end = min(max(int(c), start), tokens)
        cov[start:end] = True
        start = end
    return cov


# ---- down projection ------------------------------------------------------------

def run_down(d, tokens, hidden, f32):
    h, w = to_dev_bf16(d["h"]), to_dev_bf16(d["w_down"])
    offs = torch.from_numpy(d["offs"]).cuda()
    p = torch.from_numpy(d["probs"]).cuda()
    if f32:
        out = torch.full((tokens, hidden), SENTINEL32, dtype=torch.int32, device="cuda").view(torch.float32)
    else:
        out = torch.full((tokens, hidden), SENTINEL16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    epi.grouped_down_router_fwd(h, w, offs, p, out)
    return out


def exact_sums(h, w_down, offs, tokens, inter, hidden, experts):
    s, s_abs = oracle.grouped_gate_up(h, w_down, w_down, offs, tokens, inter, hidden, experts, with_abs_sum=True)
    return s[:, :hidden], s_abs[:, :hidden]


def check_down(d, tokens, inter, hidden, experts, what):
    o32 = run_down(d, tokens, hidden, True)
    o16 = run_down(d, tokens, hidden, False)
    torch.cuda.synchronize()
    g32 = o32.cpu().numpy()
    g16 = to_host_bits(o16)
    cov = covered_rows(d["offs"], tokens)
    assert (g32[~cov].view(np.uint32) == SENTINEL32).all(), f"{what}: fp32 rows of no expert written"
    assert (g16[~cov] == SENTINEL16).all(), f"{what}: bf16 rows of no expert written"
    want16 = torch.from_numpy(np.ascontiguousarray(g32[cov])).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(g16[cov], want16.view(np.uint16)), f"{what}: bf16 output is not bf16(fp32 output)"
    s, s_abs = exact_sums(d["h"], d["w_down"], d["offs"], tokens, inter, hidden, experts)
    p = d["probs"][cov]
    st32 = assert_down_router_within(g32[cov], True, s[cov], s_abs[cov], p, inter, f"{what} fp32")
    st16 = assert_down_router_within(g16[cov], False, s[cov], s_abs[cov], p, inter, f"{what} bf16")
    say(f"{what}: fp32 {st32}, bf16 {st16}")


@pytest.mark.parametrize("name", ["down_4096x512x1024_e5", "down_4096x512x1024_e5_f32"])
def test_small_named_workloads(name):
    w = DOWN_WORKLOADS[name]
    check_down(w.generate(), w.tokens, w.inter, w.hidden, w.experts, w.name)


# tails: tokens not a multiple of 256 per expert; inter not a multiple of 64 (a
# partial K step, its valid part shorter and longer than one 32-wide sub-step); hidden not a multiple of 256 (the block's second 128-column
# tile partial, or absent: hidden 120 and 376); one expert; many small experts
@pytest.mark.parametrize("tokens,inter,hidden,experts,split", [
    (300, 64, 256, 3, "dirichlet"), (257, 200, 136, 4, "one_empty"), (1000, 256, 512, 1, "even"),
    (129, 96, 120, 7, "dirichlet"), (640, 1032, 376, 16, "dirichlet"), (1, 8, 8, 1, "even"),
    (513, 2048, 264, 2, "dirichlet"), (200, 184, 264, 3, "dirichlet"), (333, 232, 136, 5, "dirichlet"),
    # many experts: more row tiles than one tile group holds, groups spanning experts
    (3000, 128, 1024, 64, "dirichlet"),
])
def test_down_shapes(tokens, inter, hidden, experts, split):
    w = DownWorkload(f"d_{tokens}x{inter}x{hidden}_e{experts}", tokens, inter, hidden, experts,
                     seed=tokens + inter + hidden + experts, split=split)
    check_down(w.generate(), tokens, inter, hidden, experts, w.name)


@pytest.mark.parametrize("offs", [[50, 20, 300, 100], [0, 0, 0, 257], [257, 257, 257, 257], [-5, 10, 10, 200],
                                  [100, 1000, 5, 7]])
def test_down_counts_that_are_empty_decreasing_or_too_large(offs):
    w = DownWorkload("d_offs", 257, 64, 40, 4, seed=32)
    d = w.generate()
    d["offs"] = np.array(offs, dtype=np.int32)
    check_down(d, 257, 64, 40, 4, f"offs {offs}")


def test_down_every_token_in_one_expert_of_sixteen():
    w = DownWorkload("d_skew", 2000, 96, 520, 16, seed=35)
    d = w.generate()
    d["offs"] = np.array([0] * 7 + [2000] * 9, dtype=np.int32)
    check_down(d, 2000, 96, 520, 16, "one expert holds every token")


def test_down_zero_probabilities_and_zero_rows():
    w = DownWorkload("d_zeros", 384, 128, 264, 3, seed=33)
    d = w.generate()
    d["probs"][::7] = 0.0
    d["h"][5::11] = 0x8000                    # rows of -0: every product is +-0, the sum +0
    check_down(d, 384, 128, 264, 3, "zero probs / zero rows")


@pytest.mark.parametrize("name", ["down_131072x2048x7168_e8", "down_131072x2048x7168_e8_f32"])
def test_down_full_size_sampled_rows(name):
    w = DOWN_WORKLOADS[name]
    f32 = w.out_dtype == "f32"
    say(f"{w.name}: generate")
    d = w.generate()
    say(f"{w.name}: gpu")
    out = run_down(d, w.tokens, w.hidden, f32)
    offs = d["offs"].astype(np.int64)
    starts = np.concatenate([[0], offs[:-1]])
    rng = np.random.default_rng(6)
    pick = set()
    for s0, e0 in zip(starts, offs):
        if e0 > s0:
            pick |= {s0, s0 + 1, e0 - 1, min(s0 + 255, e0 - 1), min(s0 + 256, e0 - 1)}
    pick |= set(rng.integers(0, w.tokens, 200).tolist())
    idx = np.array(sorted(pick))
    sub = out[torch.from_numpy(idx).cuda()]
    torch.cuda.synchronize()
    got = sub.cpu().numpy() if f32 else to_host_bits(sub)
    if f32:
        assert not (out.view(torch.int32) == SENTINEL32).any().item(), f"{w.name}: rows left unwritten"
    else:
        assert not (out.view(torch.int16) == SENTINEL16).any().item(), f"{w.name}: rows left unwritten"
    expert_of = np.searchsorted(offs, idx, side="right")
    sub_offs = np.array([np.sum(expert_of <= e) for e in range(w.experts)], dtype=np.int32)
    say(f"{w.name}: oracle on {idx.size} sampled rows")
    s, s_abs = exact_sums(d["h"][idx], d["w_down"], sub_offs, idx.size, w.inter, w.hidden, w.experts)
    st = assert_down_router_within(got, f32, s, s_abs, d["probs"][idx], w.inter, w.name)
    say(f"{w.name}: {st}")


def test_down_full_size_bf16_output_is_the_rounded_fp32_output_everywhere():
    """Every element at full size: both epilogues multiply the same bf16 rounding of the
    same accumulator by p in fp32, so the bf16 output must be the bf16 rounding (to
    nearest, ties to even) of the fp32 output. The sampled rows above tie the fp32
    output to the oracle."""
    w = DOWN_WORKLOADS["down_131072x2048x7168_e8"]
    say(f"{w.name}: generate")
    d = w.generate()
    say(f"{w.name}: gpu, fp32 and bf16 outputs")
    o32 = run_down(d, w.tokens, w.hidden, True)
    o16 = run_down(d, w.tokens, w.hidden, False)
    assert not (o32.view(torch.int32) == SENTINEL32).any().item(), f"{w.name}: fp32 rows left unwritten"
    same = torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))
    torch.cuda.synchronize()
    assert same, f"{w.name}: bf16 output differs from the rounded fp32 output"
    say(f"{w.name}: bf16 output == bf16(fp32 output) on all {w.tokens} x {w.hidden}")


# ---- combine ------------------------------------------------------------------------

EO_TORCH = {oracle.BF16: torch.bfloat16, oracle.F16: torch.float16, oracle.F32: torch.float32}
EO_CODE = {"bf16": oracle.BF16, "f16": oracle.F16, "f32": oracle.F32}


def eo_to_dev(eo, code):
    if code == oracle.F32:
        return torch.from_numpy(np.ascontiguousarray(eo, np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(eo).view(np.int16)).view(EO_TORCH[code]).cuda()


def eo_for_oracle(eo, code):
    return eo.view(np.float16) if code == oracle.F16 else eo


def run_combine(eo, code, row_of, hidden):
    tokens = row_of.shape[0]
    out = torch.full((tokens, hidden), SENTINEL32, dtype=torch.int32, device="cuda").view(torch.float32)
    epi.moe_combine_fwd(eo_to_dev(eo, code), torch.from_numpy(np.ascontiguousarray(row_of)).cuda(), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_combine(eo, code, row_of, rows, hidden, what):
    tokens, top_k = row_of.shape
    got = run_combine(eo, code, row_of, hidden)
    want = oracle.moe_combine(eo_for_oracle(eo, code), code, row_of, rows, tokens, top_k, hidden)
    nan_w, nan_g = np.isnan(want), np.isnan(got)
    assert np.array_equal(nan_w, nan_g), f"{what}: NaN positions differ"
    bad = ~nan_w & (got.view(np.uint32) != want.view(np.uint32))
    assert not bad.any(), f"{what}: {int(bad.sum())} of {got.size} differ (bit-exact bar)"
    say(f"{what}: {got.size} bit-exact")


def test_combine_small_named_workload():
    w = COMBINE_WORKLOADS["combine_4096x1024_k8_e64of8"]
    d = w.generate()
    check_combine(d["expert_out"], EO_CODE[w.eo_dtype], d["row_of"], d["rows"], w.hidden, w.name)


# hidden against the 1024-element row segments a block takes: one partial segment (8, 520),
# a full one and two elements (1032), seven full ones (7168), eight and a partial ninth (8200).
# top_k: one slot, chunks of eight slot indices with more local rows than are loaded at once
# (12 of 16 experts, all local), and the largest top_k accepted.
@pytest.mark.parametrize("eo_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("tokens,hidden,top_k,ge,le", [
    (777, 1032, 8, 64, 8), (300, 8, 2, 8, 4), (513, 520, 4, 16, 16), (64, 8200, 6, 32, 32), (1, 7168, 1, 4, 2),
    (200, 1032, 12, 16, 16), (3, 64, 1024, 1024, 512),
])
def test_combine_shapes_and_dtypes(eo_dtype, tokens, hidden, top_k, ge, le):
    w = CombineWorkload(f"c_{tokens}x{hidden}_k{top_k}_e{ge}of{le}_{eo_dtype}", tokens, hidden, top_k, ge, le,
                        seed=tokens + hidden + top_k, eo_dtype=eo_dtype, sigma=3.0)
    d = w.generate()
    check_combine(d["expert_out"], EO_CODE[eo_dtype], d["row_of"], d["rows"], hidden, w.name)


def test_combine_signed_zeros_infinities_and_odd_slots():
    """-0 rows (a token whose only rows are -0 gets +0), infinities (inf - inf is NaN),
    order-sensitive magnitudes, duplicated rows, and slot indices that are negative or
    past the last row."""
    rng = np.random.default_rng(40)
    rows, tokens, top_k, hidden = 12, 40, 5, 16
    eo = rng.standard_normal((rows, hidden)).astype(np.float32)
    eo[0] = -0.0
    eo[1, :4] = np.inf
    eo[2, :4] = -np.inf
    eo[3] = 2.0 ** 24
    eo[4] = 1.0
    row_of = rng.integers(-3, rows + 4, (tokens, top_k)).astype(np.int32)
    row_of[0] = [0, 0, -1, 99, 0]
    row_of[1] = [1, 2, 3, 4, 4]
    row_of[2] = [3, 4, 4, -7, 12]
    row_of[3] = [4, 4, 3, 0, 1]
    row_of[4] = [-1, -1, -1, -1, -1]
    check_combine(eo, oracle.F32, row_of, rows, hidden, "zeros / infinities / odd slots")
    got = run_combine(eo, oracle.F32, row_of, hidden)
    assert (got[0] == 0).all() and not np.signbit(got[0]).any()
    assert (got[4] == 0).all() and not np.signbit(got[4]).any()


def test_combine_no_local_rows():
    """rows == 0: every slot is another rank's; out is +0 everywhere (expert_out is empty)."""
    tokens, top_k, hidden = 33, 3, 24
    out = torch.full((tokens, hidden), 7.0, dtype=torch.float32, device="cuda")
    eo = torch.empty((0, hidden), dtype=torch.float32, device="cuda")
    row_of = torch.from_numpy(np.arange(tokens * top_k, dtype=np.int32).reshape(tokens, top_k) % 5 - 2).cuda()
    epi.moe_combine_fwd(eo, row_of, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert (got == 0).all() and not np.signbit(got).any()


def test_combine_full_size_every_token():
    w = COMBINE_WORKLOADS["combine_131072x7168_k8_e64of8"]
    say(f"{w.name}: generate")
    d = w.generate()
    code, row_of, rows = EO_CODE[w.eo_dtype], d["row_of"], d["rows"]
    say(f"{w.name}: gpu ({rows} rows)")
    out = torch.full((w.tokens, w.hidden), SENTINEL32, dtype=torch.int32,
                     device="cuda").view(torch.float32)
    epi.moe_combine_fwd(eo_to_dev(d["expert_out"], code), torch.from_numpy(row_of).cuda(), out)
    got = out.cpu().numpy()
    del out
    say(f"{w.name}: oracle on every token")
    want = oracle.moe_combine(d["expert_out"], code, row_of, rows, w.tokens, w.top_k, w.hidden)
    bad = np.flatnonzero((got.view(np.uint32) != want.view(np.uint32)).any(axis=1))
    assert bad.size == 0, f"{w.name}: {bad.size} tokens differ, first {bad[:5].tolist()}"
    n_local = (row_of >= 0).sum(1)
    say(f"{w.name}: all {w.tokens} tokens bit-exact ({int((n_local == 0).sum())} with no local row, "
        f"{int((n_local >= 3).sum())} with three or more)")


def test_the_chain_on_a_side_stream_gives_identical_results():
    """gate_up GEMM + SwiGLU -> down GEMM + router multiply (fp32) -> combine, on the default
    stream and on a side stream: bit-identical outputs (the binding passes the current stream)."""
    from moe_routed_expert_amd.workloads import GroupedWorkload
    gw = GroupedWorkload("chain", 1000, 256, 128, 4, 7.0, seed=41)
    g = gw.generate()
    rng = np.random.default_rng(42)
    wd = to_dev_bf16(((rng.standard_normal((4, 256, 128)).astype(np.float32) * 0.05).view(np.uint32) >> 16)
                     .astype(np.uint16))
    a, wg, wu = to_dev_bf16(g["a"]), to_dev_bf16(g["w_gate"]), to_dev_bf16(g["w_up"])
    offs = torch.from_numpy(g["offs"]).cuda()
    p = torch.from_numpy(g["probs"]).cuda()
    tokens, top_k = 500, 2
    row_of = torch.from_numpy(rng.permutation(1000).astype(np.int32).reshape(tokens, top_k)).cuda()

    def chain():
        y = torch.empty((1000, 128), dtype=torch.bfloat16, device="cuda")
        epi.grouped_gate_up_swiglu_fwd(a, wg, wu, offs, p, y, None, 7.0)
        o = torch.empty((1000, 256), dtype=torch.float32, device="cuda")
        epi.grouped_down_router_fwd(y, wd, offs, p, o)
        c = torch.empty((tokens, 256), dtype=torch.float32, device="cuda")
        epi.moe_combine_fwd(o, row_of, c)
        return y, o, c

    say("chain: default stream vs side stream")
    ref = chain()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = chain()
    torch.cuda.synchronize()
    for r, q in zip(ref, got):
        assert torch.equal(r.view(torch.int16) if r.dtype == torch.bfloat16 else r.view(torch.int32),
                           q.view(torch.int16) if q.dtype == torch.bfloat16 else q.view(torch.int32))
    assert torch.isfinite(ref[2]).all()


# ---- tensors of more than 2^31 elements (64-bit offsets) -----------------------------

def _sampled_rows(tokens, offs, extra, seed):
    rng = np.random.default_rng(seed)
    ends = offs.astype(np.int64)
    starts = np.concatenate([[0], ends[:-1]])
    pick = {tokens - 1}
    for s0, e0 in zip(starts, ends):
        if e0 > s0:
            pick |= {int(s0), int(e0 - 1)}
    pick |= set(rng.integers(0, tokens, extra).tolist())
    return np.array(sorted(pick))


def test_gate_up_with_more_than_2_31_activation_elements():
    tokens, hidden, inter, experts = 300000, 7168, 256, 2
    offs = np.array([150001, tokens], np.int32)
    g = torch.Generator(device="cuda").manual_seed(50)
    say(f"gate_up {tokens}x{hidden}x{inter}: generate on the device")
    a = torch.randn(tokens, hidden, device="cuda", generator=g).to(torch.bfloat16)
    assert a.numel() > 2 ** 31
    wg = (torch.randn(experts, inter, hidden, device="cuda", generator=g) * 0.05).to(torch.bfloat16)
    wu = (torch.randn(experts, inter, hidden, device="cuda", generator=g) * 0.05).to(torch.bfloat16)
    p = torch.rand(tokens, device="cuda", generator=g)
    y = torch.empty(tokens, inter, dtype=torch.bfloat16, device="cuda")
    x = torch.empty(tokens, 2 * inter, dtype=torch.bfloat16, device="cuda")
    epi.grouped_gate_up_swiglu_fwd(a, wg, wu, torch.from_numpy(offs).cuda(), p, y, x, 10.0)
    idx = _sampled_rows(tokens, offs, 60, 51)
    ti = torch.from_numpy(idx).cuda()
    a_s, x_s, y_s = to_host_bits(a[ti]), to_host_bits(x[ti]), to_host_bits(y[ti])
    p_s = p[ti].cpu().numpy()
    torch.cuda.synchronize()
    expert_of = np.searchsorted(offs.astype(np.int64), idx, side="right")
    sub_offs = np.array([np.sum(expert_of <= e) for e in range(experts)], dtype=np.int32)
    say(f"gate_up: oracle on {idx.size} sampled rows (largest row offset {idx[-1] * hidden})")
    s, s_abs = oracle.grouped_gate_up(a_s, to_host_bits(wg), to_host_bits(wu), sub_offs, idx.size, hidden, inter,
                                      experts, with_abs_sum=True)
    from tests.gpu_util import assert_bf16_parity, assert_gemm_bf16_within
    assert_gemm_bf16_within(x_s, s, s_abs, hidden, "gate_up x beyond 2^31")
    assert_bf16_parity(y_s, oracle.swiglu_clamped_fwd(x_s, p_s, idx.size, inter, 10.0), "gate_up y beyond 2^31")


def test_down_with_more_than_2_31_output_elements():
    tokens, inter, hidden, experts = 300000, 256, 7168, 2
    offs = np.array([120000, tokens], np.int32)
    g = torch.Generator(device="cuda").manual_seed(52)
    say(f"down {tokens}x{inter}x{hidden}: generate on the device")
    h = torch.randn(tokens, inter, device="cuda", generator=g).to(torch.bfloat16)
    wd = (torch.randn(experts, hidden, inter, device="cuda", generator=g) * 0.1).to(torch.bfloat16)
    p = torch.rand(tokens, device="cuda", generator=g)
    out = torch.empty(tokens, hidden, dtype=torch.float32, device="cuda")
    assert out.numel() > 2 ** 31
    epi.grouped_down_router_fwd(h, wd, torch.from_numpy(offs).cuda(), p, out)
    idx = _sampled_rows(tokens, offs, 60, 53)
    ti = torch.from_numpy(idx).cuda()
    h_s, o_s, p_s = to_host_bits(h[ti]), out[ti].cpu().numpy(), p[ti].cpu().numpy()
    torch.cuda.synchronize()
    expert_of = np.searchsorted(offs.astype(np.int64), idx, side="right")
    sub_offs = np.array([np.sum(expert_of <= e) for e in range(experts)], dtype=np.int32)
    say(f"down: oracle on {idx.size} sampled rows (largest output offset {idx[-1] * hidden})")
    s, s_abs = exact_sums(h_s, to_host_bits(wd), sub_offs, idx.size, inter, hidden, experts)
    assert_down_router_within(o_s, True, s, s_abs, p_s, inter, "down beyond 2^31")


def test_combine_with_more_than_2_31_elements():
    """Past 2^31 elements, and with 300000 x 7 (token, segment) pairs more than the grid
    holds, so blocks take several pairs each."""
    tokens, hidden, top_k = 300000, 7168, 2
    rows = 320000
    g = torch.Generator(device="cuda").manual_seed(54)
    say(f"combine {tokens}x{hidden}, {rows} rows: generate on the device")
    eo = torch.randn(rows, hidden, device="cuda", generator=g)
    assert eo.numel() > 2 ** 31
    rng = np.random.default_rng(55)
    row_of = rng.integers(-1, rows, (tokens, top_k)).astype(np.int32)
    row_of[-1] = [rows - 1, rows - 2]                     # the last rows, far past 2^31 elements
    out = torch.empty(tokens, hidden, dtype=torch.float32, device="cuda")
    epi.moe_combine_fwd(eo, torch.from_numpy(row_of).cuda(), out)
    idx = np.unique(np.concatenate([rng.integers(0, tokens, 60), [tokens - 1]]))
    used = np.unique(row_of[idx][row_of[idx] >= 0])
    eo_s = eo[torch.from_numpy(used.astype(np.int64)).cuda()].cpu().numpy()
    got = out[torch.from_numpy(idx).cuda()].cpu().numpy()
    torch.cuda.synchronize()
    remap = {int(r): i for i, r in enumerate(used)}
    ro_s = np.vectorize(lambda r: remap.get(int(r), -1))(row_of[idx]).astype(np.int32)
    say(f"combine: oracle on {idx.size} sampled tokens")
    want = oracle.moe_combine(eo_s, oracle.F32, ro_s, used.size, idx.size, top_k, hidden)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "combine beyond 2^31: sampled tokens differ"


def test_router_multiply_to_fp32_then_combine_matches_the_oracle_bit_for_bit():
    """The non-GEMM part of the path end to end: routed bf16 rows times their probabilities
    into fp32 (router_weight_mul_fwd with an fp32 output), then the combine. Both steps are
    exact definitions, so the chain must equal the oracle's chain bit for bit."""
    w = COMBINE_WORKLOADS["combine_4096x1024_k8_e64of8"]
    row_of, rows = w.row_of()
    rng = np.random.default_rng(44)
    xb = ((rng.standard_normal((rows, w.hidden)).astype(np.float32)).view(np.uint32) >> 16).astype(np.uint16)
    p = rng.random(rows, dtype=np.float32)
    say(f"router fp32 -> combine, {rows} rows x {w.hidden}")
    x_d = to_dev_bf16(xb)
    p_d = torch.from_numpy(p).cuda()
    o_d = torch.empty((rows, w.hidden), dtype=torch.float32, device="cuda")
    epi.router_weight_mul_fwd(x_d, p_d, o_d)
    c_d = torch.empty((w.tokens, w.hidden), dtype=torch.float32, device="cuda")
    epi.moe_combine_fwd(o_d, torch.from_numpy(row_of).cuda(), c_d)
    torch.cuda.synchronize()
    o_want = oracle.router_weight_mul_fwd_typed(xb, oracle.BF16, p, oracle.F32, rows, w.hidden)
    c_want = oracle.moe_combine(o_want, oracle.F32, row_of, rows, w.tokens, w.top_k, w.hidden)
    assert np.array_equal(o_d.cpu().numpy().view(np.uint32), o_want.view(np.uint32))
    assert np.array_equal(c_d.cpu().numpy().view(np.uint32), c_want.view(np.uint32))
