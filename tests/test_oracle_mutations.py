"""The pins catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle/oracle.c (a dropped term, a
wrong sign, a swapped operand or half, an exclusive mask, a clamp on the wrong
side, truncation instead of round-to-nearest-even, ...), builds it with the
oracle's own flags in a temporary directory, loads it through a fresh copy of
the oracle wrapper and runs the pin tests of tests/test_oracle_pins.py
against it. At least one pin must fail for every planted mistake. The real
oracle is never modified; everything here runs on the CPU.
"""
import importlib.util
import os
import subprocess

import pytest

import oracle as real_oracle
from oracle import build as oracle_build
from tests import test_oracle_pins as pins
from tests import test_oracle_pins_dtypes as dpins
from tests import test_oracle_pins_grouped as gpins
from tests import test_oracle_pins_next3 as npins

SRC = oracle_build.SRC

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("gate clamped from below too", "float gc = (g > L) ? L : g;",
     "float gc = (g > L) ? L : ((g < -L) ? -L : g);"),
    ("exclusive gate mask", "int mask_g = (g <= L);", "int mask_g = (g < L);"),
    ("exclusive up mask", "int mask_u = (-L <= u) && (u <= L);", "int mask_u = (-L < u) && (u < L);"),
    ("up clamped from above only", "float uc = (u > L) ? L : ((u < -L) ? -L : u);", "float uc = (u > L) ? L : u;"),
    ("sigmoid sign", "float sig = 1.0f / (1.0f + expf(-gc));", "float sig = 1.0f / (1.0f + expf(gc));"),
    ("silu of the unclamped gate", "float a = gc * sig;", "float a = g * sig;"),
    ("silu' term dropped", "float dsilu = sig * (1.0f + gc * (1.0f - sig));", "float dsilu = sig;"),
    ("silu' sign flipped", "float dsilu = sig * (1.0f + gc * (1.0f - sig));",
     "float dsilu = sig * (1.0f - gc * (1.0f - sig));"),
    ("d_gate without the probability", "out[1] = mask_g ? (t * uc) * dsilu : 0.0f;",
     "out[1] = mask_g ? (gy * uc) * dsilu : 0.0f;"),
    ("d_up with the wrong factor", "out[2] = mask_u ? t * a : 0.0f;", "out[2] = mask_u ? t * uc : 0.0f;"),
    ("masked gradient as -0", "out[2] = mask_u ? t * a : 0.0f;", "out[2] = mask_u ? t * a : -0.0f;"),
    ("probability-gradient term times p", "out[3] = gy * h;", "out[3] = gy * h * p;"),
    ("forward without the probability", "out[0] = h * p;", "out[0] = h;"),
    ("gate and up halves swapped (forward)",
     "oracle_swiglu_point(oracle_bf16_to_f32(xr[j]), oracle_bf16_to_f32(xr[inter + j]),\n                                probs[r], 0.0f, L, q);",
     "oracle_swiglu_point(oracle_bf16_to_f32(xr[inter + j]), oracle_bf16_to_f32(xr[j]),\n                                probs[r], 0.0f, L, q);"),
    ("d_gate and d_up halves swapped", "gxr[j] = oracle_f32_to_bf16(q[1]);\n            gxr[inter + j] = oracle_f32_to_bf16(q[2]);",
     "gxr[j] = oracle_f32_to_bf16(q[2]);\n            gxr[inter + j] = oracle_f32_to_bf16(q[1]);"),
    ("truncation instead of rounding", "if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))", "if (0)"),
    ("ties away from zero", "if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))", "if (dropped >= 0x8000u)"),
    ("router grad_x from x", "grad_x[r * hidden + k] = oracle_f32_to_bf16(g * probs[r]);",
     "grad_x[r * hidden + k] = oracle_f32_to_bf16(oracle_bf16_to_f32(x ? x[r * hidden + k] : grad_out[r * hidden + k]) * probs[r]);"),
    ("router grad_probs squares grad_out", "float term = g * oracle_bf16_to_f32(x[r * hidden + k]);", "float term = g * g;"),
    ("router forward skips the probability", "float v = oracle_bf16_to_f32(x[r * hidden + k]) * probs[r];",
     "float v = oracle_bf16_to_f32(x[r * hidden + k]);"),
    ("row sums in float32", "acc += (double)q[3];", "acc = (double)((float)acc + q[3]);"),
    ("float16 truncation", "if (rem > half || (rem == half && (n & 1u)))", "if (0)"),
    ("float16 ties away from zero", "if (rem > half || (rem == half && (n & 1u)))", "if (rem >= half)"),
    ("float16 exponent bias", "uint32_t out = ((uint32_t)(e + 15) << 10)", "uint32_t out = ((uint32_t)(e + 16) << 10)"),
    ("float16 subnormals flushed", "if (e < -14)\n        return (uint16_t)(sign | n);",
     "if (e < -14)\n        return sign;"),
    ("float16 widening bias", "mag = ldexpf((float)(1024u + frac), ex - 25);", "mag = ldexpf((float)(1024u + frac), ex - 24);"),
    ("typed router forward skips the probability",
     "oracle_store(out, r * hidden + k, out_dtype, oracle_load(x, r * hidden + k, x_dtype) * probs[r]);",
     "oracle_store(out, r * hidden + k, out_dtype, oracle_load(x, r * hidden + k, x_dtype));"),
    ("grouped: weights read transposed",
     "double prod = (double)oracle_bf16_to_f32(at[h]) * (double)oracle_bf16_to_f32(wj[h]);",
     "double prod = (double)oracle_bf16_to_f32(at[h]) * (double)oracle_bf16_to_f32(w[h * inter + j]);"),
    ("grouped: the previous expert's weights",
     "const uint16_t *w = (half == 0 ? w_gate : w_up) + e * inter * hidden;",
     "const uint16_t *w = (half == 0 ? w_gate : w_up) + (e > 0 ? e - 1 : 0) * inter * hidden;"),
    ("grouped: gate and up weights swapped",
     "const uint16_t *w = (half == 0 ? w_gate : w_up) + e * inter * hidden;",
     "const uint16_t *w = (half == 0 ? w_up : w_gate) + e * inter * hidden;"),
    ("grouped: offs read as per-expert counts", "int64_t end = offs[e];", "int64_t end = start + offs[e];"),
    ("grouped: decreasing counts not clamped", "if (end < start) end = start;", ";"),
    ("grouped: sums rounded through binary32", "uint16_t g = oracle_f64_to_bf16(sum_scratch[t * 2 * inter + j]);",
     "uint16_t g = oracle_f32_to_bf16((float)sum_scratch[t * 2 * inter + j]);"),
    ("grouped: epilogue on the binary32 sums, not their bf16 roundings",
     "oracle_swiglu_point(oracle_bf16_to_f32(g), oracle_bf16_to_f32(u), probs[t], 0.0f, L, q);",
     "oracle_swiglu_point((float)sum_scratch[t * 2 * inter + j], (float)sum_scratch[t * 2 * inter + inter + j], "
     "probs[t], 0.0f, L, q);"),
    ("down: probability not applied", "oracle_store(out, t * hidden + n, out_dtype, out2 * probs[t]);",
     "oracle_store(out, t * hidden + n, out_dtype, out2);"),
    ("down: sum not rounded to bf16 first", "float out2 = oracle_bf16_to_f32(oracle_f64_to_bf16(s));",
     "float out2 = (float)s;"),
    ("down: weights read transposed",
     "s += (double)oracle_bf16_to_f32(ht[i]) * (double)oracle_bf16_to_f32(wn[i]);",
     "s += (double)oracle_bf16_to_f32(ht[i]) * (double)oracle_bf16_to_f32(w[i * hidden + n]);"),
    ("combine: slots in descending order", "for (int64_t j = 0; j < top_k; ++j) {",
     "for (int64_t j = top_k - 1; j >= 0; --j) {"),
    ("combine: starts from -0", "float acc = 0.0f;", "float acc = -0.0f;"),
    ("combine: the last slot overwrites", "acc = acc + oracle_load(expert_out, r * hidden + n, eo_dtype);",
     "acc = oracle_load(expert_out, r * hidden + n, eo_dtype);"),
    ("typed backward reads grad_y as x's neighbour",
     "oracle_load(grad_y, r * inter + j, dtype), L, q);", "oracle_load(x, r * inter + j, dtype), L, q);"),
]


def _pins():
    """Every pin test, with its parameters bound, cheapest first."""
    calls = [
        ("rounding via router forward", lambda o: pins.test_oracle_rounding_matches_torch_via_router_forward(o)),
        ("hand-derived cases", lambda o: [pins.test_bwd_hand_derived_cases(c, o) for c in pins._golden_rows()]),
        ("fwd gate sweep L=7", lambda o: pins.test_fwd_every_bf16_gate_vs_float64_library(7.0, o)),
        ("fwd up sweep", lambda o: pins.test_fwd_every_bf16_up_vs_float64_library(o)),
        ("bwd gate sweep", lambda o: pins.test_bwd_every_bf16_gate_vs_autograd(o)),
        ("bwd up sweep", lambda o: pins.test_bwd_every_bf16_up_vs_autograd(o)),
        ("one-sided differences", lambda o: pins.test_bwd_one_sided_differences_at_the_limits(o)),
        ("cancellation in row sums", lambda o: pins.test_grad_probs_keep_small_terms_next_to_cancelling_large_ones(o)),
        ("central differences", lambda o: pins.test_bwd_matches_central_finite_differences(o)),
        ("brute force 4x8", lambda o: pins.test_bruteforce_4x8_dependency_structure(o)),
        ("fwd workload", lambda o: pins.test_fwd_workload_vs_float64_library("swiglu_256x128", o)),
        ("bwd workloads", lambda o: [pins.test_bwd_workload_vs_autograd(w, o) for w in
                                     (pins.WORKLOADS["swiglu_256x128"],)]),
        ("textbook swiglu", lambda o: pins.test_fwd_reduces_to_textbook_swiglu_without_clamp(o)),
        ("router fwd eager", lambda o: pins.test_router_fwd_bitwise_equals_eager_fp32_multiply(o)),
        ("router bwd exact", lambda o: pins.test_router_bwd_grad_x_bitwise_equals_eager_and_grad_probs_exact(o)),
        ("router bwd without x", lambda o: pins.test_router_bwd_without_probability_gradient_skips_x(o)),
        ("power-of-two scaling", lambda o: pins.test_power_of_two_scaling_is_exact(o)),
        ("float16 widening", lambda o: dpins.test_f16_widening_every_pattern_matches_numpy(o)),
        ("float16 rounding", lambda o: dpins.test_f16_rounding_matches_numpy_via_router_forward(o)),
        ("typed bf16 = bf16", lambda o: dpins.test_typed_bf16_equals_untyped(o)),
        ("float16 sweeps", lambda o: [dpins.test_f16_every_pattern_vs_float64_autograd(w, o) for w in ("gate", "up")]),
        ("float32 bounds", lambda o: dpins.test_f32_random_inputs_within_derived_bounds(o)),
        ("router dtypes fwd", lambda o: [dpins.test_router_typed_forward_bitwise_equals_eager(a, b, o)
                                         for a, b in ((real_oracle.BF16, real_oracle.F32),
                                                      (real_oracle.F16, real_oracle.F16))]),
        ("router fp32 grad_out", lambda o: dpins.test_router_typed_backward_fp32_grad_out(o)),
        ("binary64 rounding", lambda o: gpins.test_f64_rounding_matches_nearest_search_and_the_exact_helper(o)),
        ("grouped integer products", lambda o: [gpins.test_integer_products_per_expert_are_exact(f, o) for f in
                                                ([3, 3, 9, 14], [5, 2, 20, 14], [-4, 6, 9, 11])]),
        ("grouped float64 matmul", lambda o: gpins.test_float64_matmul_on_normal_data(o)),
        ("grouped rational sums", lambda o: gpins.test_tiny_case_exact_rational_sums_and_rounding(o)),
        ("grouped per-expert scale", lambda o: gpins.test_per_expert_power_of_two_weights_select_the_expert(o)),
        ("grouped epilogue", lambda o: gpins.test_forward_is_the_epilogue_of_the_rounded_sums(o)),
        ("grouped tie", lambda o: gpins.test_sums_next_to_a_bf16_tie_are_rounded_once(o)),
        ("grouped reading", lambda o: gpins.test_epilogue_reads_the_bf16_rounded_sums_not_the_accumulators(o)),
        ("down integer", lambda o: [npins.test_down_integer_products_and_power_of_two_probs(d, f, o)
                                    for d in (real_oracle.BF16, real_oracle.F32) for f in ([4, 4, 11], [11, 3, 20])]),
        ("down rational", lambda o: npins.test_down_exact_rational_sums_then_the_router_multiply(o)),
        ("down layout", lambda o: npins.test_down_weights_are_rows_of_hidden(o)),
        ("combine order", lambda o: npins.test_combine_adds_slots_in_ascending_order_in_binary32(o)),
        ("combine integer", lambda o: [npins.test_combine_integer_rows_match_numpy(d, o)
                                       for d in (real_oracle.BF16, real_oracle.F32)]),
    ]
    return calls


def _load_mutant(tmp_path, name, find, repl):
    src = open(SRC).read()
    assert src.count(find) >= 1, f"mutation '{name}' no longer matches oracle.c"
    mutated = src.replace(find, repl, 1)
    c_path = tmp_path / "oracle_mutant.c"
    c_path.write_text(mutated)
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", *oracle_build.CFLAGS, str(c_path), "-o", str(so), "-lm"], check=True)
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{abs(hash(name))}",
                                                  os.path.join(os.path.dirname(SRC), "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._LIB_PATH = str(so)
    mod._lib = None
    return mod


def test_the_real_oracle_passes_every_pin():
    for label, call in _pins():
        call(real_oracle)


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_every_planted_mistake_is_caught(tmp_path, name, find, repl):
    mod = _load_mutant(tmp_path, name, find, repl)
    for label, call in _pins():
        try:
            call(mod)
        except AssertionError:
            return  # caught
    pytest.fail(f"no pin catches the planted mistake: {name}")
