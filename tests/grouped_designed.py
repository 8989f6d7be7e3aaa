"""Designed inputs for the fused gate_up grouped GEMM + clamped SwiGLU epilogue
on which the two possible readings of the epilogue's inputs give different
bf16 outputs.

The page "nemo_automodel.components.quantized_experts" (`_mxfp4_base_mm`)
returns the grouped product in the activation dtype, and the clamped SwiGLU of
page "nemo_automodel.components.moe.swiglu_triton" (module description) is then
applied to that bf16 tensor. So the epilogue's gate and up are the bf16
roundings of the sums, not the fp32 accumulators. A random test cannot tell
the two apart within a 1-ulp bar; these inputs can.

Every grouped sum here is exact in binary32 whatever the order of additions
(three terms of a few significant bits each, the rest zeros) and is not a bf16
value, so the bf16 rounding of x is known exactly. Each row's probability is
chosen so that, in one target column, silu(min(g, L)) * clamp(u) * p rounds to
different bf16 values under the two readings, both at least REL_MARGIN away
(relatively) from a rounding midpoint, far more than the kernel's fp32
arithmetic can move them.
"""
import numpy as np
import torch

TOKENS, HIDDEN, INTER, EXPERTS, LIMIT = 64, 8, 16, 2, 7.0
REL_MARGIN = 1e-4

# (d1, d2): 1 + d1 + d2 is exact in binary32 and is not a bf16 value
PAIRS = [(2.0 ** -8, 2.0 ** -10), (2.0 ** -9, 2.0 ** -11), (2.0 ** -7, 2.0 ** -9), (2.0 ** -7, -(2.0 ** -10))]
UP_SCALES = [0.5, 1.0, 2.0, 4.0]            # |u| stays below LIMIT: no clamp on up
GATE_SCALES = [0.5, 1.0, 2.0, 3.0, -1.0, -2.0, 4.0, 6.0]


def bf16_bits_of_exact(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values that are bf16 numbers (asserted)."""
    f = np.asarray(v, dtype=np.float32)
    b = f.view(np.uint32)
    assert (b & 0xFFFF == 0).all() and np.array_equal(f.astype(np.float64), np.asarray(v, np.float64))
    return (b >> 16).astype(np.uint16)


def to_bf16_value(x) -> np.ndarray:
    """Nearest bf16 value (ties to even) of float64 values, as float64."""
    return torch.from_numpy(np.atleast_1d(np.asarray(x, np.float64))).to(torch.bfloat16).to(torch.float64).numpy()


def to_bf16_bits(x) -> np.ndarray:
    return torch.from_numpy(np.atleast_1d(np.asarray(x, np.float64))).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def stable(x: float) -> bool:
    """x rounds to the same bf16 value anywhere within REL_MARGIN of itself."""
    v = to_bf16_value([x * (1 - REL_MARGIN), x, x * (1 + REL_MARGIN)])
    return v[0] == v[1] == v[2]


def silu(z):
    return z / (1.0 + np.exp(-z))


def y_of(g, u, p, L):
    """The clamped SwiGLU times p, in float64, of the given gate and up."""
    return silu(np.minimum(g, L)) * np.clip(u, -L, L) * p


def build():
    """Inputs (bf16 bits / float32), the exact sums (float64) and, per row, the
    target column with the bf16 bits each reading gives there."""
    a = np.zeros((TOKENS, HIDDEN))
    a[:, :3] = 1.0
    wg = np.zeros((EXPERTS, INTER, HIDDEN))
    wu = np.zeros((EXPERTS, INTER, HIDDEN))
    for e in range(EXPERTS):
        sgn = 1.0 if e == 0 else -1.0
        for n in range(INTER):
            d1, d2 = PAIRS[n % len(PAIRS)]
            if n < INTER // 2:      # the up sum carries the difference; the gate is clamped to L
                wg[e, n, 0] = 64.0
                s = UP_SCALES[(n // len(PAIRS)) % len(UP_SCALES)] * sgn
                wu[e, n, :3] = (s, s * d1, s * d2)
            else:                   # the gate sum carries the difference; up is +-1
                wu[e, n, 0] = sgn
                s = GATE_SCALES[(n - INTER // 2) % len(GATE_SCALES)] * sgn
                wg[e, n, :3] = (s, s * d1, s * d2)
    offs = np.array([TOKENS // 2, TOKENS], dtype=np.int32)
    expert_of_row = np.repeat(np.arange(EXPERTS), TOKENS // EXPERTS)
    g_exact = np.stack([a[t] @ wg[expert_of_row[t]].T for t in range(TOKENS)])
    u_exact = np.stack([a[t] @ wu[expert_of_row[t]].T for t in range(TOKENS)])
    for v in (g_exact, u_exact):   # exact in binary32 and not bf16 numbers (the gate of up-case columns is 64)
        assert np.array_equal(v.astype(np.float32).astype(np.float64), v)
    g_b = to_bf16_value(g_exact).reshape(g_exact.shape)
    u_b = to_bf16_value(u_exact).reshape(u_exact.shape)
    assert (u_b[:, :INTER // 2] != u_exact[:, :INTER // 2]).all()
    assert (g_b[:, INTER // 2:] != g_exact[:, INTER // 2:]).all()

    probs = np.empty(TOKENS, np.float32)
    target = np.empty(TOKENS, np.int64)
    want_bits = np.empty(TOKENS, np.uint16)       # the bf16-rounded reading
    other_bits = np.empty(TOKENS, np.uint16)      # the fp32-accumulator reading
    for t in range(TOKENS):
        n = t % INTER
        for j in range(2000):
            p = float(np.float32(0.3 + 0.00731 * j))
            y_bf = float(y_of(g_b[t, n], u_b[t, n], p, LIMIT))
            y_32 = float(y_of(g_exact[t, n], u_exact[t, n], p, LIMIT))
            if stable(y_bf) and stable(y_32) and to_bf16_bits(y_bf)[0] != to_bf16_bits(y_32)[0]:
                break
        else:
            raise AssertionError(f"no probability separates the readings in row {t}")
        probs[t], target[t] = p, n
        want_bits[t], other_bits[t] = to_bf16_bits(y_bf)[0], to_bf16_bits(y_32)[0]
    return {"a": bf16_bits_of_exact(a), "w_gate": bf16_bits_of_exact(wg), "w_up": bf16_bits_of_exact(wu),
            "offs": offs, "probs": probs, "g_exact": g_exact, "u_exact": u_exact,
            "x_bits": np.concatenate([to_bf16_bits(g_exact).reshape(g_exact.shape),
                                      to_bf16_bits(u_exact).reshape(u_exact.shape)], axis=1),
            "target": target, "want_bits": want_bits, "other_bits": other_bits}
