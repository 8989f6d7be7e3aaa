"""CPU oracle for the routed-expert epilogue (ctypes wrapper of liboracle.so).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library
and its Python binding) never imports or calls it, and the two share no code.

All arrays are numpy: bfloat16 tensors travel as uint16 bit patterns, probs and
probability gradients as float32. See oracle.c for the definitions and the
passages of the pages each function follows.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(library cross-checks, exhaustive bfloat16 sweeps, finite differences, exact
sums, hand-derived cases); none is "parity unpinned".
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def default_threads() -> int:
    """Threads the oracle uses unless told otherwise (host cores, at most 16)."""
    return max(1, min(16, os.cpu_count() or 1))


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # build only if nothing is built
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_swiglu_point.argtypes = [ctypes.c_float] * 5 + [_f32p]
    lib.oracle_swiglu_point.restype = None
    lib.oracle_swiglu_clamped_fwd.argtypes = [_u16p, _f32p, _u16p, _i64, _i64, ctypes.c_float, ctypes.c_int]
    lib.oracle_swiglu_clamped_fwd.restype = None
    lib.oracle_swiglu_clamped_bwd.argtypes = [_u16p, _f32p, _u16p, _u16p, _f32p, _f64p, _i64, _i64,
                                              ctypes.c_float, ctypes.c_int]
    lib.oracle_swiglu_clamped_bwd.restype = None
    lib.oracle_router_weight_mul_fwd.argtypes = [_u16p, _f32p, _u16p, _i64, _i64, ctypes.c_int]
    lib.oracle_router_weight_mul_fwd.restype = None
    lib.oracle_router_weight_mul_bwd.argtypes = [_u16p, _u16p, _f32p, _u16p, _f32p, _f64p, _i64, _i64,
                                                 ctypes.c_int]
    lib.oracle_router_weight_mul_bwd.restype = None
    _lib = lib
    return lib


def _arr(a, dtype, shape):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    if a.size != int(np.prod(shape)):
        raise ValueError(f"expected {shape} elements, got shape {a.shape}")
    return a


def _p(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype)) if a is not None else None


# ---- scalar helpers (used by the pin tests) ------------------------------

def bf16_to_f32(b: int) -> float:
    return float(_load().oracle_bf16_to_f32(int(b)))


def f32_to_bf16(f: float) -> int:
    return int(_load().oracle_f32_to_bf16(float(f)))


def swiglu_point(g: float, u: float, p: float, gy: float, L: float):
    """(y_f32, d_gate_f32, d_up_f32, dprob_term_f32) for one element, unrounded."""
    out = (ctypes.c_float * 4)()
    _load().oracle_swiglu_point(g, u, p, gy, L, out)
    return tuple(float(v) for v in out)


def f32_to_bf16_array(a):
    """Vector form of f32_to_bf16 (loops in Python over ctypes: small inputs only)."""
    lib = _load()
    flat = np.ascontiguousarray(a, dtype=np.float32).ravel()
    return np.array([lib.oracle_f32_to_bf16(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(a))


# ---- tensor entry points --------------------------------------------------

def swiglu_clamped_fwd(x, probs, rows, inter, L, threads=None):
    """y (uint16 [rows, inter]) = bf16(silu(min(gate, L)) * clamp(up, -L, L) * p)."""
    x = _arr(x, np.uint16, (rows, 2 * inter))
    probs = _arr(probs, np.float32, (rows,))
    y = np.empty((rows, inter), dtype=np.uint16)
    _load().oracle_swiglu_clamped_fwd(_p(x, ctypes.c_uint16), _p(probs, ctypes.c_float),
                                      _p(y, ctypes.c_uint16), rows, inter, float(L),
                                      threads or default_threads())
    return y


def swiglu_clamped_bwd(x, probs, grad_y, rows, inter, L, want_grad_probs=True, threads=None,
                       with_abs_sum=False):
    """(grad_x uint16 [rows, 2*inter], grad_probs float32 [rows] or None), plus the
    per-row sum of |term| (float64) when with_abs_sum."""
    x = _arr(x, np.uint16, (rows, 2 * inter))
    probs = _arr(probs, np.float32, (rows,))
    grad_y = _arr(grad_y, np.uint16, (rows, inter))
    grad_x = np.empty((rows, 2 * inter), dtype=np.uint16)
    grad_probs = np.empty((rows,), dtype=np.float32) if want_grad_probs else None
    abs_sum = np.empty((rows,), dtype=np.float64) if with_abs_sum else None
    _load().oracle_swiglu_clamped_bwd(_p(x, ctypes.c_uint16), _p(probs, ctypes.c_float),
                                      _p(grad_y, ctypes.c_uint16), _p(grad_x, ctypes.c_uint16),
                                      _p(grad_probs, ctypes.c_float), _p(abs_sum, ctypes.c_double),
                                      rows, inter, float(L), threads or default_threads())
    if with_abs_sum:
        return grad_x, grad_probs, abs_sum
    return grad_x, grad_probs


def router_weight_mul_fwd(x, probs, rows, hidden, threads=None):
    """out (uint16 [rows, hidden]) = bf16(fp32(x) * p)."""
    x = _arr(x, np.uint16, (rows, hidden))
    probs = _arr(probs, np.float32, (rows,))
    out = np.empty((rows, hidden), dtype=np.uint16)
    _load().oracle_router_weight_mul_fwd(_p(x, ctypes.c_uint16), _p(probs, ctypes.c_float),
                                         _p(out, ctypes.c_uint16), rows, hidden,
                                         threads or default_threads())
    return out


def router_weight_mul_bwd(grad_out, x, probs, rows, hidden, want_grad_probs=True, threads=None,
                          with_abs_sum=False):
    """(grad_x uint16 [rows, hidden], grad_probs float32 [rows] or None), plus the
    per-row sum of |term| (float64) when with_abs_sum; x may be None when
    want_grad_probs is False."""
    grad_out = _arr(grad_out, np.uint16, (rows, hidden))
    if want_grad_probs:
        x = _arr(x, np.uint16, (rows, hidden))
    else:
        x = None
    probs = _arr(probs, np.float32, (rows,))
    grad_x = np.empty((rows, hidden), dtype=np.uint16)
    grad_probs = np.empty((rows,), dtype=np.float32) if want_grad_probs else None
    abs_sum = np.empty((rows,), dtype=np.float64) if (with_abs_sum and want_grad_probs) else None
    _load().oracle_router_weight_mul_bwd(_p(grad_out, ctypes.c_uint16), _p(x, ctypes.c_uint16),
                                         _p(probs, ctypes.c_float), _p(grad_x, ctypes.c_uint16),
                                         _p(grad_probs, ctypes.c_float), _p(abs_sum, ctypes.c_double),
                                         rows, hidden, threads or default_threads())
    if with_abs_sum:
        return grad_x, grad_probs, abs_sum
    return grad_x, grad_probs


# ---- float16 / float32 storage --------------------------------------------

BF16, F16, F32 = 0, 1, 2
_NP = {BF16: np.uint16, F16: np.float16, F32: np.float32}


def _typed_lib():
    lib = _load()
    if not getattr(lib, "_typed_ready", False):
        vp = ctypes.c_void_p
        lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f32.restype = ctypes.c_float
        lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_swiglu_clamped_fwd_typed.argtypes = [vp, ctypes.c_int, _f32p, vp, _i64, _i64, ctypes.c_float,
                                                        ctypes.c_int]
        lib.oracle_swiglu_clamped_bwd_typed.argtypes = [vp, ctypes.c_int, _f32p, vp, vp, _f32p, _f64p, _i64, _i64,
                                                        ctypes.c_float, ctypes.c_int]
        lib.oracle_router_weight_mul_fwd_typed.argtypes = [vp, ctypes.c_int, _f32p, vp, ctypes.c_int, _i64, _i64,
                                                           ctypes.c_int]
        lib.oracle_router_weight_mul_bwd_typed.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, _f32p, vp, _f32p,
                                                           _f64p, _i64, _i64, ctypes.c_int]
        for n in ("oracle_swiglu_clamped_fwd_typed", "oracle_swiglu_clamped_bwd_typed",
                  "oracle_router_weight_mul_fwd_typed", "oracle_router_weight_mul_bwd_typed"):
            getattr(lib, n).restype = None
        lib._typed_ready = True
    return lib


def f16_to_f32(h: int) -> float:
    return float(_typed_lib().oracle_f16_to_f32(int(h)))


def f32_to_f16(f: float) -> int:
    return int(_typed_lib().oracle_f32_to_f16(float(f)))


def _vp(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def swiglu_clamped_fwd_typed(x, dtype, probs, rows, inter, L, threads=None):
    """y ([rows, inter], same dtype as x). bf16 arrays are uint16 bit patterns."""
    x = _arr(x, _NP[dtype], (rows, 2 * inter))
    probs = _arr(probs, np.float32, (rows,))
    y = np.empty((rows, inter), dtype=_NP[dtype])
    _typed_lib().oracle_swiglu_clamped_fwd_typed(_vp(x), dtype, _p(probs, ctypes.c_float), _vp(y), rows, inter,
                                                 float(L), threads or default_threads())
    return y


def swiglu_clamped_bwd_typed(x, dtype, probs, grad_y, rows, inter, L, want_grad_probs=True, threads=None,
                             with_abs_sum=False):
    """(grad_x, grad_probs or None[, abs_sum]) with grad_x of x's dtype."""
    x = _arr(x, _NP[dtype], (rows, 2 * inter))
    probs = _arr(probs, np.float32, (rows,))
    grad_y = _arr(grad_y, _NP[dtype], (rows, inter))
    grad_x = np.empty((rows, 2 * inter), dtype=_NP[dtype])
    grad_probs = np.empty((rows,), dtype=np.float32) if want_grad_probs else None
    abs_sum = np.empty((rows,), dtype=np.float64) if with_abs_sum else None
    _typed_lib().oracle_swiglu_clamped_bwd_typed(_vp(x), dtype, _p(probs, ctypes.c_float), _vp(grad_y), _vp(grad_x),
                                                 _p(grad_probs, ctypes.c_float), _p(abs_sum, ctypes.c_double),
                                                 rows, inter, float(L), threads or default_threads())
    if with_abs_sum:
        return grad_x, grad_probs, abs_sum
    return grad_x, grad_probs


def router_weight_mul_fwd_typed(x, x_dtype, probs, out_dtype, rows, hidden, threads=None):
    x = _arr(x, _NP[x_dtype], (rows, hidden))
    probs = _arr(probs, np.float32, (rows,))
    out = np.empty((rows, hidden), dtype=_NP[out_dtype])
    _typed_lib().oracle_router_weight_mul_fwd_typed(_vp(x), x_dtype, _p(probs, ctypes.c_float), _vp(out), out_dtype,
                                                    rows, hidden, threads or default_threads())
    return out


def router_weight_mul_bwd_typed(grad_out, go_dtype, x, x_dtype, probs, rows, hidden, want_grad_probs=True,
                                threads=None, with_abs_sum=False):
    """(grad_x of x_dtype, grad_probs or None[, abs_sum]); x may be None without grad_probs."""
    grad_out = _arr(grad_out, _NP[go_dtype], (rows, hidden))
    x = _arr(x, _NP[x_dtype], (rows, hidden)) if want_grad_probs else None
    probs = _arr(probs, np.float32, (rows,))
    grad_x = np.empty((rows, hidden), dtype=_NP[x_dtype])
    grad_probs = np.empty((rows,), dtype=np.float32) if want_grad_probs else None
    abs_sum = np.empty((rows,), dtype=np.float64) if (with_abs_sum and want_grad_probs) else None
    _typed_lib().oracle_router_weight_mul_bwd_typed(_vp(grad_out), go_dtype, _vp(x), x_dtype,
                                                    _p(probs, ctypes.c_float), _vp(grad_x),
                                                    _p(grad_probs, ctypes.c_float), _p(abs_sum, ctypes.c_double),
                                                    rows, hidden, threads or default_threads())
    if with_abs_sum:
        return grad_x, grad_probs, abs_sum
    return grad_x, grad_probs


# ---- gate_up grouped GEMM with the clamped SwiGLU epilogue ----------------

def _grouped_lib():
    lib = _load()
    if not getattr(lib, "_grouped_ready", False):
        vp = ctypes.c_void_p
        lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.oracle_grouped_gate_up.argtypes = [vp, vp, vp, vp, vp, vp, _i64, _i64, _i64, _i64, ctypes.c_int]
        lib.oracle_grouped_gate_up.restype = None
        lib.oracle_grouped_swiglu_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, _i64, _i64, _i64, _i64,
                                                  ctypes.c_float, ctypes.c_int]
        lib.oracle_grouped_swiglu_fwd.restype = None
        lib._grouped_ready = True
    return lib


def f64_to_bf16(v: float) -> int:
    return int(_grouped_lib().oracle_f64_to_bf16(float(v)))


def grouped_gate_up(a, w_gate, w_up, offs, tokens, hidden, inter, experts, with_abs_sum=False, threads=None):
    """Exact grouped sums [tokens, 2*inter] (float64; rows of no expert are NaN)[, sum |a*w|].
    a: [tokens, hidden] bf16 bits; w_gate, w_up: [experts, inter, hidden] bf16 bits; offs: int32 [experts]."""
    a = _arr(a, np.uint16, (tokens, hidden))
    w_gate = _arr(w_gate, np.uint16, (experts, inter, hidden))
    w_up = _arr(w_up, np.uint16, (experts, inter, hidden))
    offs = _arr(offs, np.int32, (experts,))
    s = np.full((tokens, 2 * inter), np.nan)
    s_abs = np.full((tokens, 2 * inter), np.nan) if with_abs_sum else None
    _grouped_lib().oracle_grouped_gate_up(_vp(a), _vp(w_gate), _vp(w_up), _vp(offs), _vp(s), _vp(s_abs), tokens,
                                          hidden, inter, experts, threads or default_threads())
    return (s, s_abs) if with_abs_sum else s


def grouped_swiglu_fwd(a, w_gate, w_up, offs, probs, tokens, hidden, inter, experts, L, y_init=None,
                       x_init=None, threads=None):
    """(y [tokens, inter], x [tokens, 2*inter]) as bf16 bits. Rows of no expert keep y_init / x_init
    (default 0xFFFF, a NaN pattern no computed value takes)."""
    a = _arr(a, np.uint16, (tokens, hidden))
    w_gate = _arr(w_gate, np.uint16, (experts, inter, hidden))
    w_up = _arr(w_up, np.uint16, (experts, inter, hidden))
    offs = _arr(offs, np.int32, (experts,))
    probs = _arr(probs, np.float32, (tokens,))
    y = np.array(y_init, dtype=np.uint16) if y_init is not None else np.full((tokens, inter), 0xFFFF, np.uint16)
    x = np.array(x_init, dtype=np.uint16) if x_init is not None else np.full((tokens, 2 * inter), 0xFFFF,
                                                                            np.uint16)
    scratch = np.empty((tokens, 2 * inter), dtype=np.float64)
    _grouped_lib().oracle_grouped_swiglu_fwd(_vp(a), _vp(w_gate), _vp(w_up), _vp(offs), _vp(probs), _vp(y), _vp(x),
                                             _vp(scratch), tokens, hidden, inter, experts, float(L),
                                             threads or default_threads())
    return y, x


# ---- down projection with the router-weight multiply, and the combine -------

def _next3_lib():
    lib = _grouped_lib()
    if not getattr(lib, "_next3_ready", False):
        vp = ctypes.c_void_p
        lib.oracle_grouped_down_router_fwd.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, _i64, _i64, _i64, _i64,
                                                       ctypes.c_int]
        lib.oracle_grouped_down_router_fwd.restype = None
        lib.oracle_moe_combine.argtypes = [vp, ctypes.c_int, vp, vp, _i64, _i64, _i64, _i64, ctypes.c_int]
        lib.oracle_moe_combine.restype = None
        lib._next3_ready = True
    return lib


def grouped_down_router_fwd(h, w_down, offs, probs, tokens, inter, hidden, experts, out_dtype=BF16, out_init=None,
                            threads=None):
    """out [tokens, hidden] (bf16 bits or float32): round_out(fp32(bf16(h @ w_down[e]^T)) * p) per expert's
    rows; rows of no expert keep out_init (default: 0xFFFF bits / NaN)."""
    h = _arr(h, np.uint16, (tokens, inter))
    w_down = _arr(w_down, np.uint16, (experts, hidden, inter))
    offs = _arr(offs, np.int32, (experts,))
    probs = _arr(probs, np.float32, (tokens,))
    if out_init is not None:
        out = np.array(out_init, dtype=_NP[out_dtype])
    elif out_dtype == BF16:
        out = np.full((tokens, hidden), 0xFFFF, np.uint16)
    else:
        out = np.full((tokens, hidden), np.nan, np.float32)
    _next3_lib().oracle_grouped_down_router_fwd(_vp(h), _vp(w_down), _vp(offs), _vp(probs), _vp(out), out_dtype,
                                                tokens, inter, hidden, experts, threads or default_threads())
    return out


def moe_combine(expert_out, eo_dtype, row_of, rows, tokens, top_k, hidden, threads=None):
    """float32 [tokens, hidden]: per token, the binary32 sum in ascending slot order of its rows of expert_out."""
    expert_out = _arr(expert_out, _NP[eo_dtype], (rows, hidden))
    row_of = _arr(row_of, np.int32, (tokens, top_k))
    out = np.empty((tokens, hidden), np.float32)
    _next3_lib().oracle_moe_combine(_vp(expert_out), eo_dtype, _vp(row_of), _vp(out), rows, tokens, top_k, hidden,
                                    threads or default_threads())
    return out
