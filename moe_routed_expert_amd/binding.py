"""Python binding of libmoe_epi (ctypes; argument marshalling only).

Every step of the computation runs in the library's HIP kernels. This module
only checks that torch tensors have the dtypes, devices, shapes and
contiguity the C ABI expects, passes their device pointers and the current
HIP stream, and turns a nonzero status into an exception. PyTorch supplies
device memory and streams. There is no fallback: if libmoe_epi.so is missing
or fails to load, every call raises.

Names follow the C ABI (include/moe_epi.h):
  swiglu_clamped_fwd(x, probs, y, limit)
  swiglu_clamped_bwd(x, probs, grad_y, grad_x, grad_probs, limit)
  router_weight_mul_fwd(x, probs, out)
  router_weight_mul_bwd(grad_out, x, probs, grad_x, grad_probs)
  grouped_gate_up_swiglu_fwd(a, w_gate, w_up, offs, probs, y, x_out, limit)
  grouped_down_router_fwd(h, w_down, offs, probs, out)
  moe_combine_fwd(expert_out, row_of, out)
plus allocating helpers and torch.autograd.Function wrappers with the shapes
of the pages' SwigluClamped / _RouterWeightMulFunction.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_epi.so")

STATUS = {
    0: "MOE_EPI_SUCCESS",
    1: "MOE_EPI_ERR_NULL_POINTER",
    2: "MOE_EPI_ERR_BAD_SHAPE",
    3: "MOE_EPI_ERR_BAD_LIMIT",
    4: "MOE_EPI_ERR_ALIAS",
    5: "MOE_EPI_ERR_LAUNCH",
    6: "MOE_EPI_ERR_MISALIGNED",
    7: "MOE_EPI_ERR_BAD_DTYPE",
}

# moe_epi_dtype codes of the *_typed entry points
DTYPE_CODE = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}

_lib = None


class MoeEpiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({describe(status)})")


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m moe_routed_expert_amd.build` "
                          "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    L.swiglu_clamped_fwd.argtypes = [vp, vp, vp, i64, i64, f32, vp]
    L.swiglu_clamped_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, vp]
    L.router_weight_mul_fwd.argtypes = [vp, vp, vp, i64, i64, vp]
    L.router_weight_mul_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, vp]
    i32 = ctypes.c_int
    L.swiglu_clamped_fwd_typed.argtypes = [vp, vp, vp, i64, i64, f32, i32, vp]
    L.swiglu_clamped_bwd_typed.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, vp]
    L.router_weight_mul_fwd_typed.argtypes = [vp, i32, vp, vp, i32, i64, i64, vp]
    L.router_weight_mul_bwd_typed.argtypes = [vp, i32, vp, i32, vp, vp, vp, i64, i64, vp]
    L.grouped_gate_up_swiglu_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, vp]
    L.grouped_down_router_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, vp]
    L.moe_combine_fwd.argtypes = [vp, i32, vp, vp, i64, i64, i64, i64, vp]
    for name in ("swiglu_clamped_fwd", "swiglu_clamped_bwd", "router_weight_mul_fwd", "router_weight_mul_bwd",
                 "swiglu_clamped_fwd_typed", "swiglu_clamped_bwd_typed", "router_weight_mul_fwd_typed",
                 "router_weight_mul_bwd_typed", "grouped_gate_up_swiglu_fwd", "grouped_down_router_fwd",
                 "moe_combine_fwd"):
        getattr(L, name).restype = ctypes.c_int
    L.moe_epi_status_string.argtypes = [ctypes.c_int]
    L.moe_epi_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def describe(status: int) -> str:
    return lib().moe_epi_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise MoeEpiError(status, where)


def _stream_handle(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor | None, name: str, dtype, shape, device) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name}: expected a tensor on {device}, got {t.device}")
    if tuple(t.shape) not in [tuple(s) for s in shape]:
        raise ValueError(f"{name}: expected shape {' or '.join(str(tuple(s)) for s in shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _code(t: torch.Tensor, name: str) -> int:
    if t.dtype not in DTYPE_CODE:
        raise TypeError(f"{name}: expected bfloat16, float16 or float32, got {t.dtype}")
    return DTYPE_CODE[t.dtype]


def _rows_cols(x: torch.Tensor, name: str):
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got {tuple(x.shape)}")
    return int(x.shape[0]), int(x.shape[1])


# ---- C-ABI entry points -----------------------------------------------------

def swiglu_clamped_fwd(x, probs, y, limit: float, stream=None) -> None:
    """y[:] = silu(min(gate, L)) * clamp(up, -L, L) * probs, rounded to x's dtype;
    x = [gate | up] [rows, 2*inter] (bf16, fp16 or fp32); probs fp32 [rows] or
    [rows, 1]; y [rows, inter] of x's dtype."""
    rows, two_i = _rows_cols(x, "x")
    if two_i % 2:
        raise ValueError("x must have an even number of columns ([gate | up])")
    inter, dev, code = two_i // 2, x.device, _code(x, "x")
    _need(x, "x", x.dtype, [(rows, two_i)], dev)
    _need(probs, "probs", torch.float32, [(rows,), (rows, 1)], dev)
    _need(y, "y", x.dtype, [(rows, inter)], dev)
    st = _stream_handle(x, stream)
    if code == 0:
        status = lib().swiglu_clamped_fwd(_ptr(x), _ptr(probs), _ptr(y), rows, inter, float(limit), st)
    else:
        status = lib().swiglu_clamped_fwd_typed(_ptr(x), _ptr(probs), _ptr(y), rows, inter, float(limit), code, st)
    _check(status, "swiglu_clamped_fwd")


def swiglu_clamped_bwd(x, probs, grad_y, grad_x, grad_probs, limit: float, stream=None) -> None:
    """grad_x[:, :inter] = d_gate, grad_x[:, inter:] = d_up (x's dtype), grad_probs[:] =
    per-row probability gradient (fp32; skipped when grad_probs is None)."""
    rows, two_i = _rows_cols(x, "x")
    if two_i % 2:
        raise ValueError("x must have an even number of columns ([gate | up])")
    inter, dev, code = two_i // 2, x.device, _code(x, "x")
    _need(x, "x", x.dtype, [(rows, two_i)], dev)
    _need(probs, "probs", torch.float32, [(rows,), (rows, 1)], dev)
    _need(grad_y, "grad_y", x.dtype, [(rows, inter)], dev)
    _need(grad_x, "grad_x", x.dtype, [(rows, two_i)], dev)
    if grad_probs is not None:
        _need(grad_probs, "grad_probs", torch.float32, [(rows,), (rows, 1)], dev)
    st = _stream_handle(x, stream)
    if code == 0:
        status = lib().swiglu_clamped_bwd(_ptr(x), _ptr(probs), _ptr(grad_y), _ptr(grad_x), _ptr(grad_probs), rows,
                                          inter, float(limit), st)
    else:
        status = lib().swiglu_clamped_bwd_typed(_ptr(x), _ptr(probs), _ptr(grad_y), _ptr(grad_x), _ptr(grad_probs),
                                                rows, inter, float(limit), code, st)
    _check(status, "swiglu_clamped_bwd")


def router_weight_mul_fwd(x, probs, out, stream=None) -> None:
    """out[:] = fp32(x) * probs rounded to out's dtype; x [rows, hidden] (bf16, fp16
    or fp32), out of x's dtype or fp32; probs fp32 [rows] or [rows, 1]."""
    rows, hidden = _rows_cols(x, "x")
    dev, xc = x.device, _code(x, "x")
    _need(x, "x", x.dtype, [(rows, hidden)], dev)
    _need(probs, "probs", torch.float32, [(rows,), (rows, 1)], dev)
    _need(out, "out", out.dtype, [(rows, hidden)], dev)
    oc = _code(out, "out")
    st = _stream_handle(x, stream)
    if xc == 0 and oc == 0:
        status = lib().router_weight_mul_fwd(_ptr(x), _ptr(probs), _ptr(out), rows, hidden, st)
    else:
        status = lib().router_weight_mul_fwd_typed(_ptr(x), xc, _ptr(probs), _ptr(out), oc, rows, hidden, st)
    _check(status, "router_weight_mul_fwd")


def router_weight_mul_bwd(grad_out, x, probs, grad_x, grad_probs, stream=None) -> None:
    """grad_x[:] = fp32(grad_out) * probs rounded to grad_x's dtype (x's dtype);
    grad_probs[:] = sum_k grad_out * x (fp32). grad_out has the output's dtype.
    x and grad_probs may both be None (probabilities without gradient)."""
    rows, hidden = _rows_cols(grad_out, "grad_out")
    dev = grad_out.device
    _need(grad_out, "grad_out", grad_out.dtype, [(rows, hidden)], dev)
    _need(grad_x, "grad_x", grad_x.dtype, [(rows, hidden)], dev)
    xc, oc = _code(grad_x, "grad_x"), _code(grad_out, "grad_out")
    if grad_probs is not None:
        _need(x, "x", grad_x.dtype, [(rows, hidden)], dev)
        _need(grad_probs, "grad_probs", torch.float32, [(rows,), (rows, 1)], dev)
    _need(probs, "probs", torch.float32, [(rows,), (rows, 1)], dev)
    xp = _ptr(x) if grad_probs is not None else None
    st = _stream_handle(grad_out, stream)
    if xc == 0 and oc == 0:
        status = lib().router_weight_mul_bwd(_ptr(grad_out), xp, _ptr(probs), _ptr(grad_x), _ptr(grad_probs), rows,
                                             hidden, st)
    else:
        status = lib().router_weight_mul_bwd_typed(_ptr(grad_out), oc, xp, xc, _ptr(probs), _ptr(grad_x),
                                                   _ptr(grad_probs), rows, hidden, st)
    _check(status, "router_weight_mul_bwd")


def grouped_gate_up_swiglu_fwd(a, w_gate, w_up, offs, probs, y, x_out, limit: float, stream=None) -> None:
    """Fused gate_up grouped GEMM + clamped SwiGLU x probs. a [tokens, hidden] bf16 (rows grouped by
    expert); w_gate, w_up [experts, inter, hidden] bf16; offs int32 [experts] cumulative token counts
    (on the device); probs fp32 [tokens] or [tokens, 1]; y [tokens, inter] bf16; x_out None or
    [tokens, 2*inter] bf16 (gate | up, the backward's input)."""
    tokens, hidden = _rows_cols(a, "a")
    if w_gate.dim() != 3:
        raise ValueError(f"w_gate must be 3-D [experts, inter, hidden], got {tuple(w_gate.shape)}")
    experts, inter = int(w_gate.shape[0]), int(w_gate.shape[1])
    dev = a.device
    _need(a, "a", torch.bfloat16, [(tokens, hidden)], dev)
    _need(w_gate, "w_gate", torch.bfloat16, [(experts, inter, hidden)], dev)
    _need(w_up, "w_up", torch.bfloat16, [(experts, inter, hidden)], dev)
    _need(offs, "offs", torch.int32, [(experts,)], dev)
    _need(probs, "probs", torch.float32, [(tokens,), (tokens, 1)], dev)
    _need(y, "y", torch.bfloat16, [(tokens, inter)], dev)
    if x_out is not None:
        _need(x_out, "x_out", torch.bfloat16, [(tokens, 2 * inter)], dev)
    st = _stream_handle(a, stream)
    status = lib().grouped_gate_up_swiglu_fwd(a.data_ptr(), w_gate.data_ptr(), w_up.data_ptr(), offs.data_ptr(),
                                              probs.data_ptr(), y.data_ptr(), _ptr(x_out), tokens, hidden, inter,
                                              experts, float(limit), st)
    _check(status, "grouped_gate_up_swiglu_fwd")


def grouped_down_router_fwd(h, w_down, offs, probs, out, stream=None) -> None:
    """Fused down-projection grouped GEMM + router-weight multiply. h [tokens, inter] bf16 (rows grouped
    by expert); w_down [experts, hidden, inter] bf16; offs int32 [experts] cumulative token counts (on the
    device); probs fp32 [tokens] or [tokens, 1]; out [tokens, hidden] bf16 or fp32:
    out = out.dtype(fp32(bf16(h @ w_down[e]^T)) * probs)."""
    tokens, inter = _rows_cols(h, "h")
    if w_down.dim() != 3:
        raise ValueError(f"w_down must be 3-D [experts, hidden, inter], got {tuple(w_down.shape)}")
    experts, hidden = int(w_down.shape[0]), int(w_down.shape[1])
    dev = h.device
    _need(h, "h", torch.bfloat16, [(tokens, inter)], dev)
    _need(w_down, "w_down", torch.bfloat16, [(experts, hidden, inter)], dev)
    _need(offs, "offs", torch.int32, [(experts,)], dev)
    _need(probs, "probs", torch.float32, [(tokens,), (tokens, 1)], dev)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"out: expected bfloat16 or float32, got {out.dtype}")
    _need(out, "out", out.dtype, [(tokens, hidden)], dev)
    st = _stream_handle(h, stream)
    status = lib().grouped_down_router_fwd(h.data_ptr(), w_down.data_ptr(), offs.data_ptr(), probs.data_ptr(),
                                           out.data_ptr(), DTYPE_CODE[out.dtype], tokens, inter, hidden, experts,
                                           st)
    _check(status, "grouped_down_router_fwd")


def moe_combine_fwd(expert_out, row_of, out, stream=None) -> None:
    """out[t] = fp32 sum, in ascending slot order from +0, of expert_out[row_of[t, j]] over the slots j
    whose row is in [0, rows). expert_out [rows, hidden] bf16, fp16 or fp32; row_of int32 [tokens, top_k];
    out fp32 [tokens, hidden]."""
    rows, hidden = _rows_cols(expert_out, "expert_out")
    tokens, top_k = _rows_cols(row_of, "row_of")
    dev = out.device
    _need(expert_out, "expert_out", expert_out.dtype, [(rows, hidden)], dev)
    _need(row_of, "row_of", torch.int32, [(tokens, top_k)], dev)
    _need(out, "out", torch.float32, [(tokens, hidden)], dev)
    st = _stream_handle(out, stream)
    status = lib().moe_combine_fwd(_ptr(expert_out) if rows else None, _code(expert_out, "expert_out"),
                                   row_of.data_ptr(), out.data_ptr(), rows, tokens, top_k, hidden, st)
    _check(status, "moe_combine_fwd")


# ---- allocating helpers and autograd wrappers ------------------------------

def swiglu_clamped(x, probs, limit: float):
    y = torch.empty((x.shape[0], x.shape[1] // 2), dtype=x.dtype, device=x.device)
    swiglu_clamped_fwd(x, probs, y, limit)
    return y


def router_weight_mul(x, probs, out_dtype=None):
    out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    router_weight_mul_fwd(x, probs, out)
    return out


class SwigluClamped(torch.autograd.Function):
    """silu(clamp(gate, max=L)) * clamp(up, -L, L) * probs with the HIP forward and
    single-pass backward; saves only x and probs."""

    @staticmethod
    def forward(ctx, x, probs, limit: float):
        x = x.contiguous()
        probs = probs.contiguous()
        ctx.save_for_backward(x, probs)
        ctx.limit = float(limit)
        return swiglu_clamped(x, probs, limit)

    @staticmethod
    def backward(ctx, grad_y):
        x, probs = ctx.saved_tensors
        grad_x = torch.empty_like(x)
        grad_probs = torch.empty_like(probs) if ctx.needs_input_grad[1] else None
        swiglu_clamped_bwd(x, probs, grad_y.contiguous(), grad_x, grad_probs, ctx.limit)
        return grad_x, grad_probs, None


class RouterWeightMul(torch.autograd.Function):
    """fp32(x) * probs rounded to out_dtype (default: x's dtype; float32 for a
    scatter-add combine) with the HIP forward and a one-pass backward. x is
    saved only when probs needs a gradient (it is read only for that gradient)."""

    @staticmethod
    def forward(ctx, x, probs, out_dtype=None):
        x = x.contiguous()
        probs = probs.contiguous()
        save_x = probs.requires_grad
        ctx.save_for_backward(x if save_x else None, probs)
        ctx.save_x = save_x
        ctx.x_dtype = x.dtype
        return router_weight_mul(x, probs, out_dtype)

    @staticmethod
    def backward(ctx, grad_out):
        x, probs = ctx.saved_tensors
        grad_out = grad_out.contiguous()
        grad_x = torch.empty(grad_out.shape, dtype=ctx.x_dtype, device=grad_out.device)
        grad_probs = torch.empty_like(probs) if ctx.save_x else None
        router_weight_mul_bwd(grad_out, x, probs, grad_x, grad_probs)
        return grad_x, grad_probs, None
