"""C-ABI checks that need no GPU: the library loads, exports every function
include/moe_epi.h declares, and rejects bad arguments on the host before any
HIP call. Every call here is built to fail validation (or to have rows == 0),
so nothing is ever launched."""
import ctypes
import glob
import os
import re

import pytest
import torch

from moe_routed_expert_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Host-only checks: where a GPU is visible they are not needed (and a mistaken
# case that passed validation would launch on fake addresses), so skip there.
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="host-only checks; a GPU is visible")

OK, NULLP, SHAPE, LIMIT, ALIAS, LAUNCH, MISAL, DTYPE = range(8)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        from moe_routed_expert_amd import build
        build.build()
    return binding.lib()


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;]*\)\s*;", text, flags=re.M)
    return names


def test_header_declares_the_four_ops_and_status_string():
    assert set(declared_functions()) >= {"swiglu_clamped_fwd", "swiglu_clamped_bwd", "router_weight_mul_fwd",
                                         "router_weight_mul_bwd", "moe_epi_status_string"}


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for code in range(8):
        s = binding.describe(code)
        assert s and s != "unknown status"
    assert binding.describe(99) == "unknown status"
    assert binding.describe(0) == "success"


# The status codes as the boundary specifies them: the first six in the order
# of the specification (MOE_EPI_ERR_LAUNCH = 5), the two this library adds
# appended after them, so a caller written to the first six reads every code
# the same way.
SPEC_STATUS = {
    "MOE_EPI_SUCCESS": 0,
    "MOE_EPI_ERR_NULL_POINTER": 1,
    "MOE_EPI_ERR_BAD_SHAPE": 2,
    "MOE_EPI_ERR_BAD_LIMIT": 3,
    "MOE_EPI_ERR_ALIAS": 4,
    "MOE_EPI_ERR_LAUNCH": 5,
    "MOE_EPI_ERR_MISALIGNED": 6,
    "MOE_EPI_ERR_BAD_DTYPE": 7,
}


def test_status_code_values_pinned(L):
    text = open(os.path.join(ROOT, "include", "moe_epi.h")).read()
    body = re.search(r"typedef enum moe_epi_status \{(.*?)\} moe_epi_status;", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    header = {m.group(1): int(m.group(2)) for m in re.finditer(r"(MOE_EPI_\w+)\s*=\s*(\d+)", body)}
    assert header == SPEC_STATUS
    assert binding.STATUS == {v: k for k, v in SPEC_STATUS.items()}
    # the library's own strings say what each code means
    assert "launch" in binding.describe(5)
    assert "aligned" in binding.describe(6)
    assert "dtype" in binding.describe(7)
    assert "NULL" in binding.describe(1) or "null" in binding.describe(1)


# fake, never dereferenced device addresses (validation fails before any use)
A = 0x10_0000_0000
B = 0x20_0000_0000
C = 0x30_0000_0000
D = 0x40_0000_0000
E = 0x50_0000_0000


def sw_fwd(L, x, p, y, rows=4, inter=8, lim=7.0):
    return L.swiglu_clamped_fwd(x, p, y, rows, inter, lim, None)


def sw_bwd(L, x, p, gy, gx, gp, rows=4, inter=8, lim=7.0):
    return L.swiglu_clamped_bwd(x, p, gy, gx, gp, rows, inter, lim, None)


def test_swiglu_fwd_validation(L):
    assert sw_fwd(L, None, B, C) == NULLP
    assert sw_fwd(L, A, None, C) == NULLP
    assert sw_fwd(L, A, B, None) == NULLP
    assert sw_fwd(L, A, B, C, rows=-1) == SHAPE
    assert sw_fwd(L, A, B, C, inter=0) == SHAPE
    assert sw_fwd(L, A, B, C, inter=-3) == SHAPE
    assert sw_fwd(L, A, B, C, rows=1 << 40, inter=1 << 40) == SHAPE
    for bad in (0.0, -1.0, float("inf"), float("nan"), -0.0):
        assert sw_fwd(L, A, B, C, lim=bad) == LIMIT
    assert sw_fwd(L, A + 1, B, C) == MISAL
    assert sw_fwd(L, A, B + 2, C) == MISAL
    assert sw_fwd(L, A, B, C + 1) == MISAL
    # x is 4 x 16 bf16 = 128 bytes: y inside it, or probs inside y, is aliasing
    assert sw_fwd(L, A, B, A + 64) == ALIAS
    assert sw_fwd(L, A, B, A + 126) == ALIAS
    assert sw_fwd(L, A, C + 16, C) == ALIAS
    # rows == 0 launches nothing and accepts NULL buffers
    assert sw_fwd(L, None, None, None, rows=0) == OK
    assert sw_fwd(L, None, None, None, rows=0, lim=0.0) == LIMIT


def test_swiglu_bwd_validation(L):
    assert sw_bwd(L, None, B, C, D, E) == NULLP
    assert sw_bwd(L, A, B, None, D, E) == NULLP
    assert sw_bwd(L, A, B, C, None, E) == NULLP
    assert sw_bwd(L, A, B, C, D, E, inter=0) == SHAPE
    assert sw_bwd(L, A, B, C, D, E, lim=float("nan")) == LIMIT
    assert sw_bwd(L, A, B, C, D + 1, E) == MISAL
    assert sw_bwd(L, A, B, C, D, E + 2) == MISAL
    assert sw_bwd(L, A, B, C, A + 2, E) == ALIAS       # grad_x over x
    assert sw_bwd(L, A, B, C, C, E) == ALIAS           # grad_x over grad_y
    assert sw_bwd(L, A, B, C, D, D + 64) == ALIAS      # grad_probs inside grad_x
    assert sw_bwd(L, A, B, C, D, B) == ALIAS           # grad_probs over probs
    assert sw_bwd(L, None, None, None, None, None, rows=0) == OK


def test_router_validation(L):
    f = lambda x, p, o, rows=4, h=8: L.router_weight_mul_fwd(x, p, o, rows, h, None)
    b = lambda go, x, p, gx, gp, rows=4, h=8: L.router_weight_mul_bwd(go, x, p, gx, gp, rows, h, None)
    assert f(None, B, C) == NULLP
    assert f(A, B, C, rows=-2) == SHAPE
    assert f(A, B, C, h=0) == SHAPE
    assert f(A + 1, B, C) == MISAL
    assert f(A, B, A + 8) == ALIAS
    assert f(None, None, None, rows=0) == OK
    assert b(A, None, C, D, E) == NULLP                # grad_probs wanted but no x
    assert b(None, B, C, D, None) == NULLP
    assert b(A, B, C, D, E, h=-1) == SHAPE
    assert b(A, B, C, D + 1, E) == MISAL
    assert b(A, B, C, A + 16, E) == ALIAS              # grad_x over grad_out
    assert b(A, B, C, D, D) == ALIAS                   # grad_probs over grad_x
    assert b(A, B, C, D + 3, None) == MISAL            # odd grad_x address
    assert b(None, None, None, None, None, rows=0) == OK


def test_typed_validation(L):
    sf = lambda x, p, y, dt, rows=4, inter=8: L.swiglu_clamped_fwd_typed(x, p, y, rows, inter, 7.0, dt, None)
    sb = lambda dt: L.swiglu_clamped_bwd_typed(A, B, C, D, E, 4, 8, 7.0, dt, None)
    rf = lambda xd, od: L.router_weight_mul_fwd_typed(A, xd, B, C, od, 4, 8, None)
    rb = lambda od, xd: L.router_weight_mul_bwd_typed(A, od, B, xd, C, D, E, 4, 8, None)
    for bad in (-1, 3, 99):
        assert sf(A, B, C, bad) == DTYPE
        assert sb(bad) == DTYPE
        assert rf(bad, 0) == DTYPE and rf(0, bad) == DTYPE
        assert rb(bad, 0) == DTYPE and rb(0, bad) == DTYPE
    # the output is x's dtype or float32: other pairs are rejected
    for xd, od in ((2, 0), (2, 1), (0, 1), (1, 0)):
        assert rf(xd, od) == DTYPE and rb(od, xd) == DTYPE
    # float32 elements need 4-byte alignment
    assert sf(A + 2, B, C, 2) == MISAL
    assert sf(A, B, C + 2, 2) == MISAL
    # float32 byte sizes double: y at 64 bytes into a 4 x 16 float32 x (256 bytes) overlaps
    assert sf(A, B, A + 192, 2) == ALIAS
    assert sf(None, None, None, 2, rows=0) == OK


def test_binding_rejects_cpu_tensors_before_the_library():
    x = torch.zeros(4, 16, dtype=torch.bfloat16)
    p = torch.zeros(4, dtype=torch.float32)
    y = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.swiglu_clamped_fwd(x, p, y, 7.0)
    with pytest.raises(TypeError):
        binding.swiglu_clamped_fwd(x.double(), p, y, 7.0)
    with pytest.raises(ValueError):
        binding.router_weight_mul_fwd(x[:, :7], p, y[:, :7])


# ---- grouped gate_up GEMM + epilogue ------------------------------------------

F = 0x60_0000_0000
G = 0x70_0000_0000


def gr(L, a=A, wg=B, wu=C, offs=D, p=E, y=F, x=G, tokens=256, hidden=64, inter=32, experts=4, lim=7.0):
    return L.grouped_gate_up_swiglu_fwd(a, wg, wu, offs, p, y, x, tokens, hidden, inter, experts, lim, None)


def test_grouped_validation(L):
    for kw in ({"a": None}, {"wg": None}, {"wu": None}, {"offs": None}, {"p": None}, {"y": None}):
        assert gr(L, **kw) == NULLP, kw
    for kw in ({"tokens": -1}, {"hidden": 0}, {"inter": 0}, {"experts": 0}, {"hidden": 60}, {"inter": 36},
               {"tokens": 2 ** 31}, {"experts": 2 ** 62, "inter": 8}):
        assert gr(L, **kw) == SHAPE, kw
    for lim in (0.0, -1.0, float("inf"), float("nan")):
        assert gr(L, lim=lim) == LIMIT
    assert gr(L, tokens=0) == OK                       # nothing to do, nothing launched
    assert gr(L, tokens=0, a=None) == OK               # pointers are not needed for an empty call
    for kw in ({"a": A + 2}, {"wg": B + 8}, {"wu": C + 4}, {"y": F + 2}, {"x": G + 8}, {"offs": D + 2},
               {"p": E + 1}):
        assert gr(L, **kw) == MISAL, kw
    assert gr(L, y=A) == ALIAS                         # y on top of a
    assert gr(L, x=B) == ALIAS                         # x_out on top of w_gate
    assert gr(L, x=F + 16) == ALIAS                    # x_out overlapping y
    assert gr(L, y=D) == ALIAS                         # y on top of offs


def test_grouped_binding_rejects_bad_tensors():
    a = torch.zeros(16, 64, dtype=torch.bfloat16)
    w = torch.zeros(2, 32, 64, dtype=torch.bfloat16)
    offs = torch.tensor([8, 16], dtype=torch.int32)
    p = torch.zeros(16)
    y = torch.zeros(16, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):                    # CPU tensors
        binding.grouped_gate_up_swiglu_fwd(a, w, w, offs, p, y, None, 7.0)
    with pytest.raises(ValueError):                    # 2-D weights
        binding.grouped_gate_up_swiglu_fwd(a, w[0], w[0], offs, p, y, None, 7.0)


# ---- down projection + router multiply, and the combine ----------------------------

def dn(L, h=A, w=B, offs=D, p=E, out=F, odt=0, tokens=256, inter=64, hidden=32, experts=4):
    return L.grouped_down_router_fwd(h, w, offs, p, out, odt, tokens, inter, hidden, experts, None)


def test_down_validation(L):
    for kw in ({"h": None}, {"w": None}, {"offs": None}, {"p": None}, {"out": None}):
        assert dn(L, **kw) == NULLP, kw
    for kw in ({"tokens": -1}, {"inter": 0}, {"hidden": 0}, {"experts": 0}, {"inter": 60}, {"hidden": 36},
               {"tokens": 2 ** 31}, {"experts": 2 ** 62, "hidden": 8}):
        assert dn(L, **kw) == SHAPE, kw
    for odt in (1, 3, -1):                             # float16 output is not offered
        assert dn(L, odt=odt) == DTYPE, odt
    assert dn(L, tokens=0) == OK and dn(L, tokens=0, h=None) == OK
    for kw in ({"h": A + 2}, {"w": B + 8}, {"out": F + 4}, {"offs": D + 2}, {"p": E + 1}):
        assert dn(L, **kw) == MISAL, kw
    for kw in ({"out": A}, {"out": B}, {"out": D}, {"out": E - 16}):
        assert dn(L, **kw) == ALIAS, kw
    assert dn(L, out=E - 16, odt=2) == ALIAS           # fp32 output: twice the bytes


def cb(L, eo=A, edt=2, ro=B, out=C, rows=100, tokens=64, top_k=8, hidden=16):
    return L.moe_combine_fwd(eo, edt, ro, out, rows, tokens, top_k, hidden, None)


def test_combine_validation(L):
    for kw in ({"eo": None}, {"ro": None}, {"out": None}):
        assert cb(L, **kw) == NULLP, kw
    for kw in ({"rows": -1}, {"tokens": -1}, {"top_k": 0}, {"top_k": 1025}, {"hidden": 0}, {"hidden": 12},
               {"hidden": 2 ** 29}, {"tokens": 2 ** 60, "top_k": 8}):
        assert cb(L, **kw) == SHAPE, kw
    for edt in (3, -1):
        assert cb(L, edt=edt) == DTYPE, edt
    assert cb(L, tokens=0) == OK
    for kw in ({"eo": A + 8}, {"out": C + 4}, {"ro": B + 2}):
        assert cb(L, **kw) == MISAL, kw
    for kw in ({"out": A}, {"out": B}, {"out": A + 100 * 16 * 4 - 16}):
        assert cb(L, **kw) == ALIAS, kw


def test_down_and_combine_bindings_reject_cpu_tensors():
    h = torch.zeros(16, 64, dtype=torch.bfloat16)
    w = torch.zeros(2, 32, 64, dtype=torch.bfloat16)
    offs = torch.tensor([8, 16], dtype=torch.int32)
    p = torch.zeros(16)
    out = torch.zeros(16, 32, dtype=torch.float32)
    with pytest.raises(ValueError):
        binding.grouped_down_router_fwd(h, w, offs, p, out)
    eo = torch.zeros(10, 32)
    ro = torch.zeros(16, 4, dtype=torch.int32)
    with pytest.raises(ValueError):
        binding.moe_combine_fwd(eo, ro, out)
