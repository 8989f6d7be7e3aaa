"""GPU parity of the float16 / float32 storage paths (the *_typed entry points)
and of the router multiply's float32 output, against the oracle's typed
functions. Bars: tests/gpu_util.py."""
import sys

import numpy as np
import pytest
import torch

import moe_routed_expert_amd as epi
import oracle
from moe_routed_expert_amd.workloads import WORKLOADS, custom
from tests.gpu_util import (assert_bf16_parity, assert_dprobs, assert_f16_parity, assert_f32_within,
                            f32_swiglu_bounds, to_dev_bf16, to_dev_f32, to_host_bits)

pytestmark = pytest.mark.gpu
CODE = {"bf16": oracle.BF16, "f16": oracle.F16, "f32": oracle.F32}
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def say(msg):
    print(f"\n[gpu-dtypes] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    epi.binding.lib()
    yield
    torch.cuda.synchronize()


def to_dev(a: np.ndarray, dt: str) -> torch.Tensor:
    if dt == "bf16":
        return to_dev_bf16(a)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def to_host(t: torch.Tensor, dt: str) -> np.ndarray:
    return to_host_bits(t) if dt == "bf16" else t.cpu().numpy()


def check_swiglu(d, rows, inter, L, dt, y, gx, gp, what):
    code = CODE[dt]
    y_o = oracle.swiglu_clamped_fwd_typed(d["x"], code, d["probs"], rows, inter, L)
    gx_o, gp_o, scale = oracle.swiglu_clamped_bwd_typed(d["x"], code, d["probs"], d["grad_out"], rows, inter, L,
                                                        with_abs_sum=True)
    if dt == "f16":
        s = [assert_f16_parity(y, y_o, f"{what} y"), assert_f16_parity(gx[:, :inter], gx_o[:, :inter], f"{what} d_gate"),
             assert_f16_parity(gx[:, inter:], gx_o[:, inter:], f"{what} d_up")]
    else:
        b_y, b_dg, b_du = f32_swiglu_bounds(d["x"], d["probs"], d["grad_out"], L)
        s = [assert_f32_within(y, y_o, b_y, f"{what} y"), assert_f32_within(gx[:, :inter], gx_o[:, :inter], b_dg,
                                                                             f"{what} d_gate"),
             assert_f32_within(gx[:, inter:], gx_o[:, inter:], b_du, f"{what} d_up")]
    p = assert_dprobs(gp, gp_o, scale, f"{what} d_probs") if gp is not None else {}
    say(f"{what}: {s} d_probs {p}")


def run_swiglu(d, rows, inter, L, dt, offset=0):
    def dev(a):
        if offset == 0:
            return to_dev(a, dt)
        flat = to_dev(a.ravel(), dt)
        buf = torch.zeros(flat.numel() + offset + 8, dtype=TORCH[dt], device="cuda")
        v = buf[offset:offset + flat.numel()]
        v.copy_(flat)
        return v.view(*a.shape)
    x, gy = dev(d["x"]), dev(d["grad_out"])
    p = to_dev_f32(d["probs"])
    y = dev(np.zeros((rows, inter), d["x"].dtype))
    gx = dev(np.zeros((rows, 2 * inter), d["x"].dtype))
    gp = torch.empty((rows,), dtype=torch.float32, device="cuda")
    gx2 = dev(np.zeros((rows, 2 * inter), d["x"].dtype))
    epi.swiglu_clamped_fwd(x, p, y, L)
    epi.swiglu_clamped_bwd(x, p, gy, gx, gp, L)
    epi.swiglu_clamped_bwd(x, p, gy, gx2, None, L)   # without the probability gradient (its own launch shapes)
    torch.cuda.synchronize()
    gx_h = to_host(gx, dt)
    assert np.array_equal(to_host(gx2, dt).view(np.uint8), gx_h.view(np.uint8)), "grad_x differs without grad_probs"
    return to_host(y, dt), gx_h, gp.cpu().numpy()


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_swiglu_8192x2048(dt):
    w = WORKLOADS["swiglu_8192x2048"]
    d = w.generate(dtype=dt)
    say(f"{w.name} {dt}")
    y, gx, gp = run_swiglu(d, w.rows, w.cols, w.limit, dt)
    check_swiglu(d, w.rows, w.cols, w.limit, dt, y, gx, gp, f"{w.name} {dt}")


@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("rows,inter,offset", [(37, 8, 0), (17, 136, 0), (9, 200, 0), (300, 1536, 0), (5, 2056, 0),
                                               (3, 8200, 0), (13, 24, 1), (7, 1544, 1), (2, 3, 0), (6, 1032, 0),
                                               (9, 2048, 0), (4, 4096, 0), (3, 6144, 0), (2, 16384, 0), (5, 512, 0),
                                               (21, 1792, 0), (6, 2040, 0)])
def test_swiglu_shapes(dt, rows, inter, offset):
    w = custom("swiglu", rows, inter, limit=7.0, x_sigma=5.0, seed=3000 + rows + inter,
               x_special_frac=0.1, x_special_values=(-7.0, 7.0, 0.0, 7.03125, -7.03125),
               probs_kind="uniform_zeros", probs_zero_frac=0.1)
    d = w.generate(dtype=dt)
    say(f"swiglu {dt} rows={rows} inter={inter} offset={offset} elements")
    y, gx, gp = run_swiglu(d, rows, inter, w.limit, dt, offset)
    check_swiglu(d, rows, inter, w.limit, dt, y, gx, gp, f"swiglu {dt} {rows}x{inter}+{offset}")


def test_f16_special_values():
    L = 7.0
    sp = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 7.0, -7.0, 7.00390625, -7.00390625, 65504.0, -65504.0,
                   6e-8, -6e-8, 1e-5, -30.0, -1.28125, 3.0], dtype=np.float16)
    rng = np.random.default_rng(7)
    rows, inter = 32, 136
    x = np.concatenate([rng.choice(sp, size=(rows, inter)), rng.choice(sp, size=(rows, inter))], axis=1)
    gy = rng.choice(np.array([0.0, -0.0, 1.0, -2.5, 1e-4], np.float16), size=(rows, inter))
    d = {"x": x, "grad_out": gy, "probs": rng.choice(np.array([0.0, 0.5, 1.0, 300.0], np.float32), size=rows)}
    say("f16 special values")
    y, gx, gp = run_swiglu(d, rows, inter, L, "f16")
    y_o = oracle.swiglu_clamped_fwd_typed(d["x"], oracle.F16, d["probs"], rows, inter, L)
    gx_o, gp_o = oracle.swiglu_clamped_bwd_typed(d["x"], oracle.F16, d["probs"], d["grad_out"], rows, inter, L)
    assert_f16_parity(y, y_o, "f16 special y")
    assert_f16_parity(gx, gx_o, "f16 special grad_x")
    assert np.array_equal(np.isnan(gp), np.isnan(gp_o))


def test_typed_bf16_calls_equal_the_bf16_calls():
    w = WORKLOADS["swiglu_8192x2048"]
    d = w.generate(rows=1024)
    x, gy, p = to_dev_bf16(d["x"]), to_dev_bf16(d["grad_out"]), to_dev_f32(d["probs"])
    L = epi.binding.lib()
    st = torch.cuda.current_stream().cuda_stream
    ya, yb = torch.empty((1024, w.cols), dtype=torch.bfloat16, device="cuda"), torch.empty((1024, w.cols),
                                                                                         dtype=torch.bfloat16,
                                                                                         device="cuda")
    ga, gb = torch.empty_like(x), torch.empty_like(x)
    pa, pb = torch.empty_like(p), torch.empty_like(p)
    assert L.swiglu_clamped_fwd(x.data_ptr(), p.data_ptr(), ya.data_ptr(), 1024, w.cols, w.limit, st) == 0
    assert L.swiglu_clamped_fwd_typed(x.data_ptr(), p.data_ptr(), yb.data_ptr(), 1024, w.cols, w.limit, 0, st) == 0
    assert L.swiglu_clamped_bwd(x.data_ptr(), p.data_ptr(), gy.data_ptr(), ga.data_ptr(), pa.data_ptr(), 1024,
                                w.cols, w.limit, st) == 0
    assert L.swiglu_clamped_bwd_typed(x.data_ptr(), p.data_ptr(), gy.data_ptr(), gb.data_ptr(), pb.data_ptr(), 1024,
                                      w.cols, w.limit, 0, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    assert torch.equal(ga.view(torch.int16), gb.view(torch.int16)) and torch.equal(pa, pb)


@pytest.mark.parametrize("xd,od", [("bf16", "f32"), ("f16", "f16"), ("f16", "f32"), ("f32", "f32")])
@pytest.mark.parametrize("rows,hidden", [(4096, 7168), (13, 8), (9, 1000), (31, 7176), (5, 16384), (3, 1536),
                                         (33, 2048), (5, 2056), (7, 4096), (9, 8192), (2, 1040), (4, 12288)])
def test_router_dtype_pairs(xd, od, rows, hidden):
    w = custom("router", rows, hidden, x_sigma=1.0, seed=4000 + rows + hidden)
    d = w.generate(dtype=xd, grad_dtype=od)
    say(f"router x={xd} out={od} rows={rows} hidden={hidden}")
    x, go, p = to_dev(d["x"], xd), to_dev(d["grad_out"], od), to_dev_f32(d["probs"])
    out = torch.empty((rows, hidden), dtype=TORCH[od], device="cuda")
    gx = torch.empty((rows, hidden), dtype=TORCH[xd], device="cuda")
    gx2 = torch.empty_like(gx)
    gp = torch.empty((rows,), dtype=torch.float32, device="cuda")
    epi.router_weight_mul_fwd(x, p, out)
    epi.router_weight_mul_bwd(go, x, p, gx, gp)
    epi.router_weight_mul_bwd(go, None, p, gx2, None)
    torch.cuda.synchronize()
    out_o = oracle.router_weight_mul_fwd_typed(d["x"], CODE[xd], d["probs"], CODE[od], rows, hidden)
    gx_o, gp_o, scale = oracle.router_weight_mul_bwd_typed(d["grad_out"], CODE[od], d["x"], CODE[xd], d["probs"],
                                                           rows, hidden, with_abs_sum=True)
    bits = lambda a, dt: a if dt == "bf16" else a.view(np.uint16 if dt == "f16" else np.uint32)
    assert_bf16_parity(bits(to_host(out, od), od), bits(out_o, od), "router out", exact=True)
    assert_bf16_parity(bits(to_host(gx, xd), xd), bits(gx_o, xd), "router grad_x", exact=True)
    assert np.array_equal(bits(to_host(gx2, xd), xd), bits(gx_o, xd))
    assert_dprobs(gp.cpu().numpy(), gp_o, scale, "router d_probs")


def test_router_autograd_with_fp32_output():
    r = custom("router", 64, 512, x_sigma=1.0, seed=9).generate()
    x = to_dev_bf16(r["x"]).requires_grad_(True)
    p = to_dev_f32(r["probs"]).requires_grad_(True)
    out = epi.RouterWeightMul.apply(x, p, torch.float32)
    assert out.dtype == torch.float32
    g = torch.from_numpy(np.random.default_rng(1).standard_normal((64, 512)).astype(np.float32)).cuda()
    out.backward(g)
    out_o = oracle.router_weight_mul_fwd_typed(r["x"], oracle.BF16, r["probs"], oracle.F32, 64, 512)
    assert np.array_equal(out.detach().cpu().numpy().view(np.uint32), out_o.view(np.uint32))
    gx_o, gp_o, scale = oracle.router_weight_mul_bwd_typed(g.cpu().numpy(), oracle.F32, r["x"], oracle.BF16,
                                                           r["probs"], 64, 512, with_abs_sum=True)
    assert np.array_equal(to_host_bits(x.grad), gx_o)
    assert_dprobs(p.grad.cpu().numpy(), gp_o, scale, "autograd d_probs")
