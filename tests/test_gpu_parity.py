"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Bar: see tests/gpu_util.py. Every input comes from the seeded generator in
moe_routed_expert_amd.workloads; every expected value from oracle/.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import moe_routed_expert_amd as epi
from moe_routed_expert_amd.workloads import WORKLOADS, custom
from tests.gpu_util import (assert_bf16_parity, assert_dprobs, to_dev_bf16, to_dev_f32,
                            to_host_bits)
from tests.numerics import bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"\n[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    epi.binding.lib()  # raises if libmoe_epi.so is not built
    yield
    torch.cuda.synchronize()


def run_swiglu(d, rows, inter, L, want_grad_probs=True):
    x = to_dev_bf16(d["x"])
    p = to_dev_f32(d["probs"])
    gy = to_dev_bf16(d["grad_out"])
    y = torch.empty((rows, inter), dtype=torch.bfloat16, device="cuda")
    gx = torch.empty((rows, 2 * inter), dtype=torch.bfloat16, device="cuda")
    gp = torch.empty((rows,), dtype=torch.float32, device="cuda") if want_grad_probs else None
    epi.swiglu_clamped_fwd(x, p, y, L)
    epi.swiglu_clamped_bwd(x, p, gy, gx, gp, L)
    torch.cuda.synchronize()
    return to_host_bits(y), to_host_bits(gx), (gp.cpu().numpy() if gp is not None else None)


def check_swiglu_rows(d, rows, inter, L, y, gx, gp, what):
    y_o = oracle.swiglu_clamped_fwd(d["x"], d["probs"], rows, inter, L)
    gx_o, gp_o, scale = oracle.swiglu_clamped_bwd(d["x"], d["probs"], d["grad_out"], rows, inter, L,
                                                  with_abs_sum=True)
    s1 = assert_bf16_parity(y, y_o, f"{what} y")
    s2 = assert_bf16_parity(gx[:, :inter], gx_o[:, :inter], f"{what} d_gate")
    s3 = assert_bf16_parity(gx[:, inter:], gx_o[:, inter:], f"{what} d_up")
    s4 = assert_dprobs(gp, gp_o, scale, f"{what} d_probs") if gp is not None else {}
    say(f"{what}: y exact {s1['exact']:.5f}, d_gate exact {s2['exact']:.5f}, d_up exact {s3['exact']:.5f}, "
        f"d_probs {s4}")


@pytest.mark.parametrize("name", ["swiglu_256x128", "swiglu_8192x2048", "swiglu_100003x1536"])
def test_swiglu_named_workload_full(name):
    w = WORKLOADS[name]
    say(f"{name}: generate")
    d = w.generate()
    say(f"{name}: gpu fwd+bwd rows={w.rows} inter={w.cols} L={w.limit}")
    y, gx, gp = run_swiglu(d, w.rows, w.cols, w.limit)
    check_swiglu_rows(d, w.rows, w.cols, w.limit, y, gx, gp, name)
    say(f"{name}: bwd without probability gradient")
    _, gx2, _ = run_swiglu(d, w.rows, w.cols, w.limit, want_grad_probs=False)
    assert np.array_equal(gx, gx2)


def test_swiglu_headline_size_every_row_and_invariants():
    # The 131072 x 2048 workload at full size, every row against the oracle
    # (checked in blocks of rows to bound the host memory the comparison takes).
    w = WORKLOADS["swiglu_131072x2048"]
    rows, I, L = w.rows, w.cols, w.limit
    say(f"{w.name}: generate")
    d = w.generate()
    x = to_dev_bf16(d["x"])
    p = to_dev_f32(d["probs"])
    gy = to_dev_bf16(d["grad_out"])
    y = torch.empty((rows, I), dtype=torch.bfloat16, device="cuda")
    gx = torch.empty((rows, 2 * I), dtype=torch.bfloat16, device="cuda")
    gp = torch.empty((rows,), dtype=torch.float32, device="cuda")
    say(f"{w.name}: gpu fwd+bwd")
    epi.swiglu_clamped_fwd(x, p, y, L)
    epi.swiglu_clamped_bwd(x, p, gy, gx, gp, L)
    torch.cuda.synchronize()
    yh, gxh, gph = to_host_bits(y), to_host_bits(gx), gp.cpu().numpy()
    block = 16384
    exact = []
    for r0 in range(0, rows, block):
        r1 = min(rows, r0 + block)
        sub = {"x": d["x"][r0:r1], "probs": d["probs"][r0:r1], "grad_out": d["grad_out"][r0:r1]}
        y_o = oracle.swiglu_clamped_fwd(sub["x"], sub["probs"], r1 - r0, I, L)
        gx_o, gp_o, scale = oracle.swiglu_clamped_bwd(sub["x"], sub["probs"], sub["grad_out"], r1 - r0, I, L,
                                                      with_abs_sum=True)
        s1 = assert_bf16_parity(yh[r0:r1], y_o, f"{w.name} rows {r0}-{r1} y")
        s2 = assert_bf16_parity(gxh[r0:r1, :I], gx_o[:, :I], f"{w.name} rows {r0}-{r1} d_gate")
        s3 = assert_bf16_parity(gxh[r0:r1, I:], gx_o[:, I:], f"{w.name} rows {r0}-{r1} d_up")
        assert_dprobs(gph[r0:r1], gp_o, scale, f"{w.name} rows {r0}-{r1} d_probs")
        exact.append((s1["exact"], s2["exact"], s3["exact"]))
    say(f"{w.name}: all {rows} rows within the bar; bit-exact fractions per block (y, d_gate, d_up) "
        f"min {np.min(exact, axis=0)}")
    # properties that hold at any size, checked on every row:
    xf = bf16_bits_to_f32(d["x"])
    assert np.all(gxh[:, :I][xf[:, :I] > L] == 0)                  # masked d_gate is +0
    assert np.all(gxh[:, I:][np.abs(xf[:, I:]) > L] == 0)          # masked d_up is +0
    del xf
    say(f"{w.name}: power-of-two scaling (grad_y * 2)")
    gx2 = torch.empty_like(gx)
    gp2 = torch.empty_like(gp)
    epi.swiglu_clamped_bwd(x, p, gy * 2, gx2, gp2, L)
    torch.cuda.synchronize()
    assert torch.equal(gx2.float(), gx.float() * 2)
    assert torch.equal(gp2, gp * 2)


def test_router_full():
    w = WORKLOADS["router_65536x7168"]
    rows, H = w.rows, w.cols
    say(f"{w.name}: generate")
    d = w.generate()
    x, p, go = to_dev_bf16(d["x"]), to_dev_f32(d["probs"]), to_dev_bf16(d["grad_out"])
    out = torch.empty_like(x)
    gx = torch.empty_like(x)
    gp = torch.empty((rows,), dtype=torch.float32, device="cuda")
    say(f"{w.name}: gpu fwd+bwd")
    epi.router_weight_mul_fwd(x, p, out)
    epi.router_weight_mul_bwd(go, x, p, gx, gp)
    torch.cuda.synchronize()
    out_o = oracle.router_weight_mul_fwd(d["x"], d["probs"], rows, H)
    gx_o, gp_o, scale = oracle.router_weight_mul_bwd(d["grad_out"], d["x"], d["probs"], rows, H,
                                                     with_abs_sum=True)
    assert_bf16_parity(to_host_bits(out), out_o, "router out", exact=True)
    assert_bf16_parity(to_host_bits(gx), gx_o, "router grad_x", exact=True)
    st = assert_dprobs(gp.cpu().numpy(), gp_o, scale, "router d_probs")
    say(f"{w.name}: bit-exact out/grad_x, d_probs {st}")
    say(f"{w.name}: bwd without probability gradient")
    gx2 = torch.empty_like(x)
    epi.router_weight_mul_bwd(go, None, p, gx2, None)
    torch.cuda.synchronize()
    assert torch.equal(gx2.view(torch.int16), gx.view(torch.int16))


def _offset_view(bits: np.ndarray, offset_elems: int) -> torch.Tensor:
    """A contiguous bf16 device tensor whose data pointer is offset_elems * 2
    bytes past a 256-byte aligned allocation (offset 1 -> not 16-byte aligned)."""
    flat = bits.ravel()
    buf = torch.zeros(flat.size + offset_elems + 8, dtype=torch.bfloat16, device="cuda")
    view = buf[offset_elems:offset_elems + flat.size]
    view.copy_(to_dev_bf16(flat))
    return view.view(*bits.shape)


# Row widths reach every launch-shape bucket (vectors of 8 per row: < 64 with lane groups of 8, 16 and 32; 64;
# 65-128; 129-191; 192; 193-255; 256; 257-512; 513-1024; wider, in several passes), with ragged row counts, and the
# per-element path (widths not a multiple of 8; offset pointers).
SHAPES = [(1, 1), (3, 3), (2, 8), (37, 8), (5, 24), (64, 56), (33, 64), (17, 136), (9, 200), (40, 520),
          (7, 1544), (5, 2056), (1031, 128), (300, 1536), (129, 2048), (11, 4096), (3, 8200), (6, 1032),
          (4, 6144), (2, 16384), (5, 512), (3, 3072), (21, 1792), (6, 2040)]


@pytest.mark.parametrize("rows,inter", SHAPES)
@pytest.mark.parametrize("offset", [0, 1])
def test_swiglu_shapes_and_alignment(rows, inter, offset):
    w = custom("swiglu", rows, inter, limit=7.0, x_sigma=5.0, seed=1000 + rows * 7 + inter,
               x_special_frac=0.1, x_special_values=(-7.0, 7.0, 0.0, 7.03125, -7.03125),
               probs_kind="uniform_zeros", probs_zero_frac=0.1)
    d = w.generate()
    say(f"swiglu rows={rows} inter={inter} pointer offset={offset * 2} bytes")
    x = _offset_view(d["x"], offset)
    gy = _offset_view(d["grad_out"], offset)
    p = to_dev_f32(d["probs"])
    y = _offset_view(np.zeros((rows, inter), np.uint16), offset)
    gx = _offset_view(np.zeros((rows, 2 * inter), np.uint16), offset)
    gp = torch.empty((rows,), dtype=torch.float32, device="cuda")
    epi.swiglu_clamped_fwd(x, p, y, w.limit)
    epi.swiglu_clamped_bwd(x, p, gy, gx, gp, w.limit)
    torch.cuda.synchronize()
    check_swiglu_rows(d, rows, inter, w.limit, to_host_bits(y), to_host_bits(gx), gp.cpu().numpy(),
                      f"swiglu {rows}x{inter}+{offset}")


# hidden 4096/5120/6144/7168/8192 use 8/10/12/14/16 vectors per lane in one
# pass, 7176 rounds 15 up to 16, 16384 takes two passes of 16
@pytest.mark.parametrize("rows,hidden", [(1, 1), (3, 7), (13, 8), (64, 24), (9, 1000), (257, 7168), (31, 7176),
                                         (19, 4096), (7, 5120), (5, 6144), (9, 8192), (3, 16384), (4, 200),
                                         (7, 1536), (6, 1544), (33, 2048), (5, 2056), (3, 3072), (2, 1040),
                                         (4, 12288), (3, 1024)])
@pytest.mark.parametrize("offset", [0, 1])
def test_router_shapes_and_alignment(rows, hidden, offset):
    d = custom("router", rows, hidden, x_sigma=1.0, seed=2000 + rows * 3 + hidden).generate()
    say(f"router rows={rows} hidden={hidden} pointer offset={offset * 2} bytes")
    x = _offset_view(d["x"], offset)
    go = _offset_view(d["grad_out"], offset)
    p = to_dev_f32(d["probs"])
    out = _offset_view(np.zeros((rows, hidden), np.uint16), offset)
    gx = _offset_view(np.zeros((rows, hidden), np.uint16), offset)
    gp = torch.empty((rows,), dtype=torch.float32, device="cuda")
    epi.router_weight_mul_fwd(x, p, out)
    epi.router_weight_mul_bwd(go, x, p, gx, gp)
    torch.cuda.synchronize()
    out_o = oracle.router_weight_mul_fwd(d["x"], d["probs"], rows, hidden)
    gx_o, gp_o, scale = oracle.router_weight_mul_bwd(d["grad_out"], d["x"], d["probs"], rows, hidden,
                                                     with_abs_sum=True)
    assert_bf16_parity(to_host_bits(out), out_o, "router out", exact=True)
    assert_bf16_parity(to_host_bits(gx), gx_o, "router grad_x", exact=True)
    assert_dprobs(gp.cpu().numpy(), gp_o, scale, "router d_probs")


def test_special_values():
    # NaN, infinities, signed zeros, values at and one bf16 step beyond +-L,
    # denormals, gates far below -L, zero and large probabilities, zero grad_y.
    L = 7.0
    specials = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 7.0, -7.0, 7.03125, -7.03125, 6.96875,
                         -6.96875, 1e-39, -1e-39, -30.0, -60.0, -86.0, -87.0, -87.5, -88.0, -88.5, -89.0,
                         3.0, -1.28125, 1.0, 100.0],
                        dtype=np.float32)
    rng = np.random.default_rng(99)
    rows, inter = 64, 160
    g = rng.choice(specials, size=(rows, inter)).astype(np.float32)
    u = rng.choice(specials, size=(rows, inter)).astype(np.float32)
    gyf = rng.choice(np.array([0.0, -0.0, 1.0, -2.5, 1e-30, np.nan], np.float32), size=(rows, inter))
    tb = lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    d = {"x": np.concatenate([tb(g), tb(u)], axis=1),
         "probs": rng.choice(np.array([0.0, 0.5, 1.0, 3e5, 1e-20], np.float32), size=rows),
         "grad_out": tb(gyf)}
    say("special values")
    y, gx, gp = run_swiglu(d, rows, inter, L)
    y_o = oracle.swiglu_clamped_fwd(d["x"], d["probs"], rows, inter, L)
    gx_o, gp_o = oracle.swiglu_clamped_bwd(d["x"], d["probs"], d["grad_out"], rows, inter, L)
    assert_bf16_parity(y, y_o, "special y")
    assert_bf16_parity(gx, gx_o, "special grad_x")
    assert np.array_equal(np.isnan(gp), np.isnan(gp_o))
    fin = ~np.isnan(gp_o)
    assert np.array_equal(np.isinf(gp[fin]), np.isinf(gp_o[fin]))


def test_gate_band_where_sigma_is_subnormal():
    # Every bf16 gate in [-92, -84]. From about -87.3 down, sigma(gate) =
    # 1/(1 + e^-gate) is below 2^-126 (an fp32 subnormal), and from about
    # -88.7 e^-gate overflows and sigma is 0. In between silu(gate) = gate *
    # sigma is a normal number, so y, d_gate and d_up are nonzero wherever
    # the other factors are: a reciprocal that flushed subnormal results to
    # zero would show here as zeros where the oracle has values.
    L = 7.0
    gates = np.arange(-92.0, -83.75, 0.5, dtype=np.float32)          # bf16 spacing is 0.5 here
    ups = np.array([7.0, -7.0, 1.0, -3.0, 0.5, 6.96875, 7.03125, -0.0], np.float32)
    g, u = np.meshgrid(gates, ups, indexing="ij")
    rows = 16
    tb = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)
    gr = np.tile(g.ravel(), (rows, 1))
    ur = np.tile(u.ravel(), (rows, 1))
    gy = np.tile(np.array([1.0, -2.5, 0.75, 3.0], np.float32), (rows, gr.shape[1] // 4 + 1))[:, :gr.shape[1]]
    d = {"x": np.concatenate([tb(gr), tb(ur)], axis=1),
         "probs": np.array([1.0, 0.5, 0.25, 3.0, 0.125, 2.0, 0.75, 1.5] * 2, np.float32),
         "grad_out": tb(gy)}
    inter = gr.shape[1]
    say(f"gate band [-92, -84]: rows={rows} inter={inter}")
    y, gx, gp = run_swiglu(d, rows, inter, L)
    y_o = oracle.swiglu_clamped_fwd(d["x"], d["probs"], rows, inter, L)
    gx_o, gp_o, scale = oracle.swiglu_clamped_bwd(d["x"], d["probs"], d["grad_out"], rows, inter, L,
                                                  with_abs_sum=True)
    in_band = (gr > -88.75) & (gr < -87.25) & (ur != 0)
    assert ((y_o & 0x7FFF) != 0)[in_band].all()  # the band really gives nonzero outputs in the oracle
    assert_bf16_parity(y, y_o, "band y")
    assert_bf16_parity(gx, gx_o, "band grad_x")
    assert_dprobs(gp, gp_o, scale, "band d_probs")


def test_more_than_2_pow_31_elements():
    # x has 524291 * 4096 > 2^31 elements: the rows are a 4096-row seeded block
    # tiled on the device (copies only), so the oracle needs only the block.
    w = WORKLOADS["swiglu_131072x2048"]
    I, L = w.cols, w.limit
    block = w.generate(rows=4096)
    rows = 524291
    reps = (rows + 4095) // 4096
    say(f"> 2^31 elements: rows={rows} inter={I} (x {rows * 2 * I * 2 / 2**30:.1f} GiB)")
    x = to_dev_bf16(block["x"]).repeat(reps, 1)[:rows].contiguous()
    gy = to_dev_bf16(block["grad_out"]).repeat(reps, 1)[:rows].contiguous()
    p = to_dev_f32(block["probs"]).repeat(reps)[:rows].contiguous()
    assert x.numel() > 2**31
    y = torch.empty((rows, I), dtype=torch.bfloat16, device="cuda")
    gx = torch.empty((rows, 2 * I), dtype=torch.bfloat16, device="cuda")
    gp = torch.empty((rows,), dtype=torch.float32, device="cuda")
    epi.swiglu_clamped_fwd(x, p, y, L)
    epi.swiglu_clamped_bwd(x, p, gy, gx, gp, L)
    torch.cuda.synchronize()
    idx = np.array(sorted({0, 1, 4095, 4096, 262143, 262144, 262145, rows // 2, rows - 3, rows - 2, rows - 1}))
    src = idx % 4096
    sub = {k: v[src] for k, v in block.items()}
    yh = to_host_bits(y[torch.from_numpy(idx).cuda()])
    gxh = to_host_bits(gx[torch.from_numpy(idx).cuda()])
    gph = gp[torch.from_numpy(idx).cuda()].cpu().numpy()
    check_swiglu_rows(sub, idx.size, I, L, yh, gxh, gph, "2^31+ elements")
    del x, gy, y, gx
    torch.cuda.empty_cache()


def test_side_stream_gives_identical_results():
    w = WORKLOADS["swiglu_8192x2048"]
    d = w.generate(rows=2048)
    x, p, gy = to_dev_bf16(d["x"]), to_dev_f32(d["probs"]), to_dev_bf16(d["grad_out"])
    ya = torch.empty((2048, w.cols), dtype=torch.bfloat16, device="cuda")
    yb = torch.empty_like(ya)
    gxa, gxb = torch.empty_like(x), torch.empty_like(x)
    say("default stream vs side stream")
    epi.swiglu_clamped_fwd(x, p, ya, w.limit)
    epi.swiglu_clamped_bwd(x, p, gy, gxa, None, w.limit)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        epi.swiglu_clamped_fwd(x, p, yb, w.limit)
        epi.swiglu_clamped_bwd(x, p, gy, gxb, None, w.limit)
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    assert torch.equal(gxa.view(torch.int16), gxb.view(torch.int16))


def test_autograd_wrappers_match_the_entry_points():
    w = WORKLOADS["swiglu_256x128"]
    d = w.generate()
    x = to_dev_bf16(d["x"]).requires_grad_(True)
    p = to_dev_f32(d["probs"]).requires_grad_(True)
    gy = to_dev_bf16(d["grad_out"])
    say("autograd wrappers")
    y = epi.SwigluClamped.apply(x, p, w.limit)
    y.backward(gy)
    y2, gx2, gp2 = run_swiglu(d, w.rows, w.cols, w.limit)
    assert np.array_equal(to_host_bits(y.detach()), y2)
    assert np.array_equal(to_host_bits(x.grad), gx2)
    assert np.array_equal(p.grad.cpu().numpy(), gp2)
    # router: probs without grad -> x is not saved and no probability gradient
    r = custom("router", 33, 64, x_sigma=1.0, seed=5).generate()
    xr = to_dev_bf16(r["x"]).requires_grad_(True)
    pr = to_dev_f32(r["probs"])
    out = epi.RouterWeightMul.apply(xr, pr)
    out.backward(to_dev_bf16(r["grad_out"]))
    gx_o, _ = oracle.router_weight_mul_bwd(r["grad_out"], None, r["probs"], 33, 64, want_grad_probs=False)
    assert np.array_equal(to_host_bits(xr.grad), gx_o)
    assert np.array_equal(to_host_bits(out.detach()), oracle.router_weight_mul_fwd(r["x"], r["probs"], 33, 64))


def test_zero_rows():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    p = torch.empty((0,), dtype=torch.float32, device="cuda")
    y = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    epi.swiglu_clamped_fwd(x, p, y, 7.0)
    epi.swiglu_clamped_bwd(x, p, y, torch.empty_like(x), torch.empty_like(p), 7.0)
    epi.router_weight_mul_fwd(y, p, torch.empty_like(y))
    epi.router_weight_mul_bwd(y, y, p, torch.empty_like(y), torch.empty_like(p))
    torch.cuda.synchronize()


def test_bad_arguments_raise_without_launching():
    x = torch.zeros((4, 16), dtype=torch.bfloat16, device="cuda")
    p = torch.zeros((4,), dtype=torch.float32, device="cuda")
    y = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(epi.MoeEpiError) as e:
        epi.swiglu_clamped_fwd(x, p, y, float("nan"))
    assert e.value.status == 3
    y_over_x = x.view(-1)[:32].view(4, 8)
    with pytest.raises(epi.MoeEpiError) as e:
        epi.swiglu_clamped_fwd(x, p, y_over_x, 7.0)
    assert e.value.status == 4  # y aliases x
