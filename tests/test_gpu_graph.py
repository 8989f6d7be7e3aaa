"""The library's calls under HIP graph capture.

A serving loop or a launch-bound small step replays the path as one graph:
every entry point only launches kernels on the caller's stream (no
allocation, no memset, no host synchronisation), so it can be captured. The
whole routed-expert chain (gate_up GEMM + SwiGLU epilogue, the streaming
SwiGLU forward and backward, down GEMM + router multiply, combine, router
multiply forward and backward) is captured once and replayed several times,
with eager work and synchronisation between the replays, the outputs reset to
sentinels before each, and new inputs copied into the captured buffers before
the last. Every replay must equal the eager run on the same inputs bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import moe_routed_expert_amd as epi
from moe_routed_expert_amd.workloads import GroupedWorkload
from tests.gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu
TOKENS, HIDDEN, INTER, EXPERTS, TOP_K, L = 1000, 256, 128, 4, 2, 7.0


def say(msg):
    print(f"\n[gpu-graph] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    epi.binding.lib()
    yield
    torch.cuda.synchronize()


def bf16_normal(rng, shape, sigma):
    return to_dev_bf16(((rng.standard_normal(shape).astype(np.float32) * sigma).view(np.uint32) >> 16)
                       .astype(np.uint16))


class Chain:
    """Static input and output buffers of one step of the chain."""

    def __init__(self, seed):
        g = GroupedWorkload("graph", TOKENS, HIDDEN, INTER, EXPERTS, L, seed=seed).generate()
        rng = np.random.default_rng(seed + 1)
        dev = "cuda"
        self.a, self.wg, self.wu = to_dev_bf16(g["a"]), to_dev_bf16(g["w_gate"]), to_dev_bf16(g["w_up"])
        self.offs = torch.from_numpy(g["offs"]).to(dev)
        self.p = torch.from_numpy(g["probs"]).to(dev)
        self.wd = bf16_normal(rng, (EXPERTS, HIDDEN, INTER), 0.05)
        self.gy = bf16_normal(rng, (TOKENS, INTER), 1.0)
        self.gout = bf16_normal(rng, (TOKENS, HIDDEN), 1.0)
        self.row_of = torch.from_numpy(rng.permutation(TOKENS).astype(np.int32).reshape(-1, TOP_K)).to(dev)
        bf, f32 = torch.bfloat16, torch.float32
        self.outs = {
            "y": torch.empty((TOKENS, INTER), dtype=bf, device=dev),
            "x": torch.empty((TOKENS, 2 * INTER), dtype=bf, device=dev),
            "y_stream": torch.empty((TOKENS, INTER), dtype=bf, device=dev),
            "grad_x": torch.empty((TOKENS, 2 * INTER), dtype=bf, device=dev),
            "grad_p": torch.empty((TOKENS,), dtype=f32, device=dev),
            "down": torch.empty((TOKENS, HIDDEN), dtype=f32, device=dev),
            "combined": torch.empty((TOKENS // TOP_K, HIDDEN), dtype=f32, device=dev),
            "router_out": torch.empty((TOKENS, HIDDEN), dtype=bf, device=dev),
            "router_gx": torch.empty((TOKENS, HIDDEN), dtype=bf, device=dev),
            "router_gp": torch.empty((TOKENS,), dtype=f32, device=dev),
        }

    def step(self):
        o = self.outs
        epi.grouped_gate_up_swiglu_fwd(self.a, self.wg, self.wu, self.offs, self.p, o["y"], o["x"], L)
        epi.swiglu_clamped_fwd(o["x"], self.p, o["y_stream"], L)
        epi.swiglu_clamped_bwd(o["x"], self.p, self.gy, o["grad_x"], o["grad_p"], L)
        epi.grouped_down_router_fwd(o["y"], self.wd, self.offs, self.p, o["down"])
        epi.moe_combine_fwd(o["down"], self.row_of, o["combined"])
        epi.router_weight_mul_fwd(self.a, self.p, o["router_out"])
        epi.router_weight_mul_bwd(self.gout, self.a, self.p, o["router_gx"], o["router_gp"])

    def reset(self):
        for t in self.outs.values():   # eager fills, outside the graph
            t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).fill_(0x7FBF if t.dtype ==
                                                                                     torch.bfloat16 else 0x7FC0DEAD)

    def snapshot(self):
        return {k: v.clone() for k, v in self.outs.items()}


def assert_same(got, want, what):
    for k in want:
        g, w = got[k], want[k]
        iv = torch.int16 if w.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(g.view(iv), w.view(iv)), f"{what}: {k} differs from the eager run"


def test_the_chain_replayed_from_a_graph_equals_eager():
    c = Chain(seed=61)
    c.reset()
    c.step()
    torch.cuda.synchronize()
    want = c.snapshot()
    assert torch.isfinite(want["combined"]).all() and torch.isfinite(want["grad_p"]).all()

    # warm-up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c.step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        c.step()
    torch.cuda.synchronize()

    scratch = torch.randn((512, 512), device="cuda")
    for replay in range(3):
        c.reset()
        scratch = scratch @ scratch.t() / 512.0   # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_same(c.outs, want, f"replay {replay}")
    say("3 replays equal the eager run")

    # new inputs in the captured buffers: the graph reads them, and equals eager on them
    other = Chain(seed=62)
    for name in ("a", "p", "gy", "gout"):
        getattr(c, name).copy_(getattr(other, name))
    c.reset()
    c.step()
    torch.cuda.synchronize()
    want2 = c.snapshot()
    assert not torch.equal(want2["y"].view(torch.int16), want["y"].view(torch.int16))
    c.reset()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert_same(c.outs, want2, "replay on new inputs")
    say("replay on new inputs equals the eager run")
