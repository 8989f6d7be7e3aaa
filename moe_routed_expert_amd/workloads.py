"""Seeded synthetic inputs for the routed-expert epilogue.

This module is shared by the tests, the smoke check and the benchmark. It
holds none of the method's arithmetic: only random draws, their placement and
their rounding to the input dtypes (bfloat16 via torch's round-to-nearest-even
conversion, fp32 for probabilities). It imports nothing else from this package
and nothing from the oracle.

The five named workloads follow the shapes and value distributions of the
pages' workload ("the 16-node shape" in the nemo_automodel.components.moe
.swiglu_triton module description, whose per-GPU share gives x of about
1.1 GB) and of the router-weight multiply (nemo_automodel.components.moe
.optimized_ops, x [tokens, hidden]):

  swiglu_256x128      L=7,  x ~ N(0, 3^2), 5% of x entries exactly +-7
  swiglu_8192x2048    L=10, x ~ N(0, 4^2), probs renormalised per 8 rows (top-8)
  swiglu_131072x2048  L=10, x ~ N(0, 4^2)            (x is 131072 x 4096 bf16)
  swiglu_100003x1536  L=7,  x ~ N(0, 5^2), 10% of x entries in {-7, +7, 0},
                      20% of rows with probability exactly 0
  router_65536x7168   x ~ N(0, 1)

probs ~ U(0, 1) fp32 unless stated, grad_out ~ N(0, 1) bf16 everywhere.

Readings taken where the workload text is loose:
  - "p% of entries" is read per entry: each entry is special independently
    with probability p (Bernoulli), and the special value is drawn uniformly
    from the listed set;
  - U(0, 1) is numpy's float32 random() in [0, 1);
  - top-8 renormalisation divides each group of 8 consecutive rows by the
    group's sum, computed in float64 and rounded once to float32;
  - normals are drawn in float32, scaled by sigma in float32 and rounded to
    the storage dtype (bfloat16 or float16) to nearest-even; float32 storage
    keeps the draws as they are (so a float32 workload holds the same draws
    as its bfloat16 twin before rounding).
Draws are made in fixed chunks of 4096 rows; each chunk and each kind of draw
has its own PCG64 stream from numpy.random.SeedSequence(seed, spawn_key=(kind,
chunk)), so a workload is the same on every machine and for any thread count.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK_ROWS = 4096


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), rounded to nearest-even by torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# Storage dtypes: bfloat16 travels as uint16 bit patterns, float16 and float32
# as numpy's own types.
DTYPES = ("bf16", "f16", "f32")
ELEM_BYTES = {"bf16": 2, "f16": 2, "f32": 4}


def _to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draws -> the storage dtype (rounded to nearest-even by torch/numpy)."""
    if dtype == "bf16":
        return _to_bf16_bits(a)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float16).numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def storage_numpy_dtype(dtype: str):
    return {"bf16": np.uint16, "f16": np.float16, "f32": np.float32}[dtype]


@dataclass(frozen=True)
class Workload:
    name: str
    op: str                   # "swiglu" or "router"
    rows: int
    cols: int                 # inter (swiglu) or hidden (router)
    limit: float | None       # L for swiglu, None for router
    x_sigma: float
    seed: int
    x_special_frac: float = 0.0
    x_special_values: tuple = ()
    probs_kind: str = "uniform"   # "uniform" | "top8" | "uniform_zeros"
    probs_zero_frac: float = 0.0
    notes: str = field(default="", compare=False)

    @property
    def x_cols(self) -> int:
        return 2 * self.cols if self.op == "swiglu" else self.cols

    def fwd_bytes(self, dtype: str = "bf16", out_dtype: str | None = None) -> int:
        """Algorithmic HBM bytes of one forward pass (every input read once,
        every output written once); out_dtype is the router output's dtype."""
        e = ELEM_BYTES[dtype]
        if self.op == "swiglu":
            return self.rows * (3 * e * self.cols + 4)
        return self.rows * ((e + ELEM_BYTES[out_dtype or dtype]) * self.cols + 4)

    def bwd_bytes(self, with_grad_probs: bool = True, dtype: str = "bf16", out_dtype: str | None = None) -> int:
        """Algorithmic HBM bytes of one backward pass."""
        e = ELEM_BYTES[dtype]
        if self.op == "swiglu":
            return self.rows * (5 * e * self.cols + 4 + (4 if with_grad_probs else 0))
        eo = ELEM_BYTES[out_dtype or dtype]
        if with_grad_probs:
            return self.rows * ((eo + 2 * e) * self.cols + 8)
        return self.rows * ((eo + e) * self.cols + 4)

    def generate(self, rows: int | None = None, threads: int | None = None, dtype: str = "bf16",
                 grad_dtype: str | None = None) -> dict:
        """Inputs as numpy arrays: x ([rows, x_cols] of `dtype`), probs
        (float32 [rows]), grad_out ([rows, cols] of `grad_dtype`, default
        `dtype`). bf16 arrays are uint16 bit patterns.

        Each chunk of CHUNK_ROWS rows draws from its own streams, derived from
        (seed, stream kind, chunk index), so chunks can be drawn in parallel and
        rows < self.rows gives exactly the leading rows of the full workload."""
        n = self.rows if rows is None else int(rows)
        if n < 0 or n > self.rows:
            raise ValueError("rows out of range")
        xc, gc = self.x_cols, self.cols
        grad_dtype = grad_dtype or dtype
        x = np.empty((n, xc), dtype=storage_numpy_dtype(dtype))
        gy = np.empty((n, gc), dtype=storage_numpy_dtype(grad_dtype))
        special = np.array(self.x_special_values, dtype=np.float32)

        def rng(kind: int, chunk: int) -> np.random.Generator:
            return np.random.Generator(np.random.PCG64(np.random.SeedSequence(self.seed, spawn_key=(kind, chunk))))

        def fill(chunk: int) -> None:
            r0 = chunk * CHUNK_ROWS
            m = min(CHUNK_ROWS, n - r0)
            xf = rng(0, chunk).standard_normal((m, xc), dtype=np.float32)
            xf *= np.float32(self.x_sigma)
            if self.x_special_frac > 0.0:
                g = rng(1, chunk)
                hit = g.random((m, xc), dtype=np.float32) < np.float32(self.x_special_frac)
                xf[hit] = special[g.integers(0, len(special), size=int(hit.sum()))]
            x[r0:r0 + m] = _to_storage(xf, dtype)
            gy[r0:r0 + m] = _to_storage(rng(2, chunk).standard_normal((m, gc), dtype=np.float32), grad_dtype)

        chunks = range((n + CHUNK_ROWS - 1) // CHUNK_ROWS)
        workers = threads or max(1, min(16, os.cpu_count() or 1))
        if workers > 1 and len(chunks) > 1:
            with ThreadPoolExecutor(workers) as pool:
                list(pool.map(fill, chunks))
        else:
            for c in chunks:
                fill(c)

        probs = rng(3, 0).random(self.rows, dtype=np.float32)[:n].copy()
        if self.probs_kind == "top8":
            p64 = probs.astype(np.float64)
            for g0 in range(0, n, 8):
                p64[g0:g0 + 8] /= p64[g0:g0 + 8].sum()
            probs = p64.astype(np.float32)
        elif self.probs_kind == "uniform_zeros":
            zero = rng(4, 0).random(self.rows, dtype=np.float32)[:n] < np.float32(self.probs_zero_frac)
            probs[zero] = np.float32(0.0)
        elif self.probs_kind != "uniform":
            raise ValueError(self.probs_kind)
        return {"x": x, "probs": probs, "grad_out": gy}


WORKLOADS = {
    w.name: w for w in [
        Workload("swiglu_256x128", "swiglu", 256, 128, 7.0, 3.0, seed=1,
                 x_special_frac=0.05, x_special_values=(-7.0, 7.0)),
        Workload("swiglu_8192x2048", "swiglu", 8192, 2048, 10.0, 4.0, seed=2, probs_kind="top8"),
        Workload("swiglu_131072x2048", "swiglu", 131072, 2048, 10.0, 4.0, seed=3),
        Workload("swiglu_100003x1536", "swiglu", 100003, 1536, 7.0, 5.0, seed=4,
                 x_special_frac=0.10, x_special_values=(-7.0, 7.0, 0.0),
                 probs_kind="uniform_zeros", probs_zero_frac=0.20),
        Workload("router_65536x7168", "router", 65536, 7168, None, 1.0, seed=5),
    ]
}

# The benchmark's headline workload: the per-GPU share of the large-node shape.
HEADLINE = "swiglu_131072x2048"


# ---- gate_up grouped GEMM + epilogue ------------------------------------------
#
# Inputs of the fused grouped GEMM (pages: nemo_automodel.components.moe
# .mok_experts for the weight layout [local_experts, expert_intermediate,
# hidden]; .quantized_experts, _mxfp4_base_mm, for tokens grouped by expert with
# cumulative int32 counts offs). Readings taken where the pages give no numbers:
#   - tokens are split over the local experts by a multinomial draw with
#     Dirichlet(2, ..., 2) proportions (uneven, as routing is); "one_empty"
#     forces one expert to receive no token, "even" splits evenly;
#   - a ~ N(0, a_sigma^2) and each weight ~ N(0, (gate_up_sigma / (a_sigma *
#     sqrt(hidden)))^2), so that gate and up come out ~ N(0, gate_up_sigma^2):
#     with gate_up_sigma = 4 that is the x ~ N(0, 4^2) of the epilogue's
#     131072 x 2048 workload, and the clamps at L = 10 engage as they do there;
#   - hidden = 7168 is the router workload's width, and 8 local experts per GPU
#     is a reading (the pages give no local expert count);
#   - probs ~ U(0, 1) fp32.
# Draws use their own SeedSequence streams (kinds 10-14), chunked like the rest.

@dataclass(frozen=True)
class GroupedWorkload:
    name: str
    tokens: int
    hidden: int
    inter: int
    experts: int
    limit: float
    seed: int
    a_sigma: float = 1.0
    gate_up_sigma: float = 4.0
    split: str = "dirichlet"      # "dirichlet" | "one_empty" | "even"

    def flops(self) -> int:
        """Multiply-adds of the two products, counted as 2 flops each."""
        return 2 * self.tokens * self.hidden * 2 * self.inter

    def min_bytes(self, write_x: bool = True) -> int:
        """Algorithmic HBM bytes: a, both weight tensors, probs and offs read once,
        y (and x = [gate | up]) written once."""
        t, h, i, e = self.tokens, self.hidden, self.inter, self.experts
        return t * h * 2 + 2 * e * i * h * 2 + 4 * t + 4 * e + t * i * 2 + (t * 2 * i * 2 if write_x else 0)

    def counts(self) -> np.ndarray:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(self.seed, spawn_key=(10, 0))))
        e = self.experts
        if self.split == "even":
            c = np.full(e, self.tokens // e, dtype=np.int64)
            c[: self.tokens % e] += 1
            return c
        if self.split == "one_empty" and e > 1:
            c = g.multinomial(self.tokens, g.dirichlet(np.full(e - 1, 2.0)))
            return np.insert(c, e // 2, 0)
        if self.split not in ("dirichlet", "one_empty"):
            raise ValueError(self.split)
        return g.multinomial(self.tokens, g.dirichlet(np.full(e, 2.0)))

    def offs(self) -> np.ndarray:
        return np.cumsum(self.counts()).astype(np.int32)

    def generate(self, threads: int | None = None) -> dict:
        """a [tokens, hidden], w_gate / w_up [experts, inter, hidden] (bf16 bits as
        uint16), offs int32 [experts], probs float32 [tokens]."""
        t, h, i, e = self.tokens, self.hidden, self.inter, self.experts
        w_sigma = np.float32(self.gate_up_sigma / (self.a_sigma * np.sqrt(h)))
        a = np.empty((t, h), dtype=np.uint16)
        w_gate = np.empty((e, i, h), dtype=np.uint16)
        w_up = np.empty((e, i, h), dtype=np.uint16)

        def rng(kind: int, chunk: int) -> np.random.Generator:
            return np.random.Generator(np.random.PCG64(np.random.SeedSequence(self.seed, spawn_key=(kind, chunk))))

        def fill_a(chunk: int) -> None:
            r0 = chunk * CHUNK_ROWS
            m = min(CHUNK_ROWS, t - r0)
            f = rng(11, chunk).standard_normal((m, h), dtype=np.float32)
            f *= np.float32(self.a_sigma)
            a[r0:r0 + m] = _to_bf16_bits(f)

        def fill_w(job: tuple) -> None:
            which, ex = job
            f = rng(12 + which, ex).standard_normal((i, h), dtype=np.float32)
            f *= w_sigma
            (w_gate if which == 0 else w_up)[ex] = _to_bf16_bits(f)

        jobs_a = range((t + CHUNK_ROWS - 1) // CHUNK_ROWS)
        jobs_w = [(which, ex) for which in (0, 1) for ex in range(e)]
        workers = threads or max(1, min(16, os.cpu_count() or 1))
        with ThreadPoolExecutor(workers) as pool:
            list(pool.map(fill_a, jobs_a))
            list(pool.map(fill_w, jobs_w))
        probs = rng(14, 0).random(t, dtype=np.float32)
        return {"a": a, "w_gate": w_gate, "w_up": w_up, "offs": self.offs(), "probs": probs}


GROUPED_WORKLOADS = {
    w.name: w for w in [
        GroupedWorkload("grouped_4096x1024x512_e5", 4096, 1024, 512, 5, 10.0, seed=20, split="one_empty"),
        GroupedWorkload("grouped_131072x7168x2048_e8", 131072, 7168, 2048, 8, 10.0, seed=21),
    ]
}


def custom(op: str, rows: int, cols: int, limit: float | None = None, x_sigma: float = 4.0,
           seed: int = 0, **kw) -> Workload:
    """An ad-hoc workload (test shapes: ragged tails, tiny rows, odd widths)."""
    return Workload(f"{op}_{rows}x{cols}_s{seed}", op, rows, cols, limit, x_sigma, seed=seed, **kw)
