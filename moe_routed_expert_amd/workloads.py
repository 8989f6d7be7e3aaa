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

def expert_counts(seed: int, tokens: int, experts: int, split: str) -> np.ndarray:
    """Tokens per local expert: a multinomial over Dirichlet(2) shares ("dirichlet"), the
    same with one empty expert in the middle ("one_empty"), or as even as possible ("even")."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(10, 0))))
    if split == "even":
        c = np.full(experts, tokens // experts, dtype=np.int64)
        c[: tokens % experts] += 1
        return c
    if split == "one_empty" and experts > 1:
        c = g.multinomial(tokens, g.dirichlet(np.full(experts - 1, 2.0)))
        return np.insert(c, experts // 2, 0)
    if split not in ("dirichlet", "one_empty"):
        raise ValueError(split)
    return g.multinomial(tokens, g.dirichlet(np.full(experts, 2.0)))


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
        return expert_counts(self.seed, self.tokens, self.experts, self.split)

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


@dataclass(frozen=True)
class DownWorkload:
    """Down projection grouped GEMM + router-weight multiply: h [tokens, inter] (the SwiGLU
    output, rows grouped by expert), w_down [experts, hidden, inter], probs [tokens].

    h ~ N(0, h_sigma^2) and w ~ N(0, (out_sigma / (h_sigma * sqrt(inter)))^2), so the product's
    entries have standard deviation about out_sigma; probs ~ U(0, 1). Draw kinds: 10 expert
    counts, 15 h chunks, 16 one w_down slice per expert, 17 probs."""
    name: str
    tokens: int
    inter: int
    hidden: int
    experts: int
    seed: int
    out_dtype: str = "bf16"       # "bf16" | "f32"
    h_sigma: float = 0.5
    out_sigma: float = 1.0
    split: str = "dirichlet"

    def flops(self) -> int:
        return 2 * self.tokens * self.inter * self.hidden

    def min_bytes(self) -> int:
        """h, w_down, probs and offs read once, out written once."""
        t, i, h, e = self.tokens, self.inter, self.hidden, self.experts
        return t * i * 2 + e * h * i * 2 + 4 * t + 4 * e + t * h * ELEM_BYTES[self.out_dtype]

    def counts(self) -> np.ndarray:
        return expert_counts(self.seed, self.tokens, self.experts, self.split)

    def offs(self) -> np.ndarray:
        return np.cumsum(self.counts()).astype(np.int32)

    def generate(self, threads: int | None = None) -> dict:
        """h [tokens, inter], w_down [experts, hidden, inter] (bf16 bits), offs int32, probs float32."""
        t, i, hd, e = self.tokens, self.inter, self.hidden, self.experts
        w_sigma = np.float32(self.out_sigma / (self.h_sigma * np.sqrt(i)))
        h = np.empty((t, i), dtype=np.uint16)
        w = np.empty((e, hd, i), dtype=np.uint16)

        def rng(kind: int, chunk: int) -> np.random.Generator:
            return np.random.Generator(np.random.PCG64(np.random.SeedSequence(self.seed, spawn_key=(kind, chunk))))

        def fill_h(chunk: int) -> None:
            r0 = chunk * CHUNK_ROWS
            m = min(CHUNK_ROWS, t - r0)
            f = rng(15, chunk).standard_normal((m, i), dtype=np.float32)
            f *= np.float32(self.h_sigma)
            h[r0:r0 + m] = _to_bf16_bits(f)

        def fill_w(ex: int) -> None:
            f = rng(16, ex).standard_normal((hd, i), dtype=np.float32)
            f *= w_sigma
            w[ex] = _to_bf16_bits(f)

        workers = threads or max(1, min(16, os.cpu_count() or 1))
        with ThreadPoolExecutor(workers) as pool:
            list(pool.map(fill_h, range((t + CHUNK_ROWS - 1) // CHUNK_ROWS)))
            list(pool.map(fill_w, range(e)))
        probs = rng(17, 0).random(t, dtype=np.float32)
        return {"h": h, "w_down": w, "offs": self.offs(), "probs": probs}


@dataclass(frozen=True)
class CombineWorkload:
    """Combine of routed rows into tokens on one expert-parallel rank.

    Each token routes to top_k distinct experts out of global_experts, uniformly at random (slot
    j holds the j-th pick); this rank holds experts [0, local_experts). The slots routed here
    are numbered as the permuted rows are laid out, grouped by local expert and in token order
    inside each expert; row_of[t, j] is that row, or -1 for a slot of another rank's expert.
    expert_out ~ N(0, sigma^2) rows (the router-weighted expert outputs) of eo_dtype. Draw
    kinds: 18 routing (per chunk of tokens), 19 expert_out (per chunk of rows)."""
    name: str
    tokens: int
    hidden: int
    top_k: int
    global_experts: int
    local_experts: int
    seed: int
    eo_dtype: str = "f32"
    sigma: float = 0.05

    def _rng(self, kind: int, chunk: int) -> np.random.Generator:
        return np.random.Generator(np.random.PCG64(np.random.SeedSequence(self.seed, spawn_key=(kind, chunk))))

    def routing(self) -> np.ndarray:
        """int32 [tokens, top_k]: the expert of each slot (distinct within a token)."""
        t, k, ge = self.tokens, self.top_k, self.global_experts
        out = np.empty((t, k), dtype=np.int32)
        for chunk in range((t + CHUNK_ROWS - 1) // CHUNK_ROWS):
            r0 = chunk * CHUNK_ROWS
            m = min(CHUNK_ROWS, t - r0)
            keys = self._rng(18, chunk).random((m, ge))
            out[r0:r0 + m] = np.argsort(keys, axis=1, kind="stable")[:, :k]
        return out

    def row_of(self, experts: np.ndarray | None = None) -> tuple[np.ndarray, int]:
        """(row_of int32 [tokens, top_k], rows): local slots numbered by (expert, token)."""
        ex = self.routing() if experts is None else experts
        local = ex < self.local_experts
        t_idx, j_idx = np.nonzero(local)
        order = np.lexsort((t_idx, ex[t_idx, j_idx]))           # by expert, then token
        row_of = np.full(ex.shape, -1, dtype=np.int32)
        row_of[t_idx[order], j_idx[order]] = np.arange(order.size, dtype=np.int32)
        return row_of, int(order.size)

    def min_bytes(self, row_of: np.ndarray, rows: int) -> int:
        """Each local slot's row read once, row_of read once, out written once."""
        valid = int(((row_of >= 0) & (row_of < rows)).sum())
        return valid * self.hidden * ELEM_BYTES[self.eo_dtype] + row_of.size * 4 + self.tokens * self.hidden * 4

    def generate(self, threads: int | None = None) -> dict:
        """expert_out [rows, hidden] (bf16/f16 bits as uint16 for 16-bit dtypes, float32 otherwise),
        row_of int32 [tokens, top_k], rows."""
        row_of, rows = self.row_of()
        hd = self.hidden
        dt = np.float32 if self.eo_dtype == "f32" else np.uint16
        eo = np.empty((rows, hd), dtype=dt)

        def fill(chunk: int) -> None:
            r0 = chunk * CHUNK_ROWS
            m = min(CHUNK_ROWS, rows - r0)
            f = self._rng(19, chunk).standard_normal((m, hd), dtype=np.float32)
            f *= np.float32(self.sigma)
            if self.eo_dtype == "f32":
                eo[r0:r0 + m] = f
            elif self.eo_dtype == "bf16":
                eo[r0:r0 + m] = _to_bf16_bits(f)
            else:
                eo[r0:r0 + m] = f.astype(np.float16).view(np.uint16)

        workers = threads or max(1, min(16, os.cpu_count() or 1))
        with ThreadPoolExecutor(workers) as pool:
            list(pool.map(fill, range((rows + CHUNK_ROWS - 1) // CHUNK_ROWS)))
        return {"expert_out": eo, "row_of": row_of, "rows": rows}


DOWN_WORKLOADS = {
    w.name: w for w in [
        DownWorkload("down_4096x512x1024_e5", 4096, 512, 1024, 5, seed=22, split="one_empty"),
        DownWorkload("down_4096x512x1024_e5_f32", 4096, 512, 1024, 5, seed=23, out_dtype="f32"),
        DownWorkload("down_131072x2048x7168_e8", 131072, 2048, 7168, 8, seed=24),
        DownWorkload("down_131072x2048x7168_e8_f32", 131072, 2048, 7168, 8, seed=25, out_dtype="f32"),
    ]
}

COMBINE_WORKLOADS = {
    w.name: w for w in [
        CombineWorkload("combine_4096x1024_k8_e64of8", 4096, 1024, 8, 64, 8, seed=26),
        CombineWorkload("combine_131072x7168_k8_e64of8", 131072, 7168, 8, 64, 8, seed=27),
    ]
}

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
