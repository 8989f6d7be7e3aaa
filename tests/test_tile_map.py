"""The grouped GEMM's block -> tile mapping (csrc/grouped_map.h), checked on the CPU.

A host-only build of the library's own header walks every block of the launched grid
the way the kernel does: the grouped tile order (tile_of, for the group sizes the
kernels use and others) and the search for the row tile's expert and rows
(find_row_tile).
For random and malformed token counts per expert, both epilogue widths and
several group sizes, every row of every expert must be covered exactly once
per column tile, rows of no expert never, no tile may straddle two experts or
exceed the tile height, and every block of the grid must be visited once.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from moe_routed_expert_amd import build as hip_build

SOURCE = r'''
#include "grouped_map.h"
#include <cstdio>
#include <vector>
using namespace moe_epi;

// 0 on success, else a code naming the first violation
// the launched tile: 256 rows x 128 columns per weight tensor (x 2 in router mode)
template <int GM>
int walk(const std::vector<int32_t>& offs, int64_t tokens, int64_t n_cols, bool router) {
    constexpr int BM = 256, BN = 128;
    const int64_t experts = static_cast<int64_t>(offs.size());
    int64_t n_tiles, n_blocks;
    const int64_t grid = grouped_grid(tokens, n_cols, router ? 2 * BN : BN, experts, BM, &n_tiles, &n_blocks);
    if (grid <= 0 || grid != n_blocks) return 1;
    // expert of each row (-1: none), as the pages define the ranges
    std::vector<int64_t> expert_of(tokens, -1);
    int64_t start = 0;
    for (int64_t e = 0; e < experts; ++e) {
        int64_t end = offs[e];
        end = end < start ? start : (end > tokens ? tokens : end);
        for (int64_t t = start; t < end; ++t) expert_of[t] = e;
        start = end;
    }
    std::vector<int> seen(static_cast<size_t>(tokens * n_tiles), 0);
    std::vector<char> hit(grid, 0);
    for (int64_t b = 0; b < grid; ++b) {
        const int64_t logical = b;  // the kernel keeps the hardware's block order
        if (hit[logical]) return 2;
        hit[logical] = 1;
        if (logical >= n_blocks) continue;
        int64_t mt, nt;
        tile_of(logical, n_blocks / n_tiles, n_tiles, GM, &mt, &nt);
        if (nt < 0 || nt >= n_tiles || mt < 0) return 3;
        const TileRows tr = find_row_tile(offs.data(), tokens, experts, mt, BM);
        if (tr.rows == 0) continue;
        if (tr.rows < 0 || tr.rows > BM || tr.row0 < 0 || tr.row0 + tr.rows > tokens) return 4;
        for (int64_t t = tr.row0; t < tr.row0 + tr.rows; ++t) {
            if (expert_of[t] != tr.expert) return 5;
            ++seen[t * n_tiles + nt];
        }
    }
    for (int64_t t = 0; t < tokens; ++t)
        for (int64_t nt = 0; nt < n_tiles; ++nt)
            if (seen[t * n_tiles + nt] != (expert_of[t] >= 0 ? 1 : 0)) return 6;
    return 0;
}

int main() {
    int bad = 0, n = 0;
@CALLS@
    printf("walks %d failed %d\n", n, bad);
    return bad != 0;
}
'''


def cases():
    rng = np.random.default_rng(11)
    out = [
        (1, [1]), (255, [255]), (256, [256]), (257, [257]), (300, [50, 20, 300, 100]), (257, [0, 0, 0, 257]),
        (257, [257, 257, 257, 257]), (257, [-5, 10, 10, 200]), (257, [100, 1000, 5, 7]), (4096, [1160, 2118, 2118, 2510, 4096]),
        (1000, [0]), (700, [700, 700, 700]),
    ]
    for _ in range(12):
        experts = int(rng.integers(1, 17))
        tokens = int(rng.integers(1, 5000))
        counts = rng.multinomial(tokens, rng.dirichlet(np.full(experts, 0.7)))
        offs = np.cumsum(counts)
        if rng.random() < 0.3:  # malformed: perturb some entries
            k = int(rng.integers(0, experts))
            offs[k] = int(rng.integers(-10, tokens + 300))
        out.append((tokens, [int(v) for v in offs]))
    return out


def test_every_row_covered_once_per_column_tile(tmp_path):
    hipcc = hip_build.HIPCC
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    calls = []
    for tokens, offs in cases():
        vec = "{" + ", ".join(str(v) for v in offs) + "}"
        for n_cols, router in ((128, False), (136, False), (2048, False), (256, True), (264, True), (120, True)):
            for gm in (1, 4, 8, 32):
                calls.append(f"    {{ int r = walk<{gm}>(std::vector<int32_t>{vec}, {tokens}, {n_cols}, "
                             f"{str(router).lower()}); ++n; if (r) {{ ++bad; printf(\"tokens=%d cols=%d router=%d "
                             f"gm=%d: code %d\\n\", {tokens}, {n_cols}, {int(router)}, {gm}, r); }} }}")
    src = tmp_path / "tilemap.cpp"
    src.write_text(SOURCE.replace("@CALLS@", "\n".join(calls)))
    exe = tmp_path / "tilemap"
    cmd = [hipcc, "-x", "hip", "--cuda-host-only", "-std=c++17", "-O1", f"-I{hip_build.INCLUDE}",
           f"-I{hip_build.CSRC}", str(src), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "failed 0" in run.stdout
