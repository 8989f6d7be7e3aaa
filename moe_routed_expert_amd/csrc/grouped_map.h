// Block -> tile mapping of the grouped GEMM kernels (gfx950), callable from
// host code too, so that it can be checked on the CPU.
//
// Rows of local expert e are [start_e, end_e): start_0 = 0, end_e = offs[e]
// clamped to [start_e, tokens], start_{e+1} = end_e (the routed activations
// grouped contiguously by expert, offs the cumulative token counts). Each
// expert's rows are cut into row tiles of bm rows (the last one partial), so
// no tile straddles two experts; the output columns are cut into column tiles.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace moe_epi {

struct TileRows {
    int64_t row0;   // first token of the tile
    int rows;       // valid tokens in the tile (0: no tile)
    int64_t expert;
};

// The mt-th row tile over all experts in order. Uniform across a block.
__host__ __device__ inline TileRows find_row_tile(const int32_t* __restrict__ offs, int64_t tokens, int64_t experts,
                                                  int64_t mt, int bm) {
    int64_t start = 0, before = 0;
    for (int64_t e = 0; e < experts; ++e) {
        int64_t end = offs[e];
        end = end < start ? start : (end > tokens ? tokens : end);
        const int64_t n = (end - start + bm - 1) / bm;
        if (mt < before + n) {
            const int64_t row0 = start + (mt - before) * bm;
            const int64_t left = end - row0;
            return TileRows{row0, static_cast<int>(left < bm ? left : bm), e};
        }
        before += n;
        start = end;
    }
    return TileRows{0, 0, 0};
}

// Logical tile -> (row tile, column tile). Tiles are visited in groups of gm
// row tiles: within a group the row tile changes fastest. Blocks are handed
// to the 8 XCDs in turn, so the blocks that run together on one XCD are every
// 8th logical tile of a window of consecutive ones; that window covers a few
// groups' row tiles and a run of column tiles, and each XCD's share of it
// reuses both its A tiles and its weight tiles from L2 instead of streaming
// one and re-reading the other. All XCDs work on the same window, so their
// L2 misses meet in the shared Infinity Cache.
__host__ __device__ inline void tile_of(int64_t logical, int64_t m_tiles, int64_t n_tiles, int gm, int64_t* mt,
                                        int64_t* nt) {
    const int64_t per_group = static_cast<int64_t>(gm) * n_tiles;
    const int64_t group = logical / per_group;
    const int64_t first = group * gm;
    const int64_t rows_in_group = m_tiles - first < gm ? m_tiles - first : gm;
    const int64_t in_group = logical % per_group;
    *mt = first + in_group % rows_in_group;
    *nt = in_group / rows_in_group;
}

// Grid: row tiles (worst case ceil(tokens / bm) + experts: one partial tile
// per expert) times column tiles.
// Returns 0 when it does not fit a 1-D grid.
inline int64_t grouped_grid(int64_t tokens, int64_t n_cols, int64_t cols_per_tile, int64_t experts, int bm,
                            int64_t* n_tiles, int64_t* n_blocks) {
    *n_tiles = (n_cols + cols_per_tile - 1) / cols_per_tile;
    const int64_t m_bound = (tokens + bm - 1) / bm + experts;
    *n_blocks = m_bound * *n_tiles;
    return *n_blocks < (static_cast<int64_t>(1) << 31) ? *n_blocks : 0;
}

}  // namespace moe_epi
