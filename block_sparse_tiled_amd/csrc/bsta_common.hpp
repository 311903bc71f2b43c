// Shared device-side definitions for the block-sparse tiled attention kernels
// (gfx950 / CDNA4 only).
//
// Geometry follows the FastVideo "video_sparse_attn" page
// (construct_variable_block_sizes: ceil(dim/4) tiles per axis, the last tile
// keeps the remainder, a tile's valid-token count is the product of its three
// extents, tiles numbered time-major) and the "bsa_attn" page
// (get_tile_partition_indices: each tile lists its clipped sub-block in
// row-major order).  Inside a padded 64-slot tile the valid tokens come first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsta.h"

namespace bsta {

constexpr int kTileElems = 64;  // 4 x 4 x 4 tokens
// Size of the static device scratch behind attn_block_sparse_bwd_noalloc,
// and the device ordinals whose scratch address is cached.
constexpr int64_t kBwdScratchBytes = int64_t(64) << 20;
// Largest tile count the backward accepts (its CSR transpose keeps two ints
// per tile in the LDS of one workgroup).
constexpr int kMaxBwdTiles = 4096;
constexpr int kMaxDevices = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One segment of a packed sequence ("video_sparse_attn_h3" page, build():
// dense segments and video regions packed in one sequence): a dense segment
// of `rows` consecutive rows is cut into tiles of 64 rows; a video region is
// a (T, Y, X) token grid cut into 4x4x4 tiles as a single grid.  Dense
// segments' tiles come first in tile order (the prefix), then each region's.
struct Seg {
    int64_t tok0;             // first packed token
    int32_t tile0, ntile;     // first tile and tile count
    int32_t rows;             // dense: row count; video region: 0
    int32_t T, Y, X, nY, nX;  // video region's token grid and tiles per axis
};

// Plain-old-data geometry passed by value to every kernel.  Tiles are
// 4 x 4 x tx tokens with tx = 4 (64 tokens) or 8 (128 tokens, reading of the
// "video_sparse_attn_h3" page's tile registry: the width axis doubled).  A
// tile owns E = 16*tx consecutive slots; kernels that work on 64-slot units
// see a 128-token tile as two units (sub = E / 64).  With nseg > 0 the
// sequence is packed from seg[0..nseg) (packed order) and T, Y, X are unused.
struct Geo {
    int32_t B, H, D;
    int32_t T, Y, X;
    int32_t nT, nY, nX, Nt;
    int64_t L, Lpad;
    int32_t tx, lx;   // tile extent along X and its log2
    int32_t E, le;    // slots per tile and its log2
    int32_t sub;      // 64-slot units per tile
    int32_t full;     // every tile holds E valid tokens
    int32_t nseg;     // packed segments (0: one T x Y x X grid)
    int32_t nprefix;  // packed: tiles of the dense segments (the prefix)
    Seg seg[BSTA_MAX_SEGMENTS];
};

// Extent of tile `idx` along an axis of `dim` tokens cut into `size`s
// (size, or the remainder).
__host__ __device__ inline int axis_extent(int dim, int idx, int size = 4) {
    int r = dim - size * idx;
    return r < size ? r : size;
}

struct TileInfo {
    int a, b, c;     // tile coordinates along T, Y, X
    int st, sy, sx;  // extents
    int n;           // valid tokens
};

// Tile j of a (T, Y, X) grid with nY x nX tiles per time slab, tx wide.
__host__ __device__ inline TileInfo grid_tile_info(int T, int Y, int X, int nY, int nX, int tx,
                                                   int j) {
    TileInfo t;
    t.c = j % nX;
    int r = j / nX;
    t.b = r % nY;
    t.a = r / nY;
    t.st = axis_extent(T, t.a);
    t.sy = axis_extent(Y, t.b);
    t.sx = axis_extent(X, t.c, tx);
    t.n = t.st * t.sy * t.sx;
    return t;
}

// Raster token (of the grid) in slot r of tile t, or -1 for a pad slot.
__host__ __device__ inline int64_t grid_slot_token(const TileInfo& t, int Y, int X, int tx, int r) {
    if (r >= t.n) return -1;
    int plane = t.sy * t.sx;
    int dt = r / plane;
    int rem = r - dt * plane;
    int dy = rem / t.sx;
    int dx = rem - dy * t.sx;
    int tt = 4 * t.a + dt, yy = 4 * t.b + dy, xx = tx * t.c + dx;
    return ((int64_t)tt * Y + yy) * X + xx;
}

// (tile, slot in tile) of raster token l of a (., Y, X) grid.
__host__ __device__ inline void grid_token_slot(int64_t l, int Y, int X, int nY, int nX, int tx,
                                                int lx, int* tile, int* r) {
    int64_t plane = (int64_t)Y * X;
    int tt = (int)(l / plane);
    int rem = (int)(l - (int64_t)tt * plane);
    int yy = rem / X;
    int xx = rem - yy * X;
    int a = tt >> 2, b = yy >> 2, c = xx >> lx;
    int sy = axis_extent(Y, b), sx = axis_extent(X, c, tx);
    *tile = (a * nY + b) * nX + c;
    *r = ((tt & 3) * sy + (yy & 3)) * sx + (xx & (tx - 1));
}

// Packed: the segment holding tile j, and the one holding token l.
__host__ __device__ inline int seg_of_tile(const Geo& g, int j) {
    int s = 0;
    for (int t = 0; t < g.nseg; ++t)
        if (j >= g.seg[t].tile0 && j < g.seg[t].tile0 + g.seg[t].ntile) s = t;
    return s;
}
__host__ __device__ inline int seg_of_token(const Geo& g, int64_t l) {
    int s = 0;
    for (int t = 1; t < g.nseg; ++t)
        if (l >= g.seg[t].tok0) s = t;
    return s;
}

__host__ __device__ inline TileInfo tile_info(const Geo& g, int j) {
    return grid_tile_info(g.T, g.Y, g.X, g.nY, g.nX, g.tx, j);
}

// Valid-token count of tile j.
__host__ __device__ inline int tile_occupancy(const Geo& g, int j) {
    if (g.nseg == 0) return tile_info(g, j).n;
    const Seg& s = g.seg[seg_of_tile(g, j)];
    const int jl = j - s.tile0;
    if (s.rows > 0) return s.rows - 64 * jl < 64 ? s.rows - 64 * jl : 64;
    return grid_tile_info(s.T, s.Y, s.X, s.nY, s.nX, 4, jl).n;
}

// Valid slots of 64-slot unit u (slots [64u, 64u + 64)): the tile's valid
// tokens come first, so a tile's second unit holds what exceeds 64.
__host__ __device__ inline int unit_occupancy(const Geo& g, int u) {
    const int part = u & (g.sub - 1);
    const int n = tile_occupancy(g, u >> (g.le - 6)) - 64 * part;
    return n < 0 ? 0 : (n > 64 ? 64 : n);
}

// Token of slot s (s in [0, Lpad)), or -1 for a pad slot.
__device__ inline int64_t slot_to_token(const Geo& g, int64_t s) {
    const int j = (int)(s >> g.le);
    const int r = (int)(s & (g.E - 1));
    if (g.nseg == 0) return grid_slot_token(tile_info(g, j), g.Y, g.X, g.tx, r);
    const Seg& sg = g.seg[seg_of_tile(g, j)];
    const int jl = j - sg.tile0;
    if (sg.rows > 0) {
        const int n = sg.rows - 64 * jl < 64 ? sg.rows - 64 * jl : 64;
        return r < n ? sg.tok0 + 64 * jl + r : -1;
    }
    const int64_t t = grid_slot_token(grid_tile_info(sg.T, sg.Y, sg.X, sg.nY, sg.nX, 4, jl), sg.Y,
                                      sg.X, 4, r);
    return t < 0 ? -1 : sg.tok0 + t;
}

// Slot of token l.
__device__ inline int64_t token_to_slot(const Geo& g, int64_t l) {
    int j, r;
    if (g.nseg == 0) {
        grid_token_slot(l, g.Y, g.X, g.nY, g.nX, g.tx, g.lx, &j, &r);
        return ((int64_t)j << g.le) + r;
    }
    const Seg& sg = g.seg[seg_of_token(g, l)];
    const int64_t ll = l - sg.tok0;
    if (sg.rows > 0) return (int64_t)sg.tile0 * 64 + ll;
    grid_token_slot(ll, sg.Y, sg.X, sg.nY, sg.nX, 4, 2, &j, &r);
    return ((int64_t)(sg.tile0 + j) << 6) + r;
}

// Selection of a packed sequence: the prefix tile count, and per video
// span its tile range [a, b) and the tiles k it keeps per video query tile.
struct PackedSpans {
    int32_t n;        // video spans
    int32_t nprefix;  // prefix tiles P
    int32_t vlen;     // CSR entries of a video query row: P + sum of k
    int32_t a[BSTA_MAX_SEGMENTS], b[BSTA_MAX_SEGMENTS], k[BSTA_MAX_SEGMENTS];
};

// Pooling order shared by the fused tile+pool kernel and the standalone
// pooling kernel, so that both give the same fp32 vectors bit for bit: a
// tile's slots are cut into runs of kPoolGroupRows; each run's valid rows
// are summed in slot order from +0.0, and the run sums are added in run order
// from +0.0 (runs with no valid row add +0.0), then divided by n_j.
constexpr int kPoolGroupRows = 8;

// acc[0..7] += the eight bf16 values of w (low half of each word first).
__device__ inline void add_bf16x8(float (&acc)[8], const u32x4& w) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        acc[2 * c] += __uint_as_float(w[c] << 16);
        acc[2 * c + 1] += __uint_as_float(w[c] & 0xffff0000u);
    }
}

}  // namespace bsta
