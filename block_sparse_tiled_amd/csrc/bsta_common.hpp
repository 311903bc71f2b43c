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
constexpr int kMaxDevices = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Plain-old-data geometry passed by value to every kernel.  Tiles are
// 4 x 4 x tx tokens with tx = 4 (64 tokens) or 8 (128 tokens, reading of the
// "video_sparse_attn_h3" page's tile registry: the width axis doubled).  A
// tile owns E = 16*tx consecutive slots; kernels that work on 64-slot units
// see a 128-token tile as two units (sub = E / 64).
struct Geo {
    int32_t B, H, D;
    int32_t T, Y, X;
    int32_t nT, nY, nX, Nt;
    int64_t L, Lpad;
    int32_t tx, lx;   // tile extent along X and its log2
    int32_t E, le;    // slots per tile and its log2
    int32_t sub;      // 64-slot units per tile
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

__host__ __device__ inline TileInfo tile_info(const Geo& g, int j) {
    TileInfo t;
    t.c = j % g.nX;
    int r = j / g.nX;
    t.b = r % g.nY;
    t.a = r / g.nY;
    t.st = axis_extent(g.T, t.a);
    t.sy = axis_extent(g.Y, t.b);
    t.sx = axis_extent(g.X, t.c, g.tx);
    t.n = t.st * t.sy * t.sx;
    return t;
}

// Valid-token count of tile j.
__host__ __device__ inline int tile_occupancy(const Geo& g, int j) {
    return tile_info(g, j).n;
}

// Valid slots of 64-slot unit u (slots [64u, 64u + 64)): the tile's valid
// tokens come first, so a tile's second unit holds what exceeds 64.
__host__ __device__ inline int unit_occupancy(const Geo& g, int u) {
    const int part = u & (g.sub - 1);
    const int n = tile_occupancy(g, u >> (g.le - 6)) - 64 * part;
    return n < 0 ? 0 : (n > 64 ? 64 : n);
}

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

// Raster token of slot s (s in [0, Lpad)), or -1 for a pad slot.
__device__ inline int64_t slot_to_token(const Geo& g, int64_t s) {
    int j = (int)(s >> g.le);
    int r = (int)(s & (g.E - 1));
    TileInfo t = tile_info(g, j);
    if (r >= t.n) return -1;
    int plane = t.sy * t.sx;
    int dt = r / plane;
    int rem = r - dt * plane;
    int dy = rem / t.sx;
    int dx = rem - dy * t.sx;
    int tt = 4 * t.a + dt, yy = 4 * t.b + dy, xx = g.tx * t.c + dx;
    return ((int64_t)tt * g.Y + yy) * g.X + xx;
}

// Slot of raster token l.
__device__ inline int64_t token_to_slot(const Geo& g, int64_t l) {
    int64_t plane = (int64_t)g.Y * g.X;
    int tt = (int)(l / plane);
    int rem = (int)(l - (int64_t)tt * plane);
    int yy = rem / g.X;
    int xx = rem - yy * g.X;
    int a = tt >> 2, b = yy >> 2, c = xx >> g.lx;
    int sy = axis_extent(g.Y, b), sx = axis_extent(g.X, c, g.tx);
    int j = (a * g.nY + b) * g.nX + c;
    int r = ((tt & 3) * sy + (yy & 3)) * sx + (xx & (g.tx - 1));
    return ((int64_t)j << g.le) + r;
}

}  // namespace bsta
