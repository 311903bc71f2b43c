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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Plain-old-data geometry passed by value to every kernel.
struct Geo {
    int32_t B, H, D;
    int32_t T, Y, X;
    int32_t nT, nY, nX, Nt;
    int64_t L, Lpad;
};

// Extent of tile `idx` along an axis of `dim` tokens (4, or the remainder).
__host__ __device__ inline int axis_extent(int dim, int idx) {
    int r = dim - 4 * idx;
    return r < 4 ? r : 4;
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
    t.sx = axis_extent(g.X, t.c);
    t.n = t.st * t.sy * t.sx;
    return t;
}

// Valid-token count of tile j.
__host__ __device__ inline int tile_occupancy(const Geo& g, int j) {
    return tile_info(g, j).n;
}

// Raster token of slot s (s in [0, Lpad)), or -1 for a pad slot.
__device__ inline int64_t slot_to_token(const Geo& g, int64_t s) {
    int j = (int)(s >> 6);
    int r = (int)(s & 63);
    TileInfo t = tile_info(g, j);
    if (r >= t.n) return -1;
    int plane = t.sy * t.sx;
    int dt = r / plane;
    int rem = r - dt * plane;
    int dy = rem / t.sx;
    int dx = rem - dy * t.sx;
    int tt = 4 * t.a + dt, yy = 4 * t.b + dy, xx = 4 * t.c + dx;
    return ((int64_t)tt * g.Y + yy) * g.X + xx;
}

// Slot of raster token l.
__device__ inline int64_t token_to_slot(const Geo& g, int64_t l) {
    int64_t plane = (int64_t)g.Y * g.X;
    int tt = (int)(l / plane);
    int rem = (int)(l - (int64_t)tt * plane);
    int yy = rem / g.X;
    int xx = rem - yy * g.X;
    int a = tt >> 2, b = yy >> 2, c = xx >> 2;
    int sy = axis_extent(g.Y, b), sx = axis_extent(g.X, c);
    int j = (a * g.nY + b) * g.nX + c;
    int r = ((tt & 3) * sy + (yy & 3)) * sx + (xx & 3);
    return (int64_t)j * kTileElems + r;
}

}  // namespace bsta
