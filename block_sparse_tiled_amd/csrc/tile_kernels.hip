// Tile permutation kernels: raster [B,L,H,D] <-> zero-padded tile order
// [B,Lpad,H,D] ("bsa_attn" page: preprocess_qkv / postprocess_output with
// get_tile_partition_indices and its inverse; "video_sparse_attn_h3" page:
// tile() keeps pad positions zero).
//
// Both layouts keep a token's H*D row contiguous, so each kernel is a row
// gather: one output row per token slot, copied in 16-byte vectors.  The
// slot <-> token map is computed in closed form per row (no index tensor).
// HBM bound: read L rows, write Lpad rows (tile) or the reverse (untile).
#include "bsta_common.hpp"

namespace bsta {

// Wide rows (64 to 1024 vectors of 16 bytes): LPR lanes per output row, so
// a 256-thread workgroup copies 256/LPR rows.
// The row's source is computed once per row; each lane loads its whole share
// of the row (up to 16 vectors, all in flight) before storing it.  Loads and
// stores are non-temporal: each byte is touched once.
constexpr int kMaxVecPerLane = 16;

template <bool TO_TILES, int LPR>
__global__ __launch_bounds__(256) void permute_wide_kernel(
        Geo g, const u32x4* __restrict__ src, u32x4* __restrict__ dst, int nvec,
        int64_t total_rows) {
    const int lane = threadIdx.x % LPR;
    const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
    if (row >= total_rows) return;
    const int64_t in_rows = TO_TILES ? g.L : g.Lpad;
    const int64_t out_rows = TO_TILES ? g.Lpad : g.L;
    const int64_t b = row / out_rows;
    const int64_t pos = row - b * out_rows;
    const int64_t from = TO_TILES ? slot_to_token(g, pos) : token_to_slot(g, pos);
    const u32x4* s_row = src + (b * in_rows + (from < 0 ? 0 : from)) * nvec;
    u32x4* d_row = dst + row * nvec;
    constexpr int kVec = kMaxVecPerLane * 64 / LPR;
    u32x4 val[kVec];
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
        const int v = lane + LPR * u;
        val[u] = (u32x4){0u, 0u, 0u, 0u};
        if (from >= 0 && v < nvec) val[u] = __builtin_nontemporal_load(&s_row[v]);
    }
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
        const int v = lane + LPR * u;
        if (v < nvec) __builtin_nontemporal_store(val[u], &d_row[v]);
    }
}

// Narrow rows (fewer than 64 vectors): flat (row, vector) indexing, one
// vector per thread and step.
template <bool TO_TILES>
__global__ __launch_bounds__(256) void permute_rows_kernel(
        Geo g, const u32x4* __restrict__ src, u32x4* __restrict__ dst,
        int nvec, int rows_per_wg, int64_t total_rows) {
    const int64_t row0 = (int64_t)blockIdx.x * rows_per_wg;
    const int work = rows_per_wg * nvec;
    const int64_t in_rows = TO_TILES ? g.L : g.Lpad;
    const int64_t out_rows = TO_TILES ? g.Lpad : g.L;
    for (int e = threadIdx.x; e < work; e += 256) {
        int rl = e / nvec;
        int v = e - rl * nvec;
        int64_t row = row0 + rl;
        if (row >= total_rows) break;
        int64_t b = row / out_rows;
        int64_t pos = row - b * out_rows;
        int64_t from = TO_TILES ? slot_to_token(g, pos) : token_to_slot(g, pos);
        u32x4 val = {0u, 0u, 0u, 0u};
        if (from >= 0) val = __builtin_nontemporal_load(&src[(b * in_rows + from) * nvec + v]);
        dst[row * nvec + v] = val;
    }
}

// Tiling with the per-tile mean pooling of the top-k coarse stage ("sla"
// page, get_block_map / mean_pool) in the same pass.  One workgroup per
// (batch, tile, stripe of 64 vectors) with one wave per run of
// kPoolGroupRows rows: lane l copies vector 64*stripe + l (eight consecutive
// (head, d) values) of each valid row of its run to the row's slot (all the
// run's loads in flight), writes +0.0 to its pad rows, and sums its valid
// rows in slot order in fp32.  Wave 0 then adds the runs' sums in run order,
// starting from +0.0, and divides by n_j: the order pool_kernel uses on the
// tiled tensor, so the pooled vectors are bit for bit those
// attn_select_blocks would compute.  Short runs per wave matter: with 8
// rows per wave the kernel moves 6.1 TB/s at 40 heads x 128, against 5.4
// TB/s with one wave walking all 64 rows (same box), since the many short
// waves leave no long tail.  The stripe index varies fastest over the grid,
// so the stripes of a tile's rows are read close together in time.
template <int PARTS>
__global__ __launch_bounds__(64 * PARTS) void tile_pool_kernel(
        Geo g, const u32x4* __restrict__ src, u32x4* __restrict__ dst, float* __restrict__ pooled) {
    static_assert(PARTS * kPoolGroupRows <= 128, "a tile holds at most 128 slots");
    __shared__ int64_t tok[PARTS * kPoolGroupRows];
    __shared__ f32x4 part[PARTS][64][2];
    const int nvec = g.H * g.D / 8;
    const int nstripe = (nvec + 63) / 64;
    const int64_t bj = blockIdx.x / nstripe;
    const int stripe = (int)(blockIdx.x - bj * nstripe);
    const int b = (int)(bj / g.Nt);
    const int j = (int)(bj - (int64_t)b * g.Nt);
    const int n = tile_occupancy(g, j);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if ((int)threadIdx.x < g.E) tok[threadIdx.x] = slot_to_token(g, ((int64_t)j << g.le) + threadIdx.x);
    __syncthreads();
    const int v = stripe * 64 + lane;
    const int r0 = wave * kPoolGroupRows;
    const int re = n < r0 + kPoolGroupRows ? n : r0 + kPoolGroupRows;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (v < nvec) {
        const u32x4* sb = src + (int64_t)b * g.L * nvec + v;
        u32x4* db = dst + ((int64_t)b * g.Lpad + ((int64_t)j << g.le)) * nvec + v;
        if (re - r0 == kPoolGroupRows) {
            u32x4 w[kPoolGroupRows];
#pragma unroll
            for (int u = 0; u < kPoolGroupRows; ++u) w[u] = __builtin_nontemporal_load(&sb[tok[r0 + u] * nvec]);
#pragma unroll
            for (int u = 0; u < kPoolGroupRows; ++u) {
                __builtin_nontemporal_store(w[u], &db[(int64_t)(r0 + u) * nvec]);
                add_bf16x8(acc, w[u]);
            }
        } else {
            for (int r = r0; r < re; ++r) {
                const u32x4 w = __builtin_nontemporal_load(&sb[tok[r] * nvec]);
                __builtin_nontemporal_store(w, &db[(int64_t)r * nvec]);
                add_bf16x8(acc, w);
            }
            for (int r = (re > r0 ? re : r0); r < r0 + kPoolGroupRows; ++r)
                __builtin_nontemporal_store((u32x4){0u, 0u, 0u, 0u}, &db[(int64_t)r * nvec]);
        }
        part[wave][lane][0] = (f32x4){acc[0], acc[1], acc[2], acc[3]};
        part[wave][lane][1] = (f32x4){acc[4], acc[5], acc[6], acc[7]};
    }
    __syncthreads();
    if (wave != 0 || v >= nvec) return;
    float tot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < PARTS; ++p) {
        const f32x4 lo = part[p][lane][0], hi = part[p][lane][1];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            tot[c] += lo[c];
            tot[4 + c] += hi[c];
        }
    }
    const int col = v * 8;
    const int h = col / g.D;
    const int d0 = col - h * g.D;
    float* out = pooled + (((int64_t)b * g.H + h) * g.Nt + j) * g.D + d0;
    const float fn = (float)n;
    f32x4 lo = {tot[0] / fn, tot[1] / fn, tot[2] / fn, tot[3] / fn};
    f32x4 hi = {tot[4] / fn, tot[5] / fn, tot[6] / fn, tot[7] / fn};
    *(f32x4*)out = lo;
    *(f32x4*)(out + 4) = hi;
}

hipError_t launch_tile_pool(const Geo& g, const void* x, void* x_tiled, float* pooled,
                            hipStream_t stream) {
    const int nvec = g.H * g.D / 8;
    const int64_t groups = (int64_t)g.B * g.Nt * ((nvec + 63) / 64);
    if (groups <= 0) return hipSuccess;
    if (g.E == 64)
        hipLaunchKernelGGL(tile_pool_kernel<64 / kPoolGroupRows>, dim3((unsigned)groups),
                           dim3(64 * (64 / kPoolGroupRows)), 0, stream, g, (const u32x4*)x,
                           (u32x4*)x_tiled, pooled);
    else
        hipLaunchKernelGGL(tile_pool_kernel<128 / kPoolGroupRows>, dim3((unsigned)groups),
                           dim3(64 * (128 / kPoolGroupRows)), 0, stream, g, (const u32x4*)x,
                           (u32x4*)x_tiled, pooled);
    return hipGetLastError();
}

hipError_t launch_permute(const Geo& g, const void* src, void* dst, bool to_tiles,
                          hipStream_t stream) {
    const int nvec = g.H * g.D / 8;
    const int64_t total_rows = (int64_t)g.B * (to_tiles ? g.Lpad : g.L);
    if (total_rows <= 0) return hipSuccess;
    if (nvec >= 64 && nvec <= 64 * kMaxVecPerLane) {
        // A whole workgroup per row measured fastest (6.3 TB/s at 40 heads
        // x 128: 2.5 vectors per lane) over one or two waves per row.
        constexpr int LPR = 256;
        const int64_t blocks = (total_rows + 256 / LPR - 1) / (256 / LPR);
        if (to_tiles)
            hipLaunchKernelGGL((permute_wide_kernel<true, LPR>), dim3((unsigned)blocks), dim3(256), 0,
                               stream, g, (const u32x4*)src, (u32x4*)dst, nvec, total_rows);
        else
            hipLaunchKernelGGL((permute_wide_kernel<false, LPR>), dim3((unsigned)blocks), dim3(256), 0,
                               stream, g, (const u32x4*)src, (u32x4*)dst, nvec, total_rows);
        return hipGetLastError();
    }
    int rows_per_wg = (4096 + nvec - 1) / nvec;  // ~64 KB per workgroup
    if (rows_per_wg < 1) rows_per_wg = 1;
    const int64_t blocks = (total_rows + rows_per_wg - 1) / rows_per_wg;
    if (to_tiles)
        hipLaunchKernelGGL(permute_rows_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           g, (const u32x4*)src, (u32x4*)dst, nvec, rows_per_wg, total_rows);
    else
        hipLaunchKernelGGL(permute_rows_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           g, (const u32x4*)src, (u32x4*)dst, nvec, rows_per_wg, total_rows);
    return hipGetLastError();
}

}  // namespace bsta
