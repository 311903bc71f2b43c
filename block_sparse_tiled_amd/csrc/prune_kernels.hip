// Query pruning for gfx950 (CDNA4).
//
// Method ("bsa_attn" page: the introduction prunes redundant query tokens in
// each block; forward prunes the query blocks at a keep ratio, selects
// key-value blocks from the kept queries, attends with them, and restores
// full block length from the kept indices).  The page shows the calls but
// not their bodies; the rule built here: a tile of n valid tokens keeps
// c = min(n, max(1, floor(ratio * n))) of them, those least aligned with the
// tile's mean query (lowest cos(q_r, m), ties to the lower slot).  The kept
// set is a 64-bit mask per 64-slot unit (one per 64-token tile, two per
// 128-token tile, bit r for slot r of the unit); the kept queries' mean is
// written where the block selection reads the pooled query.
//
// One wave per (batch, head, tile): the tile's 64 or 128 rows of one head (D
// bf16 each) are staged in LDS with coalesced 16-byte loads, 64 / (D/8) rows per
// instruction; the mean, the per-row scores, the ranks and the kept mean are
// then lane-parallel over rows or over d.  The kept mean is summed in fp32
// in the pooling kernels' order, so with ratio 1 it equals their pooled
// vector bit for bit.
#include "bsta_common.hpp"

namespace bsta {

namespace {

template <int D, int SUB>
__global__ __launch_bounds__(64) void prune_kernel(Geo g, const __bf16* __restrict__ q,
                                                   double ratio, uint64_t* __restrict__ keep_mask,
                                                   int32_t* __restrict__ keep_count,
                                                   float* __restrict__ pooled) {
    constexpr int CH = D / 8;       // 16-byte chunks per row
    constexpr int E = 64 * SUB;     // slots per tile; lane l holds rows l + 64s, s < SUB
    __shared__ __attribute__((aligned(16))) uint16_t rows[E * D];
    __shared__ float mean[D];
    const int lane = threadIdx.x;
    const int64_t item = blockIdx.x;  // (b*H + h)*Nt + j
    const int j = (int)(item % g.Nt);
    const int64_t bh = item / g.Nt;
    const int h = (int)(bh % g.H);
    const int64_t b = bh / g.H;
    const int n = tile_occupancy(g, j);
    const int64_t rs = (int64_t)g.H * D;  // elements between consecutive slots
    const __bf16* base = q + (b * g.Lpad + (int64_t)j * E) * rs + (int64_t)h * D;

    // Stage the valid rows: instruction i covers 64 / CH rows.
    constexpr int RPI = 64 / CH;
    for (int r0 = 0; r0 < E; r0 += RPI) {
        const int r = r0 + lane / CH, c = lane % CH;
        if (r < n)
            *(u32x4*)&rows[r * D + c * 8] = *(const u32x4*)(base + (int64_t)r * rs + c * 8);
    }
    __syncthreads();
    auto at = [&](int r, int d) { return __uint_as_float((uint32_t)rows[r * D + d] << 16); };

    // Mean of the valid rows, d = lane + 64 i.
    for (int d = lane; d < D; d += 64) {
        float acc = 0.f;
        for (int r = 0; r < n; ++r) acc += at(r, d);
        mean[d] = acc / (float)n;
    }
    __syncthreads();
    // cos(q_r, m) of this lane's rows (0 when either vector is zero).  |m|^2
    // is summed in the same order by every lane; a lane walks its own row
    // from d = lane on, so the lanes' LDS reads fall in different banks.
    float mm = 0.f;
    for (int d = 0; d < D; ++d) mm = __builtin_fmaf(mean[d], mean[d], mm);
    float score[SUB];
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
        const int r = lane + 64 * s;
        score[s] = INFINITY;
        if (r < n) {
            float dot = 0.f, qq = 0.f;
            for (int i = 0; i < D; ++i) {
                const int d = (i + lane) & (D - 1);
                const float x = at(r, d);
                dot = __builtin_fmaf(x, mean[d], dot);
                qq = __builtin_fmaf(x, x, qq);
            }
            const float den = sqrtf(qq) * sqrtf(mm);
            score[s] = den > 0.f ? dot / den : 0.f;
        }
    }
    // Rank among the valid rows: lower scores first, ties to the lower slot.
    int rank[SUB] = {};
    for (int i = 0; i < n; ++i) {
        const float si = __shfl(score[SUB > 1 ? (i >> 6) : 0], i & 63, 64);
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            const int r = lane + 64 * s;
            rank[s] += (si < score[s] || (si == score[s] && i < r)) ? 1 : 0;
        }
    }
    const int c = (int)fmin((double)n, fmax(1.0, floor(ratio * (double)n)));
    // The kept set: one 64-bit mask per 64-slot unit of the tile.
    uint64_t kept[SUB];
#pragma unroll
    for (int s = 0; s < SUB; ++s)
        kept[s] = __builtin_amdgcn_ballot_w64(lane + 64 * s < n && rank[s] < c);
    if (lane == 0) {
#pragma unroll
        for (int s = 0; s < SUB; ++s) keep_mask[item * SUB + s] = kept[s];
        if (keep_count != nullptr) keep_count[item] = c;
    }

    // Mean of the kept rows, the tile's pooled query, in the pooling kernels'
    // order (runs of kPoolGroupRows slots, each summed from +0.0, the run
    // sums added in order from +0.0).
    for (int d = lane; d < D; d += 64) {
        float tot = 0.f;
        for (int r0 = 0; r0 < E; r0 += kPoolGroupRows) {
            float acc = 0.f;
            for (int r = r0; r < r0 + kPoolGroupRows && r < n; ++r)
                if ((kept[SUB > 1 ? (r >> 6) : 0] >> (r & 63)) & 1) acc += at(r, d);
            tot += acc;
        }
        pooled[item * D + d] = tot / (float)c;
    }
}

}  // namespace

hipError_t launch_prune(const Geo& g, const void* q_tiled, double ratio, uint64_t* keep_mask,
                        int32_t* keep_count, float* pooled_q, hipStream_t stream) {
    const unsigned blocks = (unsigned)((int64_t)g.B * g.H * g.Nt);
    const __bf16* qt = (const __bf16*)q_tiled;
    if (g.sub == 1) {
        if (g.D == 128)
            hipLaunchKernelGGL((prune_kernel<128, 1>), dim3(blocks), dim3(64), 0, stream, g, qt, ratio,
                               keep_mask, keep_count, pooled_q);
        else
            hipLaunchKernelGGL((prune_kernel<64, 1>), dim3(blocks), dim3(64), 0, stream, g, qt, ratio,
                               keep_mask, keep_count, pooled_q);
    } else {
        if (g.D == 128)
            hipLaunchKernelGGL((prune_kernel<128, 2>), dim3(blocks), dim3(64), 0, stream, g, qt, ratio,
                               keep_mask, keep_count, pooled_q);
        else
            hipLaunchKernelGGL((prune_kernel<64, 2>), dim3(blocks), dim3(64), 0, stream, g, qt, ratio,
                               keep_mask, keep_count, pooled_q);
    }
    return hipGetLastError();
}

}  // namespace bsta
