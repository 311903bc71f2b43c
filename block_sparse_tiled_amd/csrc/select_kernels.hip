// Coarse stage kernels: per-tile mean pooling, pooled scores, per-row top-k
// with CSR output, and sliding-tile-window (STA) CSR.
//
// Method ("sla" page, get_block_map / mean_pool): Q and K are mean-pooled
// per tile, the score of query tile i against key tile j is the dot product
// of the pooled vectors (no scale), and every query tile keeps its k best key
// tiles.  Window mode follows the "STA_configuration" page: a window is a
// count of tiles along t, h, w, and every query tile is charged
// prod(window) tiles.  The CSR form is the map_to_index step of the
// "video_sparse_attn_h3" page.
//
// Precision: pooled vectors are fp32 sums of the valid bf16 rows in row
// order, divided by the valid count; scores are fp32 dot products
// accumulated in fp32 by the matrix cores.  Selection is exact on those
// scores: a threshold search on
// order-preserving 32-bit keys, equal keys resolved toward the lower index.
#include "bsta_common.hpp"

namespace bsta {

// ------------------------------------------------------------------ pooling
// grid (B*Nt*stripes, tensors): one workgroup per (batch, tile, stripe of 64
// vectors of 8 (head, d) columns, tensor), one wave per run of
// kPoolGroupRows slots (bsta_common.hpp).  Each wave sums its run's valid
// rows (all loads in flight) and wave 0 adds the run sums in order: the
// fused tile+pool kernel's structure and order, without the copy.  Many
// short waves: a wave walking all 64 rows of a tile left a long tail (70%
// of HBM peak against 76%).
template <int PARTS>
__global__ __launch_bounds__(64 * PARTS) void pool_kernel(
        Geo g, const u32x4* __restrict__ q, const u32x4* __restrict__ k,
        float* __restrict__ pq, float* __restrict__ pk) {
    __shared__ f32x4 part[PARTS][64][2];
    const u32x4* src = blockIdx.y ? k : q;
    float* dst = blockIdx.y ? pk : pq;
    const int nvec = g.H * g.D / 8;
    const int nstripe = (nvec + 63) / 64;
    const int64_t bj = blockIdx.x / nstripe;
    const int stripe = (int)(blockIdx.x - bj * nstripe);
    const int b = (int)(bj / g.Nt);
    const int j = (int)(bj - (int64_t)b * g.Nt);
    const int n = tile_occupancy(g, j);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int v = stripe * 64 + lane;
    const int r0 = wave * kPoolGroupRows;
    const int re = n < r0 + kPoolGroupRows ? n : r0 + kPoolGroupRows;
    if (v < nvec) {
        const u32x4* base = src + ((int64_t)b * g.Lpad + ((int64_t)j << g.le)) * nvec + v;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (re - r0 == kPoolGroupRows) {
            u32x4 w[kPoolGroupRows];
#pragma unroll
            for (int u = 0; u < kPoolGroupRows; ++u)
                w[u] = __builtin_nontemporal_load(&base[(int64_t)(r0 + u) * nvec]);
#pragma unroll
            for (int u = 0; u < kPoolGroupRows; ++u) add_bf16x8(acc, w[u]);
        } else {
            for (int r = r0; r < re; ++r) add_bf16x8(acc, __builtin_nontemporal_load(&base[(int64_t)r * nvec]));
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
    float* out = dst + (((int64_t)b * g.H + h) * g.Nt + j) * g.D + d0;
    // Divide (not multiply by 1/n) for the correctly rounded quotient.
    const float fn = (float)n;
    f32x4 lo = {tot[0] / fn, tot[1] / fn, tot[2] / fn, tot[3] / fn};
    f32x4 hi = {tot[4] / fn, tot[5] / fn, tot[6] / fn, tot[7] / fn};
    *(f32x4*)out = lo;
    *(f32x4*)(out + 4) = hi;
}

// ------------------------------------------------------------------ scores
// S[bh] = Pq[bh] Pk[bh]^T, fp32, [Nt, Nt] per (batch, head), on the fp32
// matrix cores (v_mfma_f32_32x32x2_f32): a workgroup of four waves covers a
// 64x64 output tile, each wave a 32x32 block.  Per 8 values of d, lane l
// (row or column l%32, half h = l/32) holds the 4 values d0 + 4h + [0, 4)
// of its row; k-step s then contracts d0 + s (lanes 0..31) with d0 + 4 + s
// (lanes 32..63).  A and B use the same assignment, so the 4 steps cover
// the 8 values exactly once.  Each lane loads all of its D/8 pieces of both
// rows up front, so their latencies overlap.  Rows or columns past Nt read
// row Nt-1 and their outputs are not stored.
//
// Tiles are dealt to XCDs in contiguous runs (workgroup x runs on XCD x%8),
// so each XCD's L2 holds the pooled vectors of its own heads only.
constexpr int kScoreTile = 64;

template <int D>
__global__ __launch_bounds__(256) void score_kernel(
        int Nt, int64_t tiles, const float* __restrict__ pq, const float* __restrict__ pk,
        float* __restrict__ s) {
    const int64_t per_xcd = (tiles + 7) / 8;
    const int64_t w = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (w >= tiles) return;  // workgroup-uniform
    // w = (bh * nb + bi) * nb + bj.
    const int nb = (Nt + kScoreTile - 1) / kScoreTile;
    const int bj = (int)(w % nb);
    const int64_t rest = w / nb;
    const int bi = (int)(rest % nb);
    const int64_t bh = rest / nb;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 31, h = lane >> 5;
    const int i0 = bi * kScoreTile + (wave >> 1) * 32;
    const int j0 = bj * kScoreTile + (wave & 1) * 32;
    const int ia = i0 + r < Nt ? i0 + r : Nt - 1;
    const int jb = j0 + r < Nt ? j0 + r : Nt - 1;
    const float* arow = pq + (bh * Nt + ia) * D + 4 * h;
    const float* brow = pk + (bh * Nt + jb) * D + 4 * h;
    f32x4 a[D / 8], b[D / 8];
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
        a[c] = *(const f32x4*)(arow + 8 * c);
        b[c] = *(const f32x4*)(brow + 8 * c);
    }
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < D / 8; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[c][k], b[c][k], acc, 0, 0, 0);
    // Register q of lane l holds row 8(q/4) + 4h + q%4, column l%32.
    float* out = s + bh * Nt * Nt;
    const int j = j0 + r;
    if (j < Nt) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = i0 + 8 * (q >> 2) + 4 * h + (q & 3);
            if (i < Nt) out[(int64_t)i * Nt + j] = acc[q];
        }
    }
}

// ------------------------------------------------------------------ top-k
// Order-preserving key of an fp32 score (-0 folded onto +0).
__device__ inline uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the 256 threads of a workgroup; *total gets the sum.
__device__ inline int block_exclusive_scan(int x, int* smem4, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    if (lane == 63) smem4[wave] = incl;
    __syncthreads();
    int before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        int t = smem4[w];
        before += (w < wave) ? t : 0;
        sum += t;
    }
    __syncthreads();
    *total = sum;
    return before + incl - x;
}

// One workgroup per CSR row (b, h, i).  Keys live in LDS (Nt * 4 bytes),
// selection flags after them (Nt bytes).
__global__ __launch_bounds__(256) void topk_kernel(
        int Nt, int k, int64_t rows, const float* __restrict__ s,
        uint8_t* __restrict__ mask, int32_t* __restrict__ row_ptr,
        int32_t* __restrict__ col_idx) {
    extern __shared__ uint32_t smem[];
    uint32_t* keys = smem;
    uint8_t* flags = (uint8_t*)(keys + Nt);
    __shared__ int hist[256];
    __shared__ int scan4[4];
    __shared__ int sel_digit, sel_rest;

    const int64_t row = blockIdx.x;
    const float* srow = s + row * Nt;
    for (int j = threadIdx.x; j < Nt; j += 256) keys[j] = score_key(srow[j]);

    uint32_t prefix = 0, pmask = 0;
    int kk = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[threadIdx.x] = 0;
        __syncthreads();
        for (int j = threadIdx.x; j < Nt; j += 256) {
            uint32_t key = keys[j];
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        // Count of keys whose digit is >= this thread's digit (suffix sum).
        const int c = hist[threadIdx.x];
        int tot;
        const int excl = block_exclusive_scan(c, scan4, &tot);
        const int at_or_above = tot - excl;
        const int above = at_or_above - c;
        if (c > 0 && above < kk && kk <= at_or_above) {
            sel_digit = threadIdx.x;
            sel_rest = kk - above;
        }
        __syncthreads();
        prefix |= (uint32_t)sel_digit << shift;
        pmask |= 255u << shift;
        kk = sel_rest;
        __syncthreads();
    }
    const uint32_t thr = prefix;  // key of the k-th largest score
    const int take_eq = kk;        // how many keys equal to thr are kept

    // Contiguous chunk of j per thread so that prefix sums follow j order.
    const int chunk = (Nt + 255) / 256;
    const int j0 = min(Nt, (int)threadIdx.x * chunk);
    const int j1 = min(Nt, j0 + chunk);
    int eq = 0;
    for (int j = j0; j < j1; ++j) eq += keys[j] == thr;
    int dummy;
    int eq_before = block_exclusive_scan(eq, scan4, &dummy);
    int nsel = 0;
    for (int j = j0; j < j1; ++j) {
        uint32_t key = keys[j];
        bool sel = key > thr;
        if (key == thr) {
            sel = eq_before < take_eq;
            ++eq_before;
        }
        flags[j] = sel;
        nsel += sel;
    }
    int pos = block_exclusive_scan(nsel, scan4, &dummy);
    int32_t* out = col_idx + row * k;
    for (int j = j0; j < j1; ++j)
        if (flags[j] && pos < k) out[pos++] = j;
    __syncthreads();
    if (mask) {
        uint8_t* mrow = mask + row * Nt;
        for (int j = threadIdx.x; j < Nt; j += 256) mrow[j] = flags[j];
    }
    if (threadIdx.x == 0) {
        row_ptr[row] = (int32_t)(row * k);
        if (row == rows - 1) row_ptr[rows] = (int32_t)(rows * k);
    }
}

// The k-th largest key of a row held as key[c] = lane's score j = 64c + l
// (0 for padding): returns it, and in *take_eq how many keys equal to it
// are kept (the lowest-index ones) so that exactly k are kept.
// Only columns j in [lo, hi) take part; the caller holds key 0 everywhere
// else (the whole row: lo = 0, hi = Nt).
template <int C>
__device__ inline uint32_t kth_key(const uint32_t (&key)[C], int lo, int hi, int k, int lane,
                                   int* take_eq) {
    // Padding slots hold key 0 and every candidate below is >= 1, so they
    // never count; a real key 0 is handled by the explicit validity test in
    // the final pass.
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int c = 0; c < C; ++c) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[c] >= cand));
        if (cnt >= k) thr = cand;
    }
    int above = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int j = c * 64 + lane;
        const bool valid = j >= lo && j < hi;
        above += __builtin_popcountll(__builtin_amdgcn_ballot_w64(valid && key[c] > thr));
    }
    *take_eq = k - above;
    return thr;
}

// Writes the kept ids of a row (keys above thr, and the first take_eq keys
// equal to it in j order) to out[0, ...) in ascending j, and the row's mask
// (if any).  With j = 64c + l, walking c upward and ranking lanes by mbcnt
// visits j in increasing order, so the same ballots give the tie ranks and
// the output positions.  Returns the number written.
template <int C>
__device__ inline int write_kept(const uint32_t (&key)[C], int lo, int hi, uint32_t thr,
                                 int take_eq, int limit, uint8_t* __restrict__ mrow,
                                 int32_t* __restrict__ out, int lane) {
    int base = 0, eq_base = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int j = c * 64 + lane;
        const bool valid = j >= lo && j < hi;
        const bool eq = valid && key[c] == thr;
        const uint64_t eqm = __builtin_amdgcn_ballot_w64(eq);
        const int eq_rank = eq_base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(eqm >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)eqm, 0u));
        eq_base += __builtin_popcountll(eqm);
        const bool sel = valid && (key[c] > thr || (eq && eq_rank < take_eq));
        const uint64_t sm = __builtin_amdgcn_ballot_w64(sel);
        const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(sm >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)sm, 0u));
        base += __builtin_popcountll(sm);
        if (sel && pos < limit) out[pos] = j;
        if (mrow && valid) mrow[j] = sel;
    }
    return base;
}

// One wave per CSR row, for rows of at most 64*C scores: lane l holds
// scores j = 64c + l, c < C, in registers (coalesced loads, no LDS, no
// barriers).  The k-th largest key is found bit by bit from the top: a bit
// is kept when at least k keys are at or above the candidate (one ballot and
// popcount per register).  Then keys above it are kept, and of the keys
// equal to it the first k - (count above) in j order.
template <int C>
__device__ inline void select_row_wave(int Nt, int k, const float* __restrict__ srow,
                                       uint8_t* __restrict__ mrow, int32_t* __restrict__ out,
                                       int lane) {
    uint32_t key[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int j = c * 64 + lane;
        key[c] = j < Nt ? score_key(srow[j]) : 0u;
    }
    int take_eq;
    const uint32_t thr = kth_key<C>(key, 0, Nt, k, lane, &take_eq);
    write_kept<C>(key, 0, Nt, thr, take_eq, k, mrow, out, lane);
}

// Top-k: every row keeps k tiles; CSR row r starts at r*k.
template <int C>
__global__ __launch_bounds__(256) void topk_wave_kernel(
        int Nt, int k, int64_t rows, const float* __restrict__ s,
        uint8_t* __restrict__ mask, int32_t* __restrict__ row_ptr,
        int32_t* __restrict__ col_idx) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // wave-uniform
    select_row_wave<C>(Nt, k, s + row * Nt, mask ? mask + row * Nt : nullptr, col_idx + row * k,
                       lane);
    if (lane == 0) {
        row_ptr[row] = (int32_t)(row * k);
        if (row == rows - 1) row_ptr[rows] = (int32_t)(rows * k);
    }
}

// Packed sequence, exempt mode (one wave per CSR row): a prefix query tile
// keeps every tile; a video query tile keeps the prefix and, in each span
// [a, b), the k best tiles of that span, found by the top-k routines on the
// row's keys with every key outside the span held at 0.  Row lengths are
// fixed (Nt for prefix rows, vlen for video rows), so every row knows its
// CSR start without a scan.
template <int C>
__global__ __launch_bounds__(256) void packed_select_kernel(
        int Nt, int64_t rows, PackedSpans sp, const float* __restrict__ s,
        uint8_t* __restrict__ mask, int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // wave-uniform
    const int64_t bh = row / Nt;
    const int i = (int)(row - bh * Nt);
    const int P = sp.nprefix;
    const int64_t head_nnz = (int64_t)P * Nt + (int64_t)(Nt - P) * sp.vlen;
    const int64_t start = bh * head_nnz + (i < P ? (int64_t)i * Nt
                                                 : (int64_t)P * Nt + (int64_t)(i - P) * sp.vlen);
    int32_t* out = col_idx + start;
    uint8_t* mrow = mask ? mask + row * Nt : nullptr;
    const int whole = i < P ? Nt : P;  // leading tiles kept outright
    for (int j = lane; j < whole; j += 64) {
        out[j] = j;
        if (mrow) mrow[j] = 1;
    }
    if (i >= P) {
        const float* srow = s + row * Nt;
        uint32_t key[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int j = c * 64 + lane;
            key[c] = j < Nt ? score_key(srow[j]) : 0u;
        }
        int pos = P;
        for (int r = 0; r < sp.n; ++r) {
            const int a = sp.a[r], b = sp.b[r], k = sp.k[r];
            uint32_t kr[C];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int j = c * 64 + lane;
                kr[c] = (j >= a && j < b) ? key[c] : 0u;
            }
            int take;
            const uint32_t thr = kth_key<C>(kr, a, b, k, lane, &take);
            write_kept<C>(kr, a, b, thr, take, k, mrow, out + pos, lane);
            pos += k;
        }
    }
    if (lane == 0) {
        row_ptr[row] = (int32_t)start;
        if (row == rows - 1) row_ptr[rows] = (int32_t)(start + (i < P ? Nt : sp.vlen));
    }
}

// ------------------------------------------------------------------ cumulative threshold
// Reading of the "bsa_attn" page's key-value block selection (a cumulative
// threshold and a minimum block count; the rule is not on the page): with
// p_j = softmax_j(S_ij / sqrt(D)) over a row's key tiles, taken in
// descending score order (ties to the lower index), a row keeps the
// shortest prefix whose mass reaches threshold * sum_j p_j, and at least
// min(min_blocks, Nt) tiles.  Every such row is a top-c row of the same
// ranking; its ids are written by the routine top-k uses (write_kept).

// Sum over the wave, taken from lane 0 so that every lane sees the same
// value (the butterfly gives each lane its own rounding order).
__device__ inline float wave_sum_uniform(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

__device__ inline float wave_max_uniform(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// One wave per CSR row: counts[row] = tiles kept, and the kept ids, in
// ascending order, written over the row's own scores (read into registers
// first) for compact_rows_kernel to move into place.  p is fp32 exp2 of the
// scaled score minus the row max (the max tile has p = 1, so the total is at
// least 1).  The kept prefix ends at the largest key x whose tiles at or
// above x hold at least threshold * total, found bit by bit from the top as
// in select_row_wave; all masses come from the same per-lane order and
// summation tree, and adding non-negative terms is monotone in every term,
// so the mass is non-increasing in x and the search is exact on these fp32
// values.  Of the tiles tied at x (equal scores, equal p), the lowest-index
// ones are added one at a time until the mass is reached.  A row raised to
// the minimum count keeps the top-kmin set instead (kth_key).
template <int C>
__global__ __launch_bounds__(256) void cumulative_count_kernel(
        int Nt, int64_t rows, float* __restrict__ s, float scale_log2, float threshold,
        int kmin, uint8_t* __restrict__ mask, int32_t* __restrict__ counts) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // wave-uniform
    const float* srow = s + row * Nt;
    float sv[C];
    uint32_t key[C];
    float mloc = -INFINITY;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int j = c * 64 + lane;
        sv[c] = j < Nt ? srow[j] : -INFINITY;
        key[c] = j < Nt ? score_key(sv[c]) : 0u;
        mloc = fmaxf(mloc, sv[c]);
    }
    const float mx = wave_max_uniform(mloc);
    float p[C];
    float loc = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        p[c] = c * 64 + lane < Nt ? __builtin_amdgcn_exp2f((sv[c] - mx) * scale_log2) : 0.f;
        loc += p[c];
    }
    const float target = threshold * wave_sum_uniform(loc);
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        float m = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) m += key[c] >= cand ? p[c] : 0.f;
        if (wave_sum_uniform(m) >= target) thr = cand;
    }
    float m_above = 0.f, p_eq = 0.f;
    int above = 0, eq = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const bool valid = c * 64 + lane < Nt;
        m_above += valid && key[c] > thr ? p[c] : 0.f;
        above += __builtin_popcountll(__builtin_amdgcn_ballot_w64(valid && key[c] > thr));
        const uint64_t em = __builtin_amdgcn_ballot_w64(valid && key[c] == thr);
        eq += __builtin_popcountll(em);
        if (em != 0 && p_eq == 0.f) {
            const int src = __builtin_ctzll(em);
            p_eq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p[c]), src));
        }
    }
    float acc = wave_sum_uniform(m_above);
    int take = 0;
    while (take < eq && acc < target) {  // wave-uniform
        acc += p_eq;
        ++take;
    }
    if (take == 0 && eq > 0) take = 1;
    int cnt = above + take;
    if (cnt < kmin) {  // wave-uniform
        cnt = kmin < Nt ? kmin : Nt;
        thr = kth_key<C>(key, 0, Nt, cnt, lane, &take);
    }
    write_kept<C>(key, 0, Nt, thr, take, Nt, mask ? mask + row * Nt : nullptr, (int32_t*)(s + row * Nt),
                  lane);
    if (lane == 0) counts[row] = cnt;
}

// In-place scan of row counts into CSR offsets: on entry row_ptr[r + 1]
// holds the count of row r; on exit row_ptr[r] is the start of row r and
// row_ptr[rows] the total.  One workgroup of 1024 threads over chunks of
// 8192 rows, eight consecutive rows per thread (independent loads), a
// workgroup scan of the per-thread sums, and a carry between chunks.
__global__ __launch_bounds__(1024) void scan_counts_kernel(int64_t rows,
                                                           int32_t* __restrict__ row_ptr) {
    constexpr int E = 8;
    __shared__ int part[1024];
    const int tid = threadIdx.x;
    int64_t carry = 0;
    for (int64_t base = 0; base < rows; base += 1024 * E) {
        const int64_t r0 = base + (int64_t)tid * E;
        int v[E];
        int sum = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = r0 + e < rows ? row_ptr[r0 + e + 1] : 0;
#pragma unroll
        for (int e = 0; e < E; ++e) sum += v[e];
        part[tid] = sum;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele, inclusive
            const int add = tid >= off ? part[tid - off] : 0;
            __syncthreads();
            part[tid] += add;
            __syncthreads();
        }
        int64_t run = carry + part[tid] - sum;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            run += v[e];
            if (r0 + e < rows) row_ptr[r0 + e + 1] = (int32_t)run;
        }
        carry += part[1023];
        __syncthreads();  // part is rewritten by the next chunk
    }
    if (tid == 0) row_ptr[0] = 0;
}

// Moves each row's ids (written by cumulative_count_kernel over its scores)
// to its CSR range; one wave per row.
__global__ __launch_bounds__(256) void compact_rows_kernel(
        int Nt, int64_t rows, const float* __restrict__ s, const int32_t* __restrict__ row_ptr,
        int32_t* __restrict__ col_idx) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // wave-uniform
    const int32_t p0 = row_ptr[row];
    const int n = row_ptr[row + 1] - p0;
    const int32_t* src = (const int32_t*)(s + row * Nt);
    for (int t = lane; t < n; t += 64) col_idx[p0 + t] = src[t];
}

// ------------------------------------------------------------------ STA
struct StaArgs {
    int16_t win[BSTA_MAX_STA_HEADS][3];
    int32_t head_prefix[BSTA_MAX_STA_HEADS + 1];  // sum of prod(window) over heads < h
};

__device__ inline int sta_start(int a, int w, int n) {
    int s = a - w / 2;
    s = s < 0 ? 0 : s;
    return s > n - w ? n - w : s;
}

// One workgroup per CSR row.
__global__ __launch_bounds__(256) void sta_kernel(
        Geo g, StaArgs args, uint8_t* __restrict__ mask, int32_t* __restrict__ row_ptr,
        int32_t* __restrict__ col_idx) {
    const int64_t row = blockIdx.x;
    const int i = (int)(row % g.Nt);
    const int64_t bh = row / g.Nt;
    const int h = (int)(bh % g.H);
    const int64_t b = bh / g.H;
    const int wt = args.win[h][0], wy = args.win[h][1], wx = args.win[h][2];
    const int cnt = wt * wy * wx;
    const int64_t per_batch = (int64_t)args.head_prefix[g.H] * g.Nt;
    const int64_t start = b * per_batch + (int64_t)args.head_prefix[h] * g.Nt + (int64_t)i * cnt;
    TileInfo ti = tile_info(g, i);
    const int sa = sta_start(ti.a, wt, g.nT);
    const int sb = sta_start(ti.b, wy, g.nY);
    const int sc = sta_start(ti.c, wx, g.nX);
    for (int e = threadIdx.x; e < cnt; e += 256) {
        int dx = e % wx;
        int r = e / wx;
        int dy = r % wy;
        int dt = r / wy;
        col_idx[start + e] = ((sa + dt) * g.nY + (sb + dy)) * g.nX + (sc + dx);
    }
    if (mask) {
        uint8_t* mrow = mask + row * g.Nt;
        for (int j = threadIdx.x; j < g.Nt; j += 256) {
            TileInfo tj = tile_info(g, j);
            bool in = tj.a >= sa && tj.a < sa + wt && tj.b >= sb && tj.b < sb + wy &&
                      tj.c >= sc && tj.c < sc + wx;
            mrow[j] = in;
        }
    }
    if (threadIdx.x == 0) {
        row_ptr[row] = (int32_t)start;
        const int64_t rows = (int64_t)g.B * g.H * g.Nt;
        if (row == rows - 1) row_ptr[rows] = (int32_t)(g.B * per_batch);
    }
}

// ------------------------------------------------------------------ launchers
namespace {
hipError_t launch_pool_tensors(const Geo& g, const void* q, const void* k, float* pq, float* pk,
                               unsigned tensors, hipStream_t stream) {
    const int nvec = g.H * g.D / 8;
    const unsigned groups = (unsigned)((int64_t)g.B * g.Nt * ((nvec + 63) / 64));
    if (g.E == 64)
        hipLaunchKernelGGL(pool_kernel<64 / kPoolGroupRows>, dim3(groups, tensors),
                           dim3(64 * (64 / kPoolGroupRows)), 0, stream, g, (const u32x4*)q,
                           (const u32x4*)k, pq, pk);
    else
        hipLaunchKernelGGL(pool_kernel<128 / kPoolGroupRows>, dim3(groups, tensors),
                           dim3(64 * (128 / kPoolGroupRows)), 0, stream, g, (const u32x4*)q,
                           (const u32x4*)k, pq, pk);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_pool(const Geo& g, const void* q, const void* k, float* pq, float* pk,
                       hipStream_t stream) {
    return launch_pool_tensors(g, q, k, pq, pk, 2, stream);
}

// One tensor: the same kernel with a grid of one tensor.
hipError_t launch_pool1(const Geo& g, const void* x, float* px, hipStream_t stream) {
    return launch_pool_tensors(g, x, x, px, px, 1, stream);
}

hipError_t launch_scores(const Geo& g, const float* pq, const float* pk, float* s,
                         hipStream_t stream) {
    const int64_t nb = (g.Nt + kScoreTile - 1) / kScoreTile;
    const int64_t tiles = nb * nb * g.B * g.H;
    const unsigned blocks = (unsigned)(8 * ((tiles + 7) / 8));
    if (g.D == 128)
        hipLaunchKernelGGL(score_kernel<128>, dim3(blocks), dim3(256), 0, stream, g.Nt, tiles, pq,
                           pk, s);
    else
        hipLaunchKernelGGL(score_kernel<64>, dim3(blocks), dim3(256), 0, stream, g.Nt, tiles, pq,
                           pk, s);
    return hipGetLastError();
}

hipError_t launch_topk(const Geo& g, int k, const float* s, uint8_t* mask, int32_t* row_ptr,
                       int32_t* col_idx, hipStream_t stream) {
    const int64_t rows = (int64_t)g.B * g.H * g.Nt;
    const int chunks = (g.Nt + 63) / 64;
    const unsigned wave_blocks = (unsigned)((rows + 3) / 4);
#define BSTA_TOPK_WAVE(CC)                                                                     \
    hipLaunchKernelGGL(topk_wave_kernel<CC>, dim3(wave_blocks), dim3(256), 0, stream, g.Nt, k, \
                       rows, s, mask, row_ptr, col_idx)
    if (chunks <= 8) BSTA_TOPK_WAVE(8);
    else if (chunks <= 16) BSTA_TOPK_WAVE(16);
    else if (chunks <= 24) BSTA_TOPK_WAVE(24);
    else if (chunks <= 32) BSTA_TOPK_WAVE(32);
    else {
        const size_t lds = (size_t)g.Nt * 5 + 16;
        hipLaunchKernelGGL(topk_kernel, dim3((unsigned)rows), dim3(256), lds, stream, g.Nt, k,
                           rows, s, mask, row_ptr, col_idx);
    }
#undef BSTA_TOPK_WAVE
    return hipGetLastError();
}

hipError_t launch_packed_select(const Geo& g, const PackedSpans& sp, const float* s,
                                uint8_t* mask, int32_t* row_ptr, int32_t* col_idx,
                                hipStream_t stream) {
    const int64_t rows = (int64_t)g.B * g.H * g.Nt;
    const int chunks = (g.Nt + 63) / 64;
    const unsigned wave_blocks = (unsigned)((rows + 3) / 4);
#define BSTA_PACKED(CC)                                                                        \
    hipLaunchKernelGGL(packed_select_kernel<CC>, dim3(wave_blocks), dim3(256), 0, stream, g.Nt, \
                       rows, sp, s, mask, row_ptr, col_idx)
    if (chunks <= 8) BSTA_PACKED(8);
    else if (chunks <= 16) BSTA_PACKED(16);
    else if (chunks <= 24) BSTA_PACKED(24);
    else if (chunks <= 32) BSTA_PACKED(32);
    else return hipErrorInvalidValue;  // the caller bounds Nt by 2048
#undef BSTA_PACKED
    return hipGetLastError();
}

hipError_t launch_cumulative(const Geo& g, float threshold, int min_blocks, float* s,
                              uint8_t* mask, int32_t* row_ptr, int32_t* col_idx,
                              hipStream_t stream) {
    const int64_t rows = (int64_t)g.B * g.H * g.Nt;
    const int chunks = (g.Nt + 63) / 64;
    const unsigned wave_blocks = (unsigned)((rows + 3) / 4);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)g.D));
    const int kmin = min_blocks < g.Nt ? min_blocks : g.Nt;
#define BSTA_CUM(CC)                                                                           \
    do {                                                                                       \
        hipLaunchKernelGGL(cumulative_count_kernel<CC>, dim3(wave_blocks), dim3(256), 0, stream, \
                           g.Nt, rows, s, scale_log2, threshold, kmin, mask, row_ptr + 1);     \
        hipLaunchKernelGGL(scan_counts_kernel, dim3(1), dim3(1024), 0, stream, rows, row_ptr);  \
        hipLaunchKernelGGL(compact_rows_kernel, dim3(wave_blocks), dim3(256), 0, stream, g.Nt,  \
                           rows, (const float*)s, (const int32_t*)row_ptr, col_idx);           \
    } while (0)
    if (chunks <= 8) BSTA_CUM(8);
    else if (chunks <= 16) BSTA_CUM(16);
    else if (chunks <= 24) BSTA_CUM(24);
    else if (chunks <= 32) BSTA_CUM(32);
    else return hipErrorInvalidValue;  // the caller rejects Nt > 2048 first
#undef BSTA_CUM
    return hipGetLastError();
}

hipError_t launch_sta(const Geo& g, const int32_t* windows, uint8_t* mask, int32_t* row_ptr,
                      int32_t* col_idx, hipStream_t stream) {
    StaArgs args = {};
    int32_t acc = 0;
    for (int h = 0; h < g.H; ++h) {
        args.win[h][0] = (int16_t)windows[3 * h];
        args.win[h][1] = (int16_t)windows[3 * h + 1];
        args.win[h][2] = (int16_t)windows[3 * h + 2];
        args.head_prefix[h] = acc;
        acc += windows[3 * h] * windows[3 * h + 1] * windows[3 * h + 2];
    }
    args.head_prefix[g.H] = acc;
    const int64_t rows = (int64_t)g.B * g.H * g.Nt;
    hipLaunchKernelGGL(sta_kernel, dim3((unsigned)rows), dim3(256), 0, stream, g, args, mask,
                       row_ptr, col_idx);
    return hipGetLastError();
}

}  // namespace bsta
