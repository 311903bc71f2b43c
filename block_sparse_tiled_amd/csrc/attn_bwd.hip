// Block-sparse attention backward for gfx950 (CDNA4): gradients of
// sum(dO * O) with respect to Q, K and V for O = softmax(Q K^T / sqrt(D)) V
// over the key tiles of each query tile's CSR row.
//
// Method: the chain rule through the masked softmax of the "bsa_attn" page's
// forward (_compute_sparse_attention; the page's class targets training).
// With P the probabilities, recomputed from the forward's log-sum-exp, and
// dP = dO V^T:
//   dS = P * (dP - delta),  delta = rowsum(dO * O)   (one value per query)
//   dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D),  dV = P^T dO.
//
// Three launches:
//   delta     rowsum(dO * O) per query slot (fp32).
//   csc       per (batch, head), the transpose of the CSR: for every key
//             tile the query tiles whose rows list it, in row order, so that
//             the dK/dV sums run in a fixed order (the first workgroups of
//             the dq launch).
//   dq        one workgroup of four waves per query tile, walking its CSR
//             row: S^T = K Q^T and dP^T = V dO^T on the matrix cores (keys
//             as M, queries as N, so each lane holds one query), then
//             dQ^T += K^T dS^T with K^T read by LDS transpose reads; each
//             wave takes 32 queries and one 32-key half of every key tile,
//             and K and V arrive by direct-to-LDS DMA.
//   dkdv      one workgroup of four waves per key tile, walking its CSC
//             column: S = Q K^T and dP = dO V^T (queries as M, keys as N, so
//             each lane holds one key), then dV^T += dO^T P and
//             dK^T += Q^T dS; each wave takes 16 keys of the tile, on the
//             16x16x32 matrix instruction (its layouts are given with it).
// The walks work on 64-slot units.  A 64-token tile is one unit; a 128-token
// (4x4x8) tile is two, its valid tokens first, so its first unit holds
// min(n, 64) of them.  A dq work item is one query unit and a dkdv item one
// key unit; a CSR entry (or a column's query tile) stands for the tile's
// units, walked as consecutive entries, so every 64x64 unit pair is one
// entry of the same code.  The CSR and its transpose stay per tile.
// The dQ products use v_mfma_f32_32x32x16_bf16 with the lane layouts of the
// forward kernel (checked on hardware there): A[m][k] in lane m + 32*(k/8),
// element k%8; B[k][n] in lane n + 32*(k/8), element k%8; accumulator
// register r of lane l holds D[8*(r/4) + 4*(l/32) + r%4][l%32].  A score
// accumulator converted to bf16 in chunks of 8 registers is the B operand of
// the next product over the same 16 keys (or queries) in a fixed permuted
// order; ds_read_b64_tr_b16 reads the A operand in exactly that order (per
// 16-lane group, lane d receives element d%4 of the value addressed by lane
// d/4 + 4m, m = 0..3).
//
// Both walk kernels bring their tiles into LDS by direct-to-LDS DMA into a
// ring of half-tile slots, ahead of the products (each ring is described
// with its kernel); P and
// dS are rounded to bf16 for the second product, accumulators are fp32 and
// each gradient is rounded once to bf16 at the end.  Pad query rows and pad
// key rows contribute nothing and are written as +0.0.
#include <mutex>

#include "bsta_common.hpp"
#include "lds_dma.hpp"

namespace bsta {

namespace {

typedef short i16x4b __attribute__((ext_vector_type(4)));
typedef short i16x8b __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4b lds_i16x4b;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8b;

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline uint32_t lds_base(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ inline f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS ring layout of the dQ kernel: half-tiles of 32 rows of D bf16 (2*D
// bytes, unpadded); the 16-byte chunk c of row r sits at chunk position
// c ^ ring_swz(r).  The K tile is read both ways, by rows (ds_read_b128: row l32,
// one chunk per lane half) and transposed (ds_read_b64_tr_b16: 4 rows x 32
// bytes per 16-lane group), and ring_swz is chosen so that neither read has a
// bank conflict (64 banks of 4 bytes): ring_swz permutes the chunk positions of
// any 16 consecutive rows (row reads), and it sends 4 consecutive rows from
// a multiple of 4 to distinct 64-byte quarters of the bank range (D = 128)
// or, for D = 64 (two rows per bank range), rows of equal parity to
// distinct 64-byte halves of their 128 bytes (transpose reads).  It
// depends on the row modulo 16 only, as the DMA's offsets require.
template <int D>
__device__ inline int ring_swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 1) | (((r >> 3) & 1) << 1);
}

// LDS byte offset of element `col` (a multiple of 4) of row `row`.
template <int D>
__device__ inline uint32_t ring_off(int row, int col) {
    return (uint32_t)(row * 2 * D + ((col >> 3) ^ ring_swz<D>(row)) * 16 + (col & 7) * 2);
}

// 8 bf16 of row `row`, from element `col` (a multiple of 8), swizzled layout.
template <int D>
__device__ inline bf16x8 ring_row8(uint32_t base, int row, int col) {
    return *(const lds_bf16x8b*)(uintptr_t)(base + ring_off<D>(row, col));
}

// A operand (transposed) of a product over 16 rows of a swizzled half-tile:
// rows 16*step + 4*half + [0,4) and +8, columns 32*db + 16*dsub +
// 4*(s16%4) for source lane s16 (see the header for the transpose read).
template <int D>
__device__ inline bf16x8 ring_tr8(uint32_t base, int step, int db, int lane) {
    const int s16 = lane & 15, dsub = (lane >> 4) & 1, half = lane >> 5;
    const int row = 16 * step + 4 * half + (s16 >> 2);
    const int col = 32 * db + 16 * dsub + 4 * (s16 & 3);
    const i16x4b lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4b*)(uintptr_t)(base + ring_off<D>(row, col)));
    const i16x4b hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4b*)(uintptr_t)(base + ring_off<D>(row + 8, col)));
    const i16x8b w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
}

__device__ inline f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Item of workgroup b when chunks of c consecutive items are dealt to the 8
// XCDs in turn (the hardware deals workgroup b to XCD b % 8); a bijection on
// [0, n): the last, partial band keeps the identity.
__device__ inline int64_t chunked_item(int64_t b, int64_t n, int c) {
    const int64_t band = 8 * (int64_t)c, nb = n / band;
    if (b >= nb * band) return b;
    const int64_t x = b & 7, sl = b >> 3;
    return ((sl / c) * 8 + x) * c + sl % c;
}

}  // namespace

// ------------------------------------------------------------------ delta
// One thread per (batch, slot, head): delta = sum_d dO * O in fp32, and
// the slot's lse scaled to base 2 (log2(e) * lse) for the dK/dV walk.  A
// pad slot (row r >= n_u of its 64-slot unit), or a row that attends to no
// key (lse = -inf), gets +inf instead: its probabilities in the walk come
// out as exp2(-inf) = 0 from finite scores (pad rows of Q are zero), with
// no per-element mask.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(Geo g, const __bf16* __restrict__ o,
                                                        const __bf16* __restrict__ dO,
                                                        const float* __restrict__ lse,
                                                        float* __restrict__ delta,
                                                        float* __restrict__ lse2) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)g.B * g.Lpad * g.H;
    if (t >= total) return;
    const int h = (int)(t % g.H);
    const int64_t bs = t / g.H;
    const int64_t slot = bs % g.Lpad;
    const int64_t b = bs / g.Lpad;
    const u32x4* po = (const u32x4*)(o + t * D);
    const u32x4* pd = (const u32x4*)(dO + t * D);
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
        const u32x4 a = po[c], w = pd[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc += __uint_as_float(a[e] << 16) * __uint_as_float(w[e] << 16);
            acc += __uint_as_float(a[e] & 0xffff0000u) * __uint_as_float(w[e] & 0xffff0000u);
        }
    }
    const int64_t at = (b * g.H + h) * g.Lpad + slot;
    delta[at] = acc;
    const float l = lse[at];
    const bool row = (int)(slot & 63) < unit_occupancy(g, (int)(slot >> 6)) && l > -INFINITY;
    lse2[at] = row ? l * kLog2e : INFINITY;  // the dK/dV walk reads it by DMA
}

// ------------------------------------------------------------------ csc
// The transpose of head bh's CSR, by one workgroup of 256 threads (the
// first B*H workgroups of the dq launch run it, beside the dq walks, which
// do not read it; the dkdv launch after them does).  LDS `sm` holds 2*Nt +
// 256 ints: per-column counts (reused as fill cursors) and starts, and the
// scan's partial sums.  Column j of head bh lists, in row order, the query
// tiles whose CSR rows hold j; it occupies row_idx[col_start[bh*Nt + j] +
// [0, col_cnt[bh*Nt + j])), inside the head's own CSR range.  Row ranges
// are clamped to [0, col_len) and ids outside [0, Nt) are skipped.  A row
// that repeats an id appears that many times in the id's column (the fill
// takes its positions with an LDS atomic), so the dK/dV walk counts the
// repeat as the forward and the dQ walk do.
__device__ inline void csc_head(const Geo& g, int64_t bh, const int32_t* __restrict__ row_ptr,
                                const int32_t* __restrict__ col_idx, int64_t col_len,
                                int32_t* __restrict__ col_start, int32_t* __restrict__ col_cnt,
                                int32_t* __restrict__ row_idx, int* sm) {
    constexpr int NT = 256;
    const int Nt = g.Nt;
    int* cnt = sm;  // counts, then fill cursors
    int* start = sm + Nt;
    int* part = sm + 2 * Nt;
    const int tid = threadIdx.x;
    const int64_t base = bh * Nt;
    auto clampp = [&](int64_t p) { return p < 0 ? (int64_t)0 : (p > col_len ? col_len : p); };
    for (int j = tid; j < Nt; j += NT) cnt[j] = 0;
    __syncthreads();
    for (int i = tid; i < Nt; i += NT) {
        const int64_t p0 = clampp(row_ptr[base + i]);
        const int64_t p1 = clampp(row_ptr[base + i + 1]);
        for (int64_t p = p0; p < p1; ++p) {
            const int j = col_idx[p];
            if ((unsigned)j < (unsigned)Nt) atomicAdd(&cnt[j], 1);
        }
    }
    __syncthreads();
    // Exclusive scan of cnt: each thread a run of `per` columns.
    const int per = (Nt + NT - 1) / NT;
    const int j0 = tid * per < Nt ? tid * per : Nt;
    const int j1 = j0 + per < Nt ? j0 + per : Nt;
    int sum = 0;
    for (int j = j0; j < j1; ++j) sum += cnt[j];
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
        const int add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int run = part[tid] - sum;
    for (int j = j0; j < j1; ++j) {
        start[j] = run;
        run += cnt[j];
    }
    __syncthreads();
    const int64_t head_off = clampp(row_ptr[base]);
    for (int j = tid; j < Nt; j += NT) {
        col_start[base + j] = (int32_t)(head_off + start[j]);
        col_cnt[base + j] = cnt[j];
        cnt[j] = 0;  // the fill's cursor from here on
    }
    __syncthreads();
    // Fill in row order: one row at a time, its ids in parallel.  Repeats of
    // an id within the row take distinct positions (all holding the same row).
    for (int i = 0; i < Nt; ++i) {
        const int64_t p0 = clampp(row_ptr[base + i]);
        const int64_t p1 = clampp(row_ptr[base + i + 1]);
        for (int64_t p = p0 + tid; p < p1; p += NT) {
            const int j = col_idx[p];
            if ((unsigned)j < (unsigned)Nt) {
                const int r = atomicAdd(&cnt[j], 1);
                const int64_t pos = head_off + start[j] + r;
                if (pos < col_len) row_idx[pos] = i;
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ dq
// One workgroup of four waves per query unit.  Wave w owns query rows
// 32*(w%2) + [0, 32) and key rows 32*(w/2) + [0, 32) of every key tile it
// walks: its three products per entry (S^T and dP^T over its 32 keys, then
// dQ^T += K^T dS^T over them) need one 32-row half of K and one of V.  Two
// waves per SIMD fit in the registers this leaves, and the halves' partial
// dQ are added at the end (key half 0 + key half 1, a fixed order).
//
// K and V reach LDS by direct global->LDS DMA into a ring of kDqSlots
// half-tile slots (the swizzled layout above).  Walk entry t is sequence
// positions 4t + r, r = 0..3: K rows 0-31, K rows 32-63, V rows 0-31, V rows
// 32-63; position s sits in slot s % kDqSlots and is issued by wave s % 4.
// Before entry t is read each wave waits for its own position of t, and one
// workgroup barrier publishes all four and retires entry t-1, whose slots
// are refilled at once.
constexpr int kDqSlots = 10;

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(
        Geo g, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
        const __bf16* __restrict__ v, const __bf16* __restrict__ dO,
        const float* __restrict__ lse, const float* __restrict__ delta,
        const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t col_len,
        float scale, __bf16* __restrict__ dq, int csc_blocks, int32_t* __restrict__ col_start,
        int32_t* __restrict__ col_cnt, int32_t* __restrict__ row_idx) {
    constexpr int NDC = D / 16, NDB = D / 32;
    constexpr int HALF = 32 * D * 2;  // bytes of one half-tile slot
    constexpr int NP = HALF / 1024;   // DMA instructions per half-tile
    __shared__ __attribute__((aligned(1024))) char ring[kDqSlots * HALF];
    static_assert(2 * NDB * 16 * 64 * 4 <= kDqSlots * HALF, "partial dQ exchange fits the ring");
    static_assert((2 * kMaxBwdTiles + 256) * 4 <= kDqSlots * HALF, "the CSR transpose fits the ring");
    // The first csc_blocks workgroups transpose one head's CSR each.
    if ((int64_t)blockIdx.x < csc_blocks) {
        csc_head(g, blockIdx.x, row_ptr, col_idx, col_len, col_start, col_cnt, row_idx, (int*)ring);
        return;
    }
    // CSR reads are wave-uniform: read them through the scalar cache.
    typedef const __attribute__((address_space(4))) int32_t* cptr;
    const cptr rp_s = (cptr)row_ptr, ci_s = (cptr)col_idx;
    // Wave-uniform by construction; readfirstlane tells the compiler so, which
    // keeps the DMA bookkeeping and the tile-id reads scalar.
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, l32 = lane & 31;
    const int qb = wave & 1, kh = wave >> 1;  // query block, key half
    // A work item is one 64-slot query unit iu of tile i = iu / sub (sub = 2
    // units per 128-token tile, else 1); every CSR entry j of the tile's row
    // stands for the key units sub*j + [0, sub), walked as consecutive entries.
    const int lsub = g.le - 6, msub = g.sub - 1;
    const int nu = g.Nt << lsub;
    const int64_t item = blockIdx.x - csc_blocks;
    const int iu = (int)(item % nu);
    const int i = iu >> lsub;
    const int64_t bh = item / nu;
    const int h = (int)(bh % g.H);
    const int64_t b = bh / g.H;
    const int64_t rs = (int64_t)g.H * D;
    const int qi = qb * 32 + l32;
    const int ni = unit_occupancy(g, iu);
    const bool qvalid = qi < ni;
    const int64_t qslot = (int64_t)iu * 64 + qi;
    const int64_t qoff = ((b * g.Lpad + qslot) * g.H + h) * D;
    bf16x8 qf[NDC], df[NDC];
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
        qf[dc] = *(const bf16x8*)(q + qoff + dc * 16 + half * 8);
        df[dc] = *(const bf16x8*)(dO + qoff + dc * 16 + half * 8);
    }
    // A pad query row takes lse = +inf, so that its probabilities come out
    // as exp2(-inf) = 0 without a per-element select.
    const float lse2 = qvalid ? lse[bh * g.Lpad + qslot] * kLog2e : INFINITY;
    const float dl = qvalid ? delta[bh * g.Lpad + qslot] : 0.f;
    const float scale_log2 = scale * kLog2e;
    // The compiler cannot see the DMA below: make these loads finish first,
    // so that the waits on the DMA count only DMA.
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) asm volatile("" ::"v"(qf[dc]), "v"(df[dc]));
    asm volatile("" ::"v"(lse2), "v"(dl));
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = (f32x16){};
    int64_t p0 = rp_s[bh * g.Nt + i], p1 = rp_s[bh * g.Nt + i + 1];
    p0 = p0 < 0 ? 0 : (p0 > col_len ? col_len : p0);
    p1 = p1 < p0 ? p0 : (p1 > col_len ? col_len : p1);
    const int n = (int)(p1 - p0) << lsub;  // walk entries (key units)

    // Per-lane DMA source offsets of blocks 0..3 of a half-tile: block u
    // fills slot bytes [1024u, 1024u + 1024), row r = (1024u + 16*lane) /
    // (2D), chunk position c; the lane fetches the chunk the swizzle puts
    // there, c ^ ring_swz(r).  K and V share the layout.
    int32_t off[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int byte = u * 1024 + lane * 16;
        const int r = byte / (2 * D);
        const int c = (byte % (2 * D)) / 16;
        off[u] = 2 * ((int32_t)(r * rs) + (c ^ ring_swz<D>(r)) * 8) - (1024 * u - kDmaBias<D>);
    }
    const int64_t rs2 = rs * 2;  // bytes per slot row
    const uint64_t rows16 = (uint64_t)(16 * rs2);
    // This wave's DMA source: K (waves 0, 1) or V (waves 2, 3), rows 32*(w%2).
    const uint64_t src0 = (uint64_t)(uintptr_t)((wave < 2 ? k : v) + (b * g.Lpad * g.H + h) * D) +
                          (uint64_t)((wave & 1) * 32 * rs2);
    const uint32_t ring0 = lds_base(ring);
    // Key unit of walk entry t, or -1 for a tile id outside [0, Nt) (its
    // slots are filled from unit 0 and its products skipped).  The read of
    // the tile id and the check are apart, so that a read made ahead is not
    // waited for at once.
    auto raw_of = [&](int t) -> int { return ci_s[p0 + (t >> lsub)]; };
    auto checked = [&](int j, int t) -> int {
        return (unsigned)j < (unsigned)g.Nt ? (j << lsub) | (t & msub) : -1;
    };
    const int NSEQ = 4 * n;
    int my_next = wave, my_slot = wave;
    auto issue = [&](int j) {
        dma_half<D>(src0 + (uint64_t)(j < 0 ? 0 : j) * 64 * rs2, rows16, off,
                    ring0 + (uint32_t)my_slot * HALF);
        my_next += 4;
        my_slot = my_slot >= kDqSlots - 4 ? my_slot + 4 - kDqSlots : my_slot + 4;
    };
    while (my_next < NSEQ && my_next < kDqSlots)
        issue(checked(raw_of(my_next >> 2), my_next >> 2));
    // Tile ids are read one entry ahead of their use, at the end of the
    // entry before, so that the scalar loads' latency falls into the wait at
    // the next barrier (which drains them anyway) instead of the LDS waits
    // of the products: the id of entry t, and that of this wave's next
    // position.  In the walk a wave issues at most one position per entry
    // (the limit grows by 4 per entry, a wave's positions by 4 per issue, and
    // each entry issues up to the limit).
    int j_cur = n > 0 ? raw_of(0) : -1;
    int j_iss = my_next < NSEQ ? raw_of(my_next >> 2) : -1;

    int rslot = 0;  // slot of position 4t
    for (int t = 0; t < n; ++t) {
        // Own position of entry t done, then the barrier publishes the other
        // waves' and retires entry t-1 (its reads fed products already).
        wait_dma<NP>((my_next - (4 * t + 4 + wave)) >> 2);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int lim = 4 * t + kDqSlots < NSEQ ? 4 * t + kDqSlots : NSEQ;
        const int j = checked(j_cur, t);
        const bool issued = my_next < lim;
        if (issued) issue(checked(j_iss, my_next >> 2));
        auto read_ahead = [&]() {
            if (t + 1 < n) j_cur = raw_of(t + 1);
            if (issued && my_next < NSEQ) j_iss = raw_of(my_next >> 2);
        };
        const int kslot = rslot + kh < kDqSlots ? rslot + kh : rslot + kh - kDqSlots;
        const int vslot = rslot + 2 + kh < kDqSlots ? rslot + 2 + kh : rslot + 2 + kh - kDqSlots;
        const uint32_t kbuf = ring0 + (uint32_t)kslot * HALF, vbuf = ring0 + (uint32_t)vslot * HALF;
        rslot = rslot + 4 < kDqSlots ? rslot + 4 : rslot + 4 - kDqSlots;
        if (j >= 0) {
            // Valid keys of this half (every tile full: no lookup per entry).
            const int nk = (g.full ? 64 : unit_occupancy(g, j)) - 32 * kh;
            // S^T and dP^T over this wave's 32 keys (row l32 of the half-slot),
            // operand reads batched ahead of their products.
            bf16x8 ka[NDC], va[NDC];
#pragma unroll
            for (int dc = 0; dc < NDC; ++dc) {
                const int col = 16 * dc + 8 * half;
                ka[dc] = ring_row8<D>(kbuf, l32, col);
                va[dc] = ring_row8<D>(vbuf, l32, col);
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
            for (int dc = 0; dc < NDC; ++dc) {
                s = mma(ka[dc], qf[dc], s);
                dp = mma(va[dc], df[dc], dp);
            }
            __builtin_amdgcn_sched_barrier(0);
            // dS^T in two bf16 chunks of 16 keys (chunk c: registers 8c + [0, 8),
            // key 8*(rr/4) + 4*half + rr%4 of the half for register rr).
            // When every key of the half is valid (nk >= 32: full tiles) no key
            // is masked, so that path has no per-element compare or select.
            bf16x8 dsf[2];
            if (nk >= 32) {
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const int rr = 8 * c + r;
                        const float pr = __builtin_amdgcn_exp2f(s[rr] * scale_log2 - lse2);
                        dsf[c][r] = (__bf16)(pr * (dp[rr] - dl));
                    }
            } else {
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const int rr = 8 * c + r;
                        const int key = 8 * (rr >> 2) + 4 * half + (rr & 3);
                        const float pr =
                                key < nk ? __builtin_amdgcn_exp2f(s[rr] * scale_log2 - lse2) : 0.f;
                        dsf[c][r] = (__bf16)(pr * (dp[rr] - dl));
                    }
            }
            // dQ^T += K^T dS^T over the half's two 16-key steps.
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                bf16x8 kt2[NDB];
#pragma unroll
                for (int db = 0; db < NDB; ++db) kt2[db] = ring_tr8<D>(kbuf, c, db, lane);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int db = 0; db < NDB; ++db) acc[db] = mma(kt2[db], dsf[c], acc[db]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        read_ahead();
    }
    // Key half 1 hands its partial dQ^T to key half 0 through the ring (no
    // DMA is in flight: the last entry waited for every position).
    float* const xch = (float*)ring + (size_t)qb * NDB * 16 * 64;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) xch[(db * 16 + r) * 64 + lane] = acc[db][r];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] += xch[(db * 16 + r) * 64 + lane];
    // Lane holds dQ^T[d = 32*db + 8*(r/4) + 4*half + r%4][query qi].
    __bf16* out = dq + qoff;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(qvalid ? acc[db][4 * rb + e] * scale : 0.f);
            *(bf16x4*)(out + 32 * db + 8 * rb + 4 * half) = w;
        }
}

// ------------------------------------------------------------------ dk, dv
// One workgroup of four waves per key unit, on v_mfma_f32_16x16x32_bf16
// (lane layouts checked on hardware: A[m][k] in lane m%16 + 16*(k/8),
// element k%8; B[k][n] in lane n + 16*(k/8), element k%8; register r of
// lane l holds D[4*(l/16) + r][l%16]).  Wave w owns keys 16w + [0, 16) of
// the tile, one per lane l%16, and walks the tile's CSC column: per query
// tile, S = Q K^T and dP = dO V^T in four 16-query blocks (queries as M,
// keys as N; the key fragments stay in registers), then dV^T += dO^T P and
// dK^T += Q^T dS in two 32-query steps (d as M).  A 32-query step takes the
// two 16-query blocks' registers as its B operand, so its queries run in
// the order 4*(l/16) + [0, 4), then 16 + 4*(l/16) + [0, 4); the dO^T and Q^T
// operands come in the same order from two transpose reads (per 16-lane
// group, source lane s points at row q0 + s/4, columns c0 + 4*(s%4), and
// lane d receives rows q0 + [0, 4) of column c0 + d).  Sixteen keys per wave
// keep the accumulators and fragments well within the registers of two
// waves per SIMD.
//
// Q and dO reach LDS by direct-to-LDS DMA into a ring of kKvSlots half-tile
// slots, as in the dQ kernel: walk entry t is positions 4t + r, r = 0..3 (Q
// rows 0-31, Q rows 32-63, dO rows 0-31, dO rows 32-63), position s in slot
// s % kKvSlots, issued by wave s % 4; waves 0 and 1 also bring the query
// tile's base-2 lse and delta (64 floats each) into the 256-byte side slot of
// their position's slot.  Nine slots are the fewest with which every
// position of an entry is issued before its acquire; with the side slots
// they keep a workgroup under 80 KB, two per CU.  Every wave reads the whole
// Q and dO tiles.  The 16-byte chunk c of row r sits at position
// c ^ kv_swz(r), a map that depends on the row modulo 16 only, as the DMA's
// offsets require.  It is chosen by measurement: the bank conflict counters
// of a probe that repeats the kernel's two read shapes (ds_read_b128 of 16
// rows x 4 chunks, or x 2 for D = 64; transpose reads of 4 rows x 32 bytes
// per 16-lane group) read zero for it at both head sizes.  The maps
// 2*(r%8) + (r/8)%2 (D = 128) and (r & 6) + (r/8)%2 (D = 64), which give
// rows r and r + 8 the same chunks but for the lowest bit, are also
// conflict-free for the transpose reads but double the cycles of the row
// reads (8 instead of 4 per instruction), although a model that serves 16
// consecutive lanes together rates them free of conflicts.
template <int D>
__device__ inline int kv_swz(int r) {
    const int h = (r >> 3) & 1;
    if constexpr (D == 128) return (2 * ((r & 7) ^ (4 * h))) | h;
    else return ((r & 6) ^ (4 * h)) | h;
}

template <int D>
__device__ inline uint32_t kv_off(int row, int col) {
    return (uint32_t)(row * 2 * D + (((col >> 3) ^ kv_swz<D>(row)) * 16) + (col & 7) * 2);
}

// A operand of a 16x16x32 product by two transpose reads: rows 4G + [0, 4)
// and 16 + 4G + [0, 4) of a half-tile slot for lane group G = lane/16 (per
// 16-lane group, source lane s points at row 4G + s/4, columns c0 +
// 4*(s%4), and lane d receives the four rows' elements of column c0 + d),
// given this lane's address `a` in the first four rows and the byte
// distance `r16` of 16 rows.
__device__ inline bf16x8 kv_tr16o(uint32_t a, uint32_t r16) {
    const i16x4b lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4b*)(uintptr_t)a);
    const i16x4b hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4b*)(uintptr_t)(a + r16));
    const i16x8b w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
}

constexpr int kKvSlots = 9;

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_kernel(
        Geo g, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
        const __bf16* __restrict__ v, const __bf16* __restrict__ dO,
        const float* __restrict__ lse2, const float* __restrict__ delta,
        const int32_t* __restrict__ col_start, const int32_t* __restrict__ col_cnt,
        const int32_t* __restrict__ row_idx, int64_t col_len, float scale,
        __bf16* __restrict__ dk, __bf16* __restrict__ dv) {
    constexpr int NS = D / 32, NDB = D / 16;
    constexpr int HALF = 32 * D * 2;  // bytes of one half-tile slot
    constexpr int NP = HALF / 1024;   // DMA instructions per half-tile
    __shared__ __attribute__((aligned(1024))) char ring[kKvSlots * HALF];
    __shared__ __attribute__((aligned(16))) float side[kKvSlots * 64];
    typedef const __attribute__((address_space(4))) int32_t* cptr;
    const cptr ri_s = (cptr)row_idx;
    // Wave-uniform by construction; readfirstlane tells the compiler so, which
    // keeps the DMA bookkeeping and the tile-id reads scalar.
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = lane >> 4, l16 = lane & 15;
    // Key tiles are dealt to the XCDs in runs of 16 neighbours: the columns
    // of neighbouring key tiles hold many of the same query tiles, so the
    // workgroups that run together on an XCD share more of their Q and dO
    // reads in its L2 (2% on the 40-head 1200-tile top-120 backward).
    // A work item is one 64-slot key unit ju of tile j = ju / sub; every
    // query tile i of the tile's column stands for the query units sub*i +
    // [0, sub), walked as consecutive entries.
    const int lsub = g.le - 6, msub = g.sub - 1;
    const int nu = g.Nt << lsub;
    const int64_t item = chunked_item(blockIdx.x, (int64_t)gridDim.x, 16);
    const int ju = (int)(item % nu);
    const int j = ju >> lsub;
    const int64_t bh = item / nu;
    const int h = (int)(bh % g.H);
    const int64_t b = bh / g.H;
    const int64_t rs = (int64_t)g.H * D;
    const int kj = wave * 16 + l16;
    const bool kvalid = kj < unit_occupancy(g, ju);
    const int64_t koff = ((b * g.Lpad + (int64_t)ju * 64 + kj) * g.H + h) * D;
    bf16x8 kf[NS], vf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        kf[s] = *(const bf16x8*)(k + koff + 32 * s + 8 * G);
        vf[s] = *(const bf16x8*)(v + koff + 32 * s + 8 * G);
    }
    // The compiler cannot see the DMA below: make these loads finish first,
    // so that the waits on the DMA count only DMA.
#pragma unroll
    for (int s = 0; s < NS; ++s) asm volatile("" ::"v"(kf[s]), "v"(vf[s]));
    const float scale_log2 = scale * kLog2e;
    f32x4 adv[NDB], adk[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        adv[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
        adk[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    int64_t c0 = col_start[bh * g.Nt + j];
    int64_t c1 = c0 + col_cnt[bh * g.Nt + j];
    c0 = c0 < 0 ? 0 : (c0 > col_len ? col_len : c0);
    c1 = c1 < c0 ? c0 : (c1 > col_len ? col_len : c1);
    const int m = (int)(c1 - c0) << lsub;  // walk entries (query units)

    // Per-lane DMA source offsets of blocks 0..3 of a half-tile (as in the
    // dQ kernel, with this ring's swizzle).
    int32_t off[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int byte = u * 1024 + lane * 16;
        const int r = byte / (2 * D);
        const int c = (byte % (2 * D)) / 16;
        off[u] = 2 * ((int32_t)(r * rs) + (c ^ kv_swz<D>(r)) * 8) - (1024 * u - kDmaBias<D>);
    }
    const int64_t rs2 = rs * 2;
    const uint64_t rows16 = (uint64_t)(16 * rs2);
    // Position r of an entry: Q rows 0-31 (with the tile's lse), Q rows
    // 32-63 (with its delta), dO rows 0-31, dO rows 32-63; issued by wave r.
    const uint64_t src0 = (uint64_t)(uintptr_t)((wave < 2 ? q : dO) + (b * g.Lpad * g.H + h) * D) +
                          (uint64_t)((wave & 1) * 32 * rs2);
    const uint64_t fsrc = (uint64_t)(uintptr_t)((wave == 0 ? lse2 : delta) + bh * g.Lpad);
    const uint32_t ring0 = lds_base(ring), side0 = lds_base(side);
    // Query unit of walk entry t, or -1 for a tile id outside [0, Nt) (its
    // slots are filled from unit 0 and its products skipped).
    auto raw_of = [&](int t) -> int { return ri_s[c0 + (t >> lsub)]; };
    auto checked = [&](int i, int t) -> int {
        return (unsigned)i < (unsigned)g.Nt ? (i << lsub) | (t & msub) : -1;
    };
    // Per-lane LDS offsets inside a half-tile slot, fixed for the walk.  The
    // swizzle depends on the row modulo 16 only, so rows 16..31 of a slot
    // sit at the same offsets plus 16 rows (an immediate): row reads use row
    // l16, chunk 4s + G; transpose reads row 4G + l16/4, columns 16u +
    // 4*(l16%4).
    uint32_t ro[NS], to[NDB];
#pragma unroll
    for (int s = 0; s < NS; ++s) ro[s] = kv_off<D>(l16, 32 * s + 8 * G);
#pragma unroll
    for (int u = 0; u < NDB; ++u) to[u] = kv_off<D>(4 * G + (l16 >> 2), 16 * u + 4 * (l16 & 3));
    constexpr uint32_t R16 = 16 * 2 * D;  // bytes of 16 rows
    const int NSEQ = 4 * m;
    int my_next = wave, my_slot = wave;
    auto issue = [&](int i) {
        const int64_t ii = i < 0 ? 0 : i;
        dma_half<D>(src0 + (uint64_t)ii * 64 * rs2, rows16, off, ring0 + (uint32_t)my_slot * HALF);
        if (wave < 2) dma_floats64(fsrc + (uint64_t)ii * 256, side0 + (uint32_t)my_slot * 256);
        my_next += 4;
        my_slot = my_slot >= kKvSlots - 4 ? my_slot + 4 - kKvSlots : my_slot + 4;
    };
    while (my_next < NSEQ && my_next < kKvSlots)
        issue(checked(raw_of(my_next >> 2), my_next >> 2));
    // Query tile ids are read one entry ahead of their use, at the end of the
    // entry before, as in the dQ kernel (a wave issues at most one position
    // per entry of the walk).
    int i_cur = m > 0 ? raw_of(0) : -1;
    int i_iss = my_next < NSEQ ? raw_of(my_next >> 2) : -1;

    int rslot = 0;  // slot of position 4t
    for (int t = 0; t < m; ++t) {
        // Own position of entry t done (a position is NP DMA instructions,
        // one more for waves 0 and 1, whose side slot rides along), then the
        // barrier publishes the other waves' and retires entry t-1.
        {
            const int newer = (my_next - (4 * t + 4 + wave)) >> 2;
            if (newer <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            else if (wave < 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NP + 1) : "memory");
            else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NP) : "memory");
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int lim = 4 * t + kKvSlots < NSEQ ? 4 * t + kKvSlots : NSEQ;
        const int i = checked(i_cur, t);
        const bool issued = my_next < lim;
        if (issued) issue(checked(i_iss, my_next >> 2));
        auto read_ahead = [&]() {
            if (t + 1 < m) i_cur = raw_of(t + 1);
            if (issued && my_next < NSEQ) i_iss = raw_of(my_next >> 2);
        };
        int sl[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sl[r] = rslot + r < kKvSlots ? rslot + r : rslot + r - kKvSlots;
        const uint32_t qh0 = ring0 + (uint32_t)sl[0] * HALF, qh1 = ring0 + (uint32_t)sl[1] * HALF;
        const uint32_t dh0 = ring0 + (uint32_t)sl[2] * HALF, dh1 = ring0 + (uint32_t)sl[3] * HALF;
        const float* const lse_t = side + sl[0] * 64;
        const float* const del_t = side + sl[1] * 64;
        rslot = rslot + 4 < kKvSlots ? rslot + 4 : rslot + 4 - kKvSlots;
        if (i >= 0) {
            // S and dP in four 16-query blocks (A = row l16 of the block, d =
            // 32s + 8G + [0, 8)): register r of block mb holds query 16mb + 4G +
            // r.  Block mb+1's products are issued before block mb's P and dS
            // are taken, and block mb+2's operands are read before that.
            bf16x8 pf[2], dsf[2];
            bf16x8 qa[4][NS], da[4][NS];
            f32x4 l4[4], d4[4], s4[4], p4[4];
            auto rd = [&](int mb) {
                const uint32_t qb = mb < 2 ? qh0 : qh1, dbb = mb < 2 ? dh0 : dh1;
                const uint32_t rimm = (mb & 1) * R16;
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    qa[mb][s] = *(const lds_bf16x8b*)(uintptr_t)(qb + ro[s] + rimm);
                    da[mb][s] = *(const lds_bf16x8b*)(uintptr_t)(dbb + ro[s] + rimm);
                }
                const int q0 = 16 * mb + 4 * G;
                l4[mb] = *(const f32x4*)&lse_t[q0];
                d4[mb] = *(const f32x4*)&del_t[q0];
            };
            auto mm = [&](int mb) {
                s4[mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
                p4[mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    s4[mb] = mma16(qa[mb][s], kf[s], s4[mb]);
                    p4[mb] = mma16(da[mb][s], vf[s], p4[mb]);
                }
            };
            // A pad query row has lse2 = +inf (set by the delta kernel): its
            // probabilities are exp2(-inf) = 0 with no mask.
            auto pds = [&](int mb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float pr = __builtin_amdgcn_exp2f(s4[mb][r] * scale_log2 - l4[mb][r]);
                    pf[mb >> 1][4 * (mb & 1) + r] = (__bf16)pr;
                    dsf[mb >> 1][4 * (mb & 1) + r] = (__bf16)(pr * (p4[mb][r] - d4[mb][r]));
                }
            };
            rd(0);
            rd(1);
            __builtin_amdgcn_sched_barrier(0);
            mm(0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                if (mb + 2 < 4) rd(mb + 2);
                __builtin_amdgcn_sched_barrier(0);
                if (mb + 1 < 4) mm(mb + 1);
                __builtin_amdgcn_sched_barrier(0);
                pds(mb);
                __builtin_amdgcn_sched_barrier(0);
            }
            // dV^T += dO^T P and dK^T += Q^T dS over two 32-query steps (step ks
            // reads the ks-th half-tiles), in groups of four products over four
            // d blocks: group g is step g / (NDB/2), d blocks 4*((g/2) % (NDB/4))
            // + [0, 4), dV (g even, dO^T operands) or dK (g odd, Q^T operands).
            // The operands of group g+1 are read while group g multiplies.
            constexpr int NG = NDB;  // 2 steps x NDB/4 block groups x (dV, dK)
            bf16x8 ta[2][4];
            auto rd2 = [&](int gi) {
                const int ks = gi / (NG / 2), db0i = 4 * ((gi >> 1) % (NDB / 4));
                const uint32_t base = (gi & 1) ? (ks ? qh1 : qh0) : (ks ? dh1 : dh0);
#pragma unroll
                for (int u = 0; u < 4; ++u) ta[gi & 1][u] = kv_tr16o(base + to[db0i + u], R16);
            };
            auto mm2 = [&](int gi) {
                const int ks = gi / (NG / 2), db0i = 4 * ((gi >> 1) % (NDB / 4));
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (gi & 1)
                        adk[db0i + u] = mma16(ta[1][u], dsf[ks], adk[db0i + u]);
                    else
                        adv[db0i + u] = mma16(ta[0][u], pf[ks], adv[db0i + u]);
                }
            };
            rd2(0);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                if (gi + 1 < NG) rd2(gi + 1);
                __builtin_amdgcn_sched_barrier(0);
                mm2(gi);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        read_ahead();
    }
    // Lane holds dV^T, dK^T[d = 16*db + 4*G + r][key kj].
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        bf16x4 wv, wk;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            wv[r] = (__bf16)(kvalid ? adv[db][r] : 0.f);
            wk[r] = (__bf16)(kvalid ? adk[db][r] * scale : 0.f);
        }
        *(bf16x4*)(dv + koff + 16 * db + 4 * G) = wv;
        *(bf16x4*)(dk + koff + 16 * db + 4 * G) = wk;
    }
}

// ------------------------------------------------------------------ launcher
// Device scratch of attn_block_sparse_bwd_noalloc: the same workspace
// (rowsum(dO*O), the base-2 lse and the CSR's transpose) in a static array, so that callers
// that cannot allocate (graph capture, tight serving loops) need no
// workspace argument.  Every GPU the library runs on holds its own copy
// until the process ends.  Each call writes every word of it that its
// kernels read before they read it, so no clearing is needed; calls that
// overlap on one GPU share it and race.
static __device__ __align__(256) char scratch[kBwdScratchBytes];

// Device address of `scratch` on the current device.  On the host the
// array's name is only a host-side stand-in, so the address is looked up
// with hipGetSymbolAddress, once per device with that device current, and
// kept; callers pass it to the kernels like any workspace pointer.
hipError_t bwd_scratch(void** out) {
    static std::mutex mu;
    static void* ptrs[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

hipError_t launch_attn_bwd(const Geo& g, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len,
                           float scale, void* dq, void* dk, void* dv, float* delta,
                           int32_t* col_start, int32_t* col_cnt, int32_t* row_idx,
                           hipStream_t stream) {
    const int64_t slots = (int64_t)g.B * g.Lpad * g.H;
    // The workspace's delta region holds rowsum(dO*O), then log2(e)*lse.
    float* const lse2 = delta + (int64_t)g.B * g.H * g.Lpad;
    const unsigned dblocks = (unsigned)((slots + 255) / 256);
    const unsigned items = (unsigned)((int64_t)g.B * g.H * g.Nt * g.sub);  // 64-slot units
    const int csc_blocks = g.B * g.H;  // the dq launch's first workgroups: the CSR transpose
    const __bf16 *Q = (const __bf16*)q, *K = (const __bf16*)k, *V = (const __bf16*)v,
                 *O = (const __bf16*)o, *DO = (const __bf16*)dO;
    if (g.D == 128)
        hipLaunchKernelGGL(bwd_delta_kernel<128>, dim3(dblocks), dim3(256), 0, stream, g, O, DO, lse,
                           delta, lse2);
    else
        hipLaunchKernelGGL(bwd_delta_kernel<64>, dim3(dblocks), dim3(256), 0, stream, g, O, DO, lse,
                           delta, lse2);
    if (g.D == 128) {
        hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3(csc_blocks + items), dim3(256), 0, stream, g, Q, K,
                           V, DO, lse, (const float*)delta, row_ptr, col_idx, col_len, scale,
                           (__bf16*)dq, csc_blocks, col_start, col_cnt, row_idx);
        hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3(items), dim3(256), 0, stream, g, Q, K, V, DO,
                           (const float*)lse2, (const float*)delta, (const int32_t*)col_start,
                           (const int32_t*)col_cnt, (const int32_t*)row_idx, col_len, scale,
                           (__bf16*)dk, (__bf16*)dv);
    } else {
        hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3(csc_blocks + items), dim3(256), 0, stream, g, Q, K,
                           V, DO, lse, (const float*)delta, row_ptr, col_idx, col_len, scale,
                           (__bf16*)dq, csc_blocks, col_start, col_cnt, row_idx);
        hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3(items), dim3(256), 0, stream, g, Q, K, V, DO,
                           (const float*)lse2, (const float*)delta, (const int32_t*)col_start,
                           (const int32_t*)col_cnt, (const int32_t*)row_idx, col_len, scale,
                           (__bf16*)dk, (__bf16*)dv);
    }
    return hipGetLastError();
}

}  // namespace bsta
