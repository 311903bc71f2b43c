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
// Four kernels:
//   delta     rowsum(dO * O) per query slot (fp32).
//   csc       per (batch, head), the transpose of the CSR: for every key
//             tile the query tiles whose rows list it, in row order, so that
//             the dK/dV sums run in a fixed order.
//   dq        one workgroup of two waves per query tile, walking its CSR
//             row: S^T = K Q^T and dP^T = V dO^T on the matrix cores (keys
//             as M, queries as N, so each lane holds one query), then
//             dQ^T += K^T dS^T with K^T read by LDS transpose reads.
//   dkdv      one workgroup of two waves per key tile, walking its CSC
//             column: S = Q K^T and dP = dO V^T (queries as M, keys as N, so
//             each lane holds one key), then dV^T += dO^T P and
//             dK^T += Q^T dS.
// The products use v_mfma_f32_32x32x16_bf16 with the lane layouts of the
// forward kernel (checked on hardware there): A[m][k] in lane m + 32*(k/8),
// element k%8; B[k][n] in lane n + 32*(k/8), element k%8; accumulator
// register r of lane l holds D[8*(r/4) + 4*(l/32) + r%4][l%32].  A score
// accumulator converted to bf16 in chunks of 8 registers is the B operand of
// the next product over the same 16 keys (or queries) in a fixed permuted
// order; ds_read_b64_tr_b16 reads the A operand in exactly that order (per
// 16-lane group, lane d receives element d%4 of the value addressed by lane
// d/4 + 4m, m = 0..3).
//
// Tiles are staged in LDS (rows padded by 16 bytes) from registers loaded
// one tile ahead, so the next tile's loads overlap the products; P and
// dS are rounded to bf16 for the second product, accumulators are fp32 and
// each gradient is rounded once to bf16 at the end.  Pad query rows and pad
// key rows contribute nothing and are written as +0.0.
#include "bsta_common.hpp"

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

// 8 bf16 of LDS row `row`, starting at element `col` (16-byte aligned).
__device__ inline bf16x8 lds_row8(uint32_t base, int lstr, int row, int col) {
    return *(const lds_bf16x8b*)(uintptr_t)(base + (uint32_t)(row * lstr + 2 * col));
}

// A operand (transposed) of a product over 16 rows of an LDS tile: rows
// 16*step + 4*half + [0,4) and +8, columns 32*db + 16*dsub + 4*(s16%4) for
// source lane s16 (see the header for the transpose read).
__device__ inline bf16x8 lds_tr8(uint32_t base, int lstr, int step, int db, int lane) {
    const int s16 = lane & 15, dsub = (lane >> 4) & 1, half = lane >> 5;
    const int row = 16 * step + 4 * half + (s16 >> 2);
    const int col = 32 * db + 16 * dsub + 4 * (s16 & 3);
    const uint32_t a0 = base + (uint32_t)(row * lstr + 2 * col);
    const i16x4b lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4b*)(uintptr_t)a0);
    const i16x4b hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4b*)(uintptr_t)(a0 + 8 * lstr));
    const i16x8b w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
}

// Copy of the 64 slot rows of a tile (D bf16 each, global row stride `rs`
// elements) into LDS rows of `lstr` bytes, in two halves so that the loads
// of the next tile can be in flight while the current one is used:
// load_tile fills this thread's NCH chunks (16 bytes each) into registers,
// store_tile writes them to LDS.
template <int D>
struct TileRegs {
    static constexpr int NCH = 64 * (D / 8) / 128;  // chunks per thread (128 threads)
    u32x4 c[NCH];
};

template <int D>
__device__ inline void load_tile(TileRegs<D>& r, const __bf16* src, int64_t rs) {
    constexpr int CH = D / 8;
#pragma unroll
    for (int n = 0; n < TileRegs<D>::NCH; ++n) {
        const int c = threadIdx.x + 128 * n;
        const int row = c / CH, k = c - row * CH;
        r.c[n] = *(const u32x4*)(src + (int64_t)row * rs + k * 8);
    }
}

template <int D>
__device__ inline void store_tile(const TileRegs<D>& r, char* lds, int lstr) {
    constexpr int CH = D / 8;
#pragma unroll
    for (int n = 0; n < TileRegs<D>::NCH; ++n) {
        const int c = threadIdx.x + 128 * n;
        const int row = c / CH, k = c - row * CH;
        *(u32x4*)(lds + row * lstr + k * 16) = r.c[n];
    }
}

}  // namespace

// ------------------------------------------------------------------ delta
// One thread per (batch, slot, head): delta = sum_d dO * O in fp32.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(Geo g, const __bf16* __restrict__ o,
                                                        const __bf16* __restrict__ dO,
                                                        float* __restrict__ delta) {
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
    delta[(b * g.H + h) * g.Lpad + slot] = acc;
}

// ------------------------------------------------------------------ csc
// One workgroup of 1024 threads per (batch, head).  LDS: cnt, start, cur
// (Nt ints each).  Column j of head bh lists, in row order, the query tiles
// whose CSR rows hold j; it occupies row_idx[col_start[bh*Nt + j] + [0,
// col_cnt[bh*Nt + j])), inside the head's own CSR range.  Row ranges are
// clamped to [0, col_len) and ids outside [0, Nt) are skipped; rows must
// hold distinct ids (a repeated id leaves a slot of its column unwritten,
// which the dK/dV kernel's range check then skips or reads as some row).
__global__ __launch_bounds__(1024) void bwd_csc_kernel(Geo g, const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ col_idx,
                                                       int64_t col_len, int32_t* __restrict__ col_start,
                                                       int32_t* __restrict__ col_cnt,
                                                       int32_t* __restrict__ row_idx) {
    extern __shared__ int sm[];
    __shared__ int part[1024];
    const int Nt = g.Nt;
    int* cnt = sm;
    int* start = sm + Nt;
    int* cur = sm + 2 * Nt;
    const int tid = threadIdx.x;
    const int64_t base = (int64_t)blockIdx.x * Nt;
    auto clampp = [&](int64_t p) { return p < 0 ? (int64_t)0 : (p > col_len ? col_len : p); };
    for (int j = tid; j < Nt; j += 1024) {
        cnt[j] = 0;
        cur[j] = 0;
    }
    __syncthreads();
    for (int i = tid; i < Nt; i += 1024) {
        const int64_t p0 = clampp(row_ptr[base + i]);
        const int64_t p1 = clampp(row_ptr[base + i + 1]);
        for (int64_t p = p0; p < p1; ++p) {
            const int j = col_idx[p];
            if ((unsigned)j < (unsigned)Nt) atomicAdd(&cnt[j], 1);
        }
    }
    __syncthreads();
    // Exclusive scan of cnt: each thread a run of `per` columns.
    const int per = (Nt + 1023) / 1024;
    const int j0 = tid * per < Nt ? tid * per : Nt;
    const int j1 = j0 + per < Nt ? j0 + per : Nt;
    int s = 0;
    for (int j = j0; j < j1; ++j) s += cnt[j];
    part[tid] = s;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int run = part[tid] - s;
    for (int j = j0; j < j1; ++j) {
        start[j] = run;
        run += cnt[j];
    }
    __syncthreads();
    const int64_t head_off = clampp(row_ptr[base]);
    for (int j = tid; j < Nt; j += 1024) {
        col_start[base + j] = (int32_t)(head_off + start[j]);
        col_cnt[base + j] = cnt[j];
    }
    // Fill in row order: one row at a time, its (distinct) ids in parallel.
    for (int i = 0; i < Nt; ++i) {
        const int64_t p0 = clampp(row_ptr[base + i]);
        const int64_t p1 = clampp(row_ptr[base + i + 1]);
        for (int64_t p = p0 + tid; p < p1; p += 1024) {
            const int j = col_idx[p];
            if ((unsigned)j < (unsigned)Nt) {
                const int r = cur[j];
                cur[j] = r + 1;
                const int64_t pos = head_off + start[j] + r;
                if (pos < col_len) row_idx[pos] = i;
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ dq
template <int D>
__global__ __launch_bounds__(128) void bwd_dq_kernel(
        Geo g, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
        const __bf16* __restrict__ v, const __bf16* __restrict__ dO,
        const float* __restrict__ lse, const float* __restrict__ delta,
        const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t col_len,
        float scale, __bf16* __restrict__ dq) {
    constexpr int NDC = D / 16, NDB = D / 32, LSTR = 2 * D + 16;
    __shared__ __attribute__((aligned(16))) char kt[64 * LSTR];
    __shared__ __attribute__((aligned(16))) char vt[64 * LSTR];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t item = blockIdx.x;
    const int i = (int)(item % g.Nt);
    const int64_t bh = item / g.Nt;
    const int h = (int)(bh % g.H);
    const int64_t b = bh / g.H;
    const int64_t rs = (int64_t)g.H * D;
    const int qi = wave * 32 + l32;
    const int ni = tile_occupancy(g, i);
    const bool qvalid = qi < ni;
    const int64_t qslot = (int64_t)i * 64 + qi;
    const int64_t qoff = ((b * g.Lpad + qslot) * g.H + h) * D;
    bf16x8 qf[NDC], df[NDC];
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
        qf[dc] = *(const bf16x8*)(q + qoff + dc * 16 + half * 8);
        df[dc] = *(const bf16x8*)(dO + qoff + dc * 16 + half * 8);
    }
    const float lse2 = qvalid ? lse[bh * g.Lpad + qslot] * kLog2e : 0.f;
    const float dl = qvalid ? delta[bh * g.Lpad + qslot] : 0.f;
    const float scale_log2 = scale * kLog2e;
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = (f32x16){};
    int64_t p0 = row_ptr[bh * g.Nt + i], p1 = row_ptr[bh * g.Nt + i + 1];
    p0 = p0 < 0 ? 0 : (p0 > col_len ? col_len : p0);
    p1 = p1 < p0 ? p0 : (p1 > col_len ? col_len : p1);
    const uint32_t kb0 = lds_base(kt), vb0 = lds_base(vt);
    // Entries with ids outside [0, Nt) are skipped (workgroup-uniform).
    auto next_valid = [&](int64_t p) {
        while (p < p1 && (unsigned)col_idx[p] >= (unsigned)g.Nt) ++p;
        return p;
    };
    TileRegs<D> rk, rv;
    int64_t p = next_valid(p0);
    if (p < p1) {
        const int64_t koff = ((b * g.Lpad + (int64_t)col_idx[p] * 64) * g.H + h) * D;
        load_tile<D>(rk, k + koff, rs);
        load_tile<D>(rv, v + koff, rs);
    }
    while (p < p1) {
        const int j = col_idx[p];
        const int nj = tile_occupancy(g, j);
        __syncthreads();  // the previous tile's LDS reads are done
        store_tile<D>(rk, kt, LSTR);
        store_tile<D>(rv, vt, LSTR);
        __syncthreads();
        // Issue the next tile's loads; they complete while this one is used.
        p = next_valid(p + 1);
        if (p < p1) {
            const int64_t koff = ((b * g.Lpad + (int64_t)col_idx[p] * 64) * g.H + h) * D;
            load_tile<D>(rk, k + koff, rs);
            load_tile<D>(rv, v + koff, rs);
        }
        // Operand reads are issued as a batch ahead of their products (the
        // scheduling barriers keep the compiler from serialising each read
        // with its product).
        f32x16 s[2], dp[2];
        bf16x8 ka[2][NDC], va[2][NDC];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int dc = 0; dc < NDC; ++dc) {
                const int col = 16 * dc + 8 * half;
                ka[kb][dc] = lds_row8(kb0, LSTR, l32 + 32 * kb, col);
                va[kb][dc] = lds_row8(vb0, LSTR, l32 + 32 * kb, col);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = (f32x16){};
            dp[kb] = (f32x16){};
#pragma unroll
            for (int dc = 0; dc < NDC; ++dc) {
                s[kb] = mma(ka[kb][dc], qf[dc], s[kb]);
                dp[kb] = mma(va[kb][dc], df[dc], dp[kb]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // dS^T in four bf16 chunks of 16 keys (chunk c: key block c/2,
        // registers 8*(c%2) + [0, 8)).
        bf16x8 dsf[4];
        auto ds_chunk = [&](int c) {
            const int kb = c >> 1, r0 = (c & 1) * 8;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int rr = r0 + r;
                const int key = 32 * kb + 8 * (rr >> 2) + 4 * half + (rr & 3);
                const float pr = (qvalid && key < nj)
                                         ? __builtin_amdgcn_exp2f(s[kb][rr] * scale_log2 - lse2)
                                         : 0.f;
                dsf[c][r] = (__bf16)(pr * (dp[kb][rr] - dl));
            }
        };
        // dQ^T += K^T dS^T: the K^T reads and the dS chunk of step c+1 are
        // issued while the MFMAs of step c run.
        bf16x8 kt2[2][NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) kt2[0][db] = lds_tr8(kb0, LSTR, 0, db, lane);
        ds_chunk(0);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (c + 1 < 4) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) kt2[(c + 1) & 1][db] = lds_tr8(kb0, LSTR, c + 1, db, lane);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] = mma(kt2[c & 1][db], dsf[c], acc[db]);
            if (c + 1 < 4) ds_chunk(c + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
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
template <int D>
__global__ __launch_bounds__(128) void bwd_dkdv_kernel(
        Geo g, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
        const __bf16* __restrict__ v, const __bf16* __restrict__ dO,
        const float* __restrict__ lse, const float* __restrict__ delta,
        const int32_t* __restrict__ col_start, const int32_t* __restrict__ col_cnt,
        const int32_t* __restrict__ row_idx, int64_t col_len, float scale,
        __bf16* __restrict__ dk, __bf16* __restrict__ dv) {
    constexpr int NDC = D / 16, NDB = D / 32, LSTR = 2 * D + 16;
    __shared__ __attribute__((aligned(16))) char qt[64 * LSTR];
    __shared__ __attribute__((aligned(16))) char dt[64 * LSTR];
    __shared__ __attribute__((aligned(16))) float lse_s[64];
    __shared__ __attribute__((aligned(16))) float del_s[64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t item = blockIdx.x;
    const int j = (int)(item % g.Nt);
    const int64_t bh = item / g.Nt;
    const int h = (int)(bh % g.H);
    const int64_t b = bh / g.H;
    const int64_t rs = (int64_t)g.H * D;
    const int kj = wave * 32 + l32;
    const bool kvalid = kj < tile_occupancy(g, j);
    const int64_t koff = ((b * g.Lpad + (int64_t)j * 64 + kj) * g.H + h) * D;
    bf16x8 kf[NDC], vf[NDC];
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
        kf[dc] = *(const bf16x8*)(k + koff + dc * 16 + half * 8);
        vf[dc] = *(const bf16x8*)(v + koff + dc * 16 + half * 8);
    }
    const float scale_log2 = scale * kLog2e;
    f32x16 adv[NDB], adk[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        adv[db] = (f32x16){};
        adk[db] = (f32x16){};
    }
    int64_t c0 = col_start[bh * g.Nt + j];
    int64_t c1 = c0 + col_cnt[bh * g.Nt + j];
    c0 = c0 < 0 ? 0 : (c0 > col_len ? col_len : c0);
    c1 = c1 < c0 ? c0 : (c1 > col_len ? col_len : c1);
    const uint32_t qb0 = lds_base(qt), db0 = lds_base(dt);
    auto next_valid = [&](int64_t e) {
        while (e < c1 && (unsigned)row_idx[e] >= (unsigned)g.Nt) ++e;
        return e;
    };
    TileRegs<D> rq, rd;
    float nl = 0.f, nd = 0.f;
    auto prefetch = [&](int i) {
        const int64_t qoff = ((b * g.Lpad + (int64_t)i * 64) * g.H + h) * D;
        load_tile<D>(rq, q + qoff, rs);
        load_tile<D>(rd, dO + qoff, rs);
        if (threadIdx.x < 64) {
            const int t = threadIdx.x;
            const int64_t at = bh * g.Lpad + (int64_t)i * 64 + t;
            const bool ok = t < tile_occupancy(g, i);
            nl = ok ? lse[at] * kLog2e : 0.f;
            nd = ok ? delta[at] : 0.f;
        }
    };
    int64_t e = next_valid(c0);
    if (e < c1) prefetch(row_idx[e]);
    while (e < c1) {
        const int i = row_idx[e];
        const int ni = tile_occupancy(g, i);
        __syncthreads();
        store_tile<D>(rq, qt, LSTR);
        store_tile<D>(rd, dt, LSTR);
        if (threadIdx.x < 64) {
            lse_s[threadIdx.x] = nl;
            del_s[threadIdx.x] = nd;
        }
        __syncthreads();
        e = next_valid(e + 1);
        if (e < c1) prefetch(row_idx[e]);
        // Operand reads in batches of kBatch k-steps ahead of their products
        // (the scheduling barriers keep each read from being serialised
        // with its product).
        constexpr int kBatch = NDC < 8 ? NDC : 8;
        f32x16 s[2], dp[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            s[mb] = (f32x16){};
            dp[mb] = (f32x16){};
#pragma unroll
            for (int d0 = 0; d0 < NDC; d0 += kBatch) {
                bf16x8 qa[kBatch], da[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int col = 16 * (d0 + u) + 8 * half;
                    qa[u] = lds_row8(qb0, LSTR, l32 + 32 * mb, col);
                    da[u] = lds_row8(db0, LSTR, l32 + 32 * mb, col);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    s[mb] = mma(qa[u], kf[d0 + u], s[mb]);
                    dp[mb] = mma(da[u], vf[d0 + u], dp[mb]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // P and dS in bf16 chunks of 16 queries (chunk c: query block c/2,
        // registers 8*(c%2) + [0, 8); register rr holds query
        // 32*(c/2) + 8*(rr/4) + 4*half + rr%4).
        bf16x8 pf[4], dsf[4];
        auto p_chunk = [&](int c) {
            const int mb = c >> 1, r0 = (c & 1) * 8;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int q0 = 32 * mb + 8 * ((r0 >> 2) + rb) + 4 * half;
                const f32x4 l4 = *(const f32x4*)&lse_s[q0];
                const f32x4 d4 = *(const f32x4*)&del_s[q0];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int rr = r0 + 4 * rb + e;
                    const float pr = q0 + e < ni
                                             ? __builtin_amdgcn_exp2f(s[mb][rr] * scale_log2 - l4[e])
                                             : 0.f;
                    pf[c][4 * rb + e] = (__bf16)pr;
                    dsf[c][4 * rb + e] = (__bf16)(pr * (dp[mb][rr] - d4[e]));
                }
            }
        };
        // dV^T += dO^T P and dK^T += Q^T dS; the P and dS chunk of step c+1
        // is computed while the MFMAs of step c run.
        p_chunk(0);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bf16x8 ta[NDB];
#pragma unroll
            for (int db = 0; db < NDB; ++db) ta[db] = lds_tr8(db0, LSTR, c, db, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int db = 0; db < NDB; ++db) adv[db] = mma(ta[db], pf[c], adv[db]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int db = 0; db < NDB; ++db) ta[db] = lds_tr8(qb0, LSTR, c, db, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int db = 0; db < NDB; ++db) adk[db] = mma(ta[db], dsf[c], adk[db]);
            if (c + 1 < 4) p_chunk(c + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // Lane holds dV^T, dK^T[d = 32*db + 8*(r/4) + 4*half + r%4][key kj].
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            bf16x4 wv, wk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wv[e] = (__bf16)(kvalid ? adv[db][4 * rb + e] : 0.f);
                wk[e] = (__bf16)(kvalid ? adk[db][4 * rb + e] * scale : 0.f);
            }
            *(bf16x4*)(dv + koff + 32 * db + 8 * rb + 4 * half) = wv;
            *(bf16x4*)(dk + koff + 32 * db + 8 * rb + 4 * half) = wk;
        }
}

// ------------------------------------------------------------------ launcher
hipError_t launch_attn_bwd(const Geo& g, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len,
                           float scale, void* dq, void* dk, void* dv, float* delta,
                           int32_t* col_start, int32_t* col_cnt, int32_t* row_idx,
                           hipStream_t stream) {
    const int64_t slots = (int64_t)g.B * g.Lpad * g.H;
    const unsigned dblocks = (unsigned)((slots + 255) / 256);
    const unsigned items = (unsigned)((int64_t)g.B * g.H * g.Nt);
    const size_t csc_lds = (size_t)3 * g.Nt * sizeof(int);
    const __bf16 *Q = (const __bf16*)q, *K = (const __bf16*)k, *V = (const __bf16*)v,
                 *O = (const __bf16*)o, *DO = (const __bf16*)dO;
    if (g.D == 128)
        hipLaunchKernelGGL(bwd_delta_kernel<128>, dim3(dblocks), dim3(256), 0, stream, g, O, DO, delta);
    else
        hipLaunchKernelGGL(bwd_delta_kernel<64>, dim3(dblocks), dim3(256), 0, stream, g, O, DO, delta);
    hipLaunchKernelGGL(bwd_csc_kernel, dim3((unsigned)(g.B * g.H)), dim3(1024), csc_lds, stream, g,
                       row_ptr, col_idx, col_len, col_start, col_cnt, row_idx);
    if (g.D == 128) {
        hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3(items), dim3(128), 0, stream, g, Q, K, V, DO, lse,
                           (const float*)delta, row_ptr, col_idx, col_len, scale, (__bf16*)dq);
        hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3(items), dim3(128), 0, stream, g, Q, K, V, DO,
                           lse, (const float*)delta, (const int32_t*)col_start,
                           (const int32_t*)col_cnt, (const int32_t*)row_idx, col_len, scale,
                           (__bf16*)dk, (__bf16*)dv);
    } else {
        hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3(items), dim3(128), 0, stream, g, Q, K, V, DO, lse,
                           (const float*)delta, row_ptr, col_idx, col_len, scale, (__bf16*)dq);
        hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3(items), dim3(128), 0, stream, g, Q, K, V, DO,
                           lse, (const float*)delta, (const int32_t*)col_start,
                           (const int32_t*)col_cnt, (const int32_t*)row_idx, col_len, scale,
                           (__bf16*)dk, (__bf16*)dv);
    }
    return hipGetLastError();
}

}  // namespace bsta
