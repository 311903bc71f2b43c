// Fused block-sparse flash-attention forward for gfx950 (CDNA4).
//
// Method ("bsa_attn" page, forward / _compute_sparse_attention; __init__
// fixes the scale to 1/sqrt(d) and rules out causal masking): for query tile
// i of head h, attention runs over the valid tokens of the key tiles listed
// in CSR row (b*H + h)*Nt + i, with an online (streaming) softmax.
//
// Work decomposition: a workgroup of two wave64s owns one query tile (64
// rows); wave w owns query rows 32w..32w+31 for the whole key list.  Four
// such workgroups share a CU, so each SIMD runs two waves whose softmax and
// MFMA phases overlap.  Per selected key tile:
//   1. K and V arrive in LDS by direct global->LDS DMA (global_load_lds_
//      dwordx4, 1 KB per instruction; each wave issues half of the blocks)
//      into a ring of five half-tile slots (32 keys x D): K low half, K high
//      half, V low, V high, then the next tile.  Before a slot is read, one
//      workgroup barrier both publishes it and retires the previous slot,
//      which is then refilled with the half-tile five places ahead, so up to
//      four half-tiles are in flight while one is read.  Rows are XOR-
//      swizzled in 16-byte chunks so every read below is free of bank
//      conflicts (64 banks).
//   2. S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys as M, queries as N): each
//      lane ends up holding the scores of a single query.
//   3. Online softmax in the exp2 domain (log2(e)/sqrt(D) folded into the
//      scale); the row max needs one cross-lane exchange (lane ^ 32), the row
//      sum stays per lane until the end.  The reference max is raised (and
//      O, l rescaled) only when a row max exceeds it by more than 2^8.
//   4. O^T += V^T P^T on the same MFMA.  The accumulator layout of step 2 is
//      the B-operand layout this product needs, up to a fixed permutation of
//      the 16 keys of each k-step; the A operand (V^T) comes from row-major V
//      through the LDS transpose read ds_read_b64_tr_b16, four keys at a time
//      in exactly that permuted order.
// Partial key tiles (n_j < 64) mask keys r >= n_j to -inf; padded query rows
// are written as +0.0.  Out-of-range tile ids contribute nothing.
//
// Lane layouts used (gfx950, checked on hardware):
//   v_mfma_f32_32x32x16_bf16: A[m][k] in lane m + 32*(k/8), element k%8;
//     B[k][n] in lane n + 32*(k/8), element k%8; register r of lane l holds
//     D[8*(r/4) + 4*(l/32) + r%4][l%32].
//   ds_read_b64_tr_b16, per 16-lane group: if lane s addresses 4 elements
//     C_s, lane d receives C_{d/4 + 4m}[d%4] for m = 0..3.
//   global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + 16*l.
#include "bsta_common.hpp"

namespace bsta {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kRing = 5;  // half-tile slots per wave

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// XOR swizzles of 16-byte chunks, as a function of the row inside a 32-row
// half-tile.  Chosen (and checked against both a 32-bank and a 64-bank LDS
// model) so that the 16-byte K operand reads and the 8-byte V transpose
// reads of a wave hit distinct banks.
template <int D>
__device__ inline int k_phys(int r, int c) {
    if constexpr (D == 128) return c ^ (r & 15);
    else return c ^ ((r ^ (r >> 3)) & 7);
}

template <int D>
__device__ inline int v_phys(int r, int c) {
    if constexpr (D == 128) return c ^ ((r & 3) * 2 + (r & 1) * 8);
    else return c ^ ((r & 3) << 1);
}

// LDS byte address of a __shared__ object.
__device__ inline uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Issue this wave's NI blocks (1 KB each) of one half-tile (32 rows x D bf16)
// by direct-to-LDS DMA: its block u lands at LDS byte lds0 + 2048*u (the two
// waves interleave).  `voff` holds the per-lane source byte offsets from
// `base`.  Written as inline asm so that the compiler does
// not guard every later LDS read with a wait for all outstanding DMA; the
// kernel waits on vmcnt itself.  M0 (the DMA's LDS base) is saved and
// restored around the block.
template <int NI>
__device__ inline void dma_half(const __bf16* base_any, const int32_t* voff, uint32_t lds_any) {
    // Both bases are wave-uniform; make them SGPRs.  (readfirstlane returns
    // int: go through uint32_t so the low half is never sign-extended.)
    const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane(lds_any);
    const uint64_t b64 = (uint64_t)(uintptr_t)base_any;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64);
    const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
    uint32_t saved;
    if constexpr (NI == 4) {
        asm volatile(
            "s_mov_b32 %[t], m0\n\t"
            "s_mov_b32 m0, %[l]\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[v0], %[b]\n\t"
            "s_add_u32 m0, m0, 2048\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[v1], %[b]\n\t"
            "s_add_u32 m0, m0, 2048\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[v2], %[b]\n\t"
            "s_add_u32 m0, m0, 2048\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[v3], %[b]\n\t"
            "s_mov_b32 m0, %[t]"
            : [t] "=&s"(saved)
            : [l] "s"(lds0), [b] "s"(base), [v0] "v"(voff[0]), [v1] "v"(voff[1]),
              [v2] "v"(voff[2]), [v3] "v"(voff[3])
            : "memory", "scc");
    } else {
        static_assert(NI == 2, "half-tile of 32 x 64 or 32 x 128 bf16, two waves");
        asm volatile(
            "s_mov_b32 %[t], m0\n\t"
            "s_mov_b32 m0, %[l]\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[v0], %[b]\n\t"
            "s_add_u32 m0, m0, 2048\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[v1], %[b]\n\t"
            "s_mov_b32 m0, %[t]"
            : [t] "=&s"(saved)
            : [l] "s"(lds0), [b] "s"(base), [v0] "v"(voff[0]), [v1] "v"(voff[1])
            : "memory", "scc");
    }
}

// Wait until at most `newer` half-tiles issued after the one about to be
// read are still in flight (each half-tile is NI DMA instructions).
template <int NI>
__device__ inline void wait_dma(int newer) {
    if constexpr (NI == 4) {
        switch (newer) {
            case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
            case 1: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
            case 2: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
            default: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
        }
    } else {
        switch (newer) {
            case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
            case 1: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
            case 2: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
            default: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
        }
    }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(
        Geo g, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
        const __bf16* __restrict__ v, const int32_t* __restrict__ row_ptr,
        const int32_t* __restrict__ col_idx, int64_t col_len, float scale_log2,
        __bf16* __restrict__ o, float* __restrict__ lse, int64_t items_per_xcd) {
    constexpr int NDC = D / 16;                    // MFMA k-steps for S (16 d each)
    constexpr int NDB = D / 32;                    // 32-row d blocks of O^T
    constexpr int HALF_ELEMS = 32 * D;             // one half-tile slot
    constexpr int NI = HALF_ELEMS * 2 / 1024 / 2;  // DMA instructions per wave per half-tile
    __shared__ __attribute__((aligned(1024))) __bf16 ring[kRing * HALF_ELEMS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, half = lane >> 5;
    const int64_t rs = (int64_t)g.H * D;  // elements between consecutive tokens

    // Per-lane DMA source offsets (bytes, relative to the half-tile's first
    // row) of this wave's blocks: block t = wave + 2u covers slot bytes
    // [1024t, 1024t+1024), i.e. row r = (1024t + 16*lane) / (2D), physical
    // chunk p; the lane fetches the logical chunk the swizzle stores at p.
    int32_t koff[NI], voff[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const int byte = (wave + 2 * u) * 1024 + lane * 16;
        const int r = byte / (2 * D);
        const int p = (byte % (2 * D)) / 16;
        koff[u] = 2 * ((int32_t)(r * rs) + k_phys<D>(r, p) * 8);
        voff[u] = 2 * ((int32_t)(r * rs) + v_phys<D>(r, p) * 8);
    }
    const uint32_t ring_lds = lds_addr(ring) + wave * 1024;

    // V^T transpose-read addresses inside a half-tile slot: lane group
    // G = lane/16 covers d = db*32 + 16*(G%2) + [0,16) and keys
    // 16*(kc%2) + 4*half + [0,4) (+8 for the second read); source lane
    // s = lane%16 points at key row kbase + s/4, d offset 4*(s%4).  The
    // swizzle depends on the row only through r%4, equal for all of them.
    const int s16 = lane & 15, dsub = (lane >> 4) & 1;
    const int vrow0 = 4 * half + (s16 >> 2);     // + 16*(kc%2) (+8)
    const int vcol = 16 * dsub + 4 * (s16 & 3);  // + db*32
    int vaddr[NDB];                              // element offsets for kc%2 = 0, first read
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int c = db * 32 + vcol;
        vaddr[db] = vrow0 * D + v_phys<D>(vrow0, c >> 3) * 8 + (c & 7);
    }
    const int qi = wave * 32 + l32;  // this lane's query row in the tile

    // Persistent, XCD-aware schedule.  Workgroups are dealt round-robin over
    // the 8 XCDs, so workgroup w runs on XCD w%8.  XCD e owns the contiguous
    // run [e*items_per_xcd, (e+1)*items_per_xcd) of query tiles in (b, h, i)
    // order; its resident workgroups take them in rounds of S.
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int S = gridDim.x >> 3;
    const int64_t n_items = (int64_t)g.B * g.H * g.Nt;
    const int64_t first = (int64_t)xcd * items_per_xcd;
    const int64_t last = first + items_per_xcd < n_items ? first + items_per_xcd : n_items;

    for (int64_t item = first + slot; item < last; item += S) {
        const int bh = (int)(item / g.Nt);
        const int i = (int)(item - (int64_t)bh * g.Nt);
        const int b = bh / g.H, h = bh - b * g.H;
        const int64_t head_off = (int64_t)h * D;
        const int64_t batch_row0 = (int64_t)b * g.Lpad;

        int64_t p0 = row_ptr[item], p1 = row_ptr[item + 1];
        p0 = p0 < 0 ? 0 : (p0 > col_len ? col_len : p0);
        p1 = p1 < p0 ? p0 : (p1 > col_len ? col_len : p1);
        const int n = (int)(p1 - p0);
        const int nseq = 4 * n;  // half-tiles in consumption order

        // Tile id at CSR position p, or -1 when out of range (then tile 0 is
        // fetched and fully masked, keeping the pipeline uniform).
        auto tile_at = [&](int64_t p) -> int {
            const int j = col_idx[p];
            return (unsigned)j < (unsigned)g.Nt ? j : -1;
        };
        auto tile_rows = [&](int j) -> const int64_t {
            return (batch_row0 + (int64_t)(j < 0 ? 0 : j) * 64) * rs + head_off;
        };
        // Half-tiles are consumed in the order K0lo K0hi V0lo V0hi K1lo ...;
        // half-tile s lives in ring slot s % kRing.
        const uint32_t slot_bytes = HALF_ELEMS * 2;
        auto dma = [&](const __bf16* src, const int32_t* off, int slot_idx) {
            dma_half<NI>(src, off, ring_lds + (uint32_t)slot_idx * slot_bytes);
        };
        // Wait for this wave's DMA of the half-tile about to be read (with
        // `newer` later half-tiles allowed in flight) and for its own reads of
        // the previous slot, then barrier: the half-tile is visible to both
        // waves and the previous slot is retired.
        auto acquire = [&](int newer) {
            wait_dma<NI>(newer);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
        };

        // Query fragment (B operand of S^T = K Q^T): query row qi,
        // d = 16*dc + 8*half.
        bf16x8 qf[NDC];
        const __bf16* qrow = q + (batch_row0 + (int64_t)i * 64 + qi) * rs + head_off;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) qf[dc] = *(const bf16x8*)(qrow + dc * 16 + half * 8);
        // Make the compiler wait for the query loads here, before the DMA: it
        // cannot see the DMA issued by inline asm, and a wait for these loads
        // placed inside the key loop would also drain the in-flight DMA.
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) asm volatile("" ::"v"(qf[dc]));

        // Prologue: half-tiles 0..3 (all of tile 0) into slots 0..3.  Every
        // slot of the previous item was retired behind a barrier.
        int slot0 = 0;  // ring slot of half-tile 4t
        if (n > 0) {
            const int64_t r0 = tile_rows(tile_at(p0));
            dma(k + r0, koff, 0);
            dma(k + r0 + 32 * rs, koff, 1);
            dma(v + r0, voff, 2);
            dma(v + r0 + 32 * rs, voff, 3);
        }

        f32x16 oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
        float m_run = -INFINITY, l_run = 0.f;
        int jt = n > 0 ? tile_at(p0) : -1;

        for (int t = 0; t < n; ++t) {
            const bool more = t + 1 < n;  // tile t+1 exists: its 4 half-tiles are issued now
            const int jn = more ? tile_at(p0 + t + 1) : -1;
            const int64_t rn = tile_rows(jn);
            const int nj = jt < 0 ? 0 : tile_occupancy(g, jt);
            // Slots: half-tile 4t+p in (slot0 + p) % 5; 4(t+1)+p in (slot0 + 4 + p) % 5.
            const int sl1 = slot0 == 4 ? 0 : slot0 + 1;
            const int sl2 = sl1 == 4 ? 0 : sl1 + 1;
            const int sl3 = sl2 == 4 ? 0 : sl2 + 1;
            const int sl4 = sl3 == 4 ? 0 : sl3 + 1;
            const int sls[4] = {slot0, sl1, sl2, sl3};
            // Issue order of tile t+1: Klo -> slot sl4, Khi -> slot0, Vlo -> sl1, Vhi -> sl2.
            // In flight before reading half-tile 4t+p: through 4t+3+p.
            const int in_flight = more ? 3 : 0;  // later half-tiles of the sequence

            // S^T = K Q^T, key block kb from half-tile 4t + kb.
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                acquire(more ? 3 : 3 - kb);  // tile t: 4t+kb..4t+3 issued, maybe 4t+4..
                if (more) {
                    if (kb == 0) dma(k + rn, koff, sl4);           // K lo of t+1 into retired slot
                    else dma(k + rn + 32 * rs, koff, slot0);       // K hi of t+1
                }
                const __bf16* kslot = ring + sls[kb] * HALF_ELEMS;
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
                for (int d0 = 0; d0 < NDC; d0 += 4) {
                    bf16x8 a[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        a[u] = *(const bf16x8*)(kslot + l32 * D + k_phys<D>(l32, (d0 + u) * 2 + half) * 8);
#pragma unroll
                    for (int u = 0; u < 4; ++u) sacc[kb] = mfma32(a[u], qf[d0 + u], sacc[kb]);
                }
            }

            // Online softmax for query qi on raw scores (the scale is > 0), with
            // a lazily raised reference max.  Key of (kb, r): 32kb + 8(r/4) +
            // 4half + r%4.
            if (nj < 64) {  // partial tile: mask keys r >= n_j (tile-uniform)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                        if (key >= nj) sacc[kb][r] = -INFINITY;
                    }
            }
            float mx = sacc[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = (kb == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = fmaxf(mx, wave_xor32(mx)) * scale_log2;
            const bool raise = mx > m_run + 8.0f;
            if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform, rare
                const float m_new = raise ? mx : m_run;
                const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            }
            const float neg_m = m_run == -INFINITY ? 0.f : -m_run;  // all masked so far: p = 0
            float psum = 0.f;
            bf16x8 pf[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], scale_log2, neg_m));
                    psum += pv;
                    pf[kb * 2 + (r >> 3)][r & 7] = (__bf16)pv;
                }
            l_run += psum;

            // O^T += V^T P^T: 16-key steps kc; keys 0..31 in half-tile 4t+2,
            // keys 32..63 in half-tile 4t+3.
#pragma unroll
            for (int vh = 0; vh < 2; ++vh) {
                acquire(more ? 3 : 1 - vh);
                if (more) {
                    if (vh == 0) dma(v + rn, voff, sl1);
                    else dma(v + rn + 32 * rs, voff, sl2);
                }
                const __bf16* vslot = ring + sls[2 + vh] * HALF_ELEMS;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    bf16x8 av[NDB];
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const __bf16* a0 = vslot + vaddr[db] + kk * 16 * D;
                        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a0);
                        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 8 * D));
                        const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        av[db] = __builtin_bit_cast(bf16x8, w);
                    }
#pragma unroll
                    for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(av[db], pf[vh * 2 + kk], oacc[db]);
                }
            }
            (void)in_flight;
            slot0 = sl4;
            jt = jn;
        }
        // Retire the last slot before the next item refills the ring.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();

        // Finalise: l is split over lanes l and l^32.
        const int ni = tile_occupancy(g, i);
        const float l_tot = l_run + wave_xor32(l_run);
        const bool valid = qi < ni && l_tot > 0.f;
        const float inv = valid ? 1.0f / l_tot : 0.f;
        __bf16* orow = o + (batch_row0 + (int64_t)i * 64 + qi) * rs + head_off;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 outv;
#pragma unroll
                for (int u = 0; u < 4; ++u)  // pad rows: +0.0
                    outv[u] = (__bf16)(valid ? oacc[db][r4 * 4 + u] * inv : 0.f);
                *(bf16x4*)(orow + db * 32 + r4 * 8 + half * 4) = outv;
            }
        if (lse != nullptr && half == 0) {
            const float val = valid ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
            lse[(int64_t)bh * g.Lpad + (int64_t)i * 64 + qi] = val;
        }
    }
}

namespace {

// Workgroups of the attention kernel resident per XCD on the current device
// (computed once per device and kernel).
int resident_per_xcd(const void* kernel) {
    static int cache[2][64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 16;
    const int which = kernel == (const void*)attn_fwd_kernel<128> ? 0 : 1;
    if (cache[which][dev] > 0) return cache[which][dev];
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 128, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0) {
        cus = 256;
        per_cu = 4;
    }
    const int r = (cus / 8) * per_cu;
    cache[which][dev] = r > 0 ? r : 1;
    return cache[which][dev];
}

}  // namespace

hipError_t launch_attn_fwd(const Geo& g, const void* q, const void* k, const void* v,
                           const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len,
                           float scale, void* o, float* lse, hipStream_t stream) {
    const float scale_log2 = scale * 1.4426950408889634f;
    const void* kernel =
        g.D == 128 ? (const void*)attn_fwd_kernel<128> : (const void*)attn_fwd_kernel<64>;
    const int64_t n_items = (int64_t)g.B * g.H * g.Nt;
    const int64_t items_per_xcd = (n_items + 7) / 8;
    int64_t per_xcd = resident_per_xcd(kernel);
    if (per_xcd > items_per_xcd) per_xcd = items_per_xcd;
    const unsigned blocks = (unsigned)(8 * per_xcd);
    if (g.D == 128)
        hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3(blocks), dim3(128), 0, stream, g,
                           (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, row_ptr, col_idx,
                           col_len, scale_log2, (__bf16*)o, lse, items_per_xcd);
    else
        hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3(blocks), dim3(128), 0, stream, g,
                           (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, row_ptr, col_idx,
                           col_len, scale_log2, (__bf16*)o, lse, items_per_xcd);
    return hipGetLastError();
}

}  // namespace bsta
