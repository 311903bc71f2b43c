// Fused block-sparse flash-attention forward for gfx950 (CDNA4).
//
// Method ("bsa_attn" page, forward / _compute_sparse_attention; __init__
// fixes the scale to 1/sqrt(d) and rules out causal masking): for query tile
// i of head h, attention runs over the valid tokens of the key tiles listed
// in CSR row (b*H + h)*Nt + i, with an online (streaming) softmax.
//
// Work decomposition: one workgroup of two wave64s per query tile (64
// rows); wave w owns query rows 32w..32w+31 for the whole key list.  For each
// selected key tile:
//   1. K and V (64 x D each) arrive in LDS by direct global->LDS DMA
//      (global_load_lds_dwordx4): no register staging.  Both are row-major
//      with an XOR swizzle of 16-byte chunks, chosen so that the reads below
//      are free of bank conflicts.  The next tile's K is fetched while this
//      tile's softmax and P.V run; the next tile's V while the next S runs.
//   2. S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys as M, queries as N): each
//      lane ends up holding scores of a single query.
//   3. Online softmax in the exp2 domain (log2(e)/sqrt(D) folded into the
//      scale); the row max needs one cross-lane exchange (lane ^ 32), the row
//      sum stays per lane until the end.
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
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// XOR swizzles of 16-byte chunks.  Chosen (and checked against both a
// 32-bank and a 64-bank LDS model) so that the 16-byte K operand reads and the
// 8-byte V transpose reads of each wave hit distinct banks.
// K row r, logical chunk c (D/8 chunks per row).
template <int D>
__device__ inline int k_phys(int r, int c) {
    if constexpr (D == 128) return c ^ (r & 15);
    else return c ^ ((r ^ (r >> 3)) & 7);
}

// V row r, logical chunk c.
template <int D>
__device__ inline int v_phys(int r, int c) {
    if constexpr (D == 128) return c ^ ((r & 3) * 2 + (r & 1) * 8);
    else return c ^ ((r & 3) << 1);
}

// LDS byte address of a __shared__ object.
__device__ inline uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Issue this wave's share of one 64 x D tile as 1 KB direct-to-LDS blocks:
// block u of the wave lands at LDS byte lds0 + 2048*u (the two waves
// interleave).  `voff` holds the per-lane source byte offsets from `base`.
// Written as inline asm so that the compiler does not guard every later LDS
// read with a wait for all outstanding DMA; the kernel waits on vmcnt
// itself.  M0 (the DMA's LDS base) is saved and restored around the block.
template <int NB>
__device__ inline void dma_tile(const __bf16* base_any, const int32_t* voff, uint32_t lds_any) {
    // Both the LDS base and the global base are wave-uniform; make them SGPRs.
    // (readfirstlane returns int: go through uint32_t so that the low half is
    // zero-extended, never sign-extended into the high half.)
    const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane(lds_any);
    const uint64_t b64 = (uint64_t)(uintptr_t)base_any;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64);
    const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
    uint32_t saved;
    if constexpr (NB == 8) {
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
            "s_add_u32 m0, m0, 2048\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[v4], %[b]\n\t"
            "s_add_u32 m0, m0, 2048\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[v5], %[b]\n\t"
            "s_add_u32 m0, m0, 2048\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[v6], %[b]\n\t"
            "s_add_u32 m0, m0, 2048\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[v7], %[b]\n\t"
            "s_mov_b32 m0, %[t]"
            : [t] "=&s"(saved)
            : [l] "s"(lds0), [b] "s"(base), [v0] "v"(voff[0]), [v1] "v"(voff[1]),
              [v2] "v"(voff[2]), [v3] "v"(voff[3]), [v4] "v"(voff[4]), [v5] "v"(voff[5]),
              [v6] "v"(voff[6]), [v7] "v"(voff[7])
            : "memory", "scc");
    } else {
        static_assert(NB == 4, "tile of 64 x 64 or 64 x 128 bf16");
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
    }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd_kernel(
        Geo g, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
        const __bf16* __restrict__ v, const int32_t* __restrict__ row_ptr,
        const int32_t* __restrict__ col_idx, int64_t col_len, float scale_log2,
        __bf16* __restrict__ o, float* __restrict__ lse, int64_t items_per_xcd) {
    constexpr int NDC = D / 16;   // MFMA k-steps for S (16 d each)
    constexpr int NDB = D / 32;   // 32-row d blocks of O^T
    constexpr int NBLK = 64 * D * 2 / 1024 / 2;  // DMA blocks per wave per tensor
    __shared__ __attribute__((aligned(1024))) __bf16 ks[64 * D];
    __shared__ __attribute__((aligned(1024))) __bf16 vs[64 * D];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, half = lane >> 5;
    const int64_t rs = (int64_t)g.H * D;  // elements between consecutive tokens

    // Per-lane source offsets (bytes, relative to the tile's first row) of
    // this wave's DMA blocks: block t covers LDS bytes [1024t, 1024t+1024),
    // i.e. row r = (1024t + 16*lane) / (2D), physical chunk p; the lane
    // fetches the logical chunk that the swizzle stores at p.
    int32_t koff[NBLK], voff[NBLK];
#pragma unroll
    for (int u = 0; u < NBLK; ++u) {
        const int t = wave + 2 * u;
        const int byte = t * 1024 + lane * 16;
        const int r = byte / (2 * D);
        const int p = (byte % (2 * D)) / 16;
        koff[u] = 2 * ((int32_t)(r * rs) + k_phys<D>(r, p) * 8);
        voff[u] = 2 * ((int32_t)(r * rs) + v_phys<D>(r, p) * 8);
    }
    const uint32_t ks_lds = lds_addr(ks) + wave * 1024;
    const uint32_t vs_lds = lds_addr(vs) + wave * 1024;

    // LDS transpose-read addresses (elements) for the V^T operand: lane group
    // G = lane/16 covers d = db*32 + 16*(G%2) + [0,16) and keys
    // kc*16 + 4*half + [0,4) (+8 for the second read); source lane s = lane%16
    // points at key row kbase + s/4, d offset 4*(s%4).
    const int s16 = lane & 15, dsub = (lane >> 4) & 1;
    const int vrow0 = 4 * half + (s16 >> 2);                  // + kc*16 (+8)
    const int vcol = 16 * dsub + 4 * (s16 & 3);               // + db*32
    const int qi = wave * 32 + l32;                           // this lane's query row

    // Persistent, XCD-aware schedule.  Workgroups are dealt round-robin over
    // the 8 XCDs, so workgroup w runs on XCD w%8.  XCD e owns the contiguous
    // run [e*items_per_xcd, (e+1)*items_per_xcd) of query tiles in (b, h, i)
    // order, and its resident workgroups take them in rounds: round r gives
    // slot s the item r*S + s.  All rows of a round start together and sweep
    // their ascending key-tile lists at the same pace, so the key tiles in use
    // on an XCD at any moment cluster around one tile id and stay in its L2.
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

        // Tile id at CSR position p, or -1 when out of range (then tile 0 is
        // fetched and fully masked, keeping the pipeline uniform).
        auto tile_at = [&](int64_t p) -> int {
            const int j = col_idx[p];
            return (unsigned)j < (unsigned)g.Nt ? j : -1;
        };
        auto tile_base = [&](const __bf16* t, int j) {
            return t + (batch_row0 + (int64_t)(j < 0 ? 0 : j) * 64) * rs + head_off;
        };

        // Query fragment (B operand of S^T = K Q^T): query row qi, d = 16*dc + 8*half.
        const __bf16* qrow = q + (batch_row0 + (int64_t)i * 64 + qi) * rs + head_off;
        bf16x8 qf[NDC];
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) qf[dc] = *(const bf16x8*)(qrow + dc * 16 + half * 8);
        // Make the compiler wait for the query loads here, before the DMA: it
        // cannot see the DMA issued by inline asm, and a wait for these loads
        // placed inside the key loop would also drain the in-flight DMA.
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) asm volatile("" ::"v"(qf[dc]));

        // The previous item ended with a barrier after its last LDS read, so
        // the buffers are free.
        int j = p0 < p1 ? tile_at(p0) : -1;
        if (p0 < p1) {
            dma_tile<NBLK>(tile_base(k, j), koff, ks_lds);
            dma_tile<NBLK>(tile_base(v, j), voff, vs_lds);
        }

        f32x16 oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
        float m_run = -INFINITY, l_run = 0.f;

        for (int64_t p = p0; p < p1; ++p) {
            const int jn = p + 1 < p1 ? tile_at(p + 1) : -2;  // -2: no next tile
            const int nj = j < 0 ? 0 : tile_occupancy(g, j);

            // K_j landed (V_j may still be in flight).
            if constexpr (NBLK == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
            __builtin_amdgcn_s_barrier();

            // S^T = K Q^T: two 32-key blocks; K operand row kb*32 + l32,
            // logical chunk dc*2 + half.
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
                const int krow = kb * 32 + l32;
#pragma unroll
                for (int dc = 0; dc < NDC; ++dc) {
                    bf16x8 a = *(const bf16x8*)(ks + krow * D + k_phys<D>(krow, dc * 2 + half) * 8);
                    sacc[kb] = mfma32(a, qf[dc], sacc[kb]);
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();  // every wave is done reading K_j
            if (jn != -2) dma_tile<NBLK>(tile_base(k, jn), koff, ks_lds);

            // Online softmax for query qi.  Key of (kb, r): 32kb + 8(r/4) + 4half + r%4.
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float s = sacc[kb][r] * scale_log2;
                    if (nj < 64) {
                        const int key = kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                        if (key >= nj) s = -INFINITY;
                    }
                    sacc[kb][r] = s;
                    mx = fmaxf(mx, s);
                }
            mx = fmaxf(mx, wave_xor32(mx));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;  // fully masked so far
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            m_run = m_new;
            float psum = 0.f;
            bf16x8 pf[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pv = __builtin_amdgcn_exp2f(sacc[kb][r] - m_use);
                    psum += pv;
                    pf[kb * 2 + (r >> 3)][r & 7] = (__bf16)pv;
                }
            l_run = l_run * alpha + psum;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

            // V_j landed (K_{j+1} may still be in flight).
            if (jn != -2) {
                if constexpr (NBLK == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
                else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            __builtin_amdgcn_s_barrier();

            // O^T += V^T P^T: four 16-key steps per 32-row d block.
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const int r0 = kc * 16 + vrow0, r1 = r0 + 8;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int c = db * 32 + vcol;  // d of this lane's 4-element source
                    const __bf16* a0 = vs + r0 * D + v_phys<D>(r0, c >> 3) * 8 + (c & 7);
                    const __bf16* a1 = vs + r1 * D + v_phys<D>(r1, c >> 3) * 8 + (c & 7);
                    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a0);
                    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a1);
                    typedef short i16x8 __attribute__((ext_vector_type(8)));
                    i16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    oacc[db] = mfma32(__builtin_bit_cast(bf16x8, av), pf[kc], oacc[db]);
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();  // every wave is done reading V_j
            if (jn != -2) dma_tile<NBLK>(tile_base(v, jn), voff, vs_lds);
            j = jn;
        }

        // Finalise: l is split over lanes l and l^32.
        const float l_tot = l_run + wave_xor32(l_run);
        const int ni = tile_occupancy(g, i);
        const bool valid = qi < ni && l_tot > 0.f;
        const float inv = valid ? 1.0f / l_tot : 0.f;
        __bf16* orow = o + (batch_row0 + (int64_t)i * 64 + qi) * rs + head_off;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 outv;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    outv[u] = (__bf16)(valid ? oacc[db][r4 * 4 + u] * inv : 0.f);  // pad rows: +0.0
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
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 64;
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
    const void* kernel = g.D == 128 ? (const void*)attn_fwd_kernel<128> : (const void*)attn_fwd_kernel<64>;
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
