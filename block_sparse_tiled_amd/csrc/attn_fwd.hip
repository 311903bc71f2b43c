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
//   1. K (64 x D) is staged to LDS row-major with an XOR swizzle of 16-byte
//      chunks; V is staged transposed (D x 64) with its keys permuted inside
//      every 16-key group so that one 16-byte LDS read feeds one MFMA operand.
//   2. S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys as M, queries as N), so
//      each lane ends up holding scores of a single query.
//   3. Online softmax in the exp2 domain (log2(e)/sqrt(D) folded into the
//      scale); the row max needs one cross-lane exchange (lane ^ 32), the row
//      sum stays per lane until the end.
//   4. O^T += V^T P^T on the same MFMA, P converted to bf16 in registers:
//      the accumulator layout of step 2 is exactly the B-operand layout this
//      product needs, up to a fixed permutation of the 16 keys of each
//      k-step, which the transposed V layout in LDS absorbs.
// Partial key tiles (n_j < 64) mask keys r >= n_j to -inf; padded query rows
// are written as zero.
//
// MFMA 32x32x16 bf16 lane layout (gfx950): A[m][k] in lane m + 32*(k/8),
// element k%8; B[k][n] in lane n + 32*(k/8), element k%8; D[m][n] in lane
// n, register 8*(m/8)... precisely reg r of lane l holds
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
#include "bsta_common.hpp"

namespace bsta {

namespace {

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// Physical 16-byte chunk of K row `row` (D/8 chunks per row).
template <int D>
__device__ inline int k_chunk(int row, int c) { return c ^ (row & (D / 8 - 1)); }

// Physical 16-byte chunk of V^T row `d` (8 chunks of 8 keys per row).
__device__ inline int vt_chunk(int d, int c) { return c ^ (d & 7); }

}  // namespace

template <int D>
__global__ __launch_bounds__(128) void attn_fwd_kernel(
        Geo g, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
        const __bf16* __restrict__ v, const int32_t* __restrict__ row_ptr,
        const int32_t* __restrict__ col_idx, int64_t col_len, float scale_log2,
        __bf16* __restrict__ o, float* __restrict__ lse, int per_xcd) {
    constexpr int NDC = D / 16;   // MFMA k-steps for S (16 d each)
    constexpr int NDB = D / 32;   // 32-row d blocks of O^T
    constexpr int CPR = D / 8;    // 16-byte chunks per K row
    __shared__ __attribute__((aligned(16))) __bf16 ks[64 * D];
    __shared__ __attribute__((aligned(16))) __bf16 vts[D * 64];

    // XCD-aware placement: workgroups are dealt round-robin over the 8 XCDs;
    // give each XCD a contiguous run of query tiles of one head at a time so
    // that concurrently resident tiles share key tiles in that XCD's L2.
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int bh = slot / per_xcd;
    const int i = xcd * per_xcd + (slot - bh * per_xcd);
    if (i >= g.Nt || bh >= g.B * g.H) return;
    const int b = bh / g.H, h = bh - b * g.H;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, half = lane >> 5;
    const int64_t rs = (int64_t)g.H * D;  // elements between consecutive tokens
    const int64_t head_off = (int64_t)h * D;
    const int64_t batch_row0 = (int64_t)b * g.Lpad;

    // Query fragment (B operand of S^T = K Q^T): query row qi, d = 16*dc + 8*half.
    const int qi = wave * 32 + l32;
    const __bf16* qrow = q + (batch_row0 + (int64_t)i * 64 + qi) * rs + head_off;
    bf16x8 qf[NDC];
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) qf[dc] = *(const bf16x8*)(qrow + dc * 16 + half * 8);

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int64_t row = (int64_t)bh * g.Nt + i;
    int64_t p0 = row_ptr[row], p1 = row_ptr[row + 1];
    p0 = p0 < 0 ? 0 : (p0 > col_len ? col_len : p0);
    p1 = p1 < p0 ? p0 : (p1 > col_len ? col_len : p1);

    for (int64_t p = p0; p < p1; ++p) {
        const int j = col_idx[p];
        if ((unsigned)j >= (unsigned)g.Nt) continue;  // uniform over the workgroup
        const int nj = tile_occupancy(g, j);
        const int64_t tile_row0 = batch_row0 + (int64_t)j * 64;
        const __bf16* kt = k + tile_row0 * rs + head_off;
        const __bf16* vt = v + tile_row0 * rs + head_off;

        __syncthreads();  // previous tile's LDS reads are done
        // Stage K: 64 rows x CPR chunks.
#pragma unroll
        for (int e = tid; e < 64 * CPR; e += 128) {
            const int r = e / CPR, c = e - r * CPR;
            u32x4 val = *(const u32x4*)(kt + r * rs + c * 8);
            *(u32x4*)(ks + r * D + k_chunk<D>(r, c) * 8) = val;
        }
        // Stage V^T: an 8-key x 8-d block per thread, transposed in registers.
        // Key group kg (0..7) = 16-key chunk kc = kg/2, half hh = kg%2, holding
        // keys 16kc + 4hh + {0..3} and 16kc + 8 + 4hh + {0..3}.
#pragma unroll
        for (int e = tid; e < 8 * CPR; e += 128) {
            const int dg = e % CPR, kg = e / CPR;
            const int kbase = (kg >> 1) * 16 + (kg & 1) * 4;
            u32x4 in[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int key = kbase + (u & 3) + (u >> 2) * 8;
                in[u] = *(const u32x4*)(vt + key * rs + dg * 8);
            }
#pragma unroll
            for (int dv = 0; dv < 8; ++dv) {
                u32x4 out;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t x0 = in[2 * w][dv >> 1], x1 = in[2 * w + 1][dv >> 1];
                    out[w] = (dv & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u))
                                      : ((x0 & 0xffffu) | (x1 << 16));
                }
                const int d = dg * 8 + dv;
                *(u32x4*)(vts + d * 64 + vt_chunk(d, kg) * 8) = out;
            }
        }
        __syncthreads();

        // S^T = K Q^T: two 32-key blocks.
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
            const int krow = kb * 32 + l32;
#pragma unroll
            for (int dc = 0; dc < NDC; ++dc) {
                bf16x8 a = *(const bf16x8*)(ks + krow * D + k_chunk<D>(krow, dc * 2 + half) * 8);
                sacc[kb] = mfma32(a, qf[dc], sacc[kb]);
            }
        }

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
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
        bf16x8 pf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pv = __builtin_amdgcn_exp2f(sacc[kb][r] - m_new);
                psum += pv;
                pf[kb * 2 + (r >> 3)][r & 7] = (__bf16)pv;
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

        // O^T += V^T P^T: four 16-key steps per 32-row d block.
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int drow = db * 32 + l32;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                bf16x8 a = *(const bf16x8*)(vts + drow * 64 + vt_chunk(drow, kc * 2 + half) * 8);
                oacc[db] = mfma32(a, pf[kc], oacc[db]);
            }
        }
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

hipError_t launch_attn_fwd(const Geo& g, const void* q, const void* k, const void* v,
                           const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len,
                           float scale, void* o, float* lse, hipStream_t stream) {
    const int per_xcd = (g.Nt + 7) / 8;
    const int64_t blocks = (int64_t)8 * per_xcd * g.B * g.H;
    const float scale_log2 = scale * 1.4426950408889634f;
    if (g.D == 128)
        hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3((unsigned)blocks), dim3(128), 0, stream, g,
                           (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, row_ptr, col_idx,
                           col_len, scale_log2, (__bf16*)o, lse, per_xcd);
    else
        hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3((unsigned)blocks), dim3(128), 0, stream, g,
                           (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, row_ptr, col_idx,
                           col_len, scale_log2, (__bf16*)o, lse, per_xcd);
    return hipGetLastError();
}

}  // namespace bsta
