// Direct global->LDS DMA of half-tiles (32 rows x D bf16) for gfx950, shared
// by the attention forward and backward kernels.
#pragma once

#include <cstdint>

namespace bsta {

// Issue one whole half-tile (32 rows x D bf16, NB = D/16 blocks of 1 KB)
// from the calling wave by direct-to-LDS DMA: block u lands at LDS byte
// slot + 1024*u.  The DMA's LDS address is M0 + the instruction's immediate
// offset + 16*lane, and the same immediate is added to the global address
// (checked on hardware), so M0 is set once, to slot + kDmaBias<D>, and block
// u uses offset 1024*u - kDmaBias<D> (inside the signed 13-bit range).
// `voff` holds the per-lane source byte offsets of blocks 0..3 from `base`
// with their immediates already subtracted; for D = 128 blocks 4..7 (rows
// 16..31) reuse them from a second base 16 rows further (less 4096, the
// extra immediate), since the LDS swizzles depend on the row only modulo 16.
// Written as inline asm so that the compiler does not guard every later LDS
// read with a wait for all outstanding DMA; the kernel waits on vmcnt itself.
// M0 is saved and restored around the block.
template <int D>
constexpr int kDmaBias = D == 128 ? 3584 : 1536;

template <int D>
__device__ inline void dma_half(uint64_t base_any, uint64_t rows16, const int32_t* voff,
                                uint32_t slot_lds) {
    // Both bases are wave-uniform; make them SGPRs.  (readfirstlane returns
    // int: go through uint32_t so the low half is never sign-extended.)
    const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane(slot_lds + kDmaBias<D>);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(base_any >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base_any);
    const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
    uint32_t saved;
    if constexpr (D == 128) {
        const uint64_t base16 = base + rows16 - 4096;
        asm volatile(
            "s_mov_b32 %[t], m0\n\t"
            "s_mov_b32 m0, %[l]\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[v0], %[b] offset:-3584\n\t"
            "global_load_lds_dwordx4 %[v1], %[b] offset:-2560\n\t"
            "global_load_lds_dwordx4 %[v2], %[b] offset:-1536\n\t"
            "global_load_lds_dwordx4 %[v3], %[b] offset:-512\n\t"
            "global_load_lds_dwordx4 %[v0], %[c] offset:512\n\t"
            "global_load_lds_dwordx4 %[v1], %[c] offset:1536\n\t"
            "global_load_lds_dwordx4 %[v2], %[c] offset:2560\n\t"
            "global_load_lds_dwordx4 %[v3], %[c] offset:3584\n\t"
            "s_mov_b32 m0, %[t]"
            : [t] "=&s"(saved)
            : [l] "s"(m0v), [b] "s"(base), [c] "s"(base16), [v0] "v"(voff[0]),
              [v1] "v"(voff[1]), [v2] "v"(voff[2]), [v3] "v"(voff[3])
            : "memory");
    } else {
        static_assert(D == 64, "head dim 64 or 128");
        (void)rows16;
        asm volatile(
            "s_mov_b32 %[t], m0\n\t"
            "s_mov_b32 m0, %[l]\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %[v0], %[b] offset:-1536\n\t"
            "global_load_lds_dwordx4 %[v1], %[b] offset:-512\n\t"
            "global_load_lds_dwordx4 %[v2], %[b] offset:512\n\t"
            "global_load_lds_dwordx4 %[v3], %[b] offset:1536\n\t"
            "s_mov_b32 m0, %[t]"
            : [t] "=&s"(saved)
            : [l] "s"(m0v), [b] "s"(base), [v0] "v"(voff[0]), [v1] "v"(voff[1]),
              [v2] "v"(voff[2]), [v3] "v"(voff[3])
            : "memory");
    }
}

// 64 consecutive floats (256 bytes) from `base_any` to LDS byte address
// `lds` by direct-to-LDS DMA: lane l's 4 bytes land at lds + 4*l (one
// instruction of the calling wave).
__device__ inline void dma_floats64(uint64_t base_any, uint32_t lds) {
    const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane(lds);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(base_any >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base_any);
    const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
    const int32_t voff = 4 * (int32_t)(threadIdx.x & 63);
    uint32_t saved;
    asm volatile(
            "s_mov_b32 %[t], m0\n\t"
            "s_mov_b32 m0, %[l]\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dword %[v], %[b]\n\t"
            "s_mov_b32 m0, %[t]"
            : [t] "=&s"(saved)
            : [l] "s"(m0v), [b] "s"(base), [v] "v"(voff)
            : "memory");
}

// Wait until at most `newer` (0..2) half-tiles this wave issued after the
// one about to be read are still in flight (each half-tile is NP DMA
// instructions of the issuing wave).
template <int NP>
__device__ inline void wait_dma(int newer) {
    if (newer <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (newer == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NP) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NP) : "memory");
}

}  // namespace bsta
