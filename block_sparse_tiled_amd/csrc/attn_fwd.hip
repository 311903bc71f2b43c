// Fused block-sparse flash-attention forward for gfx950 (CDNA4).
//
// Method ("bsa_attn" page, forward / _compute_sparse_attention; __init__
// fixes the scale to 1/sqrt(d) and rules out causal masking): for query tile
// i of head h, attention runs over the valid tokens of the key tiles listed
// in CSR row (b*H + h)*Nt + i, with an online (streaming) softmax.
//
// Work decomposition: a workgroup owns one query tile; wave w owns query
// rows 32w..32w+31 for the whole key list.  A 64-token tile takes two
// wave64s, and four such workgroups share a CU, so each SIMD runs two waves
// whose softmax and MFMA phases overlap (a wave raises its priority for the
// score/softmax phase below, so that phase's VALU work issues first).  A
// 128-token tile takes four wave64s, two workgroups per CU, all four waves
// reading the key tiles that waves 0 and 1 bring in.  Per selected key
// tile:
//   1. K and V arrive in LDS by direct global->LDS DMA (global_load_lds_
//      dwordx4, 1 KB per instruction; each half-tile is issued whole by one
//      wave, the low halves by wave 0 and the high halves by wave 1)
//      into a ring of five half-tile slots (32 keys x D), consumed in pairs:
//      K(t+1) low and high, then V(t) low and high.  Before a pair is read,
//      one workgroup barrier publishes it and retires the previous pair,
//      whose slots are refilled right away, so up to three half-tiles are in
//      flight while a pair is read.  Rows are XOR-swizzled in 16-byte chunks
//      so every read below is free of bank conflicts (64 banks).
//   2. S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys as M, queries as N): each
//      lane ends up holding the scores of a single query.
//   3. Online softmax in the exp2 domain (log2(e)/sqrt(D) folded into the
//      scale) against a reference max m taken from the first tile with a
//      valid key; the row sum stays per lane until the end.  m is raised
//      (and O, l rescaled; the row max then needs one cross-lane exchange,
//      lane ^ 32) only when some lane's probability sum for a tile exceeds
//      2^64 or is not finite, which keeps every p within fp32 and bf16.
//   4. O^T += V^T P^T on the same MFMA.  The accumulator layout of step 2 is
//      the B-operand layout this product needs, up to a fixed permutation of
//      the 16 keys of each k-step; the A operand (V^T) comes from row-major V
//      through the LDS transpose read ds_read_b64_tr_b16, four keys at a time
//      in exactly that permuted order.
// Partial key tiles (n_j < 64) mask keys r >= n_j to -inf; padded query rows
// are written as +0.0.  Out-of-range tile ids contribute nothing.  The output
// goes to the tiled tensor, or (raster) straight to each token's row of the
// [B, L, H, D] tensor, pad slots writing nothing.
//
// Lane layouts used (gfx950, checked on hardware):
//   v_mfma_f32_32x32x16_bf16: A[m][k] in lane m + 32*(k/8), element k%8;
//     B[k][n] in lane n + 32*(k/8), element k%8; register r of lane l holds
//     D[8*(r/4) + 4*(l/32) + r%4][l%32].
//   ds_read_b64_tr_b16, per 16-lane group: if lane s addresses 4 elements
//     C_s, lane d receives C_{d/4 + 4m}[d%4] for m = 0..3.
//   global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + 16*l.
#include <atomic>

#include "bsta_common.hpp"
#include "lds_dma.hpp"

namespace bsta {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

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

// Per-XCD sweep counters (one 128-byte line each): key tiles processed on
// that XCD, bumped by 16 every 16 steps and by the rest of a row at its
// end (few atomics on one line: loads of a line that takes many atomic
// adds queue behind them).  Only the key order within rows
// depends on them (see the kernel), so calls that overlap on one device, or
// a counter that wraps, change speed, never results' validity.
__device__ unsigned int g_sweep[8 * 32];

// Sweep target (a key tile id in [0, nt)) for sweep clock value c.
__device__ inline int sweep_target(uint32_t c, uint32_t period, int nt) {
    return (int)(((uint64_t)(c % period) * (uint64_t)nt) / period);
}

// Read of the sweep clock: an atomic load, which is served by the XCD's L2
// (where the counter's atomic adds happen), not by a CU's L1.  The caller
// takes the value with readfirstlane where it needs it, so that the load's
// latency can overlap other work.
__device__ inline uint32_t sweep_load(const unsigned int* ctr) {
    return __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

}  // namespace

// SUB = 64-slot units per tile: 1 for 64-token tiles, 2 for 128-token tiles.
// A work item is one query tile (one CSR row).  With 128-token tiles waves 0
// and 1 hold query unit 0 of the tile and waves 2 and 3 unit 1, and each CSR
// entry j stands for the key units 2j and 2j+1, walked as consecutive key
// steps.
template <int D, int SUB>
__global__ __launch_bounds__(128 * SUB) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(
        Geo g, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
        const __bf16* __restrict__ v, const int32_t* __restrict__ row_ptr,
        const int32_t* __restrict__ col_idx, int64_t col_len, float scale_log2,
        __bf16* __restrict__ o, float* __restrict__ lse, const uint64_t* __restrict__ keep,
        int64_t items_per_xcd, int rotate, int raster) {
    constexpr int NDC = D / 16;                    // MFMA k-steps for S (16 d each)
    constexpr int NDB = D / 32;                    // 32-row d blocks of O^T
    constexpr int HALF_ELEMS = 32 * D;             // one half-tile slot
    constexpr int NP = HALF_ELEMS * 2 / 1024;      // DMA instructions per half-tile (one wave)
    constexpr int SLOT_BYTES = HALF_ELEMS * 2;
    __shared__ __attribute__((aligned(1024))) __bf16 ring[kRing * HALF_ELEMS];

    // CSR reads are wave-uniform: read them through the scalar cache.
    typedef const __attribute__((address_space(4))) int32_t* cptr;
    const cptr rp_s = (cptr)row_ptr;
    const cptr ci_s = (cptr)col_idx;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave-uniform by construction; readfirstlane tells the compiler so.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    const int64_t rs = (int64_t)g.H * D;  // elements between consecutive tokens
    const int64_t rs2 = rs * 2;           // bytes
    const bool all_full = g.full != 0;
    const int NU = g.Nt * SUB;  // 64-slot units per (batch, head)
    // Waves 0 and 1 hold rows 0-31 and 32-63 of query unit 0 and issue the
    // DMA; with 128-token tiles waves 2 and 3 hold those of unit 1 and only
    // read the ring, so each key tile crosses into LDS once for 128 rows.
    const bool issuer = SUB == 1 || wave < 2;

    // Per-lane DMA source offsets (bytes, relative to the half-tile's first
    // row) of blocks 0..3: block u covers slot bytes [1024u, 1024u+1024),
    // i.e. row r = (1024u + 16*lane) / (2D), physical chunk p; the lane
    // fetches the logical chunk the swizzle stores at p.
    int32_t koff[4], voff[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int byte = u * 1024 + lane * 16;
        const int r = byte / (2 * D);
        const int p = (byte % (2 * D)) / 16;
        const int imm = 1024 * u - kDmaBias<D>;  // the block's immediate offset
        koff[u] = 2 * ((int32_t)(r * rs) + k_phys<D>(r, p) * 8) - imm;
        voff[u] = 2 * ((int32_t)(r * rs) + v_phys<D>(r, p) * 8) - imm;
    }
    const uint64_t rows16 = (uint64_t)(16 * rs2);

    // LDS read addresses (bytes) inside slot 0; a slot adds a constant.
    // K operand for k-step dc: row l32, logical chunk 2*dc + half.
    // V^T transpose reads: lane group G = lane/16 covers d = db*32 +
    // 16*(G%2) + [0,16) and keys 16*kk + 4*half + [0,4) (+8 for the second
    // read); source lane s = lane%16 points at key row 16*kk + 4*half + s/4,
    // d offset 4*(s%4).  The V swizzle depends on the row only through r%4,
    // equal for all of them.
    const uint32_t ring0 = lds_addr(ring);
    uint32_t kaddr[NDC];
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) kaddr[dc] = ring0 + 2 * (l32 * D + k_phys<D>(l32, 2 * dc + half) * 8);
    const int s16 = lane & 15, dsub = (lane >> 4) & 1;
    const int vrow0 = 4 * half + (s16 >> 2);
    const int vcol = 16 * dsub + 4 * (s16 & 3);
    uint32_t vaddr[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int c = db * 32 + vcol;
        vaddr[db] = ring0 + 2 * (vrow0 * D + v_phys<D>(vrow0, c >> 3) * 8 + (c & 7));
    }
    const int qi = (SUB == 1 ? wave : (wave & 1)) * 32 + l32;  // query row in its unit
    const int qsub = SUB == 1 ? 0 : wave >> 1;                  // unit within the tile
    const int half4 = 4 * half;

    // Persistent, XCD-aware schedule.  Workgroups are dealt round-robin over
    // the 8 XCDs, so workgroup w runs on XCD w%8.  XCD e owns a contiguous
    // run of query units in (b, h, i) order (below); its resident
    // workgroups take them in rounds of S.
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int S = gridDim.x >> 3;
    const int64_t n_rows = (int64_t)g.B * g.H * g.Nt;  // CSR rows
    const int64_t n_items = n_rows;  // a work item is one query tile
    int64_t nnz = rp_s[n_rows];
    nnz = nnz < 0 ? 0 : (nnz > col_len ? col_len : nnz);
    // Rows of equal length (every top-k CSR): the even split, items_per_xcd
    // units each.  Otherwise XCD e owns the rows [r_e, r_e+1), r_e the first
    // row whose CSR start reaches e/8 of the entries, so that every XCD
    // walks the same number of key tiles (window rows differ per head, and
    // threshold rows per row).  Both of the XCD's boundaries are found at
    // once, each by a 32-way search in one half of the wave (a row_ptr
    // that decreases somewhere, which the interface rules out, can only
    // make two XCDs share rows, never leave one out).
    int64_t first, last;
    const int64_t len0 = (int64_t)rp_s[1] - (int64_t)rp_s[0];
    if (rp_s[0] == 0 && len0 * n_rows == (int64_t)rp_s[n_rows]) {
        first = (int64_t)xcd * items_per_xcd;
        last = first + items_per_xcd < n_items ? first + items_per_xcd : n_items;
    } else {
        const int hsel = lane >> 5, j = lane & 31;
        const int64_t target = nnz * (xcd + hsel) / 8;
        int64_t lo = 0, hi = n_rows;  // smallest r with r == n_rows or row_ptr[r] >= target
        int iters = 1;
        for (int64_t span = 32; span <= n_rows; span *= 32) ++iters;
        for (int it = 0; it <= iters; ++it) {
            const int64_t step = (hi - lo + 31) / 32 > 0 ? (hi - lo + 31) / 32 : 1;
            const int64_t p = lo + step * j < hi ? lo + step * j : hi;
            const bool ge = p >= n_rows || (int64_t)row_ptr[p] >= target;
            const uint64_t m = (__builtin_amdgcn_ballot_w64(ge) >> (32 * hsel)) & 0xffffffffull;
            const int js = m ? __builtin_ctzll(m) : 32;
            const int64_t pj = lo + step * js < hi ? lo + step * js : hi;
            if (js > 0) lo = lo + step * (js - 1) + 1;
            hi = js < 32 ? pj : hi;
            if (lo > hi) lo = hi;
        }
        // The first and last boundaries are fixed: trailing empty rows (and
        // rows before a negative start) still get their outputs written.
        const int64_t r0 = xcd == 0 ? 0 : __builtin_amdgcn_readlane((int)lo, 0);
        int64_t r1 = xcd == 7 ? n_rows : __builtin_amdgcn_readlane((int)lo, 32);
        if (r1 < r0) r1 = r0;
        first = r0;
        last = r1;
    }

    // Key-order rotation for L2 reuse.  The rows' key tiles are scattered
    // over the whole head, so the K/V working set of one XCD's resident
    // workgroups is the entire head, far beyond its L2.  Walking every row
    // in ascending order shares cache lines only while the workgroups stay
    // in step, and they drift apart.  Instead each row starts at the first
    // key tile at or above a target id that sweeps 0..Nt-1 once per average
    // item duration, measured in key tiles processed on the XCD (one period
    // is S workgroups times the mean row length).  Concurrent workgroups
    // then touch neighbouring key ids whatever their start times.  Any
    // rotation visits the same set of keys, so only rounding depends on it.
    unsigned int* const sweep = &g_sweep[xcd * 32];
    // rotate: 0 = CSR order, 2 = always rotated, 1 = rotated where it pays.
    // The rotation shares cache lines among workgroups whose rows scatter
    // over a head too large for the caches.  A head of at most two L2s of
    // K and V, or rows that keep to a part of the key range (sliding
    // windows), reuse lines in CSR order already, and there the walk's
    // handoff and counter traffic cost more than they save.  The XCD's first
    // row stands for the rest: its first and last ids span under 3/4 of the
    // head's tiles in a window selection, nearly all of them otherwise.
    if (rotate == 1) {
        const uint64_t head_bytes = (uint64_t)NU * 64 * D * 2 * 2;
        bool wide = head_bytes > (8ull << 20);
        if (wide && first < last) {
            const int64_t r = first;
            int64_t a = rp_s[r], e = rp_s[r + 1];
            a = a < 0 ? 0 : (a > col_len ? col_len : a);
            e = e < a ? a : (e > col_len ? col_len : e);
            if (e - a >= 2) wide = (int64_t)4 * ((int64_t)ci_s[e - 1] - ci_s[a]) >= (int64_t)3 * g.Nt;
        }
        rotate = wide ? 1 : 0;
    }
    const uint64_t per_raw = (uint64_t)S * SUB * (uint64_t)nnz / (uint64_t)(n_rows > 0 ? n_rows : 1);
    const uint32_t period = per_raw == 0 ? 1u : (per_raw > 0x7fffffffu ? 0x7fffffffu : (uint32_t)per_raw);
    // Wave 0 hands each item's rotation start to wave 1 through the first
    // word of the last ring slot: between an item's final barrier and the
    // next item's first acquire the prologue fills only the first three
    // slots, so that word is free, and the ring keeps the workgroup's LDS at
    // exactly five slots (four workgroups per CU).
    int* const handoff = (int*)&ring[(kRing - 1) * HALF_ELEMS];

    for (int64_t item = first + slot; item < last; item += S) {
        const int bh = (int)(item / g.Nt);
        const int i = (int)(item - (int64_t)bh * g.Nt);  // query tile
        const int iu = i * SUB + qsub;                   // this wave's query unit
        const int b = bh / g.H, h = bh - b * g.H;
        const int64_t head_off = (int64_t)h * D;
        const int64_t batch_row0 = (int64_t)b * g.Lpad;
        const uint64_t kbase = (uint64_t)(uintptr_t)(k + batch_row0 * rs + head_off);
        const uint64_t vbase = (uint64_t)(uintptr_t)(v + batch_row0 * rs + head_off);

        const int64_t row = (int64_t)bh * g.Nt + i;
        int64_t p0 = rp_s[row], p1 = rp_s[row + 1];
        p0 = p0 < 0 ? 0 : (p0 > col_len ? col_len : p0);
        p1 = p1 < p0 ? p0 : (p1 > col_len ? col_len : p1);
        const int ne = (int)(p1 - p0);  // CSR entries
        const int n = ne * SUB;         // key steps

        // Rotation start k0: the step at the same fraction of the row as the
        // sweep target is of the key range, target * n / NU.  For a row
        // whose ids spread evenly over the head that is about the first
        // entry at or above the target, without reading the row's ids (an
        // exact count, one pass over them, measured 1.5-3% slower per call);
        // any start visits the same entries.  With rotation off
        // (deterministic mode) every row is walked from its first entry.
        int k0 = 0;
        const bool rot = rotate && n > 1;  // workgroup-uniform
        // The sweep clock is read first, so that its latency overlaps the
        // check of the row's ids below.
        const uint32_t clock_v = rot && wave == 0 ? sweep_load(sweep) : 0u;
        // A clean row (every tile full, every id in range) needs no key
        // masking, so its steps skip the tile lookup that masking needs.
        // The ids of the first 128 entries are loaded here and checked after
        // the first acquire, whose wait for K(0) hides their latency (the
        // rest of a longer row is checked there too).  Both waves read the
        // same ids and reach the same verdict.
        bool clean = all_full;
        int idc0 = 0, idc1 = 0;
        if (all_full) {
            idc0 = lane < ne ? col_idx[p0 + lane] : 0;
            idc1 = 64 + lane < ne ? col_idx[p0 + 64 + lane] : 0;
        }
        if (rot) {
            if (wave == 0) {
                const int target = sweep_target(__builtin_amdgcn_readfirstlane(clock_v), period, NU);
                const int cnt = (int)(((int64_t)target * n) / NU);
                if (lane == 0) *handoff = cnt < n ? cnt : 0;
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            k0 = __builtin_amdgcn_readfirstlane(*(volatile int*)handoff);
        }

        // Tile id of step t (CSR position p0 + (k0 + t) mod n), or -1 when t
        // is past the row or the id is out of range (then tile 0 is fetched
        // and fully masked).
        auto tile_id = [&](int t) -> int {
            if (t >= n) return -1;
            const int r = t + k0 < n ? t + k0 : t + k0 - n;
            const int j = ci_s[p0 + r / SUB];
            return (unsigned)j < (unsigned)g.Nt ? j * SUB + r % SUB : -1;
        };
        // Byte offset of a tile's first row from the head's base.
        auto tile_bytes = [&](int j) -> uint64_t { return (uint64_t)((int64_t)(j < 0 ? 0 : j) * 64 * rs2); };

        // Query fragment (B operand of S^T = K Q^T): query row qi,
        // d = 16*dc + 8*half.
        bf16x8 qf[NDC];
        const __bf16* qrow = q + (batch_row0 + (int64_t)iu * 64 + qi) * rs + head_off;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) qf[dc] = *(const bf16x8*)(qrow + dc * 16 + half * 8);
        // The compiler cannot see the DMA issued below: make it finish the
        // query loads first, so that no wait inside the key loop drains the
        // DMA queue on their account.
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) asm volatile("" ::"v"(qf[dc]));

        // Half-tiles are consumed in the order K0lo K0hi, then per key tile
        // t: K(t+1)lo K(t+1)hi V(t)lo V(t)hi (no K after the last tile);
        // sequence position s sits in ring slot s % kRing.  Wave w issues
        // the positions of parity w (the low halves, or the high ones), each
        // as one whole half-tile.
        const int NSEQ = 4 * n;
        int my_next = wave;               // next position this wave issues
        int my_slot = wave;               // and its ring slot
        const uint64_t hi_off = wave ? (uint64_t)(32 * rs2) : 0;
        // Byte offsets of the tiles of the last K step issued and of the one
        // before: each tile id is looked up once, at this wave's half of its
        // K; V(t) then reuses it (the last V follows its own K).
        uint64_t off_k = 0, off_km1 = 0;
        // (Producer and acquire are statement macros: captured by closures,
        // this state would be kept in memory.)
        //
        // Position s: K(0) at 0, 1; then K(t+1) at s % 4 in {2, 3} and V(t)
        // at s % 4 in {0, 1}; V(n-1) at NSEQ-2, NSEQ-1.  The half is s & 1
        // throughout, i.e. this wave's.  (The element-wise select of the
        // offsets keeps both arrays in registers.)
#define BSTA_ISSUE_NEXT()                                                                  \
    do {                                                                                   \
        const int s_ = my_next;                                                            \
        const bool tail_ = s_ >= NSEQ - 2;                                                 \
        const bool is_k_ = s_ < 2 || (!tail_ && (s_ & 2) != 0);                            \
        if (is_k_) {                                                                       \
            off_km1 = off_k;                                                               \
            off_k = tile_bytes(tile_id(s_ < 2 ? 0 : ((s_ - 2) >> 2) + 1));                 \
        }                                                                                  \
        const uint64_t src_ = (is_k_ ? kbase : vbase) + (is_k_ || tail_ ? off_k : off_km1) + \
                              hi_off;                                                      \
        int32_t offs_[4];                                                                  \
        _Pragma("unroll") for (int u_ = 0; u_ < 4; ++u_) offs_[u_] =                       \
            is_k_ ? koff[u_] : voff[u_];                                                   \
        dma_half<D>(src_, rows16, offs_, ring0 + (uint32_t)my_slot * SLOT_BYTES);          \
        my_next += 2;                                                                      \
        my_slot = my_slot >= kRing - 2 ? my_slot + 2 - kRing : my_slot + 2;                \
    } while (0)
        // Consumer: pairs of positions (one per wave).  Acquiring waits for
        // this wave's position of the pair (its later ones may stay in
        // flight), then a barrier makes the pair visible to both waves and
        // retires the previous pair, whose slots are refilled right away.
        // Gives the pair's first slot (the second is the next one,
        // cyclically).
        int read_pos = 0, read_slot = 0;
#define BSTA_ACQUIRE(sl_out)                                                               \
    do {                                                                                   \
        if (issuer) wait_dma<NP>((my_next - (read_pos + wave) - 2) >> 1);                  \
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");                                 \
        __builtin_amdgcn_s_barrier();                                                      \
        const int lim_ = read_pos + kRing < NSEQ ? read_pos + kRing : NSEQ;                \
        if (issuer)                                                                        \
            while (my_next < lim_) BSTA_ISSUE_NEXT();                                      \
        (sl_out) = read_slot;                                                              \
        read_pos += 2;                                                                     \
        read_slot = read_slot >= kRing - 2 ? read_slot + 2 - kRing : read_slot + 2;        \
    } while (0)
        auto next_slot_of = [](int sl) { return sl == kRing - 1 ? 0 : sl + 1; };
        // Steady state (at least two key tiles after step t's).  The
        // generic acquire then always does the same thing: each wave issues
        // exactly one half-tile (wave 0 the low half of K(t+2) at the K
        // acquire and of V(t+1) at the V acquire; wave 1 the high half of
        // V(t), then of K(t+2)), and at the wait wave 0 has one newer
        // half-tile of its own in flight, wave 1 none.  This fixed form
        // drops the generic loop's position bookkeeping, about a quarter of
        // the scalar instructions per key tile.  `do_k` selects the K issue;
        // `jraw2` is the unchecked id of tile t+2, loaded before the waits.
#define BSTA_ACQUIRE_STEADY(sl_out, do_k)                                                  \
    do {                                                                                   \
        if (wave == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NP) : "memory");          \
        else if (SUB == 1 || wave == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   \
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");                                 \
        __builtin_amdgcn_s_barrier();                                                      \
        const uint32_t slot_ = ring0 + (uint32_t)my_slot * SLOT_BYTES;                     \
        if (issuer) {                                                                      \
            if (do_k) {                                                                    \
                off_km1 = off_k;                                                           \
                off_k = (unsigned)jraw2 < (unsigned)g.Nt                                   \
                            ? (uint64_t)(jraw2 * SUB + (r2 % SUB)) * tile_stride : 0;        \
                dma_half<D>(kbase + off_k + hi_off, rows16, koff, slot_);                  \
            } else {                                                                       \
                dma_half<D>(vbase + off_km1 + hi_off, rows16, voff, slot_);                \
            }                                                                              \
        }                                                                                  \
        my_next += 2;                                                                      \
        my_slot = my_slot >= kRing - 2 ? my_slot + 2 - kRing : my_slot + 2;                \
        (sl_out) = read_slot;                                                              \
        read_pos += 2;                                                                     \
        read_slot = read_slot >= kRing - 2 ? read_slot + 2 - kRing : read_slot + 2;        \
    } while (0)
        // Prologue: positions 0..2.  Every slot of the previous item was
        // retired behind a barrier.
        if (issuer)
            while (my_next < 3 && my_next < NSEQ) BSTA_ISSUE_NEXT();

        f32x16 oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
        // Reference max m (exp2 domain) of this lane's query and the lane's
        // part of the softmax denominator (lanes l and l^32 hold different
        // keys of the same query).
        float m_run = 0.f, l_run = 0.f;
        bool m_init = false;

        // S^T = K Q^T of one key tile from the K half-tiles in slots
        // (sl, next), as four groups of four k-steps; `between(g)` runs after
        // group g's MFMAs are issued (the scheduling barriers keep the
        // compiler from hoisting all operand reads).
        auto scores = [&](int sl, f32x16 (&sc)[2], auto&& between) {
            const uint32_t sb0 = (uint32_t)sl * SLOT_BYTES;
            const uint32_t sb1 = (uint32_t)next_slot_of(sl) * SLOT_BYTES;
            sc[0] = (f32x16){};
            sc[1] = (f32x16){};
            constexpr int NG = 2 * NDC / 4;
            auto load_k = [&](int gidx, bf16x8 (&a)[4]) {
                const int kb = gidx / (NDC / 4), d0 = (gidx % (NDC / 4)) * 4;
                const uint32_t sb = kb == 0 ? sb0 : sb1;
#pragma unroll
                for (int u = 0; u < 4; ++u) a[u] = *(const lds_bf16x8*)(uintptr_t)(kaddr[d0 + u] + sb);
            };
            bf16x8 ka[2][4];
            load_k(0, ka[0]);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                if (gi + 1 < NG) load_k(gi + 1, ka[(gi + 1) & 1]);
                const int kb = gi / (NDC / 4), d0 = (gi % (NDC / 4)) * 4;
#pragma unroll
                for (int u = 0; u < 4; ++u) sc[kb] = mfma32(ka[gi & 1][u], qf[d0 + u], sc[kb]);
                between(gi);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // Keys of tile j at or beyond its valid count score -inf.  Key of
        // (kb, r): 32kb + 8(r/4) + 4half + r%4, compared as
        // 4half >= n_j - (32kb + 8(r/4) + r%4) with a scalar right side.
        auto mask = [&](f32x16 (&sc)[2], int j) {
            const int nj = j < 0 ? 0 : (all_full ? 64 : unit_occupancy(g, j));
            if (nj < 64) {  // tile-uniform
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int lim = nj - (kb * 32 + (r >> 2) * 8 + (r & 3));
                        if (half4 >= lim) sc[kb][r] = -INFINITY;
                    }
            }
            return nj;
        };
        // p = exp2(s*c - m) for the 8 accumulator registers [8c, 8c+8) of
        // key block kb = c/2 as one bf16x8 B operand of the PV product (key
        // order of the accumulator), adding the rounded p to the lane's sum.
        auto probs_chunk = [&](const f32x16 (&sc)[2], int c, float neg_m, bf16x8& pfc, float& ps) {
            const int kb = c >> 1, r0 = (c & 1) * 8;
#pragma unroll
            for (int r = 0; r < 8; r += 2) {
                const bf16x2 pp = {
                    (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r0 + r], scale_log2, neg_m)),
                    (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r0 + r + 1], scale_log2, neg_m))};
                pfc[r] = pp[0];
                pfc[r + 1] = pp[1];
                ps = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, ps, false);
            }
        };

        f32x16 sc_cur[2];
        int nj_cur = 0;
        // CSR index of tile t+2 in the rotated walk (used only while t+2 <
        // n, and then in [0, n)).
        const cptr rowp = ci_s + p0;
        const uint64_t tile_stride = (uint64_t)(64 * rs2);
        int r2 = k0 + 2;
        r2 = r2 >= n ? r2 - n : r2;
        if (n > 0) {
            int sl;
            BSTA_ACQUIRE(sl);
            if (all_full) {
                clean = __builtin_amdgcn_ballot_w64((unsigned)idc0 >= (unsigned)g.Nt ||
                                                    (unsigned)idc1 >= (unsigned)g.Nt) == 0;
                for (int base = 128; base < ne; base += 64) {
                    const int idx = base + lane;
                    const int j = idx < ne ? col_idx[p0 + idx] : 0;
                    clean = clean && __builtin_amdgcn_ballot_w64((unsigned)j >= (unsigned)g.Nt) == 0;
                }
            }
            scores(sl, sc_cur, [](int) {});
            nj_cur = clean ? 64 : mask(sc_cur, tile_id(0));
        }
        for (int t = 0; t < n; ++t) {
            const bool more = t + 1 < n;
            const bool steady = t + 2 < n;
            // Raw id of tile t+2 (checked after the barrier, so that the
            // scalar load's latency hides behind the waits).
            const int jraw2 = steady ? rowp[r2 / SUB] : -1;
            // Probabilities of tile t, overlapped with the scores of tile t+1.
            bf16x8 pf[4];
            float ps[4] = {0.f, 0.f, 0.f, 0.f};
            const float neg_m = -m_run;
            f32x16 sc_next[2];
            if (more) {
                // Four probability chunks spread over the score groups (two
                // groups per chunk pair when D = 64).
                constexpr int NG = 2 * NDC / 4;
                int sl;
                // This phase (scores of t+1 interleaved with the
                // probabilities of t) runs at raised wave priority, so its
                // VALU-heavy stream issues ahead of the other resident wave,
                // whose MFMAs keep the matrix pipe busy meanwhile; 3-6%
                // faster than equal priorities at 40 heads x 1200 tiles,
                // top-120 rows.
                __builtin_amdgcn_s_setprio(1);
                if (steady) BSTA_ACQUIRE_STEADY(sl, wave == 0);
                else BSTA_ACQUIRE(sl);
                scores(sl, sc_next, [&](int gi) {
#pragma unroll
                    for (int c = gi * 4 / NG; c < (gi + 1) * 4 / NG; ++c)
                        probs_chunk(sc_cur, c, neg_m, pf[c], ps[c]);
                });
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) probs_chunk(sc_cur, c, neg_m, pf[c], ps[c]);
            }
            __builtin_amdgcn_s_setprio(0);
            float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
            // The reference max starts from the first tile with a valid key
            // (m_init, wave-uniform); after that the probabilities are
            // accepted unless some lane's sum is above 2^64 (or not
            // finite): then m is raised to this tile's max first (rare).
            // Lanes l and l^32 hold keys of the same query and always share
            // m, so every decision below uses the pair's maximum.
            const bool bad = !(psum <= 0x1p64f);
            if (!m_init || __builtin_amdgcn_ballot_w64(bad) != 0) {
                float mx = fmaxf(sc_cur[0][0], sc_cur[1][0]);
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(sc_cur[0][r], sc_cur[1][r]));
                mx = fmaxf(mx, wave_xor32(mx)) * scale_log2;  // tile max of s*c
                const float m_new = !m_init ? (mx == -INFINITY ? m_run : mx) : fmaxf(m_run, mx);
                const float alpha = !m_init ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                m_run = m_new;
                psum = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) probs_chunk(sc_cur, c, -m_new, pf[c], psum);
                m_init = m_init || nj_cur > 0;
            }
            l_run += psum;

            // O^T += V(t)^T P(t)^T: 16-key steps kk of the V half-tiles; the
            // V^T operands of step g+1 are read while step g multiplies.
            {
                int sl;
                if (steady) BSTA_ACQUIRE_STEADY(sl, wave == 1);
                else BSTA_ACQUIRE(sl);
                // Advance the XCD's sweep clock (no return value: nothing
                // waits for it).
                if (rotate && (t & 15) == 15 && tid == 0)
                    __hip_atomic_fetch_add(sweep, 16u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                const uint32_t sbv[2] = {(uint32_t)sl * SLOT_BYTES, (uint32_t)next_slot_of(sl) * SLOT_BYTES};
                auto load_v = [&](int gidx, bf16x8 (&av)[NDB]) {
                    const uint32_t sb = sbv[gidx >> 1] + (gidx & 1) * 32 * D;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const uint32_t a0 = vaddr[db] + sb;
                        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a0);
                        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(a0 + 16 * D));
                        const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        av[db] = __builtin_bit_cast(bf16x8, w);
                    }
                };
                bf16x8 va[2][NDB];
                load_v(0, va[0]);
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    if (gi + 1 < 4) load_v(gi + 1, va[(gi + 1) & 1]);
#pragma unroll
                    for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(va[gi & 1][db], pf[gi], oacc[db]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            r2 = r2 + 1 >= n ? r2 + 1 - n : r2 + 1;
            if (more) {
                nj_cur = clean ? 64 : mask(sc_next, tile_id(t + 1));
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) sc_cur[kb] = sc_next[kb];
            }
        }
#undef BSTA_ACQUIRE
#undef BSTA_ACQUIRE_STEADY
#undef BSTA_ISSUE_NEXT
        if (rotate && (n & 15) != 0 && tid == 0)
            __hip_atomic_fetch_add(sweep, (unsigned)(n & 15), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        // Retire the last slots before the next item refills the ring.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();

        // Finalise: l is split over lanes l and l^32.  With a keep mask (query
        // pruning) a row outside it is written like a pad row.
        const int ni = unit_occupancy(g, iu);
        const float l_tot = l_run + wave_xor32(l_run);
        const bool kept = keep == nullptr || ((keep[(int64_t)bh * NU + iu] >> qi) & 1) != 0;
        const bool valid = qi < ni && l_tot > 0.f && kept;
        const float inv = valid ? 1.0f / l_tot : 0.f;
        // Output row: slot i*64 + qi of the tiled tensor, or with `raster`
        // the token that slot holds in [B, L, H, D] (a pad slot has none).
        int64_t orow_idx = batch_row0 + (int64_t)iu * 64 + qi;
        bool has_row = true;
        if (raster) {
            const int64_t tok = slot_to_token(g, (int64_t)iu * 64 + qi);
            has_row = tok >= 0;
            orow_idx = (int64_t)b * g.L + (tok < 0 ? 0 : tok);
        }
        __bf16* orow = o + orow_idx * rs + head_off;
        if (has_row) {
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
        }
        if (lse != nullptr && half == 0) {
            const float val = valid ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
            lse[(int64_t)bh * g.Lpad + (int64_t)iu * 64 + qi] = val;
        }
    }
}

namespace {

// Workgroups of the attention kernel resident per XCD on the current device
// (computed once per device and kernel variant).  Host threads may race here:
// each entry is an atomic, and racing threads store the same value.
int resident_per_xcd(const void* kernel, int which, int block) {
    static std::atomic<int> cache[4][64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 16;
    const int known = cache[which][dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0) {
        cus = 256;
        per_cu = 512 / block;
    }
    const int r = (cus / 8) * per_cu > 0 ? (cus / 8) * per_cu : 1;
    cache[which][dev].store(r, std::memory_order_relaxed);
    return r;
}

template <int D, int SUB>
hipError_t launch_variant(const Geo& g, const void* q, const void* k, const void* v,
                          const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len,
                          float scale_log2, void* o, float* lse, const uint64_t* keep, int rotate,
                          bool raster, hipStream_t stream) {
    const void* kernel = (const void*)attn_fwd_kernel<D, SUB>;
    const int64_t n_items = (int64_t)g.B * g.H * g.Nt;  // one query tile per item
    const int64_t items_per_xcd = (n_items + 7) / 8;
    int64_t per_xcd = resident_per_xcd(kernel, (D == 128 ? 0 : 1) + (SUB == 2 ? 2 : 0), 128 * SUB);
    if (per_xcd > items_per_xcd) per_xcd = items_per_xcd;
    const unsigned blocks = (unsigned)(8 * per_xcd);
    hipLaunchKernelGGL((attn_fwd_kernel<D, SUB>), dim3(blocks), dim3(128 * SUB), 0, stream, g,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, row_ptr, col_idx,
                       col_len, scale_log2, (__bf16*)o, lse, keep, items_per_xcd, rotate,
                       raster ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const Geo& g, const void* q, const void* k, const void* v,
                           const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len,
                           float scale, void* o, float* lse, const uint64_t* keep, int rotate,
                           bool raster, hipStream_t stream) {
    const float sl2 = scale * 1.4426950408889634f;
    if (g.D == 128 && g.sub == 1)
        return launch_variant<128, 1>(g, q, k, v, row_ptr, col_idx, col_len, sl2, o, lse, keep,
                                      rotate, raster, stream);
    if (g.D == 64 && g.sub == 1)
        return launch_variant<64, 1>(g, q, k, v, row_ptr, col_idx, col_len, sl2, o, lse, keep,
                                     rotate, raster, stream);
    if (g.D == 128)
        return launch_variant<128, 2>(g, q, k, v, row_ptr, col_idx, col_len, sl2, o, lse, keep,
                                      rotate, raster, stream);
    return launch_variant<64, 2>(g, q, k, v, row_ptr, col_idx, col_len, sl2, o, lse, keep, rotate,
                                 raster, stream);
}

}  // namespace bsta
