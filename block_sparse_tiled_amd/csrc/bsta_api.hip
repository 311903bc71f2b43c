// C ABI of libbsta.so: argument checks, geometry, and kernel launches.
//
// Every entry point validates on the host before touching HIP, so the checks
// (and the host-only helpers) work on a machine without a GPU.  Argument
// rules follow the "bsa_attn" page (__init__: no grouped-query attention, no
// causal mode, scale must be 1/sqrt(d) within rel 1e-4 / abs 1e-5; forward:
// sequence length must match the tiling) and the "video_sparse_attn_h3" page
// (tile(): ValueError on a sequence-length mismatch; build(): tile size from
// a fixed registry).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <cmath>

#include "bsta_common.hpp"

namespace bsta {
hipError_t launch_permute(const Geo& g, const void* src, void* dst, bool to_tiles,
                          hipStream_t stream);
hipError_t launch_tile_pool(const Geo& g, const void* x, void* x_tiled, float* pooled,
                            hipStream_t stream);
hipError_t launch_pool1(const Geo& g, const void* x, float* px, hipStream_t stream);
hipError_t launch_pool(const Geo& g, const void* q, const void* k, float* pq, float* pk,
                       hipStream_t stream);
hipError_t launch_scores(const Geo& g, const float* pq, const float* pk, float* s,
                         hipStream_t stream);
hipError_t launch_topk(const Geo& g, int k, const float* s, uint8_t* mask, int32_t* row_ptr,
                       int32_t* col_idx, hipStream_t stream);
hipError_t launch_sta(const Geo& g, const int32_t* windows, uint8_t* mask, int32_t* row_ptr,
                      int32_t* col_idx, hipStream_t stream);
hipError_t launch_cumulative(const Geo& g, float threshold, int min_blocks, float* s,
                              uint8_t* mask, int32_t* row_ptr, int32_t* col_idx,
                              hipStream_t stream);
hipError_t launch_packed_select(const Geo& g, const PackedSpans& sp, const float* s,
                                uint8_t* mask, int32_t* row_ptr, int32_t* col_idx,
                                hipStream_t stream);
hipError_t bwd_scratch(void** out);
hipError_t launch_attn_bwd(const Geo& g, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len,
                           float scale, void* dq, void* dk, void* dv, float* delta,
                           int32_t* col_start, int32_t* col_cnt, int32_t* row_idx,
                           hipStream_t stream);
hipError_t launch_attn_fwd(const Geo& g, const void* q, const void* k, const void* v,
                           const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len,
                           float scale, void* o, float* lse, const uint64_t* keep, int rotate,
                           bool raster, hipStream_t stream);
hipError_t launch_prune(const Geo& g, const void* q_tiled, double ratio, uint64_t* keep_mask,
                        int32_t* keep_count, float* pooled_q, hipStream_t stream);
}  // namespace bsta

using bsta::Geo;
using bsta::Seg;

namespace {

thread_local char g_err[512] = "";

// Process-wide key-order mode of attn_block_sparse_fwd (attn_set_deterministic:
// 0 = rotated where it pays, 1 = CSR order, 2 = rotated on every row).
std::atomic<int> g_deterministic{0};

// The kernel's rotate argument for a mode: 0 CSR order, 1 rotated where it
// pays (the kernel decides), 2 rotated always.
int walk_of(int mode) { return mode == 1 ? 0 : (mode == 2 ? 2 : 1); }

// Largest tile count top-k selection accepts (its per-row keys and flags
// live in LDS: 5 bytes per tile).
constexpr int kMaxTopkTiles = 12288;
// Largest tile count the cumulative-threshold selection accepts (one wave
// holds a row in registers, 32 scores per lane).
constexpr int kMaxCumulativeTiles = 2048;
// Largest grid side (tile coordinates travel as int16 in window mode).
constexpr int kMaxDim = 1 << 15;

int32_t fail(int32_t code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int32_t ok() {
    g_err[0] = '\0';
    return BSTA_OK;
}

int32_t hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(BSTA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Sizes every launch must stay within (offsets are 64-bit in the kernels;
// grid sizes 32-bit).
int32_t check_sizes(const Geo* g) {
    const double elems = (double)g->B * (double)g->Lpad * (double)g->H * (double)g->D;
    if (elems > 9.0e15) return fail(BSTA_ERR_SHAPE, "tensor too large");
    if ((double)g->B * g->H * g->Nt * 8.0 > 4.0e9)
        return fail(BSTA_ERR_SHAPE, "B*H*Nt too large for one launch");
    return BSTA_OK;
}

// The packed-sequence part of make_geo: token segments (empty dense ones
// dropped, regions divided by the patch), dense tiles first, then regions.
int32_t make_packed(const bsta_segments* sg, Geo* g) {
    if (g->tx != 4)
        return fail(BSTA_ERR_UNSUPPORTED, "packed sequences use 64-token (4x4x4) tiles");
    if (sg->count < 1 || sg->count > BSTA_MAX_SEGMENTS)
        return fail(BSTA_ERR_SHAPE, "segment count %d outside 1..%d", sg->count, BSTA_MAX_SEGMENTS);
    for (int ax = 0; ax < 3; ++ax)
        if (sg->patch[ax] < 1) return fail(BSTA_ERR_SHAPE, "patch size must be >= 1");
    int n = 0, regions = 0;
    int64_t tok = 0;
    for (int i = 0; i < sg->count; ++i) {
        Seg s = {};
        s.tok0 = tok;
        if (sg->kind[i] == 0) {
            if (sg->rows[i] < 0) return fail(BSTA_ERR_SHAPE, "segment %d: %d rows", i, sg->rows[i]);
            if (sg->rows[i] > (1 << 28)) return fail(BSTA_ERR_SHAPE, "segment %d too long", i);
            if (sg->rows[i] == 0) continue;  // dropped
            s.rows = sg->rows[i];
            s.ntile = (s.rows + 63) / 64;
            tok += s.rows;
        } else if (sg->kind[i] == 1) {
            int d[3];
            for (int ax = 0; ax < 3; ++ax) {
                const int v = sg->shape[i][ax];
                if (v <= 0 || v % sg->patch[ax] != 0)
                    return fail(BSTA_ERR_SHAPE,
                                "segment %d: latent shape %dx%dx%d is not a positive multiple of "
                                "patch %dx%dx%d", i, sg->shape[i][0], sg->shape[i][1],
                                sg->shape[i][2], sg->patch[0], sg->patch[1], sg->patch[2]);
                d[ax] = v / sg->patch[ax];
                if (d[ax] > kMaxDim) return fail(BSTA_ERR_SHAPE, "segment %d: side above %d", i, kMaxDim);
            }
            s.T = d[0];
            s.Y = d[1];
            s.X = d[2];
            s.nY = (d[1] + 3) / 4;
            s.nX = (d[2] + 3) / 4;
            s.ntile = ((d[0] + 3) / 4) * s.nY * s.nX;
            tok += (int64_t)d[0] * d[1] * d[2];
            ++regions;
        } else {
            return fail(BSTA_ERR_SHAPE, "segment %d: kind %d (0 dense, 1 video region)", i,
                        sg->kind[i]);
        }
        g->seg[n++] = s;
    }
    if (regions == 0) return fail(BSTA_ERR_SHAPE, "a packed sequence needs a video region");
    g->nseg = n;
    int64_t tiles = 0;
    bool full = true;
    for (int pass = 0; pass < 2; ++pass)  // dense segments first, then regions
        for (int i = 0; i < n; ++i) {
            Seg& s = g->seg[i];
            if ((s.rows > 0) != (pass == 0)) continue;
            s.tile0 = (int32_t)tiles;
            tiles += s.ntile;
            if (tiles > (1 << 26)) return fail(BSTA_ERR_SHAPE, "tile count too large");
            full = full && (s.rows > 0 ? s.rows % 64 == 0
                                       : (s.T % 4 == 0 && s.Y % 4 == 0 && s.X % 4 == 0));
            if (pass == 0) g->nprefix = (int32_t)tiles;
        }
    g->Nt = (int32_t)tiles;
    g->L = tok;
    g->Lpad = tiles * 64;
    g->full = full ? 1 : 0;
    g->T = g->Y = g->X = 0;
    g->nT = g->nY = g->nX = 0;
    return check_sizes(g);
}

// Validate a geometry and fill the derived fields.
int32_t make_geo(const bsta_geom* in, Geo* g) {
    if (in == nullptr) return fail(BSTA_ERR_NULL, "geometry pointer is NULL");
    if (in->tile_t != 4 || in->tile_y != 4 || (in->tile_x != 4 && in->tile_x != 8))
        return fail(BSTA_ERR_UNSUPPORTED,
                    "tile %dx%dx%d unsupported: 4x4x4 (64 tokens) or 4x4x8 (128 tokens)",
                    in->tile_t, in->tile_y, in->tile_x);
    if (in->D != 64 && in->D != 128)
        return fail(BSTA_ERR_UNSUPPORTED, "head dim D=%d unsupported: must be 64 or 128", in->D);
    if (in->B < 1 || in->H < 1)
        return fail(BSTA_ERR_SHAPE, "B=%d H=%d: both must be >= 1", in->B, in->H);
    *g = Geo{};
    g->B = in->B;
    g->H = in->H;
    g->D = in->D;
    g->tx = in->tile_x;
    g->lx = in->tile_x == 8 ? 3 : 2;
    g->E = 16 * in->tile_x;
    g->le = in->tile_x == 8 ? 7 : 6;
    g->sub = g->E / 64;
    if (in->segments != nullptr) return make_packed(in->segments, g);
    if (in->T < 1 || in->Y < 1 || in->X < 1)
        return fail(BSTA_ERR_SHAPE, "B=%d H=%d T=%d Y=%d X=%d: all must be >= 1", in->B, in->H,
                    in->T, in->Y, in->X);
    if (in->T > kMaxDim || in->Y > kMaxDim || in->X > kMaxDim)
        return fail(BSTA_ERR_SHAPE, "grid side above %d", kMaxDim);
    g->T = in->T;
    g->Y = in->Y;
    g->X = in->X;
    g->nT = (in->T + 3) / 4;
    g->nY = (in->Y + 3) / 4;
    g->nX = (in->X + g->tx - 1) / g->tx;
    const int64_t nt = (int64_t)g->nT * g->nY * g->nX;
    if (nt > (1 << 26)) return fail(BSTA_ERR_SHAPE, "tile count %lld too large", (long long)nt);
    g->Nt = (int32_t)nt;
    g->L = (int64_t)in->T * in->Y * in->X;
    g->Lpad = nt * g->E;
    g->full = (in->T % 4 == 0 && in->Y % 4 == 0 && in->X % g->tx == 0) ? 1 : 0;
    return check_sizes(g);
}

int32_t check_windows(const Geo& g, const int32_t* w, int64_t* per_batch) {
    if (g.nseg > 0)
        return fail(BSTA_ERR_UNSUPPORTED, "window mode needs a single grid, not a packed sequence");
    if (w == nullptr) return fail(BSTA_ERR_NULL, "sta_windows_host is NULL in window mode");
    if (g.H > BSTA_MAX_STA_HEADS)
        return fail(BSTA_ERR_SHAPE, "H=%d above %d heads in window mode", g.H, BSTA_MAX_STA_HEADS);
    int64_t sum = 0;
    const int n[3] = {g.nT, g.nY, g.nX};
    for (int h = 0; h < g.H; ++h) {
        int64_t prod = 1;
        for (int ax = 0; ax < 3; ++ax) {
            const int v = w[3 * h + ax];
            if (v < 1 || v > n[ax])
                return fail(BSTA_ERR_SHAPE, "head %d window %d,%d,%d outside tile grid %d,%d,%d", h,
                            w[3 * h], w[3 * h + 1], w[3 * h + 2], n[0], n[1], n[2]);
            prod *= v;
        }
        sum += prod;
    }
    *per_batch = sum;
    return BSTA_OK;
}

// CSR entry count of a selection, or a negative status.
// The selection kind without the BSTA_SELECT_PREPOOLED flag, or -1 when the
// flag is set on anything but top-k.
int32_t base_mode(int32_t mode) {
    if (mode & BSTA_SELECT_PREPOOLED) {
        const int32_t m = mode & ~BSTA_SELECT_PREPOOLED;
        return m == BSTA_SELECT_TOPK || m == BSTA_SELECT_CUMULATIVE ? m : -1;
    }
    return mode;
}

int64_t capacity_of(const Geo& g, int32_t mode_in, int32_t topk, const int32_t* windows) {
    int64_t nnz;
    const int32_t mode = base_mode(mode_in);
    if (mode == BSTA_SELECT_TOPK) {
        if (topk < 1 || topk > g.Nt)
            return fail(BSTA_ERR_SHAPE, "topk=%d outside [1, Nt=%d]", topk, g.Nt);
        nnz = (int64_t)g.B * g.H * g.Nt * topk;
    } else if (mode == BSTA_SELECT_STA) {
        int64_t per_batch = 0;
        int32_t st = check_windows(g, windows, &per_batch);
        if (st != BSTA_OK) return st;
        nnz = (int64_t)g.B * g.Nt * per_batch;
    } else if (mode == BSTA_SELECT_CUMULATIVE) {
        // Data-dependent row lengths: room for every row to keep all tiles.
        nnz = (int64_t)g.B * g.H * g.Nt * g.Nt;
    } else {
        return fail(BSTA_ERR_UNSUPPORTED, "selection mode %d unknown", mode_in);
    }
    if (nnz > 0x7fffffffLL)
        return fail(BSTA_ERR_SHAPE, "%lld CSR entries overflow int32 row_ptr", (long long)nnz);
    return nnz;
}

// Tiles a span of n keeps at keep fraction `keep`: floor(keep * n) in
// double precision, clamped to [1, n].
int32_t span_keep(int32_t n, double keep) {
    const double f = std::floor(keep * (double)n);
    return f < 1.0 ? 1 : (f > (double)n ? n : (int32_t)f);
}

// The selection of a packed sequence: spans and their keep counts (exempt
// mode) or the single k of compete mode, and the CSR entry count.
int64_t packed_plan(const Geo& g, double sparsity, double ref_keep_rate, int32_t exempt,
                    bsta::PackedSpans* sp, int32_t* compete_k) {
    if (g.nseg == 0)
        return fail(BSTA_ERR_UNSUPPORTED, "a packed selection needs a packed geometry");
    if (!std::isfinite(sparsity) || sparsity > 1.0)
        return fail(BSTA_ERR_SHAPE, "sparsity %g must be finite and <= 1", sparsity);
    *sp = bsta::PackedSpans{};
    sp->nprefix = g.nprefix;
    for (int t = 0; t < g.nseg; ++t)
        if (g.seg[t].rows == 0) {
            sp->a[sp->n] = g.seg[t].tile0;
            sp->b[sp->n] = g.seg[t].tile0 + g.seg[t].ntile;
            ++sp->n;
        }
    int64_t nnz;
    if (!exempt) {
        if (sp->n != 1)
            return fail(BSTA_ERR_UNSUPPORTED,
                        "compete mode supports one video region, the sequence has %d", sp->n);
        *compete_k = sparsity <= 0.0 ? g.Nt : span_keep(g.Nt, 1.0 - sparsity);
        nnz = (int64_t)g.B * g.H * g.Nt * *compete_k;
    } else {
        const bool dense = sparsity <= 0.0;
        if (sp->n > 1 && !(ref_keep_rate >= 0.0 && ref_keep_rate <= 1.0))
            return fail(BSTA_ERR_SHAPE, "ref_keep_rate %g outside [0, 1] with %d regions",
                        ref_keep_rate, sp->n);
        if (g.Nt > kMaxCumulativeTiles)
            return fail(BSTA_ERR_SHAPE, "packed selection supports at most %d tiles, got %d",
                        kMaxCumulativeTiles, g.Nt);
        sp->vlen = sp->nprefix;
        for (int r = 0; r < sp->n; ++r) {
            const int32_t n = sp->b[r] - sp->a[r];
            const double keep = dense ? 1.0 : (r + 1 < sp->n ? ref_keep_rate : 1.0 - sparsity);
            sp->k[r] = span_keep(n, keep);
            sp->vlen += sp->k[r];
        }
        nnz = (int64_t)g.B * g.H *
              ((int64_t)sp->nprefix * g.Nt + (int64_t)(g.Nt - sp->nprefix) * sp->vlen);
    }
    if (nnz > 0x7fffffffLL)
        return fail(BSTA_ERR_SHAPE, "%lld CSR entries overflow int32 row_ptr", (long long)nnz);
    return nnz;
}

int64_t workspace_of(const Geo& g, int32_t mode_in) {
    const int32_t mode = base_mode(mode_in);
    if (mode == BSTA_SELECT_STA) return 0;
    if (mode != BSTA_SELECT_TOPK && mode != BSTA_SELECT_CUMULATIVE)
        return fail(BSTA_ERR_UNSUPPORTED, "selection mode %d unknown", mode_in);
    const int64_t pooled = (int64_t)2 * g.B * g.H * g.Nt * g.D;
    const int64_t scores = (int64_t)g.B * g.H * g.Nt * g.Nt;
    return (pooled + scores) * (int64_t)sizeof(float);
}

}  // namespace

namespace {
// Backward workspace: delta fp32 [B*H*Lpad], col_start and col_cnt int32
// [B*H*Nt] each, row_idx int32 [col_len]; every part 256-byte aligned.
struct BwdLayout {
    int64_t delta, col_start, col_cnt, row_idx, total;
};

BwdLayout bwd_layout(const Geo& g, int64_t col_len) {
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    BwdLayout l;
    l.delta = 0;
    // rowsum(dO*O) per query slot, then log2(e)*lse per query slot.
    l.col_start = up(l.delta + (int64_t)2 * g.B * g.H * g.Lpad * 4);
    l.col_cnt = up(l.col_start + (int64_t)g.B * g.H * g.Nt * 4);
    l.row_idx = up(l.col_cnt + (int64_t)g.B * g.H * g.Nt * 4);
    l.total = up(l.row_idx + (col_len > 0 ? col_len : 0) * 4);
    return l;
}

int32_t check_scale(const Geo& g, float softmax_scale, int32_t causal) {
    if (causal != 0)
        return fail(BSTA_ERR_UNSUPPORTED, "causal=%d: block-sparse attention is bidirectional only",
                    causal);
    const double expected = 1.0 / sqrt((double)g.D);
    const double diff = fabs((double)softmax_scale - expected);
    const double tol = fmax(1e-4 * fmax(fabs((double)softmax_scale), expected), 1e-5);
    if (!(diff <= tol))
        return fail(BSTA_ERR_UNSUPPORTED, "softmax_scale %g must be 1/sqrt(D) = %g",
                    (double)softmax_scale, expected);
    return BSTA_OK;
}

int32_t block_sparse_fwd(const char* name, const bsta_geom* gin, const void* q_tiled,
                         const void* k_tiled, const void* v_tiled, const int32_t* row_ptr,
                         const int32_t* col_idx, int64_t col_len, float softmax_scale,
                         int32_t causal, const uint64_t* keep, void* o, float* lse, bool raster,
                         void* stream) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    if (q_tiled == nullptr || k_tiled == nullptr || v_tiled == nullptr || o == nullptr ||
        row_ptr == nullptr || col_idx == nullptr)
        return fail(BSTA_ERR_NULL, "%s: NULL tensor or index pointer", name);
    st = check_scale(g, softmax_scale, causal);
    if (st != BSTA_OK) return st;
    if (col_len < 0) return fail(BSTA_ERR_SHAPE, "col_len %lld < 0", (long long)col_len);
    return hip_status(bsta::launch_attn_fwd(g, q_tiled, k_tiled, v_tiled, row_ptr, col_idx,
                                            col_len, softmax_scale, o, lse, keep,
                                            walk_of(g_deterministic.load(std::memory_order_relaxed)),
                                            raster, (hipStream_t)stream),
                      name);
}
}  // namespace

extern "C" {

const char* attn_status_string(int32_t status) {
    switch (status) {
        case BSTA_OK: return "ok";
        case BSTA_ERR_NULL: return "null pointer";
        case BSTA_ERR_SHAPE: return "shape or size outside the specification";
        case BSTA_ERR_UNSUPPORTED: return "unsupported argument";
        case BSTA_ERR_CAPACITY: return "output or workspace too small";
        case BSTA_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

const char* attn_last_error(void) { return g_err; }

int32_t attn_geometry(const bsta_geom* gin, int32_t* num_tiles, int64_t* padded_len,
                      int32_t* occupancy) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    if (num_tiles) *num_tiles = g.Nt;
    if (padded_len) *padded_len = g.Lpad;
    if (occupancy)
        for (int j = 0; j < g.Nt; ++j) occupancy[j] = bsta::tile_occupancy(g, j);
    return ok();
}

int64_t attn_select_capacity(const bsta_geom* gin, int32_t mode, int32_t topk,
                             const int32_t* sta_windows_host) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    int64_t n = capacity_of(g, mode, topk, sta_windows_host);
    if (n >= 0) ok();
    return n;
}

int64_t attn_workspace_bytes(const bsta_geom* gin, int32_t mode) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    int64_t n = workspace_of(g, mode);
    if (n >= 0) ok();
    return n;
}

int32_t attn_tile(const bsta_geom* gin, const void* x, void* x_tiled, void* stream) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    if (x == nullptr || x_tiled == nullptr) return fail(BSTA_ERR_NULL, "attn_tile: NULL tensor");
    return hip_status(bsta::launch_permute(g, x, x_tiled, true, (hipStream_t)stream), "attn_tile");
}

int32_t attn_tile_pool(const bsta_geom* gin, const void* x, void* x_tiled, float* pooled,
                       void* stream) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    if (x == nullptr || x_tiled == nullptr || pooled == nullptr)
        return fail(BSTA_ERR_NULL, "attn_tile_pool: NULL tensor");
    return hip_status(bsta::launch_tile_pool(g, x, x_tiled, pooled, (hipStream_t)stream),
                      "attn_tile_pool");
}

int32_t attn_pool(const bsta_geom* gin, const void* x_tiled, float* pooled, void* stream) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    if (x_tiled == nullptr || pooled == nullptr) return fail(BSTA_ERR_NULL, "attn_pool: NULL tensor");
    return hip_status(bsta::launch_pool1(g, x_tiled, pooled, (hipStream_t)stream), "attn_pool");
}

int32_t attn_untile(const bsta_geom* gin, const void* y_tiled, void* y, void* stream) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    if (y == nullptr || y_tiled == nullptr) return fail(BSTA_ERR_NULL, "attn_untile: NULL tensor");
    return hip_status(bsta::launch_permute(g, y_tiled, y, false, (hipStream_t)stream),
                      "attn_untile");
}

int32_t attn_select_blocks(const bsta_geom* gin, const void* q_tiled, const void* k_tiled,
                           int32_t mode, int32_t topk, const int32_t* sta_windows_host,
                           uint8_t* block_mask, int32_t* row_ptr, int32_t* col_idx,
                           int64_t col_capacity, void* workspace, int64_t workspace_bytes,
                           void* stream) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    if (row_ptr == nullptr || col_idx == nullptr)
        return fail(BSTA_ERR_NULL, "attn_select_blocks: NULL row_ptr or col_idx");
    const int64_t need = capacity_of(g, mode, topk, sta_windows_host);
    if (need < 0) return (int32_t)need;
    if (col_capacity < need)
        return fail(BSTA_ERR_CAPACITY, "col_capacity %lld < %lld entries needed",
                    (long long)col_capacity, (long long)need);
    hipStream_t s = (hipStream_t)stream;
    const bool prepooled = (mode & BSTA_SELECT_PREPOOLED) != 0;
    mode = base_mode(mode);
    if (mode == BSTA_SELECT_CUMULATIVE)
        return fail(BSTA_ERR_UNSUPPORTED,
                    "attn_select_blocks: the cumulative-threshold mode is attn_select_cumulative");
    if (mode == BSTA_SELECT_STA)
        return hip_status(bsta::launch_sta(g, sta_windows_host, block_mask, row_ptr, col_idx, s),
                          "attn_select_blocks(window)");
    if (!prepooled && (q_tiled == nullptr || k_tiled == nullptr))
        return fail(BSTA_ERR_NULL, "attn_select_blocks: NULL q_tiled or k_tiled in top-k mode");
    if (g.Nt > kMaxTopkTiles)
        return fail(BSTA_ERR_SHAPE, "top-k selection supports at most %d tiles, got %d",
                    kMaxTopkTiles, g.Nt);
    const int64_t ws = workspace_of(g, mode);
    if (workspace == nullptr) return fail(BSTA_ERR_NULL, "attn_select_blocks: NULL workspace");
    if (workspace_bytes < ws)
        return fail(BSTA_ERR_CAPACITY, "workspace %lld bytes < %lld needed",
                    (long long)workspace_bytes, (long long)ws);
    float* pq = (float*)workspace;
    float* pk = pq + (int64_t)g.B * g.H * g.Nt * g.D;
    float* sc = pk + (int64_t)g.B * g.H * g.Nt * g.D;
    hipError_t e = prepooled ? hipSuccess : bsta::launch_pool(g, q_tiled, k_tiled, pq, pk, s);
    if (e == hipSuccess) e = bsta::launch_scores(g, pq, pk, sc, s);
    if (e == hipSuccess) e = bsta::launch_topk(g, topk, sc, block_mask, row_ptr, col_idx, s);
    return hip_status(e, "attn_select_blocks(top-k)");
}

int32_t attn_select_cumulative(const bsta_geom* gin, const void* q_tiled, const void* k_tiled,
                               int32_t flags, float threshold, int32_t min_blocks,
                               uint8_t* block_mask, int32_t* row_ptr, int32_t* col_idx,
                               int64_t col_capacity, void* workspace, int64_t workspace_bytes,
                               void* stream) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    if (flags != 0 && flags != BSTA_SELECT_PREPOOLED)
        return fail(BSTA_ERR_UNSUPPORTED, "attn_select_cumulative: flags %d unknown", flags);
    const bool prepooled = flags == BSTA_SELECT_PREPOOLED;
    if (row_ptr == nullptr || col_idx == nullptr)
        return fail(BSTA_ERR_NULL, "attn_select_cumulative: NULL row_ptr or col_idx");
    if (!prepooled && (q_tiled == nullptr || k_tiled == nullptr))
        return fail(BSTA_ERR_NULL, "attn_select_cumulative: NULL q_tiled or k_tiled");
    if (!(threshold > 0.f && threshold <= 1.f))
        return fail(BSTA_ERR_SHAPE, "threshold %g outside (0, 1]", (double)threshold);
    if (min_blocks < 0) return fail(BSTA_ERR_SHAPE, "min_blocks %d < 0", min_blocks);
    if (g.Nt > kMaxCumulativeTiles)
        return fail(BSTA_ERR_SHAPE, "cumulative selection supports at most %d tiles, got %d",
                    kMaxCumulativeTiles, g.Nt);
    const int64_t need = capacity_of(g, BSTA_SELECT_CUMULATIVE, 0, nullptr);
    if (need < 0) return (int32_t)need;
    if (col_capacity < need)
        return fail(BSTA_ERR_CAPACITY, "col_capacity %lld < %lld entries (every row may keep all tiles)",
                    (long long)col_capacity, (long long)need);
    const int64_t ws = workspace_of(g, BSTA_SELECT_CUMULATIVE);
    if (workspace == nullptr)
        return fail(BSTA_ERR_NULL, "attn_select_cumulative: NULL workspace");
    if (workspace_bytes < ws)
        return fail(BSTA_ERR_CAPACITY, "workspace %lld bytes < %lld needed",
                    (long long)workspace_bytes, (long long)ws);
    hipStream_t s = (hipStream_t)stream;
    float* pq = (float*)workspace;
    float* pk = pq + (int64_t)g.B * g.H * g.Nt * g.D;
    float* sc = pk + (int64_t)g.B * g.H * g.Nt * g.D;
    hipError_t e = prepooled ? hipSuccess : bsta::launch_pool(g, q_tiled, k_tiled, pq, pk, s);
    if (e == hipSuccess) e = bsta::launch_scores(g, pq, pk, sc, s);
    if (e == hipSuccess)
        e = bsta::launch_cumulative(g, threshold, min_blocks, sc, block_mask, row_ptr, col_idx, s);
    return hip_status(e, "attn_select_cumulative");
}

int32_t attn_packed_info(const bsta_geom* gin, int32_t* num_prefix, int32_t* num_regions,
                         int32_t* spans, int64_t* packed_len) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    if (g.nseg == 0) return fail(BSTA_ERR_UNSUPPORTED, "attn_packed_info: not a packed geometry");
    int r = 0;
    for (int t = 0; t < g.nseg; ++t)
        if (g.seg[t].rows == 0) {
            if (spans) {
                spans[2 * r] = g.seg[t].tile0;
                spans[2 * r + 1] = g.seg[t].tile0 + g.seg[t].ntile;
            }
            ++r;
        }
    if (num_prefix) *num_prefix = g.nprefix;
    if (num_regions) *num_regions = r;
    if (packed_len) *packed_len = g.L;
    return ok();
}

int64_t attn_packed_capacity(const bsta_geom* gin, double sparsity, double ref_keep_rate,
                             int32_t exempt) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    bsta::PackedSpans sp;
    int32_t k = 0;
    const int64_t n = packed_plan(g, sparsity, ref_keep_rate, exempt, &sp, &k);
    if (n >= 0) ok();
    return n;
}

int32_t attn_select_packed(const bsta_geom* gin, const void* q_tiled, const void* k_tiled,
                           int32_t flags, double sparsity, double ref_keep_rate, int32_t exempt,
                           uint8_t* block_mask, int32_t* row_ptr, int32_t* col_idx,
                           int64_t col_capacity, void* workspace, int64_t workspace_bytes,
                           void* stream) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    if (flags != 0 && flags != BSTA_SELECT_PREPOOLED)
        return fail(BSTA_ERR_UNSUPPORTED, "attn_select_packed: flags %d unknown", flags);
    const bool prepooled = flags == BSTA_SELECT_PREPOOLED;
    if (row_ptr == nullptr || col_idx == nullptr)
        return fail(BSTA_ERR_NULL, "attn_select_packed: NULL row_ptr or col_idx");
    if (!prepooled && (q_tiled == nullptr || k_tiled == nullptr))
        return fail(BSTA_ERR_NULL, "attn_select_packed: NULL q_tiled or k_tiled");
    bsta::PackedSpans sp;
    int32_t k = 0;
    const int64_t need = packed_plan(g, sparsity, ref_keep_rate, exempt, &sp, &k);
    if (need < 0) return (int32_t)need;
    if (col_capacity < need)
        return fail(BSTA_ERR_CAPACITY, "col_capacity %lld < %lld entries needed",
                    (long long)col_capacity, (long long)need);
    if (g.Nt > kMaxTopkTiles)
        return fail(BSTA_ERR_SHAPE, "packed selection supports at most %d tiles, got %d",
                    kMaxTopkTiles, g.Nt);
    const int64_t ws = workspace_of(g, BSTA_SELECT_TOPK);
    if (workspace == nullptr) return fail(BSTA_ERR_NULL, "attn_select_packed: NULL workspace");
    if (workspace_bytes < ws)
        return fail(BSTA_ERR_CAPACITY, "workspace %lld bytes < %lld needed",
                    (long long)workspace_bytes, (long long)ws);
    hipStream_t s = (hipStream_t)stream;
    float* pq = (float*)workspace;
    float* pk = pq + (int64_t)g.B * g.H * g.Nt * g.D;
    float* sc = pk + (int64_t)g.B * g.H * g.Nt * g.D;
    hipError_t e = prepooled ? hipSuccess : bsta::launch_pool(g, q_tiled, k_tiled, pq, pk, s);
    if (e == hipSuccess) e = bsta::launch_scores(g, pq, pk, sc, s);
    if (e == hipSuccess)
        e = exempt ? bsta::launch_packed_select(g, sp, sc, block_mask, row_ptr, col_idx, s)
                   : bsta::launch_topk(g, k, sc, block_mask, row_ptr, col_idx, s);
    return hip_status(e, "attn_select_packed");
}

int32_t attn_block_sparse_fwd(const bsta_geom* gin, const void* q_tiled, const void* k_tiled,
                              const void* v_tiled, const int32_t* row_ptr, const int32_t* col_idx,
                              int64_t col_len, float softmax_scale, int32_t causal,
                              void* o_tiled, float* lse, void* stream) {
    return block_sparse_fwd("attn_block_sparse_fwd", gin, q_tiled, k_tiled, v_tiled, row_ptr,
                            col_idx, col_len, softmax_scale, causal, nullptr, o_tiled, lse, false,
                            stream);
}

int32_t attn_block_sparse_fwd_raster(const bsta_geom* gin, const void* q_tiled,
                                     const void* k_tiled, const void* v_tiled,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     int64_t col_len, float softmax_scale, int32_t causal, void* o,
                                     float* lse, void* stream) {
    return block_sparse_fwd("attn_block_sparse_fwd_raster", gin, q_tiled, k_tiled, v_tiled,
                            row_ptr, col_idx, col_len, softmax_scale, causal, nullptr, o, lse, true,
                            stream);
}

int32_t attn_prune_queries(const bsta_geom* gin, const void* q_tiled, double keep_ratio,
                           uint64_t* keep_mask, int32_t* keep_count, float* pooled_q,
                           void* stream) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    if (q_tiled == nullptr || keep_mask == nullptr || pooled_q == nullptr)
        return fail(BSTA_ERR_NULL, "attn_prune_queries: NULL q_tiled, keep_mask or pooled_q");
    if (g.nseg > 0)
        return fail(BSTA_ERR_UNSUPPORTED, "attn_prune_queries: a single grid only (not packed)");
    if (!(keep_ratio > 0.0 && keep_ratio <= 1.0))
        return fail(BSTA_ERR_SHAPE, "keep_ratio %g outside (0, 1]", keep_ratio);
    return hip_status(bsta::launch_prune(g, q_tiled, keep_ratio, keep_mask, keep_count, pooled_q,
                                         (hipStream_t)stream),
                      "attn_prune_queries");
}

int32_t attn_block_sparse_fwd_pruned(const bsta_geom* gin, const void* q_tiled,
                                     const void* k_tiled, const void* v_tiled,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     int64_t col_len, float softmax_scale, int32_t causal,
                                     const uint64_t* keep_mask, int32_t raster, void* o,
                                     float* lse, void* stream) {
    if (keep_mask == nullptr)
        return fail(BSTA_ERR_NULL, "attn_block_sparse_fwd_pruned: NULL keep_mask");
    if (gin != nullptr && gin->segments != nullptr)
        return fail(BSTA_ERR_UNSUPPORTED,
                    "attn_block_sparse_fwd_pruned: a single grid only (not packed)");
    return block_sparse_fwd("attn_block_sparse_fwd_pruned", gin, q_tiled, k_tiled, v_tiled,
                            row_ptr, col_idx, col_len, softmax_scale, causal, keep_mask, o, lse,
                            raster != 0, stream);
}

int64_t attn_bwd_workspace_bytes(const bsta_geom* gin, int64_t col_len) {
    Geo g;
    int32_t st = make_geo(gin, &g);
    if (st != BSTA_OK) return st;
    if (col_len < 0) return fail(BSTA_ERR_SHAPE, "col_len %lld < 0", (long long)col_len);
    ok();
    return bwd_layout(g, col_len).total;
}

}  // extern "C"

namespace {

// Argument checks shared by the two backward entry points.
int32_t check_bwd(const bsta_geom* gin, Geo* g, const void* q_tiled, const void* k_tiled,
                  const void* v_tiled, const void* o_tiled, const void* do_tiled, const float* lse,
                  const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len,
                  float softmax_scale, int32_t causal, void* dq_tiled, void* dk_tiled,
                  void* dv_tiled, const char* who) {
    int32_t st = make_geo(gin, g);
    if (st != BSTA_OK) return st;
    if (q_tiled == nullptr || k_tiled == nullptr || v_tiled == nullptr || o_tiled == nullptr ||
        do_tiled == nullptr || lse == nullptr || row_ptr == nullptr || col_idx == nullptr ||
        dq_tiled == nullptr || dk_tiled == nullptr || dv_tiled == nullptr)
        return fail(BSTA_ERR_NULL, "%s: NULL tensor, lse or index pointer", who);
    st = check_scale(*g, softmax_scale, causal);
    if (st != BSTA_OK) return st;
    if (col_len < 0) return fail(BSTA_ERR_SHAPE, "col_len %lld < 0", (long long)col_len);
    if (col_len > 0x7fffffffLL)
        return fail(BSTA_ERR_SHAPE, "col_len %lld overflows int32 offsets", (long long)col_len);
    if (g->Nt > bsta::kMaxBwdTiles)
        return fail(BSTA_ERR_SHAPE, "the backward supports at most %d tiles, got %d", bsta::kMaxBwdTiles,
                    g->Nt);
    return BSTA_OK;
}

int32_t run_bwd(const Geo& g, const BwdLayout& l, char* ws, const void* q_tiled,
                const void* k_tiled, const void* v_tiled, const void* o_tiled, const void* do_tiled,
                const float* lse, const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len,
                float softmax_scale, void* dq_tiled, void* dk_tiled, void* dv_tiled, void* stream,
                const char* who) {
    return hip_status(
            bsta::launch_attn_bwd(g, q_tiled, k_tiled, v_tiled, o_tiled, do_tiled, lse, row_ptr,
                                  col_idx, col_len, softmax_scale, dq_tiled, dk_tiled, dv_tiled,
                                  (float*)(ws + l.delta), (int32_t*)(ws + l.col_start),
                                  (int32_t*)(ws + l.col_cnt), (int32_t*)(ws + l.row_idx),
                                  (hipStream_t)stream),
            who);
}

}  // namespace

extern "C" {

int32_t attn_block_sparse_bwd(const bsta_geom* gin, const void* q_tiled, const void* k_tiled,
                              const void* v_tiled, const void* o_tiled, const void* do_tiled,
                              const float* lse, const int32_t* row_ptr, const int32_t* col_idx,
                              int64_t col_len, float softmax_scale, int32_t causal,
                              void* dq_tiled, void* dk_tiled, void* dv_tiled, void* workspace,
                              int64_t workspace_bytes, void* stream) {
    Geo g;
    int32_t st = check_bwd(gin, &g, q_tiled, k_tiled, v_tiled, o_tiled, do_tiled, lse, row_ptr,
                           col_idx, col_len, softmax_scale, causal, dq_tiled, dk_tiled, dv_tiled,
                           "attn_block_sparse_bwd");
    if (st != BSTA_OK) return st;
    const BwdLayout l = bwd_layout(g, col_len);
    if (workspace == nullptr) return fail(BSTA_ERR_NULL, "attn_block_sparse_bwd: NULL workspace");
    if (workspace_bytes < l.total)
        return fail(BSTA_ERR_CAPACITY, "workspace %lld bytes < %lld needed",
                    (long long)workspace_bytes, (long long)l.total);
    return run_bwd(g, l, (char*)workspace, q_tiled, k_tiled, v_tiled, o_tiled, do_tiled, lse,
                   row_ptr, col_idx, col_len, softmax_scale, dq_tiled, dk_tiled, dv_tiled, stream,
                   "attn_block_sparse_bwd");
}

int32_t attn_block_sparse_bwd_noalloc(const bsta_geom* gin, const void* q_tiled,
                                      const void* k_tiled, const void* v_tiled,
                                      const void* o_tiled, const void* do_tiled, const float* lse,
                                      const int32_t* row_ptr, const int32_t* col_idx,
                                      int64_t col_len, float softmax_scale, int32_t causal,
                                      void* dq_tiled, void* dk_tiled, void* dv_tiled,
                                      void* stream) {
    Geo g;
    int32_t st = check_bwd(gin, &g, q_tiled, k_tiled, v_tiled, o_tiled, do_tiled, lse, row_ptr,
                           col_idx, col_len, softmax_scale, causal, dq_tiled, dk_tiled, dv_tiled,
                           "attn_block_sparse_bwd_noalloc");
    if (st != BSTA_OK) return st;
    const BwdLayout l = bwd_layout(g, col_len);
    if (l.total > bsta::kBwdScratchBytes)
        return fail(BSTA_ERR_CAPACITY,
                    "attn_block_sparse_bwd_noalloc: needs %lld bytes of scratch, the static "
                    "scratch holds %lld (use attn_block_sparse_bwd with a workspace)",
                    (long long)l.total, (long long)bsta::kBwdScratchBytes);
    void* ws = nullptr;
    st = hip_status(bsta::bwd_scratch(&ws), "attn_block_sparse_bwd_noalloc: scratch address");
    if (st != BSTA_OK) return st;
    return run_bwd(g, l, (char*)ws, q_tiled, k_tiled, v_tiled, o_tiled, do_tiled, lse, row_ptr,
                   col_idx, col_len, softmax_scale, dq_tiled, dk_tiled, dv_tiled, stream,
                   "attn_block_sparse_bwd_noalloc");
}

int32_t attn_set_deterministic(int32_t enable) {
    const int mode = enable == 0 ? 0 : (enable == 2 ? 2 : 1);
    return g_deterministic.exchange(mode, std::memory_order_relaxed);
}

}  // extern "C"
