// Driver for the host-only AddressSanitizer / UndefinedBehaviorSanitizer
// build of the C ABI's argument validation (bsta_api.hip with the launcher
// stubs of stubs.cpp; no GPU code is built or run).  Every call either is
// host-only or stops at validation, except the accepted ones, which reach a
// stub launcher.  Pointers are dummies that the host code never
// dereferences.  Prints "OK <checks>" and exits 0, or reports the first
// failed check and exits 1.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <thread>
#include <vector>

#include "bsta.h"

int stub_launches();

namespace {

int g_checks = 0;
int g_failed = 0;

void check(bool ok, const char* what, int line) {
    ++g_checks;
    if (!ok && !g_failed) {
        fprintf(stderr, "FAILED line %d: %s (last error: %s)\n", line, what, attn_last_error());
        g_failed = 1;
    }
}
#define CHECK(x) check((x), #x, __LINE__)

void* const F = (void*)0x1000;
uint8_t* const FU8 = (uint8_t*)0x1000;
int32_t* const FI = (int32_t*)0x1000;
uint64_t* const FU64 = (uint64_t*)0x1000;
float* const FF = (float*)0x1000;

bsta_geom geom(int B, int H, int D, int T, int Y, int X, int tx = 4) {
    bsta_geom g = {B, H, D, T, Y, X, 4, 4, tx};
    return g;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

void geometry_checks() {
    const int grids[][3] = {{8, 8, 8}, {21, 30, 52}, {20, 48, 80}, {5, 6, 7}, {1, 1, 1}, {3, 9, 19}};
    for (const auto& gr : grids) {
        for (int tx : {4, 8}) {
            bsta_geom g = geom(1, 2, 64, gr[0], gr[1], gr[2], tx);
            int32_t nt = -1;
            int64_t lpad = -1;
            CHECK(attn_geometry(&g, &nt, &lpad, nullptr) == BSTA_OK);
            const int want = ceil_div(gr[0], 4) * ceil_div(gr[1], 4) * ceil_div(gr[2], tx);
            CHECK(nt == want);
            CHECK(lpad == (int64_t)want * 16 * tx);
            std::vector<int32_t> occ(nt);
            CHECK(attn_geometry(&g, nullptr, nullptr, occ.data()) == BSTA_OK);
            int64_t sum = 0;
            for (int32_t n : occ) {
                CHECK(n >= 1 && n <= 16 * tx);
                sum += n;
            }
            CHECK(sum == (int64_t)gr[0] * gr[1] * gr[2]);
        }
    }
    bsta_geom bad = geom(1, 2, 96, 8, 8, 8);
    CHECK(attn_geometry(&bad, nullptr, nullptr, nullptr) == BSTA_ERR_UNSUPPORTED);
    bad = geom(0, 2, 64, 8, 8, 8);
    CHECK(attn_geometry(&bad, nullptr, nullptr, nullptr) == BSTA_ERR_SHAPE);
    bad = geom(1, 2, 64, 8, 8, 8, 16);
    CHECK(attn_geometry(&bad, nullptr, nullptr, nullptr) == BSTA_ERR_UNSUPPORTED);
    CHECK(attn_geometry(nullptr, nullptr, nullptr, nullptr) == BSTA_ERR_NULL);
    CHECK(strlen(attn_last_error()) > 0);
    for (int s = 0; s >= -6; --s) CHECK(strlen(attn_status_string(s)) > 0);
}

void select_checks() {
    bsta_geom g = geom(1, 2, 64, 8, 8, 8);  // 8 tiles
    CHECK(attn_select_capacity(&g, BSTA_SELECT_TOPK, 3, nullptr) == 1 * 2 * 8 * 3);
    CHECK(attn_select_capacity(&g, BSTA_SELECT_TOPK, 9, nullptr) == BSTA_ERR_SHAPE);
    const int32_t win[] = {1, 1, 1, 2, 2, 2};
    CHECK(attn_select_capacity(&g, BSTA_SELECT_STA, 0, win) == 8 * 1 + 8 * 8);
    const int32_t badwin[] = {1, 1, 1, 3, 1, 1};
    CHECK(attn_select_capacity(&g, BSTA_SELECT_STA, 0, badwin) == BSTA_ERR_SHAPE);
    const int64_t ws = attn_workspace_bytes(&g, BSTA_SELECT_TOPK);
    CHECK(ws == (int64_t)(2 * 2 * 8 * 64 + 2 * 8 * 8) * 4);
    const int before = stub_launches();
    CHECK(attn_select_blocks(&g, F, F, BSTA_SELECT_TOPK, 3, nullptr, FU8, FI, FI, 48, F, ws, nullptr) ==
          BSTA_OK);
    CHECK(stub_launches() > before);
    const int after_ok = stub_launches();
    CHECK(attn_select_blocks(&g, F, F, BSTA_SELECT_TOPK, 3, nullptr, FU8, FI, FI, 47, F, ws, nullptr) ==
          BSTA_ERR_CAPACITY);
    CHECK(attn_select_blocks(&g, F, F, BSTA_SELECT_TOPK, 3, nullptr, FU8, FI, FI, 48, F, ws - 1,
                             nullptr) == BSTA_ERR_CAPACITY);
    CHECK(attn_select_blocks(&g, nullptr, F, BSTA_SELECT_TOPK, 3, nullptr, FU8, FI, FI, 48, F, ws,
                             nullptr) == BSTA_ERR_NULL);
    CHECK(attn_select_blocks(&g, F, F, BSTA_SELECT_TOPK, 0, nullptr, FU8, FI, FI, 48, F, ws, nullptr) ==
          BSTA_ERR_SHAPE);
    CHECK(attn_select_blocks(&g, F, F, 7, 3, nullptr, FU8, FI, FI, 48, F, ws, nullptr) ==
          BSTA_ERR_UNSUPPORTED);
    CHECK(attn_select_blocks(&g, F, F, BSTA_SELECT_STA, 0, badwin, FU8, FI, FI, 1000, F, ws, nullptr) ==
          BSTA_ERR_SHAPE);
    CHECK(attn_select_cumulative(&g, F, F, 0, 0.0f, 0, FU8, FI, FI, 128, F, ws, nullptr) ==
          BSTA_ERR_SHAPE);
    CHECK(attn_select_cumulative(&g, F, F, 0, NAN, 0, FU8, FI, FI, 128, F, ws, nullptr) ==
          BSTA_ERR_SHAPE);
    CHECK(attn_select_cumulative(&g, F, F, 0, 0.5f, -1, FU8, FI, FI, 128, F, ws, nullptr) ==
          BSTA_ERR_SHAPE);
    CHECK(attn_select_cumulative(&g, F, F, 0, 0.5f, 0, FU8, FI, FI, 127, F, ws, nullptr) ==
          BSTA_ERR_CAPACITY);
    CHECK(stub_launches() == after_ok);  // nothing rejected reached a launch
    CHECK(attn_select_cumulative(&g, F, F, 0, 0.5f, 0, FU8, FI, FI, 128, F, ws, nullptr) == BSTA_OK);
}

void path_checks() {
    bsta_geom g = geom(1, 2, 128, 5, 6, 7);
    const float s = 1.0f / sqrtf(128.0f);
    int base = stub_launches();
    CHECK(attn_tile(&g, F, F, nullptr) == BSTA_OK);
    CHECK(attn_tile_pool(&g, F, F, FF, nullptr) == BSTA_OK);
    CHECK(attn_pool(&g, F, FF, nullptr) == BSTA_OK);
    CHECK(attn_untile(&g, F, F, nullptr) == BSTA_OK);
    CHECK(stub_launches() == base + 4);
    base = stub_launches();
    CHECK(attn_tile(&g, nullptr, F, nullptr) == BSTA_ERR_NULL);
    CHECK(attn_tile_pool(&g, F, F, nullptr, nullptr) == BSTA_ERR_NULL);
    CHECK(attn_pool(&g, nullptr, FF, nullptr) == BSTA_ERR_NULL);
    CHECK(attn_untile(&g, F, nullptr, nullptr) == BSTA_ERR_NULL);
    CHECK(attn_block_sparse_fwd(&g, F, F, F, FI, FI, 16, s, 1, F, nullptr, nullptr) ==
          BSTA_ERR_UNSUPPORTED);
    CHECK(attn_block_sparse_fwd(&g, F, F, F, FI, FI, 16, 0.5f, 0, F, nullptr, nullptr) ==
          BSTA_ERR_UNSUPPORTED);
    CHECK(attn_block_sparse_fwd_raster(&g, F, nullptr, F, FI, FI, 16, s, 0, F, nullptr, nullptr) ==
          BSTA_ERR_NULL);
    CHECK(attn_block_sparse_fwd(&g, F, F, F, FI, FI, -1, s, 0, F, nullptr, nullptr) == BSTA_ERR_SHAPE);
    CHECK(attn_prune_queries(&g, F, 0.0, FU64, nullptr, FF, nullptr) == BSTA_ERR_SHAPE);
    CHECK(attn_prune_queries(&g, F, 1.5, FU64, nullptr, FF, nullptr) == BSTA_ERR_SHAPE);
    CHECK(attn_block_sparse_fwd_pruned(&g, F, F, F, FI, FI, 16, s, 0, nullptr, 1, F, nullptr,
                                       nullptr) == BSTA_ERR_NULL);
    CHECK(stub_launches() == base);
    CHECK(attn_block_sparse_fwd(&g, F, F, F, FI, FI, 16, s, 0, F, FF, nullptr) == BSTA_OK);
    CHECK(attn_block_sparse_fwd_raster(&g, F, F, F, FI, FI, 16, s, 0, F, nullptr, nullptr) == BSTA_OK);
    CHECK(attn_prune_queries(&g, F, 0.5, FU64, FI, FF, nullptr) == BSTA_OK);
    CHECK(attn_block_sparse_fwd_pruned(&g, F, F, F, FI, FI, 16, s, 0, FU64, 0, F, FF, nullptr) ==
          BSTA_OK);
    CHECK(stub_launches() == base + 4);
    bsta_geom g8 = geom(1, 2, 128, 5, 6, 19, 8);
    CHECK(attn_block_sparse_fwd_raster(&g8, F, F, F, FI, FI, 16, s, 0, F, nullptr, nullptr) == BSTA_OK);
    CHECK(attn_prune_queries(&g8, F, 0.5, FU64, FI, FF, nullptr) == BSTA_OK);
}

void bwd_checks() {
    bsta_geom g = geom(1, 2, 64, 8, 8, 8);
    const float s = 1.0f / 8.0f;
    const int64_t need = attn_bwd_workspace_bytes(&g, 16);
    CHECK(need > 0);
    CHECK(attn_bwd_workspace_bytes(&g, -1) == BSTA_ERR_SHAPE);
    const int base = stub_launches();
    CHECK(attn_block_sparse_bwd(&g, F, F, F, F, F, FF, FI, FI, 16, s, 0, F, F, F, F, need - 1, nullptr) ==
          BSTA_ERR_CAPACITY);
    CHECK(attn_block_sparse_bwd(&g, F, F, F, F, F, FF, FI, FI, 16, s, 0, F, F, F, nullptr, need,
                                nullptr) == BSTA_ERR_NULL);
    CHECK(attn_block_sparse_bwd(&g, F, F, F, F, F, FF, FI, FI, 16, s, 1, F, F, F, F, need, nullptr) ==
          BSTA_ERR_UNSUPPORTED);
    CHECK(attn_block_sparse_bwd_noalloc(&g, F, F, F, F, F, FF, FI, FI, int64_t(17) << 20, s, 0, F, F, F,
                                        nullptr) == BSTA_ERR_CAPACITY);
    CHECK(stub_launches() == base);
    CHECK(attn_block_sparse_bwd(&g, F, F, F, F, F, FF, FI, FI, 16, s, 0, F, F, F, F, need, nullptr) ==
          BSTA_OK);
    CHECK(attn_block_sparse_bwd_noalloc(&g, F, F, F, F, F, FF, FI, FI, 16, s, 0, F, F, F, nullptr) ==
          BSTA_OK);
    CHECK(stub_launches() == base + 2);
}

// The detail message is thread-local: concurrent failing calls each see
// their own.
void thread_checks() {
    std::vector<std::thread> ts;
    std::vector<int> ok(8, 0);
    for (int i = 0; i < 8; ++i)
        ts.emplace_back([i, &ok] {
            bsta_geom g = geom(1, 2, 64, 8, 8, 8);
            int good = 1;
            for (int r = 0; r < 200; ++r) {
                const int32_t st = (i & 1) ? attn_tile(&g, nullptr, F, nullptr)
                                           : attn_select_capacity(&g, BSTA_SELECT_TOPK, 100, nullptr);
                const char* e = attn_last_error();
                good &= (i & 1) ? (st == BSTA_ERR_NULL && strstr(e, "attn_tile") != nullptr)
                                : (st == BSTA_ERR_SHAPE && strstr(e, "attn_tile") == nullptr);
            }
            ok[i] = good;
        });
    for (auto& t : ts) t.join();
    for (int i = 0; i < 8; ++i) CHECK(ok[i] == 1);
    CHECK(attn_set_deterministic(1) == 0);
    CHECK(attn_set_deterministic(0) == 1);
}

// Packed sequences: layout, capacity, argument checks, and that an accepted
// selection reaches its launches (pool, scores, select).
void packed_checks() {
    bsta_segments sg = {};
    sg.count = 4;
    sg.patch[0] = sg.patch[1] = sg.patch[2] = 1;
    sg.kind[0] = 0; sg.rows[0] = 5;
    sg.kind[1] = 1; sg.shape[1][0] = 1; sg.shape[1][1] = 2; sg.shape[1][2] = 5;
    sg.kind[2] = 0; sg.rows[2] = 3;
    sg.kind[3] = 1; sg.shape[3][0] = 2; sg.shape[3][1] = 2; sg.shape[3][2] = 2;
    bsta_geom g = geom(1, 2, 64, 0, 0, 0);
    g.segments = &sg;
    int32_t nt = 0;
    int64_t lpad = 0;
    CHECK(attn_geometry(&g, &nt, &lpad, nullptr) == BSTA_OK);
    CHECK(nt == 5 && lpad == 320);
    std::vector<int32_t> occ(nt);
    CHECK(attn_geometry(&g, nullptr, nullptr, occ.data()) == BSTA_OK);
    CHECK(occ[0] == 5 && occ[1] == 3 && occ[2] == 8 && occ[3] == 2 && occ[4] == 8);
    int32_t npre = 0, nreg = 0, spans[4] = {};
    int64_t plen = 0;
    CHECK(attn_packed_info(&g, &npre, &nreg, spans, &plen) == BSTA_OK);
    CHECK(npre == 2 && nreg == 2 && plen == 26);
    CHECK(spans[0] == 2 && spans[1] == 4 && spans[2] == 4 && spans[3] == 5);
    // per head: 2 prefix rows of 5, 3 video rows of 2 + 1 + 1
    const int64_t cap = attn_packed_capacity(&g, 0.5, 0.5, 1);
    CHECK(cap == 2 * (2 * 5 + 3 * 4));
    CHECK(attn_packed_capacity(&g, 0.5, 0.5, 0) == BSTA_ERR_UNSUPPORTED);
    CHECK(attn_packed_capacity(&g, 0.5, NAN, 1) == BSTA_ERR_SHAPE);
    CHECK(attn_packed_capacity(&g, NAN, 0.5, 1) == BSTA_ERR_SHAPE);
    const int64_t ws = attn_workspace_bytes(&g, BSTA_SELECT_TOPK);
    const int before = stub_launches();
    CHECK(attn_select_packed(&g, F, F, 0, 0.5, 0.5, 1, FU8, FI, FI, cap - 1, F, ws, nullptr) ==
          BSTA_ERR_CAPACITY);
    CHECK(attn_select_packed(&g, F, F, 0, 0.5, 0.5, 1, FU8, FI, FI, cap, F, ws - 1, nullptr) ==
          BSTA_ERR_CAPACITY);
    CHECK(attn_select_packed(&g, nullptr, F, 0, 0.5, 0.5, 1, FU8, FI, FI, cap, F, ws, nullptr) ==
          BSTA_ERR_NULL);
    CHECK(stub_launches() == before);
    CHECK(attn_select_packed(&g, F, F, 0, 0.5, 0.5, 1, FU8, FI, FI, cap, F, ws, nullptr) == BSTA_OK);
    CHECK(stub_launches() == before + 3);
    CHECK(attn_select_packed(&g, nullptr, nullptr, BSTA_SELECT_PREPOOLED, 0.5, 0.5, 1, FU8, FI, FI,
                             cap, F, ws, nullptr) == BSTA_OK);
    CHECK(stub_launches() == before + 5);
    // the most segments, each its own region, and one past it
    bsta_segments big = {};
    big.patch[0] = big.patch[1] = big.patch[2] = 2;
    big.count = BSTA_MAX_SEGMENTS;
    for (int i = 0; i < BSTA_MAX_SEGMENTS; ++i) {
        big.kind[i] = 1;
        big.shape[i][0] = big.shape[i][1] = big.shape[i][2] = 8;
    }
    g.segments = &big;
    CHECK(attn_geometry(&g, &nt, nullptr, nullptr) == BSTA_OK);
    CHECK(nt == BSTA_MAX_SEGMENTS);
    CHECK(attn_packed_capacity(&g, 0.5, 0.5, 1) == 2 * 16 * 16);
    big.count = BSTA_MAX_SEGMENTS + 1;
    CHECK(attn_geometry(&g, nullptr, nullptr, nullptr) == BSTA_ERR_SHAPE);
    big.count = 1;
    big.shape[0][1] = 7;  // not a multiple of the patch
    CHECK(attn_geometry(&g, nullptr, nullptr, nullptr) == BSTA_ERR_SHAPE);
    // single grid: no packed info
    bsta_geom single = geom(1, 2, 64, 8, 8, 8);
    CHECK(attn_packed_info(&single, nullptr, nullptr, nullptr, nullptr) == BSTA_ERR_UNSUPPORTED);
}

}  // namespace

int main() {
    geometry_checks();
    select_checks();
    path_checks();
    bwd_checks();
    thread_checks();
    packed_checks();
    if (g_failed) return 1;
    printf("OK %d checks, %d stub launches\n", g_checks, stub_launches());
    return 0;
}
