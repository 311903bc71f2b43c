/*
 * bsta.h -- block-sparse tiled video attention on MI355X (gfx950).
 *
 * C ABI of libbsta.so.  The path, in call order:
 *
 *   attn_tile            raster [B,L,H,D] -> zero-padded tile order [B,Lpad,H,D]
 *   attn_select_blocks   per-tile mean pooling of Q and K, pooled scores, top-k
 *                        key tiles per query tile (or a sliding tile window),
 *                        block mask and CSR index map
 *                        (attn_select_cumulative: the same with a cumulative
 *                        probability threshold instead of a fixed k)
 *   attn_block_sparse_fwd  softmax(q k^T / sqrt(D)) v over the selected tiles
 *   attn_untile          tile order -> raster order
 *
 * On the top-k path attn_tile_pool may replace attn_tile for Q and K: it
 * also writes the pooled vectors, and attn_select_blocks then runs with
 * BSTA_SELECT_PREPOOLED and skips its own pooling pass.  Likewise
 * attn_block_sparse_fwd_raster writes the output in raster order and
 * replaces attn_block_sparse_fwd followed by attn_untile.
 * attn_block_sparse_bwd gives the gradients of the forward for training.
 *
 * Conventions shared by every call:
 *   - Tensors are bfloat16, contiguous, in the layout [B, L, H, D] that the
 *     FastVideo attention backends use ("bsa_attn" page, forward: query, key
 *     and value are [B, L, num_heads, D]).  Q, K and V share H: grouped-query
 *     attention is not expressible.
 *   - The latent grid is (T, Y, X) with L = T*Y*X tokens in raster order
 *     (token l = (t*Y + y)*X + x).  Tiles are 4x4x4 = 64 tokens; there are
 *     Nt = ceil(T/4)*ceil(Y/4)*ceil(X/4) tiles and Lpad = 64*Nt slots.
 *   - Every tensor, mask and index pointer is a DEVICE pointer unless its
 *     comment says host.  The caller allocates and owns all memory and the
 *     stream.  The library allocates nothing, frees nothing, never
 *     synchronises, and enqueues every kernel on the given stream (a
 *     hipStream_t passed as void*; NULL = the null stream).  Its device
 *     state is a small static array of counters that attn_block_sparse_fwd
 *     uses to order its walk over each row's key tiles (see there; it
 *     never decides which keys are attended), and the static scratch of
 *     attn_block_sparse_bwd_noalloc, used by that call alone.
 *   - Every call checks its arguments on the host before any HIP call and
 *     returns a status (0 = BSTA_OK).  On failure nothing is enqueued and
 *     attn_last_error() returns a thread-local message with the detail.
 *     A failed launch returns BSTA_ERR_HIP.
 */
#ifndef BSTA_H
#define BSTA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest number of segments of a packed sequence. */
#define BSTA_MAX_SEGMENTS 16

/*
 * A packed sequence ("video_sparse_attn_h3" page, build()): dense segments
 * and video regions packed in one sequence, in this order.  kind[s] = 0: a
 * dense segment of rows[s] rows (0 rows: the segment is dropped); kind[s] =
 * 1: a video region whose latent shape shape[s] = (t, h, w) must be a
 * positive multiple of patch and becomes a token grid of shape / patch.  At
 * least one region is required.  Tiles (64 tokens): each dense segment is
 * cut into tiles of 64 consecutive rows, the last one partial, and these
 * tiles come first in tile order (the prefix, in packed order); then each
 * region is cut into 4x4x4 tiles as a single grid, region by region in
 * packed order, each region's tiles forming its span.  (The page gives the
 * arguments and checks of build(), not the layout; this is the reading.)
 */
typedef struct bsta_segments {
    int32_t count;                        /* 1 .. BSTA_MAX_SEGMENTS       */
    int32_t patch[3];                     /* patch size (t, h, w), >= 1   */
    int32_t kind[BSTA_MAX_SEGMENTS];      /* 0 dense, 1 video region      */
    int32_t rows[BSTA_MAX_SEGMENTS];      /* dense rows (kind 0)          */
    int32_t shape[BSTA_MAX_SEGMENTS][3];  /* latent t, h, w (kind 1)      */
} bsta_segments;

/* Problem geometry.  D must be 64 or 128; tile_t = tile_y = 4 and tile_x =
 * 4 (64-token tiles) or 8 (128-token tiles).  segments = NULL: one latent
 * grid T x Y x X.  segments != NULL (host memory, read during the call):
 * a packed sequence, 64-token tiles only; T, Y and X are then ignored and
 * L is the packed length (attn_packed_info). */
typedef struct bsta_geom {
    int32_t B, H, D;            /* batch, heads, head dim                  */
    int32_t T, Y, X;            /* latent token grid                       */
    int32_t tile_t, tile_y, tile_x;
    const bsta_segments* segments;
} bsta_geom;

enum {
    BSTA_OK = 0,
    BSTA_ERR_NULL = -1,         /* a required pointer is NULL               */
    BSTA_ERR_SHAPE = -2,        /* sizes, k or a window outside the spec    */
    BSTA_ERR_UNSUPPORTED = -3,  /* causal, a non-default scale, D, tile     */
    BSTA_ERR_CAPACITY = -4,     /* an output or workspace is too small      */
    BSTA_ERR_HIP = -5           /* a HIP launch failed                      */
};

enum { BSTA_SELECT_TOPK = 0, BSTA_SELECT_STA = 1, BSTA_SELECT_CUMULATIVE = 2 };
/* Flag for BSTA_SELECT_TOPK and BSTA_SELECT_CUMULATIVE: the workspace
 * already holds pooled Q and K (written by attn_tile_pool); see
 * attn_select_blocks and attn_select_cumulative. */
enum { BSTA_SELECT_PREPOOLED = 0x100 };

/* Largest head count a sliding-tile-window call accepts (windows travel as
 * kernel arguments). */
#define BSTA_MAX_STA_HEADS 256

/*
 * attn_geometry (host only, no HIP call).
 * Tile counts and valid tokens per tile, as the "video_sparse_attn" page's
 * construct_variable_block_sizes defines them: per axis ceil(dim/4) tiles,
 * the last one keeping the remainder; the count of a tile is the product of
 * its three extents; tiles are numbered j = (a*nY + b)*nX + c.
 *   num_tiles  [out, host, may be NULL]  Nt
 *   padded_len [out, host, may be NULL]  Lpad = 64*Nt (128*Nt for 4x4x8 tiles)
 *   occupancy  [out, host int32 [Nt], may be NULL]  valid tokens of tile j
 * With 4x4x8 tiles the x axis is cut into ceil(X/8) tiles of 8; for a
 * packed sequence the tiles are those of its layout (see bsta_segments),
 * dense segments' tiles first.
 */
int32_t attn_geometry(const bsta_geom* g, int32_t* num_tiles, int64_t* padded_len,
                      int32_t* occupancy);

/*
 * attn_tile: raster -> tile order ("bsa_attn" page, preprocess_qkv and
 * get_tile_partition_indices; "video_sparse_attn_h3" page, tile()).
 *   x        [in]  bf16 [B, L, H, D]
 *   x_tiled  [out] bf16 [B, Lpad, H, D]
 * Token (t,y,x) in tile j = (a,b,c) = (t/4, y/4, x/4) goes to slot
 * 64*j + (dt*s_y + dy)*s_x + dx, where (dt,dy,dx) = (t,y,x) mod 4 and s_y,
 * s_x are the tile's extents: the valid tokens of a tile come first, in the
 * row-major order of its clipped sub-block.  Every pad slot is written with
 * +0.0, so x_tiled needs no clearing and a reused buffer keeps no stale rows.
 * x and x_tiled must not overlap.
 */
int32_t attn_tile(const bsta_geom* g, const void* x, void* x_tiled, void* stream);

/*
 * attn_tile_pool: attn_tile and, in the same pass over x, the per-tile mean
 * pooling of the top-k coarse stage ("sla" page, get_block_map and
 * mean_pool): pooled[b,h,j] is the fp32 mean of the n_j valid rows of tile
 * j, summed in slot order, bit for bit the value attn_select_blocks computes
 * from x_tiled.  Reading x once instead of reading x_tiled again saves one
 * pass over Q and K on the top-k path.
 *   x        [in]  bf16 [B, L, H, D]
 *   x_tiled  [out] bf16 [B, Lpad, H, D], as from attn_tile
 *   pooled   [out] fp32 [B, H, Nt, D]; for attn_select_blocks with
 *            BSTA_SELECT_PREPOOLED, the first (Q) or second (K) slab of its
 *            workspace
 * x, x_tiled and pooled must not overlap.
 */
int32_t attn_tile_pool(const bsta_geom* g, const void* x, void* x_tiled, float* pooled,
                       void* stream);

/*
 * attn_pool: the per-tile mean of the valid rows of one tiled tensor
 * ("sla" section of the backends page, mean_pool inside get_block_map; the
 * pooling step attn_select_blocks runs on Q and K before scoring).
 *   x_tiled [in]  bf16 [B, Lpad, H, D]
 *   pooled  [out] fp32 [B, H, Nt, D]: the sum of tile j's n_j valid rows
 *           divided by n_j, summed in fp32 in the order the fused
 *           attn_tile_pool uses (runs of 8 slots summed from +0.0 in slot
 *           order, run sums added in order), so the two give the same
 *           vectors bit for bit.
 * Errors: ERR_NULL, ERR_UNSUPPORTED (geometry), ERR_HIP.
 */
int32_t attn_pool(const bsta_geom* g, const void* x_tiled, float* pooled, void* stream);

/*
 * attn_untile: tile -> raster order ("bsa_attn" page, postprocess_output and
 * get_reverse_tile_partition_indices).  Pad slots are dropped.
 *   y_tiled  [in]  bf16 [B, Lpad, H, D]
 *   y        [out] bf16 [B, L, H, D]
 */
int32_t attn_untile(const bsta_geom* g, const void* y_tiled, void* y, void* stream);

/*
 * attn_select_capacity (host only): number of CSR entries a selection
 * produces, B*H*Nt*k for top-k and Nt*B*sum_h prod(window_h) for windows;
 * for BSTA_SELECT_CUMULATIVE, whose row lengths depend on the data, the
 * bound B*H*Nt*Nt; a negative status on bad arguments.
 */
int64_t attn_select_capacity(const bsta_geom* g, int32_t mode, int32_t topk,
                             const int32_t* sta_windows_host);

/*
 * attn_workspace_bytes (host only): bytes of device workspace
 * attn_select_blocks needs in the given mode (0 for windows; for top-k and
 * for the cumulative threshold the pooled Q and K, fp32 [2, B, H, Nt, D],
 * then the pooled scores fp32 [B, H, Nt, Nt]); a negative status on bad
 * arguments.
 */
int64_t attn_workspace_bytes(const bsta_geom* g, int32_t mode);

/*
 * attn_select_blocks: the coarse stage.
 * Top-k mode ("sla" page, get_block_map and mean_pool): Pq[b,h,j] and
 * Pk[b,h,j] are the means of the n_j valid rows of tile j (fp32); the score
 * of query tile i against key tile j is Pq[i].Pk[j] (no scale); each query
 * tile keeps the k best key tiles, ties going to the lower index.
 * Window mode ("STA_configuration" page: a window is a count of tiles along
 * t, h and w): query tile (a,b,c) of head h keeps the key tiles whose
 * coordinate on each axis lies in [s, s+w) with s = clamp(a - w/2, 0, n - w)
 * (integer division), so every row holds prod(window) tiles.
 * Then map_to_index ("video_sparse_attn_h3" page): row r = (b*H + h)*Nt + i
 * of the CSR lists the kept key tiles of query tile i in ascending order.
 *   q_tiled, k_tiled  [in]  bf16 [B, Lpad, H, D] from attn_tile (pad rows 0);
 *                           unused (may be NULL) in window mode
 *   mode              BSTA_SELECT_TOPK or BSTA_SELECT_STA; BSTA_SELECT_TOPK |
 *                     BSTA_SELECT_PREPOOLED skips the pooling: the
 *                     workspace already holds pooled Q then pooled K (from
 *                     attn_tile_pool), and q_tiled, k_tiled are unused (may
 *                     be NULL)
 *   topk              1 <= k <= Nt (top-k mode)
 *   sta_windows_host  [in, host int32 [H][3]] windows (window mode),
 *                     1 <= w <= tiles on that axis; H <= BSTA_MAX_STA_HEADS
 *   block_mask        [out, uint8 [B, H, Nt, Nt], may be NULL] 1 = kept
 *   row_ptr           [out, int32 [B*H*Nt + 1]]
 *   col_idx           [out, int32 [col_capacity]]
 *   col_capacity      entries col_idx can hold (>= attn_select_capacity)
 *   workspace         [scratch, >= attn_workspace_bytes; NULL allowed in
 *                     window mode]; after a top-k call it holds the pooled
 *                     Q, K and scores described above
 * Returns BSTA_ERR_CAPACITY when col_capacity or workspace_bytes is short.
 */
int32_t attn_select_blocks(const bsta_geom* g, const void* q_tiled, const void* k_tiled,
                           int32_t mode, int32_t topk, const int32_t* sta_windows_host,
                           uint8_t* block_mask, int32_t* row_ptr, int32_t* col_idx,
                           int64_t col_capacity, void* workspace, int64_t workspace_bytes,
                           void* stream);

/*
 * attn_select_cumulative: the coarse stage with a cumulative probability
 * threshold.  The "bsa_attn" page's forward selects key-value blocks from a
 * cumulative threshold and a minimum block count without showing the rule;
 * the reading implemented here: pooling and pooled scores S as in top-k
 * mode, then per query tile p_j = softmax_j(S_ij / sqrt(D)) over the key
 * tiles; with the tiles in descending score order (ties to the lower
 * index), the row keeps the shortest prefix whose mass reaches
 * threshold * sum_j p_j, and at least min(min_blocks, Nt) tiles.  The CSR
 * row lengths therefore vary; row_ptr is their running sum.
 *   q_tiled, k_tiled  [in]  bf16 [B, Lpad, H, D] from attn_tile; unused (may
 *                           be NULL) with BSTA_SELECT_PREPOOLED
 *   flags             0 or BSTA_SELECT_PREPOOLED (the workspace already
 *                     holds pooled Q then pooled K, from attn_tile_pool)
 *   threshold         in (0, 1]
 *   min_blocks        >= 0 (values above Nt keep every tile)
 *   block_mask        [out, uint8 [B, H, Nt, Nt], may be NULL] 1 = kept
 *   row_ptr           [out, int32 [B*H*Nt + 1]]; row_ptr[B*H*Nt] is the
 *                     number of entries written
 *   col_idx           [out, int32 [col_capacity]], ascending per row
 *   col_capacity      >= B*H*Nt*Nt (attn_select_capacity with
 *                     BSTA_SELECT_CUMULATIVE), since any row may keep
 *                     every tile
 *   workspace         [scratch, >= attn_workspace_bytes(g,
 *                     BSTA_SELECT_CUMULATIVE)]; afterwards it holds the
 *                     pooled Q and K; the score rows are overwritten (each
 *                     row's kept ids are staged there)
 * Requires Nt <= 2048 (a row of scores lives in one wave's registers);
 * larger grids return BSTA_ERR_SHAPE.  Probabilities and their sums are
 * fp32, so a row whose prefix mass lies within rounding of the threshold
 * may keep one tile more or less than an exact computation would.
 */
int32_t attn_select_cumulative(const bsta_geom* g, const void* q_tiled, const void* k_tiled,
                               int32_t flags, float threshold, int32_t min_blocks,
                               uint8_t* block_mask, int32_t* row_ptr, int32_t* col_idx,
                               int64_t col_capacity, void* workspace, int64_t workspace_bytes,
                               void* stream);

/*
 * attn_packed_info (host only, no HIP call): the layout of a packed
 * sequence (g->segments != NULL; see bsta_segments).
 *   num_prefix  [out, host, may be NULL]  tiles of the dense segments
 *   num_regions [out, host, may be NULL]  video regions R
 *   spans       [out, host int32 [2*R], may be NULL]  tile range
 *               [spans[2r], spans[2r+1]) of region r, in packed order
 *   packed_len  [out, host, may be NULL]  L, tokens of the packed sequence
 * BSTA_ERR_UNSUPPORTED for a single-grid geometry.
 */
int32_t attn_packed_info(const bsta_geom* g, int32_t* num_prefix, int32_t* num_regions,
                         int32_t* spans, int64_t* packed_len);

/*
 * attn_packed_capacity (host only): CSR entries attn_select_packed writes
 * for these arguments, or a negative status.
 */
int64_t attn_packed_capacity(const bsta_geom* g, double sparsity, double ref_keep_rate,
                             int32_t exempt);

/*
 * attn_select_packed: the coarse stage of a packed sequence
 * ("video_sparse_attn_h3" page, build() and its sparsity, ref_keep_rate and
 * compete/exempt arguments; the page shows the call, not the rule; the
 * reading implemented here).  Pooling and pooled scores S as in top-k mode,
 * over the packed tiles (a tile's mean is over its valid rows).  With
 * P prefix tiles and the video spans [a_r, b_r) of n_r tiles:
 *   exempt != 0 (the default on the page): a prefix query tile keeps every
 *     tile; a video query tile keeps every prefix tile and, in each span r,
 *     the k_r tiles of highest S (ties to the lower index), with
 *     k_r = min(n_r, max(1, floor(keep_r * n_r))), keep_r = ref_keep_rate
 *     for a reference region (every region but the last) and
 *     1 - sparsity for the last (generated) region; sparsity <= 0 keeps
 *     every tile.  Prefix rows hold Nt entries, video rows P + sum_r k_r.
 *   exempt == 0 (compete): one region only; every query tile keeps the
 *     min(Nt, max(1, floor((1 - sparsity) * Nt))) tiles of highest S over
 *     the whole sequence (every tile if sparsity <= 0).
 *   q_tiled, k_tiled  [in]  bf16 [B, Lpad, H, D] from attn_tile; unused (may
 *                           be NULL) with BSTA_SELECT_PREPOOLED
 *   flags             0 or BSTA_SELECT_PREPOOLED
 *   sparsity          finite, <= 1
 *   ref_keep_rate     in [0, 1] when there is more than one region (the
 *                     page requires it then); otherwise unused
 *   block_mask        [out, uint8 [B, H, Nt, Nt], may be NULL] 1 = kept
 *   row_ptr           [out, int32 [B*H*Nt + 1]]
 *   col_idx           [out, int32 [col_capacity]], ascending per row
 *   col_capacity      >= attn_packed_capacity(g, sparsity, ref_keep_rate,
 *                     exempt)
 *   workspace         [scratch, >= attn_workspace_bytes(g,
 *                     BSTA_SELECT_TOPK)]; afterwards it holds the pooled
 *                     Q and K and the scores
 * Needs a packed geometry with Nt <= 2048 in exempt mode (a score row lives
 * in one wave's registers); BSTA_ERR_SHAPE otherwise.  keep_r * n_r is
 * evaluated in double precision.
 */
int32_t attn_select_packed(const bsta_geom* g, const void* q_tiled, const void* k_tiled,
                           int32_t flags, double sparsity, double ref_keep_rate, int32_t exempt,
                           uint8_t* block_mask, int32_t* row_ptr, int32_t* col_idx,
                           int64_t col_capacity, void* workspace, int64_t workspace_bytes,
                           void* stream);

/*
 * attn_block_sparse_fwd: fused block-sparse flash attention forward
 * ("bsa_attn" page, forward and _compute_sparse_attention; __init__ fixes
 * the scale to 1/sqrt(d) and rejects causal attention).
 * For every query tile i of head h in batch b and every valid row r < n_i:
 *   o = softmax(q k^T * softmax_scale) v
 * over the valid tokens of the key tiles listed in CSR row (b*H + h)*Nt + i.
 * Rows r >= n_i (padding) are written as +0.0 with lse = -inf; a row whose
 * CSR list is empty is written the same way.
 *   q_tiled, k_tiled, v_tiled [in]  bf16 [B, Lpad, H, D], pad rows 0
 *   row_ptr  [in] int32 [B*H*Nt + 1], non-decreasing
 *   col_idx  [in] int32 [col_len]; entries must lie in [0, Nt).  The kernel
 *            clamps row ranges to [0, col_len) and skips out-of-range tile
 *            ids, so bad indices cannot read outside the tensors.
 *   softmax_scale  must equal 1/sqrt(D) within rel 1e-4 / abs 1e-5
 *   causal   must be 0
 *   o_tiled  [out] bf16 [B, Lpad, H, D]
 *   lse      [out, fp32 [B, H, Lpad], may be NULL] natural-log softmax
 *            normaliser of the scaled scores
 * Key order.  The softmax is a sum over the row's key tiles, so their order
 * changes only rounding.  By default, when a head's K and V exceed 8 MiB
 * and rows spread over most of the head (top-k and threshold selections),
 * each row is walked cyclically from a start that depends on how far the
 * GPU has progressed through the call (a device-side counter), so that
 * workgroups running at the same time read neighbouring key tiles and share
 * them in cache; results then agree with any other order to rounding but
 * are not bitwise reproducible from call to call.  Smaller heads and rows
 * that keep to part of the key range (sliding windows) are walked in CSR
 * order.  attn_set_deterministic(1) walks every row in CSR order,
 * attn_set_deterministic(2) every row rotated.
 */
int32_t attn_block_sparse_fwd(const bsta_geom* g, const void* q_tiled, const void* k_tiled,
                              const void* v_tiled, const int32_t* row_ptr, const int32_t* col_idx,
                              int64_t col_len, float softmax_scale, int32_t causal,
                              void* o_tiled, float* lse, void* stream);

/*
 * attn_block_sparse_fwd_raster: attn_block_sparse_fwd followed by
 * attn_untile in one pass ("bsa_attn" page, forward then
 * postprocess_output): the output row of each valid query slot is written
 * straight to the token it holds in raster order, and pad slots write
 * nothing, which saves a read and a write of the output.  Arguments and key
 * order as attn_block_sparse_fwd, except
 *   o    [out] bf16 [B, L, H, D], raster order (every row written once)
 *   lse  [out, fp32 [B, H, Lpad], may be NULL] in slot order, as above
 */
int32_t attn_block_sparse_fwd_raster(const bsta_geom* g, const void* q_tiled,
                                     const void* k_tiled, const void* v_tiled,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     int64_t col_len, float softmax_scale, int32_t causal, void* o,
                                     float* lse, void* stream);

/*
 * attn_prune_queries: the query half of bidirectional sparse attention
 * ("bsa_attn" page: the introduction prunes redundant query tokens in each
 * block; forward prunes the query blocks at a keep ratio, selects key-value
 * blocks from the kept queries and attends with them only).  The page shows
 * the calls, not the rule; the rule here: a tile with n valid tokens keeps
 * c = min(n, max(1, floor(keep_ratio * n))) of them, those with the lowest
 * cos(q_r, m), m the mean of the tile's valid queries of that head (0 when
 * either vector is zero), ties to the lower slot.
 *   q_tiled    [in]  bf16 [B, Lpad, H, D] tiled queries
 *   keep_ratio [in]  in (0, 1] (host double; floor(keep_ratio * n) is taken
 *              in double precision)
 *   keep_mask  [out] uint64 [B, H, Nt * U], U = 1 for 64-token tiles and 2
 *              for 128-token tiles: word u of a tile covers its slots 64u +
 *              [0, 64), bit r set iff slot 64u + r is kept (pad slots never
 *              are)
 *   keep_count [out] int32 [B, H, Nt] kept tokens per tile, or NULL
 *   pooled_q   [out] fp32 [B, H, Nt, D]: the mean of each tile's kept
 *              queries (fp32 sum in slot order, one division).  Pass the
 *              pooled-Q part of a selection workspace (the first
 *              B*H*Nt*D floats) and pool K with attn_tile_pool into the
 *              second part; attn_select_blocks (BSTA_SELECT_TOPK |
 *              BSTA_SELECT_PREPOOLED) or attn_select_cumulative (prepooled)
 *              then select key tiles from the kept queries.
 * Errors: ERR_NULL (q_tiled, keep_mask or pooled_q NULL), ERR_SHAPE (ratio
 * outside (0, 1]), ERR_UNSUPPORTED (a packed sequence), ERR_HIP.  One wave
 * per (batch, head, tile); computed in fp32.
 */
int32_t attn_prune_queries(const bsta_geom* g, const void* q_tiled, double keep_ratio,
                           uint64_t* keep_mask, int32_t* keep_count, float* pooled_q,
                           void* stream);

/*
 * attn_block_sparse_fwd_pruned: attn_block_sparse_fwd (raster = 0) or
 * attn_block_sparse_fwd_raster (raster != 0) for pruned queries: only slots
 * in keep_mask (from attn_prune_queries) are output rows; every other slot
 * is written as +0.0 with lse = -inf, as the "bsa_attn" page's forward
 * restores full length from the kept positions (reading: pruned positions
 * hold zero).  Arguments otherwise as attn_block_sparse_fwd; keep_mask is
 * uint64 [B, H, Nt * U] (the layout attn_prune_queries writes) on the
 * device (ERR_NULL if NULL).  Pruned rows are masked, not skipped: the call
 * costs what the unpruned one does.  ERR_UNSUPPORTED for packed sequences.
 */
int32_t attn_block_sparse_fwd_pruned(const bsta_geom* g, const void* q_tiled,
                                     const void* k_tiled, const void* v_tiled,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     int64_t col_len, float softmax_scale, int32_t causal,
                                     const uint64_t* keep_mask, int32_t raster, void* o,
                                     float* lse, void* stream);

/*
 * attn_bwd_workspace_bytes (host only): bytes of device workspace
 * attn_block_sparse_bwd needs for a CSR of col_len entries (per query slot
 * rowsum(dO*O) and the lse scaled to base 2, and the CSR's transpose); a
 * negative status on bad arguments.
 */
int64_t attn_bwd_workspace_bytes(const bsta_geom* g, int64_t col_len);

/*
 * attn_block_sparse_bwd: gradients of the block-sparse attention of
 * attn_block_sparse_fwd for training (the "bsa_attn" page's method targets
 * training; the "video_sparse_attn_h3" page keeps a gradient route through
 * its tiling).  For the loss sum(dO * O) over the tiled output O:
 *   dS = P * (dO V^T - rowsum(dO * O)),  dQ = dS K * softmax_scale,
 *   dK = dS^T Q * softmax_scale,  dV = P^T dO,
 * with P the softmax probabilities of each query row over the valid keys of
 * its CSR row's tiles, recomputed from the forward's lse.
 *   q_tiled, k_tiled, v_tiled [in] bf16 [B, Lpad, H, D], as given to the
 *            forward
 *   o_tiled  [in] bf16 [B, Lpad, H, D], the forward's tiled output
 *   do_tiled [in] bf16 [B, Lpad, H, D], gradient of the loss w.r.t. O; pad
 *            rows must be finite (attn_tile writes them as zero) and do not
 *            change the result
 *   lse      [in] fp32 [B, H, Lpad], the forward's lse
 *   row_ptr, col_idx, col_len  the forward's CSR.  Ranges are clamped and
 *            out-of-range ids skipped as in the forward; an id repeated in
 *            a row counts once per occurrence, as in the forward (every
 *            selection here lists distinct ids).
 *   softmax_scale, causal  as the forward (1/sqrt(D), 0)
 *   dq_tiled, dk_tiled, dv_tiled [out] bf16 [B, Lpad, H, D]; pad rows and
 *            key tiles that no row selects are written as +0.0
 *   workspace [scratch, >= attn_bwd_workspace_bytes(g, col_len)]
 * Requires Nt <= 4096 (BSTA_ERR_SHAPE otherwise).  Tiles of 64 or 128
 * tokens, a single grid or a packed sequence; a 128-token tile is walked as
 * its two 64-slot units (valid tokens first), in unit order.  Gradients
 * accumulate in fp32, key tiles in CSR row order for dQ and query tiles in
 * ascending order for dK and dV, so equal inputs give bitwise equal
 * gradients; P and dS are rounded to bf16 for the second products.
 */
int32_t attn_block_sparse_bwd(const bsta_geom* g, const void* q_tiled, const void* k_tiled,
                              const void* v_tiled, const void* o_tiled, const void* do_tiled,
                              const float* lse, const int32_t* row_ptr, const int32_t* col_idx,
                              int64_t col_len, float softmax_scale, int32_t causal,
                              void* dq_tiled, void* dk_tiled, void* dv_tiled, void* workspace,
                              int64_t workspace_bytes, void* stream);

/*
 * attn_block_sparse_bwd_noalloc: attn_block_sparse_bwd without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving or training loops, harnesses that forbid
 * hipMalloc).  It validates its arguments exactly as attn_block_sparse_bwd,
 * runs the same kernels in the same order (so its gradients equal that
 * call's bit for bit), and calls no hipMalloc, hipFree or other allocating
 * routine.  Its workspace is a static device array of the library, 64 MiB
 * (67108864 bytes) per GPU, held on every GPU the library runs on until
 * the process ends; its address is looked up once per device on the first
 * call made with that device current.
 *   Arguments: as attn_block_sparse_bwd, without workspace and
 *            workspace_bytes.
 *   Errors: as attn_block_sparse_bwd; BSTA_ERR_CAPACITY (nothing enqueued)
 *            when attn_bwd_workspace_bytes(g, col_len) exceeds 64 MiB;
 *            BSTA_ERR_HIP when the scratch address cannot be obtained.
 * Every call on a GPU uses that GPU's one array, which keeps the last
 * call's contents (each call writes every word its kernels read, so
 * nothing needs clearing).  Calls that overlap on one GPU race: serialise
 * them, for instance on one stream.
 */
int32_t attn_block_sparse_bwd_noalloc(const bsta_geom* g, const void* q_tiled,
                                      const void* k_tiled, const void* v_tiled,
                                      const void* o_tiled, const void* do_tiled, const float* lse,
                                      const int32_t* row_ptr, const int32_t* col_idx,
                                      int64_t col_len, float softmax_scale, int32_t causal,
                                      void* dq_tiled, void* dk_tiled, void* dv_tiled,
                                      void* stream);

/*
 * attn_set_deterministic (host only, no HIP call): process-wide key order of
 * attn_block_sparse_fwd for calls made after it returns.  0 (the default):
 * the rotated walk where it pays, CSR order elsewhere (see the key order
 * above); 1 (or any value other than 0 and 2): every row in CSR order, so
 * equal inputs give bitwise equal outputs; 2: every row rotated.  Returns
 * the previous setting (0, 1 or 2).  Thread-safe; calls already enqueued
 * keep the mode they were made with.
 */
int32_t attn_set_deterministic(int32_t enable);

/* Text of a status code (static storage). */
const char* attn_status_string(int32_t status);

/* Detail of the last failure on the calling thread ("" when none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSTA_H */
