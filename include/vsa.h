/*
 * vsa.h -- C ABI of libvsa: gated, tile-sparse video attention for one
 * video-DiT layer on AMD Instinct MI355X (gfx950).
 *
 * The method (web pages cited by title and section):
 *   [SnackOnAI] "ComfyUI-Ref2VA-VSA proves a sparse attention gate can be
 *               transplanted ..." -- "The Architecture, Unpacked", "The Code,
 *               Annotated" (snippets one and two), "It In Action".
 *   [News]      "Ref2VA VSA: Sparse Attention Node for H3 Reference-to-Video"
 *               -- "The two-tier attention patch".
 *   [Veda]      "Veda Sparse Attention" news item -- "ComfyUI node" inputs.
 *
 * Video tokens are regrouped into 3D spatio-temporal tiles behind a prefix of
 * segment-pure text / reference tiles. A coarse pass mean-pools Q, K and V per
 * tile, scores video tiles against each other and keeps, per head and video
 * query tile, the top-k video key tiles; prefix key tiles are always kept and
 * prefix query tiles attend densely. A fine pass runs block-sparse softmax
 * attention over the kept tiles, and the output is
 *     out = O_fine + g (elementwise) O_coarse[tile of the token],
 * where g = x . W_gate^T is a bias-free linear gate projection of the layer
 * input and O_coarse is tile-level attention over the pooled Q, K, V.
 *
 * Conventions for every function:
 *  - Returns VSA_OK (0) or a negative status; vsa_last_error() then holds a
 *    thread-local message. All arguments are checked before any GPU work is
 *    enqueued, so a failed call enqueues nothing. There is no fallback path.
 *  - "host" pointers are CPU memory; "device" pointers are HIP device memory
 *    on the current device. The caller owns every buffer and the stream; the
 *    library allocates no device memory and keeps no pointer after returning.
 *  - GPU functions only enqueue work on `stream` (a hipStream_t; NULL = the
 *    null stream). Results are valid once the stream has completed.
 *  - Tensors are bf16 (raw 16-bit patterns) unless stated. Natural token
 *    order = prefix segments in order, then the video flattened t-major, then
 *    h, then w. [S][H][D] means token-major, then head, then head_dim.
 *  - Supported on device: head_dim in {64, 128}; tile rows B in {64, 128}.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status -- */
#define VSA_OK 0
#define VSA_ERR_ARG (-1)          /* null pointer, bad size, k out of range, NaN, ...  */
#define VSA_ERR_UNSUPPORTED (-2)  /* head_dim / tile rows / device not supported        */
#define VSA_ERR_PLAN (-3)         /* plan arrays inconsistent or untile map not injective */
#define VSA_ERR_DEVICE (-4)       /* a HIP runtime or launch error                      */

/* Short description of a status code (static string). */
const char *vsa_status_string(int status);
/* Detail of the last failing call on this thread ("" if none). */
const char *vsa_last_error(void);

/* ------------------------------------------------------------- plan -- */
typedef struct vsa_plan_info {
    int32_t grid[3];         /* video latent grid (T, H, W)                       */
    int32_t tile[3];         /* tile shape (t, h, w)                              */
    int32_t tile_rows;       /* B = tile[0] * tile[1] * tile[2]                   */
    int32_t n_prefix_tiles;  /* P: tiles [0, P) hold the prefix segments          */
    int32_t n_video_tiles;   /* n_v: tiles [P, n_t) hold the video                */
    int32_t n_tiles;         /* n_t = P + n_v                                     */
    int64_t rows_real;       /* S: number of tokens                               */
    int64_t rows_padded;     /* S_pad = n_t * B                                   */
    int64_t prefix_rows;     /* tokens in the prefix segments                     */
} vsa_plan_info;

/*
 * vsa_plan_tiles -- the tile plan ("geometry"), computed on the host.
 * [SnackOnAI] "The Code, Annotated", snippet one; "The Architecture,
 * Unpacked" (segment-pure prefix tiles); [News] "The two-tier attention
 * patch", item 1.
 *
 * Each prefix segment (text, reference image, reference audio, ...) starts
 * a new tile and fills tiles of B rows; its last tile may be short. The video
 * (grid T x H x W, flattened t-major) is cut into tiles of tile_t x tile_h x
 * tile_w, enumerated t-major then h then w, with partial tiles at the grid
 * edges. Inside a tile, real tokens take rows 0.. in (dt, dy, dx) order and
 * padding rows come last.
 *
 * prefix_seg_lens: host [n_prefix_segs] token counts (>= 0; zero adds no
 *   tile; may be NULL if n_prefix_segs == 0).
 * info: out, always filled on success.
 * untile_index: out host int32 [S]: padded row of each token, or NULL.
 * row_src: out host int32 [S_pad]: token of each padded row, -1 = padding, or NULL.
 * block_len: out host int32 [n_t]: real rows per tile, or NULL.
 * Pass all three arrays as NULL to query sizes first.
 * Errors: VSA_ERR_ARG (non-positive grid/tile, negative segment, S_pad >= 2^31).
 */
int vsa_plan_tiles(const int64_t *prefix_seg_lens, int32_t n_prefix_segs,
                   int32_t grid_t, int32_t grid_h, int32_t grid_w,
                   int32_t tile_t, int32_t tile_h, int32_t tile_w,
                   vsa_plan_info *info, int32_t *untile_index, int32_t *row_src,
                   int32_t *block_len);

/*
 * vsa_plan_validate -- checks host plan arrays against `info` before they are
 * trusted: untile is injective and is the inverse of row_src, every tile has
 * 1..B real rows packed first, block_len sums to S, and no tile mixes two
 * prefix segments or prefix and video ([SnackOnAI] snippet one: a mis-tiling
 * must fail loudly, never scramble tokens).
 * prefix_seg_lens as for vsa_plan_tiles. Returns VSA_OK or VSA_ERR_PLAN.
 */
int vsa_plan_validate(const vsa_plan_info *info, const int64_t *prefix_seg_lens,
                      int32_t n_prefix_segs, const int32_t *untile_index,
                      const int32_t *row_src, const int32_t *block_len);

/*
 * vsa_keep_count -- number k of video key tiles kept per video query tile.
 * [SnackOnAI] snippet two: keep ratio = clamp(1 - sparsity, 0, 1);
 * [Veda] "ComfyUI node": an integer keeps exactly that many key tiles.
 * keep_k >= 0: k = keep_k (VSA_ERR_ARG if keep_k > n_v).
 * keep_k < 0: k = floor(clamp(1 - sparsity, 0, 1) * n_v + 0.5)
 *             (VSA_ERR_ARG if sparsity is NaN).
 */
int vsa_keep_count(const vsa_plan_info *info, double sparsity, int64_t keep_k, int32_t *k_out);

/*
 * vsa_tile_pair_fraction -- share of the n_t^2 dense tile pairs that the sparse
 * pass computes: n_v query tiles see P + k key tiles, P prefix query tiles see
 * all n_t ([SnackOnAI] "It In Action", step three). Host only.
 */
int vsa_tile_pair_fraction(const vsa_plan_info *info, int32_t k, double *fraction);

/*
 * Reference sparsity. [Veda] "ComfyUI node" inputs table: reference_sparsity
 * applies the same top-k setting to the reference tokens (0 % = full
 * attention). Reading taken here: the prefix (reference) tiles stop being
 * sinks; every query tile, prefix or video, keeps its k_ref highest-scoring
 * prefix key tiles and its k_gen highest-scoring video key tiles.
 *
 * vsa_ref_keep_count -- k_ref over the P prefix tiles, by the vsa_keep_count
 * rule: ref_keep_k >= 0 gives k_ref = ref_keep_k (VSA_ERR_ARG above P), else
 * floor(clamp(1 - ref_sparsity, 0, 1) * P + 0.5) (VSA_ERR_ARG if NaN).
 * vsa_tile_pair_fraction_ref -- (k_ref + k_gen) / n_t, the share of dense
 * tile pairs computed in this mode. Both host only.
 */
int vsa_ref_keep_count(const vsa_plan_info *info, double ref_sparsity, int64_t ref_keep_k,
                       int32_t *k_out);
int vsa_tile_pair_fraction_ref(const vsa_plan_info *info, int32_t k_ref, int32_t k_gen,
                               double *fraction);

/* ------------------------------------------------------- workspace -- */
/*
 * The workspace (device memory, caller-owned) holds what the coarse pass
 * produces for the fine pass; it must survive between vsa_coarse_topk and
 * vsa_sparse_attn_fwd. Byte offsets (each 256-byte aligned):
 *   k_tiled, v_tiled: bf16 K and V in tile order, [H][n_t][B/64] blocks of
 *     64 rows, each block stored as (D/16)*2 fragments of 64 lanes x 8 bf16:
 *       K block, fragment f = kb*(D/16) + c (kb in {0,1}, c < D/16): lane l,
 *         element e = K[row 32*kb + l%32][d = 16*c + 8*(l/32) + e];
 *       V block, fragment f = db*4 + c (db < D/32, c < 4): lane l, element e =
 *         V[row 16*c + (e<4 ? 4*(l/32) + e : 8 + 4*(l/32) + e-4)][d = 32*db + l%32].
 *     Padding rows are zero.
 *   q_mean, k_mean, v_mean: fp32 [H][n_t][D] tile means over real rows.
 *   scores: fp32 coarse scores, [H][n_v][n_v] (video query tile i, video key
 *     tile j) after vsa_coarse_topk, [H][n_t][n_t] (every query tile, every
 *     key tile) after vsa_coarse_topk_ref; sized for the larger.
 *   k_i8, k_scale: INT8 K codes and fp32 block scales written by
 *     vsa_sparse_attn_fwd_i8 (layout there).
 *   part_o, part_ml (last): scratch for the fine pass when it splits each key
 *     list into C chunks by tile id modulo C: per chunk, bf16 O / l and the
 *     fp32 running max and sum of every 64 query rows. Empty when C = 1.
 * Everything before part_o is independent of C; the coarse stage needs only
 * those `part_o` bytes, the fine stage the whole `total_bytes`.
 *
 * split_chunks (here and in every fine / backward entry point): the C a call
 * uses; 0 = automatic (a function of the plan and head_dim only: 1 while one
 * head's K and V fit in 16 MiB, else 8 * ceil(K+V / 96 MiB), at least 16 for
 * 64-row tiles beyond 32 MiB, at most 64),
 * 1 = never split, 2..64 = that many chunks. It is a tuning choice: the
 * result depends on it only through fp32 rounding. A workspace serves the
 * fine calls made with the split count it was laid out for (or a smaller
 * layout); there is no process-wide setting. VSA_ERR_ARG outside [0, 64].
 */
typedef struct vsa_ws_layout {
    size_t k_tiled, v_tiled, q_mean, k_mean, v_mean, scores;
    size_t k_i8, k_scale;    /* INT8 fine pass: K codes and block scales */
    size_t part_o, part_ml;  /* fine-pass chunk partials (empty when not split) */
    size_t total_bytes;
    int32_t split_chunks;    /* the resolved C of this layout */
} vsa_ws_layout;

int vsa_workspace_layout(const vsa_plan_info *info, int32_t heads, int32_t head_dim,
                         int32_t split_chunks, vsa_ws_layout *layout);

/* ------------------------------------------------------ coarse pass -- */
/*
 * vsa_coarse_topk -- coarse stage: tile means, coarse scores, top-k video key
 * tiles, and the coarse attention output. Enqueued on `stream`.
 *
 *  1. Tile means ("mean-pooled Q/K", plus V for the coarse output) over the
 *     real rows of every tile: a sequential fp32 sum over rows in ascending
 *     row order from +0, then one fp32 division by block_len. K and V are
 *     also written in tile order to the workspace for the fine pass.
 *  2. Coarse score of video key tile j for video query tile i: the unscaled
 *     dot product of their mean Q and K, as a chain of fp32 fused
 *     multiply-adds over ascending d from +0.
 *  3. Top-k ([News] "The two-tier attention patch", item 2: only video key
 *     tiles are pruned): per head and video query tile, the k video key tiles
 *     with the largest score; equal scores keep the lower tile index; -0 and
 *     +0 are equal. keep_idx[h][i][0..k) holds them as ascending global tile
 *     ids (P + j). Scores must be finite.
 *  4. O_coarse[h][i] = sum_j softmax_j(scale * qmean_i . kmean_j) vmean_j over
 *     all n_t key tiles, for every tile i (prefix and video).
 *
 * info: host plan (as filled by vsa_plan_tiles).
 * row_src_dev, block_len_dev: device copies of the plan arrays.
 * heads (H), head_dim (D in {64,128}).
 * sparsity / keep_k: as vsa_keep_count. scale <= 0 means D^-1/2.
 * q, k, v: device bf16 [S][H][D]; or all three NULL when the workspace
 *   already holds the tiled K/V and the three tile means of these tokens
 *   (written by vsa_qkv_gate_proj for the same plan, heads and head_dim):
 *   step 1 is then skipped and steps 2-4 read them.
 * workspace: device, >= vsa_workspace_layout().part_o bytes, 256-byte aligned.
 * keep_idx_dev: out device int32 [H][n_v][k] (may be NULL when k == 0).
 * o_coarse_dev: out device fp32 [H][n_t][D].
 * Errors: VSA_ERR_ARG, VSA_ERR_UNSUPPORTED, VSA_ERR_DEVICE.
 */
int vsa_coarse_topk(const vsa_plan_info *info, const int32_t *row_src_dev,
                    const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                    double sparsity, int64_t keep_k, float scale,
                    const void *q, const void *k, const void *v,
                    void *workspace, size_t workspace_bytes,
                    int32_t *keep_idx_dev, float *o_coarse_dev, void *stream);

/*
 * vsa_coarse_topk_ref -- the coarse stage with reference sparsity (see
 * vsa_ref_keep_count). Steps 1 and 4 as vsa_coarse_topk; step 2 scores every
 * query tile against every key tile (same FMA chain); step 3 selects, per
 * head and query tile i (all n_t of them), the k_ref best prefix key tiles
 * and the k_gen best video key tiles (ties to the lower index), written as
 * keep_idx[h][i][0..k_ref) = prefix ids ascending, then
 * keep_idx[h][i][k_ref..k_ref+k_gen) = video ids ascending.
 * ref_sparsity / ref_keep_k: as vsa_ref_keep_count; sparsity / keep_k: as
 * vsa_keep_count (for k_gen). keep_idx_dev: out device int32
 * [H][n_t][k_ref + k_gen]; NULL allowed only when k_ref + k_gen == 0 (which
 * vsa_sparse_attn_fwd_ref then rejects). Other arguments and errors as
 * vsa_coarse_topk.
 */
int vsa_coarse_topk_ref(const vsa_plan_info *info, const int32_t *row_src_dev,
                        const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                        double sparsity, int64_t keep_k, double ref_sparsity, int64_t ref_keep_k,
                        float scale, const void *q, const void *k, const void *v,
                        void *workspace, size_t workspace_bytes,
                        int32_t *keep_idx_dev, float *o_coarse_dev, void *stream);

/* -------------------------------------------------------- fine pass -- */
/*
 * vsa_sparse_attn_fwd -- fine block-sparse attention plus the gated coarse
 * term, written in natural token order. Enqueued on `stream`.
 * [SnackOnAI] snippet two: prefix key tiles are always kept (sink blocks
 * [0, P)); prefix query tiles attend to every tile (sink queries [0, P));
 * block_len keeps padding rows out of the softmax; scale = D^-1/2.
 *
 * For each head h and real token t in tile i:
 *   keys(i)  = real rows of all tiles            if i < P,
 *            = real rows of tiles [0, P) and keep_idx[h][i-P][0..k)  otherwise;
 *   O_fine   = sum_u softmax_u(scale * q_t . k_u) v_u   (bf16 inputs, fp32 accumulation);
 *   out[t][h][:] = bf16_rne(O_fine + g[t][h][:] * o_coarse[h][i][:]).
 *
 * workspace: as filled by vsa_coarse_topk for the same plan, heads, head_dim
 *   and K/V (k_tiled / v_tiled are read), at least
 *   vsa_workspace_layout(..., split_chunks).total_bytes long (the chunk
 *   partials are written when the key lists split).
 * k: keep count used by vsa_coarse_topk; keep_idx_dev: its output.
 * split_chunks: see the workspace section (0 = automatic).
 * q: device bf16 [S][H][D]. gate: device bf16 [S][H*D] (g, natural order).
 * out: device bf16 [S][H][D]; only real tokens are written.
 * Errors: VSA_ERR_ARG (also: empty key set, i.e. P == 0 and k == 0),
 * VSA_ERR_UNSUPPORTED, VSA_ERR_DEVICE.
 */
int vsa_sparse_attn_fwd(const vsa_plan_info *info, const int32_t *row_src_dev,
                        const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                        int32_t k, float scale, int32_t split_chunks, const void *q,
                        const void *workspace, size_t workspace_bytes,
                        const int32_t *keep_idx_dev, const float *o_coarse_dev,
                        const void *gate, void *out, void *stream);

/*
 * vsa_sparse_attn_fwd_ref -- the fine pass with reference sparsity: for each
 * head h and real token t in tile i, keys(i) = the real rows of the tiles
 * keep_idx[h][i][0..k_ref + k_gen) (as written by vsa_coarse_topk_ref), for
 * prefix and video query tiles alike; O_fine and the gated output as
 * vsa_sparse_attn_fwd. k_ref, k_gen: the counts used by vsa_coarse_topk_ref.
 * Errors as vsa_sparse_attn_fwd; VSA_ERR_ARG also when k_ref + k_gen == 0.
 */
int vsa_sparse_attn_fwd_ref(const vsa_plan_info *info, const int32_t *row_src_dev,
                            const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                            int32_t k_ref, int32_t k_gen, float scale, int32_t split_chunks,
                            const void *q,
                            const void *workspace, size_t workspace_bytes,
                            const int32_t *keep_idx_dev, const float *o_coarse_dev,
                            const void *gate, void *out, void *stream);

/*
 * vsa_sparse_attn_fwd_i8 -- the fine pass with INT8 scores. [Veda] "How Veda
 * works" and its performance table: the tile-skip kernel computes attention
 * in INT8; the pages give no scheme, and the one below is this library's
 * reading. Q and K of each head are quantised in blocks of 64 rows of the
 * tiled layout (padding rows are zero), all in fp32:
 *   a = max |x| over the block, scale = a / 127,
 *   code = round-half-even(x * (127 / a)) clamped to [-127, 127]
 *   (a block with a = 0 has scale 0 and zero codes).
 * For a query in block bq and a key in block bk the score is
 *   scale_attn * s_q[bq] * s_k[bk] * (exact integer dot product of the codes);
 * the softmax, P.V (P in bf16, fp32 accumulation) and the gated combination
 * are those of vsa_sparse_attn_fwd.
 * k_ref < 0: default mode (key sets as vsa_sparse_attn_fwd with k = k_gen);
 * k_ref >= 0: reference-sparsity mode (key sets as vsa_sparse_attn_fwd_ref).
 * The K codes and scales are first written to the workspace regions k_i8
 * (int8 [H][n_t][B/64] blocks of 2*(D/32) fragments of 64 lanes x 16 codes:
 * fragment f = kb*(D/32) + c, lane l, byte e = code of K[row 32*kb + l%32]
 * [d = 32*c + 16*(l/32) + e]) and k_scale (fp32 [H][n_t][B/64]) from
 * k_tiled, so the workspace is written here; Q is quantised inside the
 * fine kernel. Other arguments and errors as vsa_sparse_attn_fwd(_ref).
 */
int vsa_sparse_attn_fwd_i8(const vsa_plan_info *info, const int32_t *row_src_dev,
                           const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                           int32_t k_ref, int32_t k_gen, float scale, int32_t split_chunks,
                           const void *q,
                           void *workspace, size_t workspace_bytes,
                           const int32_t *keep_idx_dev, const float *o_coarse_dev,
                           const void *gate, void *out, void *stream);

/* ------------------------------------------------ per-head tile shapes -- */
/*
 * [Veda] "How Veda works": tile shapes are chosen per layer and per head, so
 * that heads that mix mostly within a frame and heads that mix mostly across
 * frames each get a suitable tile within the same budget. Here a layer's
 * heads are split into groups of consecutive heads, each group with its own
 * tile plan (any tile shape the single-plan path supports); a group runs the
 * single-plan path (vsa_coarse_topk(_ref) then vsa_sparse_attn_fwd(_ref|_i8))
 * on its heads, so for every head h of group i the output is exactly what the
 * single-plan path computes for head h with plan i.
 *
 * vsa_head_group (host struct; the pointers in it are device pointers unless
 * marked host):
 *   info                 host: the group's plan (vsa_plan_tiles); all groups
 *                        plan the same token count S.
 *   row_src_dev, block_len_dev: the plan's arrays on the device.
 *   head_first, heads    the group's heads [head_first, head_first + heads) of
 *                        the heads_total heads of each token row; groups must
 *                        not overlap (heads no group covers are not written).
 *   sparsity, keep_k     keep rule for video key tiles (vsa_keep_count).
 *   ref, ref_sparsity, ref_keep_k: ref != 0 selects reference sparsity with
 *                        k_ref from vsa_ref_keep_count.
 *   int8                 != 0: the fine pass with INT8 scores (vsa_sparse_attn_fwd_i8).
 *   split_chunks         the group's fine-pass split (0 = automatic).
 *   workspace, workspace_bytes: vsa_workspace_layout(info, heads, head_dim,
 *                        split_chunks).
 *   keep_idx_dev         int32 [heads][n_v][k] (default) or [heads][n_t][k_ref + k]
 *                        (reference sparsity); may be null when that is empty.
 *   o_coarse_dev         fp32 [heads][n_t][head_dim].
 * All of these stay owned by the caller.
 */
typedef struct vsa_head_group {
    const vsa_plan_info *info;
    const int32_t *row_src_dev, *block_len_dev;
    int32_t head_first, heads;
    double sparsity;
    int64_t keep_k;
    int32_t ref, int8;
    double ref_sparsity;
    int64_t ref_keep_k;
    int32_t split_chunks;
    void *workspace;
    size_t workspace_bytes;
    int32_t *keep_idx_dev;
    float *o_coarse_dev;
} vsa_head_group;

/*
 * vsa_layer_fwd_groups -- the layer with per-head tile shapes, enqueued on
 * `stream`, group after group. q, k, v: device bf16 [S][heads_total][head_dim];
 * gate: device bf16 [S][heads_total * head_dim]; out: device bf16
 * [S][heads_total][head_dim] (each group writes its own heads). scale <= 0
 * means head_dim^-1/2. Every group is validated before anything is enqueued
 * (VSA_ERR_ARG for no groups, a head range outside [0, heads_total) or shared
 * by two groups, plans of different token counts, or a bad keep rule); errors
 * of a group's own stages name the group. VSA_ERR_UNSUPPORTED, VSA_ERR_DEVICE
 * as the single-plan entry points.
 */
int vsa_layer_fwd_groups(const vsa_head_group *groups, int32_t n_groups, int32_t heads_total,
                         int32_t head_dim, float scale, const void *q, const void *k,
                         const void *v, const void *gate, void *out, void *stream);

/* --------------------------------------------------------- backward -- */
/*
 * Backward pass: the gradient of the layer with the keep sets held fixed (a
 * top-k selection has no gradient; [SnackOnAI] "References": VSA trains end
 * to end). For each head and real token t of tile i, with the forward above:
 *   dg[t]   = dout[t] * O_coarse[i];
 *   dO_c[i] = sum_{t in i} dout[t] * g[t], back through the tile softmax to
 *             the tile means, and each real row of tile i receives the
 *             mean's share (gradient / block_len);
 *   dq, dk, dv also receive the fine attention's gradient over the same key
 *             lists (the log-sum-exp and the softmax-gradient row term
 *             D_t = dout[t] . O_fine[t] come from the training forward when
 *             it saved them, else the fine forward is recomputed for them; P
 *             and dS are rounded to bf16 for the matrix products).
 *
 * vsa_bwd_layout -- scratch regions (device, caller-owned, 256-byte aligned):
 * fragment copies (V / Q / dO rows, K / Q / dO columns), per-row log-sum-exp and D_t,
 * the coarse-path gradients, the transposed key lists ([H][n_t][n_t]) and the
 * bit matrix they are built from ([H][n_t][ceil(n_t / 32)] words), and,
 * when the forward splits its key lists, fp32 dQ partials of 8 key chunks,
 * fp32 dK / dV partials of 8 query chunks and the fp32 O_fine ([H][S_pad][D],
 * tile order) that vsa_sparse_attn_fwd_train saves.
 */
typedef struct vsa_bwd_layout {
    size_t vrow, kcol, qcol, docol, qrow, dorow, lse, dt, doc, dqm, dkm, dvm, lsec, dcc, tlist,
        tcount, tbits, part_dq, part_dkv, ofine;
    size_t total_bytes;
    int32_t split_chunks;    /* the resolved forward split of this layout */
} vsa_bwd_layout;

/* split_chunks: the forward's (as for vsa_workspace_layout); a backward with
 * C > 1 also splits its dQ and dK/dV passes into 8 XCD-affine chunks. */
int vsa_bwd_workspace_layout(const vsa_plan_info *info, int32_t heads, int32_t head_dim,
                             int32_t split_chunks, vsa_bwd_layout *layout);

/*
 * vsa_sparse_attn_bwd -- enqueues the backward pass on `stream`.
 * k_ref < 0: the default mode (keep_idx [H][n_v][k_gen] from vsa_coarse_topk);
 * k_ref >= 0: reference sparsity (keep_idx [H][n_t][k_ref + k_gen] from
 * vsa_coarse_topk_ref). q, k, v, dout: device bf16 [S][H][D]; gate:
 * device bf16 [S][H*D]; workspace / keep_idx / o_coarse: as left by the
 * coarse pass for the same inputs (the tiled K and the tile means are read).
 * split_chunks: the forward's split (0 = automatic); the workspaces are laid
 * out for it. bwd_workspace: >= vsa_bwd_workspace_layout().total_bytes.
 * dq, dk, dv: out device fp32 [S][H][D]; dgate: out device fp32 [S][H*D].
 * saved_stats != 0: bwd_workspace holds the lse and O_fine that
 * vsa_sparse_attn_fwd_train wrote for this same forward (same inputs, keep
 * lists and workspace); the backward then skips recomputing the fine forward.
 * 0: they are recomputed. It has no effect on heads too small to split their
 * key lists (those always recompute). The saved values stay valid until the
 * next training forward on the same bwd_workspace.
 * Errors: as vsa_sparse_attn_fwd(_ref), plus VSA_ERR_ARG for a small
 * backward workspace.
 */
int vsa_sparse_attn_bwd(const vsa_plan_info *info, const int32_t *row_src_dev,
                        const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                        int32_t k_ref, int32_t k_gen, float scale, int32_t split_chunks,
                        const void *q, const void *k, const void *v, const void *gate,
                        const void *dout,
                        const void *workspace, size_t workspace_bytes,
                        const int32_t *keep_idx_dev, const float *o_coarse_dev,
                        void *bwd_workspace, size_t bwd_workspace_bytes, float *dq, float *dk,
                        float *dv, float *dgate, int32_t saved_stats, void *stream);

/*
 * vsa_sparse_attn_fwd_train -- the fine pass of a training step: the same
 * output as vsa_sparse_attn_fwd (k_ref < 0; keep_idx [H][n_v][k_gen]) or
 * vsa_sparse_attn_fwd_ref (k_ref >= 0), and, for heads whose key lists are
 * split, the per-row log-sum-exp (log2 domain) and the fp32 O_fine written to
 * bwd_workspace (regions lse and ofine of vsa_bwd_workspace_layout) for a
 * following vsa_sparse_attn_bwd(..., saved_stats = 1). Arguments as
 * vsa_sparse_attn_fwd(_ref); bwd_workspace: device, >= the backward layout's
 * total_bytes, 256-byte aligned. Errors: as vsa_sparse_attn_fwd(_ref), plus
 * VSA_ERR_ARG for a small or misaligned bwd_workspace.
 */
int vsa_sparse_attn_fwd_train(const vsa_plan_info *info, const int32_t *row_src_dev,
                              const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                              int32_t k_ref, int32_t k_gen, float scale, int32_t split_chunks,
                              const void *q, const void *workspace, size_t workspace_bytes,
                              const int32_t *keep_idx_dev, const float *o_coarse_dev,
                              const void *gate, void *out, void *bwd_workspace,
                              size_t bwd_workspace_bytes, void *stream);

/* ------------------------------------------------- chunked producer -- */
/*
 * vsa_qkv_gate_proj -- the layer's four projections from its input x in one
 * GEMM whose rows are taken in tile order, writing what the attention stages
 * read directly ([SnackOnAI] "The Code, Annotated", snippet two: tile the
 * hidden states before projecting, so no sequence-sized copies follow;
 * "Why This Design Works": a chunked QKV producer that avoids the padded full
 * projection). bf16 inputs, fp32 accumulation, one bf16 rounding per output
 * (the arithmetic of vsa_gate_proj, so each projected value is the one
 * vsa_gate_proj gives for the same weight rows, bit for bit):
 *   q    = x . W_q^T   -> q, natural order, device bf16 [S][H][D];
 *   g    = x . W_g^T   -> gate, natural order, device bf16 [S][H*D];
 *   k, v = x . W_k^T, x . W_v^T -> the workspace's k_tiled / v_tiled, in the
 *          fragment layout vsa_coarse_topk writes (padding rows zero);
 *   and the tile means of q, k and v in the workspace's q_mean / k_mean /
 *   v_mean, in the canonical order of vsa_coarse_topk step 1 over the bf16
 *   values above.
 * Follow it with vsa_coarse_topk(..., q = k = v = NULL, ...) and the fine pass
 * (which reads q and gate). Only real rows are projected and stored.
 * x: device bf16 [S][hidden]; w_qkvg: device bf16 [4][H*D][hidden], the
 * stacked W_q, W_k, W_v, W_gate (nn.Linear weights, bias-free).
 * workspace: >= vsa_workspace_layout().part_o bytes, 256-byte aligned.
 * Errors: VSA_ERR_ARG (null pointers, small workspace), VSA_ERR_UNSUPPORTED
 * (head_dim not 64 or 128, hidden not a multiple of 64, H*D not a multiple
 * of 128, S*hidden*2 bytes of input beyond 4 GiB), VSA_ERR_DEVICE.
 */
int vsa_qkv_gate_proj(const vsa_plan_info *info, const int32_t *row_src_dev,
                      const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                      int32_t hidden, const void *x, const void *w_qkvg, void *q, void *gate,
                      void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------- layer without allocation -- */
/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the layer
 * of vsa_coarse_topk followed by vsa_sparse_attn_fwd (default mode, key lists
 * never split, i.e. split_chunks = 1), with the workspace taken from a static
 * device array of VSA_STATIC_WORKSPACE_BYTES inside the library instead of
 * from the caller. Each device the library runs on holds one such array until
 * the process ends; its address is looked up on the first call on a device.
 *
 * The results are those of vsa_coarse_topk + vsa_sparse_attn_fwd(...,
 * split_chunks = 1, ...) on the same arguments, bit for bit. The caller still
 * owns and passes every input and output: q, k, v (bf16 [S][H][D]), gate
 * (bf16 [S][H*D]), keep_idx_dev (out int32 [H][n_v][k]; NULL allowed when k
 * is 0), o_coarse_dev (out fp32 [H][n_t][D]) and out (bf16 [S][H][D]).
 * This call allocates nothing (no hipMalloc, no allocating library routine).
 *
 * All calls on one device share that device's array: calls that overlap in
 * time on one device (other streams, other threads) race and give undefined
 * results; serialise them. Every region the layer reads is written first in
 * the same call, so a call never depends on what an earlier call left there.
 * Errors: as vsa_coarse_topk / vsa_sparse_attn_fwd, plus VSA_ERR_ARG when the
 * layer's workspace (vsa_workspace_layout(..., 1, ...).total_bytes) exceeds
 * VSA_STATIC_WORKSPACE_BYTES (for example: 8 heads x 128 x 5,397 tokens
 * needs about 30 MB and fits; a 42-head 100k-token layer does not).
 */
#define VSA_STATIC_WORKSPACE_BYTES (64u << 20)

int vsa_layer_fwd_static(const vsa_plan_info *info, const int32_t *row_src_dev,
                         const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                         double sparsity, int64_t keep_k, float scale, const void *q,
                         const void *k, const void *v, const void *gate,
                         int32_t *keep_idx_dev, float *o_coarse_dev, void *out, void *stream);

/* -------------------------------------------------- gate projection -- */
/*
 * vsa_gate_proj -- g = bf16_rne(x . W_gate^T), the bias-free gate projection
 * ([SnackOnAI] snippets two and three: to_gate_compress is an nn.Linear
 * without bias, weight [heads*head_dim][hidden]). bf16 inputs, fp32 accumulation.
 * x: device bf16 [rows][hidden]; w_gate: device bf16 [out_features][hidden];
 * g: out device bf16 [rows][out_features]. hidden and out_features must be
 * multiples of 64. Errors: VSA_ERR_ARG, VSA_ERR_UNSUPPORTED, VSA_ERR_DEVICE.
 */
int vsa_gate_proj(const void *x, const void *w_gate, int64_t rows, int32_t hidden,
                  int32_t out_features, void *g, void *stream);

/* ---------------------------------------------------- kernel timing -- */
/*
 * Measurement support, not part of the method: per-kernel device time of this
 * library's own launches, for benchmarks that must report one kernel's time
 * when an entry point launches several.
 *
 * Timing is kept per stream: enabling it on one stream changes nothing for
 * launches on any other stream.
 *
 * vsa_timing_enable -- for `stream` (a hipStream_t; NULL = the null stream):
 * 1 clears its earlier records and starts timing; 0 stops. While on, every
 * kernel launch the library makes on that stream is bracketed by two HIP
 * events recorded on it (events are created on first use and reused; do not
 * enable timing on a stream that is being captured into a graph).
 *
 * vsa_timing_read -- for the kernel named `kernel` (one of "gate_gemm",
 * "gather_pool", "video_scores", "coarse_attn", "topk", "fine_attn",
 * "merge", "bwd_gather", "bwd_prep", "bwd_coarse", "bwd_tlist", "bwd_dq",
 * "bwd_dkdv", "bwd_stats", "quant_k", "qkv_proj"), waits for the launches recorded on
 * `stream` since its last enable (call it after those entry points have
 * returned) and returns their number in *launches and their summed duration
 * in *total_ms (host pointers); 0 and 0.0 for a stream never timed.
 * Errors: VSA_ERR_ARG for a null pointer or an unknown name, VSA_ERR_DEVICE
 * if an event query fails.
 */
int vsa_timing_enable(void *stream, int32_t enable);
int vsa_timing_read(void *stream, const char *kernel, int32_t *launches, double *total_ms);

#ifdef __cplusplus
}
#endif
#endif /* VSA_H */
