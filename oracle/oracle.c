/*
 * oracle.c -- plain, slow CPU reference for gated, tile-sparse video attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library path loads this file: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg call it.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Built with gcc -O2 -ffp-contract=off (no fast-math, no FMA contraction), so
 * every float expression below is evaluated exactly as written: fp32 adds and
 * divides are IEEE round-to-nearest, fmaf() is a correctly rounded fused
 * multiply-add, and all attention arithmetic is fp64.
 *
 * Sources (web pages, cited by title and section):
 *   [SnackOnAI]  "ComfyUI-Ref2VA-VSA proves a sparse attention gate can be
 *                transplanted ..." (snackonai.com) -- "The Architecture,
 *                Unpacked"; "The Code, Annotated" snippets one to four;
 *                "It In Action"; "References".
 *   [News]       "Ref2VA VSA: Sparse Attention Node for H3 Reference-to-Video"
 *                (comfyui-wiki.com) -- "The two-tier attention patch".
 *   [README]     ComfyUI-Ref2VA-VSA README (pickgithub project payload) --
 *                "Technical Architecture".
 *   [Veda]       "Veda Sparse Attention" news item (comfyui-wiki.com, ja) --
 *                "How Veda works"; "ComfyUI node" inputs table.
 *
 * Where the pages leave a step open, the reading taken is stated at the step.
 * Pins (tests/test_oracle_*.py) tie each function to values the pages print,
 * closed forms, library routines or brute force. One function is marked
 * "parity unpinned" where only its special cases can be pinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ bf16 -- */

/* bf16 -> fp32 is exact: a bf16 is the upper half of an fp32. */
static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a double to the nearest bf16, ties to even (one rounding, from fp64).
 * bf16 keeps 8 significant bits; below 2^-126 its spacing is fixed at 2^-133. */
uint16_t orc_bf16_round(double x)
{
    if (isnan(x)) return 0x7FC0;
    if (isinf(x)) return x > 0 ? 0x7F80 : 0xFF80;
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    int e;
    frexp(x, &e);                       /* |x| in [2^(e-1), 2^e) */
    int q = e - 1;
    if (q < -126) q = -126;
    double ulp = ldexp(1.0, q - 7);
    double r = nearbyint(x / ulp) * ulp; /* default mode: nearest, ties to even */
    if (fabs(r) >= ldexp(1.0, 128)) return x > 0 ? 0x7F80 : 0xFF80;
    float f = (float)r;                  /* exact: r fits in 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

double orc_bf16_value(uint16_t b) { return (double)bf16_to_float(b); }

/* -------------------------------------------------------------- O1: plan -- */
/*
 * Tile plan. [SnackOnAI] "The Code, Annotated", snippet one, and "The
 * Architecture, Unpacked" (segment-pure prefix tiles); [News] "The two-tier
 * attention patch" item 1.
 *
 *  - Prefix: the segments (text, reference image, reference audio, ...) are
 *    laid out in order; each segment starts a new tile and fills tiles of B
 *    rows; its last tile may be short (block_len < B), the rest is padding.
 *    Prefix tiles are tiles [0, P).
 *  - Video: tokens are flattened t-major, then h, then w, i.e. video token
 *    v = (t*Hg + y)*Wg + x. Tiles are enumerated t0 (outer), h0, w0 (inner) in
 *    steps of the tile shape. Reading: ceil tiling, so edge tiles may be partial
 *    (pinned by the worked example's 660 = 10*6*11 tiles for a 37x24x42 grid).
 *    Reading: inside a tile, real tokens take rows 0.. in lexicographic
 *    (dt, dy, dx) order and padding goes last (the pages elide this loop).
 *  - untile[token] = padded row; row_src[row] = token or -1 (padding);
 *    block_len[tile] = number of real rows.
 *
 * sizes_out[0..4] = S (real rows), P, n_v, n_t, B. Arrays may be NULL (size
 * query). Returns 0, or -1 on invalid arguments.
 */
int orc_plan(const int64_t *seg, int32_t n_seg, int32_t T, int32_t Hg, int32_t Wg,
             int32_t tt, int32_t th, int32_t tw, int64_t *sizes_out,
             int32_t *untile, int32_t *row_src, int32_t *block_len)
{
    if (n_seg < 0 || T <= 0 || Hg <= 0 || Wg <= 0 || tt <= 0 || th <= 0 || tw <= 0) return -1;
    int64_t B = (int64_t)tt * th * tw;
    int64_t P = 0, s_prefix = 0;
    for (int32_t s = 0; s < n_seg; ++s) {
        if (seg[s] < 0) return -1;
        P += (seg[s] + B - 1) / B;
        s_prefix += seg[s];
    }
    int64_t nT = (T + tt - 1) / tt, nH = (Hg + th - 1) / th, nW = (Wg + tw - 1) / tw;
    int64_t n_v = nT * nH * nW;
    int64_t n_t = P + n_v;
    int64_t S = s_prefix + (int64_t)T * Hg * Wg;
    sizes_out[0] = S;
    sizes_out[1] = P;
    sizes_out[2] = n_v;
    sizes_out[3] = n_t;
    sizes_out[4] = B;
    if (!untile || !row_src || !block_len) return 0;

    for (int64_t r = 0; r < n_t * B; ++r) row_src[r] = -1;
    int64_t tile = 0, src = 0;
    for (int32_t s = 0; s < n_seg; ++s) {
        int64_t left = seg[s];
        while (left > 0) {
            int64_t n = left < B ? left : B;
            for (int64_t r = 0; r < n; ++r) {
                row_src[tile * B + r] = (int32_t)(src + r);
                untile[src + r] = (int32_t)(tile * B + r);
            }
            block_len[tile] = (int32_t)n;
            src += n;
            left -= n;
            ++tile;
        }
    }
    for (int64_t t0 = 0; t0 < T; t0 += tt)
        for (int64_t h0 = 0; h0 < Hg; h0 += th)
            for (int64_t w0 = 0; w0 < Wg; w0 += tw) {
                int64_t cnt = 0;
                for (int64_t dt = 0; dt < tt; ++dt)
                    for (int64_t dy = 0; dy < th; ++dy)
                        for (int64_t dx = 0; dx < tw; ++dx) {
                            int64_t t = t0 + dt, y = h0 + dy, x = w0 + dx;
                            if (t >= T || y >= Hg || x >= Wg) continue;
                            int64_t token = s_prefix + (t * Hg + y) * Wg + x;
                            row_src[tile * B + cnt] = (int32_t)token;
                            untile[token] = (int32_t)(tile * B + cnt);
                            ++cnt;
                        }
                block_len[tile] = (int32_t)cnt;
                ++tile;
            }
    return 0;
}

/* -------------------------------------------------------- O2: keep count -- */
/*
 * Number of video key tiles kept per video query tile.
 * [SnackOnAI] snippet two: keep ratio = max(0, min(1, 1 - sparsity)).
 * [Veda] "ComfyUI node" inputs table: an integer keeps exactly that many key
 * tiles. Readings: k = round-half-up(keep ratio * n_v) in double; an integer
 * above n_v (or negative) is an error rather than a clamp.
 * keep_k >= 0 selects the integer form. Returns 0 or -1.
 */
int orc_keep_count(int32_t n_v, double sparsity, int64_t keep_k, int32_t *k_out)
{
    if (n_v < 0) return -1;
    if (keep_k >= 0) {
        if (keep_k > n_v) return -1;
        *k_out = (int32_t)keep_k;
        return 0;
    }
    if (isnan(sparsity)) return -1;
    double keep = 1.0 - sparsity;
    if (keep < 0.0) keep = 0.0;
    if (keep > 1.0) keep = 1.0;
    *k_out = (int32_t)floor(keep * (double)n_v + 0.5);
    return 0;
}

/* ------------------------------------------------------ O3: tile means -- */
/*
 * Mean-pooled Q, K or V per tile, for one head: mean[tile][d] over the tile's
 * real rows (padding never counts: [SnackOnAI] snippet two, block_len).
 * Reading (evaluation order, fixed so two implementations can agree bit for
 * bit): start from +0.0f, add the fp32 value of each real row in ascending row
 * order with fp32 round-to-nearest adds, then one IEEE fp32 division by the
 * number of real rows.
 * X is bf16 [S][H][D]; mean is fp32 [n_t][D].
 */
void orc_tile_means(const uint16_t *X, int32_t H, int32_t D, int32_t h,
                    const int32_t *row_src, const int32_t *block_len, int32_t n_t, int32_t B,
                    float *mean)
{
#pragma omp parallel for schedule(static)
    for (int32_t tile = 0; tile < n_t; ++tile) {
        for (int32_t d = 0; d < D; ++d) {
            float acc = 0.0f;
            int32_t n = 0;
            for (int32_t r = 0; r < B; ++r) {
                int32_t tok = row_src[(int64_t)tile * B + r];
                if (tok < 0) continue;
                acc = acc + bf16_to_float(X[((int64_t)tok * H + h) * D + d]);
                ++n;
            }
            (void)block_len;
            mean[(int64_t)tile * D + d] = acc / (float)n;
        }
    }
}

/* ---------------------------------------------------- O4: coarse scores -- */
/*
 * Coarse score of video key tile j for video query tile i, one head: the dot
 * product of the tiles' mean-pooled Q and K. (The coarse stage scores tiles
 * from pooled Q/K: [SnackOnAI] "References", the VSA paper's coarse tile
 * selection.) Reading: unscaled (the positive softmax scale cannot change the
 * ranking except through rounding), evaluated as a chain of correctly rounded
 * fp32 fused multiply-adds over ascending d starting from +0.0f.
 * qmean/kmean are fp32 [n_t][D]; query and key indices below are video-tile
 * positions 0..n_v-1 (global tile P + i). rows lists the query positions to
 * score (n_rows of them); scores is fp32 [n_rows][n_v].
 */
void orc_video_scores(const float *qmean, const float *kmean, int32_t P, int32_t n_v, int32_t D,
                      const int32_t *rows, int32_t n_rows, float *scores)
{
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < n_rows; ++r) {
        const float *q = qmean + (int64_t)(P + rows[r]) * D;
        for (int32_t j = 0; j < n_v; ++j) {
            const float *k = kmean + (int64_t)(P + j) * D;
            float acc = 0.0f;
            for (int32_t d = 0; d < D; ++d) acc = fmaf(q[d], k[d], acc);
            scores[(int64_t)r * n_v + j] = acc;
        }
    }
}

/*
 * Reference-sparsity variant ([Veda] "ComfyUI node" inputs table: the
 * reference_sparsity input applies the same top-k setting to the reference
 * tokens). Reading: the reference (prefix) tiles lose their sink status; every
 * query tile, prefix or video, is scored against every key tile with the same
 * unscaled FMA chain as above, so the ranking within each key group uses one
 * definition of the score. rows lists global query tile ids; scores is fp32
 * [n_rows][n_t] over global key tile ids 0..n_t-1.
 */
void orc_all_scores(const float *qmean, const float *kmean, int32_t n_t, int32_t D,
                    const int32_t *rows, int32_t n_rows, float *scores)
{
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < n_rows; ++r) {
        const float *q = qmean + (int64_t)rows[r] * D;
        for (int32_t j = 0; j < n_t; ++j) {
            const float *k = kmean + (int64_t)j * D;
            float acc = 0.0f;
            for (int32_t d = 0; d < D; ++d) acc = fmaf(q[d], k[d], acc);
            scores[(int64_t)r * n_t + j] = acc;
        }
    }
}

/* ----------------------------------------------------------- O5: top-k -- */
/*
 * Kept video key tiles for one video query tile: the k largest coarse scores
 * ([News] "The two-tier attention patch" item 2: top-k prunes only generated
 * video key tiles; [Veda] "How Veda works": per-head top-k gives the tile mask).
 * Reading: equal scores keep the lower tile index; -0 and +0 are equal;
 * scores must be finite. Output: the k kept tiles as ascending global tile ids
 * (P + j). Method: a full sort by (score descending, index ascending).
 * Returns 0, or -1 on a non-finite score or k outside [0, n_v].
 */
typedef struct { float s; int32_t j; } orc_scored;

static int orc_by_score_then_index(const void *pa, const void *pb)
{
    const orc_scored *a = (const orc_scored *)pa, *b = (const orc_scored *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int orc_ascending(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

int orc_topk_rows(const float *scores, int32_t n_rows, int32_t n_v, int32_t k, int32_t P,
                  int32_t *keep)
{
    if (k < 0 || k > n_v) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int32_t r = 0; r < n_rows; ++r) {
        const float *s = scores + (int64_t)r * n_v;
        orc_scored *tmp = (orc_scored *)malloc(sizeof(orc_scored) * (size_t)(n_v > 0 ? n_v : 1));
        for (int32_t j = 0; j < n_v; ++j) {
            if (!isfinite(s[j])) bad = 1;
            tmp[j].s = s[j];
            tmp[j].j = j;
        }
        qsort(tmp, (size_t)n_v, sizeof(orc_scored), orc_by_score_then_index);
        int32_t *out = keep + (int64_t)r * k;
        for (int32_t i = 0; i < k; ++i) out[i] = tmp[i].j;
        qsort(out, (size_t)k, sizeof(int32_t), orc_ascending);
        for (int32_t i = 0; i < k; ++i) out[i] += P;
        free(tmp);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------ O6: coarse attention -- */
/*
 * O_coarse for one head: tile-level softmax attention of each tile's pooled
 * query over the pooled keys of all tiles, applied to the pooled values.
 * The pages pass the gate as the kernel's coarse-gate input ([SnackOnAI]
 * snippet two) but never define the coarse output. Reading: for every query
 * tile i (prefix and video), O_coarse[i] = sum_j softmax_j(scale * qm_i . km_j)
 * vm_j over all n_t key tiles, unweighted by block_len, in fp64 from the fp32
 * means; scale = D^-1/2 as in the fine pass (snippet two).
 * PARITY UNPINNED by the pages as a definition; its evaluation is pinned by
 * closed forms (1x1x1 tiles reduce it to dense token attention; equal keys
 * give the plain mean of vm).
 * rows lists the query tiles to evaluate; out is fp64 [n_rows][D].
 */
void orc_coarse_attn(const float *qm, const float *km, const float *vm, int32_t n_t, int32_t D,
                     double scale, const int32_t *rows, int32_t n_rows, double *out)
{
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < n_rows; ++r) {
        int32_t i = rows[r];
        double *z = (double *)malloc(sizeof(double) * (size_t)n_t);
        double zmax = -INFINITY;
        for (int32_t j = 0; j < n_t; ++j) {
            double dot = 0.0;
            for (int32_t d = 0; d < D; ++d)
                dot += (double)qm[(int64_t)i * D + d] * (double)km[(int64_t)j * D + d];
            z[j] = scale * dot;
            if (z[j] > zmax) zmax = z[j];
        }
        double denom = 0.0;
        for (int32_t j = 0; j < n_t; ++j) {
            z[j] = exp(z[j] - zmax);
            denom += z[j];
        }
        for (int32_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int32_t j = 0; j < n_t; ++j) acc += z[j] * (double)vm[(int64_t)j * D + d];
            out[(int64_t)r * D + d] = acc / denom;
        }
        free(z);
    }
}

/* -------------------------------------------------- O7: fine attention -- */
/*
 * Fine attention output of individual query tokens, one head.
 * [SnackOnAI] snippet two: keys of the prefix tiles are always kept (sink
 * blocks [0, P)) and prefix query tiles attend densely (sink queries [0, P));
 * a video query tile attends to the prefix tiles plus its kept video tiles;
 * block_len masks padding so it never scores; scale = D^-1/2.
 * For query token t in tile i: keys = the real rows of tiles 0..n_t-1 if
 * i < P, else of tiles [0, P) and keep[i - P][0..k). out[t] = sum_u
 * softmax_u(scale * q_t . k_u) v_u in fp64.
 * keep is [n_v][k] global tile ids for this head. out is fp64 [n_tok][D].
 * Returns 0, or -1 if some query has no key.
 */
int orc_fine_tokens(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int32_t H, int32_t D,
                    int32_t h, const int32_t *untile, const int32_t *row_src, int32_t n_t, int32_t B,
                    int32_t P, const int32_t *keep, int32_t k, double scale, const int64_t *tokens,
                    int64_t n_tok, double *out)
{
    if (D > 256) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t qi = 0; qi < n_tok; ++qi) {
        int64_t t = tokens[qi];
        int32_t tile = untile[t] / B;
        int32_t n_keys_tiles = tile < P ? n_t : P + k;
        double q[256];
        for (int32_t d = 0; d < D; ++d) q[d] = (double)bf16_to_float(Q[(t * H + h) * D + d]);
        double *z = (double *)malloc(sizeof(double) * (size_t)n_keys_tiles * (size_t)B);
        int64_t *u_of = (int64_t *)malloc(sizeof(int64_t) * (size_t)n_keys_tiles * (size_t)B);
        int64_t nk = 0;
        double zmax = -INFINITY;
        for (int32_t a = 0; a < n_keys_tiles; ++a) {
            int32_t j = (tile < P || a < P) ? a : keep[(int64_t)(tile - P) * k + (a - P)];
            for (int32_t r = 0; r < B; ++r) {
                int32_t u = row_src[(int64_t)j * B + r];
                if (u < 0) continue;
                double dot = 0.0;
                for (int32_t d = 0; d < D; ++d)
                    dot += q[d] * (double)bf16_to_float(K[((int64_t)u * H + h) * D + d]);
                z[nk] = scale * dot;
                u_of[nk] = u;
                if (z[nk] > zmax) zmax = z[nk];
                ++nk;
            }
        }
        if (nk == 0) {
            bad = 1;
        } else {
            double denom = 0.0;
            for (int64_t a = 0; a < nk; ++a) {
                z[a] = exp(z[a] - zmax);
                denom += z[a];
            }
            for (int32_t d = 0; d < D; ++d) out[qi * D + d] = 0.0;
            for (int64_t a = 0; a < nk; ++a) {
                const uint16_t *v = V + (u_of[a] * H + h) * D;
                for (int32_t d = 0; d < D; ++d) out[qi * D + d] += z[a] * (double)bf16_to_float(v[d]);
            }
            for (int32_t d = 0; d < D; ++d) out[qi * D + d] /= denom;
        }
        free(z);
        free(u_of);
    }
    return bad ? -1 : 0;
}

/*
 * Reference-sparsity variant of O7: every query tile i has an explicit key
 * list lists[i][0..L) of global tile ids (its kept reference tiles followed
 * by its kept video tiles); a query token attends to the real rows of exactly
 * those tiles. Padding never scores; scale and fp64 arithmetic as in O7.
 * lists is int32 [n_t][L] for this head. out is fp64 [n_tok][D].
 * Returns 0, or -1 if some query has no key (L = 0 or only empty tiles).
 */
int orc_fine_tokens_lists(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int32_t H,
                          int32_t D, int32_t h, const int32_t *untile, const int32_t *row_src,
                          int32_t n_t, int32_t B, const int32_t *lists, int32_t L, double scale,
                          const int64_t *tokens, int64_t n_tok, double *out)
{
    if (D > 256) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t qi = 0; qi < n_tok; ++qi) {
        int64_t t = tokens[qi];
        int32_t tile = untile[t] / B;
        double q[256];
        for (int32_t d = 0; d < D; ++d) q[d] = (double)bf16_to_float(Q[(t * H + h) * D + d]);
        size_t cap = (size_t)(L > 0 ? L : 1) * (size_t)B;
        double *z = (double *)malloc(sizeof(double) * cap);
        int64_t *u_of = (int64_t *)malloc(sizeof(int64_t) * cap);
        int64_t nk = 0;
        double zmax = -INFINITY;
        for (int32_t a = 0; a < L; ++a) {
            int32_t j = lists[(int64_t)tile * L + a];
            if (j < 0 || j >= n_t) {
                bad = 1;
                continue;
            }
            for (int32_t r = 0; r < B; ++r) {
                int32_t u = row_src[(int64_t)j * B + r];
                if (u < 0) continue;
                double dot = 0.0;
                for (int32_t d = 0; d < D; ++d)
                    dot += q[d] * (double)bf16_to_float(K[((int64_t)u * H + h) * D + d]);
                z[nk] = scale * dot;
                u_of[nk] = u;
                if (z[nk] > zmax) zmax = z[nk];
                ++nk;
            }
        }
        if (nk == 0) {
            bad = 1;
        } else {
            double denom = 0.0;
            for (int64_t a = 0; a < nk; ++a) {
                z[a] = exp(z[a] - zmax);
                denom += z[a];
            }
            for (int32_t d = 0; d < D; ++d) out[qi * D + d] = 0.0;
            for (int64_t a = 0; a < nk; ++a) {
                const uint16_t *v = V + (u_of[a] * H + h) * D;
                for (int32_t d = 0; d < D; ++d) out[qi * D + d] += z[a] * (double)bf16_to_float(v[d]);
            }
            for (int32_t d = 0; d < D; ++d) out[qi * D + d] /= denom;
        }
        free(z);
        free(u_of);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------- INT8 fine pass (NEXT) -- */
/*
 * [Veda] "How Veda works" and its performance table: the tile-skip kernel
 * computes attention in INT8. The pages give no scheme; the reading taken
 * here is the plain symmetric one: Q and K of a head are quantised in blocks
 * of 64 rows of the tiled layout (padding rows are zero), one fp32 scale per
 * block, and only the score product q.k uses the INT8 codes; the softmax and
 * the P.V product keep full precision.
 *
 * Block quantisation, all in fp32:
 *   a     = max over the block of |x|           (exact: a bf16 is an fp32)
 *   scale = a / 127                             (0 when a == 0)
 *   code  = round-half-even(x * (127 / a)), clamped to [-127, 127]
 *                                               (0 when a == 0)
 * codes: int8 [n_t * B][D] in tiled row order; scales: fp32 [n_t * B / 64].
 * Returns 0, or -1 if B is not a multiple of 64.
 */
int orc_quant_blocks_i8(const uint16_t *X, int32_t H, int32_t D, int32_t h, const int32_t *row_src,
                        int32_t n_t, int32_t B, int8_t *codes, float *scales)
{
    if (B % 64 != 0) return -1;
    const int64_t n_blocks = (int64_t)n_t * B / 64;
    for (int64_t b = 0; b < n_blocks; ++b) {
        float a = 0.0f;
        for (int32_t r = 0; r < 64; ++r) {
            int32_t u = row_src[b * 64 + r];
            if (u < 0) continue;
            for (int32_t d = 0; d < D; ++d) {
                float x = fabsf(bf16_to_float(X[((int64_t)u * H + h) * D + d]));
                if (x > a) a = x;
            }
        }
        float inv = a > 0.0f ? 127.0f / a : 0.0f;
        scales[b] = a > 0.0f ? a / 127.0f : 0.0f;
        for (int32_t r = 0; r < 64; ++r) {
            int32_t u = row_src[b * 64 + r];
            int8_t *c = codes + (b * 64 + r) * D;
            for (int32_t d = 0; d < D; ++d) {
                float y = u < 0 ? 0.0f : rintf(bf16_to_float(X[((int64_t)u * H + h) * D + d]) * inv);
                if (y > 127.0f) y = 127.0f;
                if (y < -127.0f) y = -127.0f;
                c[d] = (int8_t)y;
            }
        }
    }
    return 0;
}

/*
 * O_fine with INT8 scores, for the given query tokens of head h over CSR key
 * lists (tiles lst[off[i]..off[i+1]) for query tile i): for a query in block
 * bq and a key in block bk,
 *   z = scale * sq[bq] * sk[bk] * (integer dot product of their codes),
 * then softmax and P.V in fp64 as O7. Returns 0, or -1 on an empty key list
 * or a bad argument.
 */
int orc_fine_tokens_i8(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int32_t H, int32_t D,
                       int32_t h, const int32_t *untile, const int32_t *row_src, int32_t n_t, int32_t B,
                       const int32_t *off, const int32_t *lst, double scale, const int64_t *tokens,
                       int64_t n_tok, double *out)
{
    if (D > 256 || B % 64 != 0) return -1;
    const int64_t rows = (int64_t)n_t * B;
    int8_t *cq = (int8_t *)malloc((size_t)rows * (size_t)D);
    int8_t *ck = (int8_t *)malloc((size_t)rows * (size_t)D);
    float *sq = (float *)malloc(sizeof(float) * (size_t)(rows / 64));
    float *sk = (float *)malloc(sizeof(float) * (size_t)(rows / 64));
    int bad = 0;
    if (!cq || !ck || !sq || !sk) {
        bad = 1;
        goto done;
    }
    orc_quant_blocks_i8(Q, H, D, h, row_src, n_t, B, cq, sq);
    orc_quant_blocks_i8(K, H, D, h, row_src, n_t, B, ck, sk);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t qi = 0; qi < n_tok; ++qi) {
        const int64_t rq = untile[tokens[qi]];
        const int32_t tile = (int32_t)(rq / B);
        const int8_t *a = cq + rq * D;
        const int32_t n_keys_tiles = off[tile + 1] - off[tile];
        size_t cap = (size_t)(n_keys_tiles > 0 ? n_keys_tiles : 1) * (size_t)B;
        double *z = (double *)malloc(sizeof(double) * cap);
        int64_t *u_of = (int64_t *)malloc(sizeof(int64_t) * cap);
        int64_t nk = 0;
        double zmax = -INFINITY;
        for (int32_t e = off[tile]; e < off[tile + 1]; ++e) {
            const int32_t j = lst[e];
            if (j < 0 || j >= n_t) {
                bad = 1;
                continue;
            }
            for (int32_t r = 0; r < B; ++r) {
                const int64_t rk = (int64_t)j * B + r;
                const int32_t u = row_src[rk];
                if (u < 0) continue;
                const int8_t *b = ck + rk * D;
                int64_t dot = 0;
                for (int32_t d = 0; d < D; ++d) dot += (int64_t)a[d] * (int64_t)b[d];
                z[nk] = scale * (double)sq[rq / 64] * (double)sk[rk / 64] * (double)dot;
                u_of[nk] = u;
                if (z[nk] > zmax) zmax = z[nk];
                ++nk;
            }
        }
        if (nk == 0) {
            bad = 1;
        } else {
            double denom = 0.0;
            for (int64_t x = 0; x < nk; ++x) {
                z[x] = exp(z[x] - zmax);
                denom += z[x];
            }
            for (int32_t d = 0; d < D; ++d) out[qi * D + d] = 0.0;
            for (int64_t x = 0; x < nk; ++x) {
                const uint16_t *v = V + (u_of[x] * H + h) * D;
                for (int32_t d = 0; d < D; ++d) out[qi * D + d] += z[x] * (double)bf16_to_float(v[d]);
            }
            for (int32_t d = 0; d < D; ++d) out[qi * D + d] /= denom;
        }
        free(z);
        free(u_of);
    }
done:
    free(cq);
    free(ck);
    free(sq);
    free(sk);
    return bad ? -1 : 0;
}

/* ------------------------------------------------------ backward (NEXT) -- */
/*
 * Gradient of the layer for one head. The method is trainable ([SnackOnAI]
 * "References": VSA trains end to end with its sparse kernel); the keep sets
 * come from a top-k and are held fixed, as a selection has no gradient.
 * Forward, for a real token t in tile i (fp64 throughout):
 *   O_fine[t]  = sum_{u in keys(i)} softmax_u(scale q_t.k_u) v_u
 *   O_c[i]     = sum_j softmax_j(scale qm_i.km_j) vm_j  over all n_t tiles,
 *                qm/km/vm the tile means of the real rows
 *   out[t]     = O_fine[t] + g[t] * O_c[i]   (elementwise)
 * Given dout (bf16), this returns (all fp64 [S][D] for head h):
 *   dg[t]  = dout[t] * O_c[i]
 *   dq, dk, dv = fine-attention gradients (chain rule through both softmaxes)
 *                plus the coarse path: dO_c[i] = sum_{t in i} dout[t] * g[t],
 *                back through the tile softmax to dqm/dkm/dvm, and each real
 *                row t of tile i receives dqm_i / n_i (the mean's derivative).
 * Key lists are given per query tile in CSR form: tiles lst[off[i]..off[i+1]).
 * The tile means are the fp32 canonical ones (orc_tile_means) read as fp64,
 * the same values the forward uses. Returns 0, or -1 on an empty key list.
 */
int orc_layer_bwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const uint16_t *G,
                  const uint16_t *dOut, int32_t H, int32_t D, int32_t h, const int32_t *untile,
                  const int32_t *row_src, const int32_t *block_len, int32_t n_t, int32_t B,
                  const int32_t *off, const int32_t *lst, const float *qm, const float *km,
                  const float *vm, double scale, double *dq, double *dk, double *dv, double *dg)
{
    if (D > 256) return -1;
    (void)untile;
    int64_t n_rows = (int64_t)n_t * B;
#define X(A, t, d) ((double)bf16_to_float((A)[((int64_t)(t) * H + h) * D + (d)]))
#define GV(t, d) ((double)bf16_to_float(G[(int64_t)(t) * H * D + (int64_t)h * D + (d)]))
    /* ---- coarse forward and its gradient inputs */
    double *Pc = (double *)malloc(sizeof(double) * (size_t)n_t * (size_t)n_t);
    double *Oc = (double *)calloc((size_t)n_t * (size_t)D, sizeof(double));
    double *dOc = (double *)calloc((size_t)n_t * (size_t)D, sizeof(double));
    double *dqm = (double *)calloc((size_t)n_t * (size_t)D, sizeof(double));
    double *dkm = (double *)calloc((size_t)n_t * (size_t)D, sizeof(double));
    double *dvm = (double *)calloc((size_t)n_t * (size_t)D, sizeof(double));
    for (int32_t i = 0; i < n_t; ++i) {
        double zmax = -INFINITY;
        for (int32_t j = 0; j < n_t; ++j) {
            double dot = 0.0;
            for (int32_t d = 0; d < D; ++d) dot += (double)qm[(int64_t)i * D + d] * (double)km[(int64_t)j * D + d];
            Pc[(int64_t)i * n_t + j] = scale * dot;
            if (scale * dot > zmax) zmax = scale * dot;
        }
        double den = 0.0;
        for (int32_t j = 0; j < n_t; ++j) {
            double e = exp(Pc[(int64_t)i * n_t + j] - zmax);
            Pc[(int64_t)i * n_t + j] = e;
            den += e;
        }
        for (int32_t j = 0; j < n_t; ++j) {
            Pc[(int64_t)i * n_t + j] /= den;
            for (int32_t d = 0; d < D; ++d) Oc[(int64_t)i * D + d] += Pc[(int64_t)i * n_t + j] * (double)vm[(int64_t)j * D + d];
        }
    }
    /* dg and dO_c */
    for (int64_t r = 0; r < n_rows; ++r) {
        int32_t t = row_src[r];
        if (t < 0) continue;
        int32_t i = (int32_t)(r / B);
        for (int32_t d = 0; d < D; ++d) {
            double go = X(dOut, t, d);
            dg[(int64_t)t * D + d] = go * Oc[(int64_t)i * D + d];
            dOc[(int64_t)i * D + d] += go * GV(t, d);
        }
    }
    /* coarse backward: dZ_ij = Pc_ij (dOc_i . vm_j - Dc_i) */
    for (int32_t i = 0; i < n_t; ++i) {
        double Dc = 0.0;
        for (int32_t d = 0; d < D; ++d) Dc += dOc[(int64_t)i * D + d] * Oc[(int64_t)i * D + d];
        for (int32_t j = 0; j < n_t; ++j) {
            double p = Pc[(int64_t)i * n_t + j];
            double dp = 0.0;
            for (int32_t d = 0; d < D; ++d) dp += dOc[(int64_t)i * D + d] * (double)vm[(int64_t)j * D + d];
            double dz = p * (dp - Dc);
            for (int32_t d = 0; d < D; ++d) {
                dqm[(int64_t)i * D + d] += scale * dz * (double)km[(int64_t)j * D + d];
                dkm[(int64_t)j * D + d] += scale * dz * (double)qm[(int64_t)i * D + d];
                dvm[(int64_t)j * D + d] += p * dOc[(int64_t)i * D + d];
            }
        }
    }
    /* ---- fine attention: the mean-pooling gradient first, then the fine part */
    for (int64_t r = 0; r < n_rows; ++r) {
        int32_t t = row_src[r];
        if (t < 0) continue;
        int32_t i = (int32_t)(r / B);
        double inv = 1.0 / (double)block_len[i];
        for (int32_t d = 0; d < D; ++d) {
            dq[(int64_t)t * D + d] = dqm[(int64_t)i * D + d] * inv;
            dk[(int64_t)t * D + d] = dkm[(int64_t)i * D + d] * inv;
            dv[(int64_t)t * D + d] = dvm[(int64_t)i * D + d] * inv;
        }
    }
    int bad = 0;
    /* per query token: softmax over its keys, O_fine, D_t, then dS */
    for (int64_t r = 0; r < n_rows; ++r) {
        int32_t t = row_src[r];
        if (t < 0) continue;
        int32_t i = (int32_t)(r / B);
        int64_t nk = 0;
        for (int32_t a = off[i]; a < off[i + 1]; ++a) nk += block_len[lst[a]];
        if (nk == 0) {
            bad = 1;
            continue;
        }
        double *z = (double *)malloc(sizeof(double) * (size_t)nk);
        int32_t *u_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)nk);
        int64_t n = 0;
        double zmax = -INFINITY;
        for (int32_t a = off[i]; a < off[i + 1]; ++a) {
            int32_t j = lst[a];
            for (int32_t rr = 0; rr < B; ++rr) {
                int32_t u = row_src[(int64_t)j * B + rr];
                if (u < 0) continue;
                double dot = 0.0;
                for (int32_t d = 0; d < D; ++d) dot += X(Q, t, d) * X(K, u, d);
                z[n] = scale * dot;
                u_of[n] = u;
                if (z[n] > zmax) zmax = z[n];
                ++n;
            }
        }
        double den = 0.0;
        for (int64_t a = 0; a < n; ++a) {
            z[a] = exp(z[a] - zmax);
            den += z[a];
        }
        double o[256], go[256];
        for (int32_t d = 0; d < D; ++d) {
            o[d] = 0.0;
            go[d] = X(dOut, t, d);
        }
        for (int64_t a = 0; a < n; ++a) {
            z[a] /= den;
            for (int32_t d = 0; d < D; ++d) o[d] += z[a] * X(V, u_of[a], d);
        }
        double Dt = 0.0;
        for (int32_t d = 0; d < D; ++d) Dt += go[d] * o[d];
        for (int64_t a = 0; a < n; ++a) {
            int32_t u = u_of[a];
            double dp = 0.0;
            for (int32_t d = 0; d < D; ++d) dp += go[d] * X(V, u, d);
            double ds = z[a] * (dp - Dt);
            for (int32_t d = 0; d < D; ++d) {
                dq[(int64_t)t * D + d] += scale * ds * X(K, u, d);
                dk[(int64_t)u * D + d] += scale * ds * X(Q, t, d);
                dv[(int64_t)u * D + d] += z[a] * go[d];
            }
        }
        free(z);
        free(u_of);
    }
#undef X
#undef GV
    free(Pc);
    free(Oc);
    free(dOc);
    free(dqm);
    free(dkm);
    free(dvm);
    return bad ? -1 : 0;
}

/*
 * dq of selected query tokens only (the same gradient as orc_layer_bwd, for
 * checks at full size): the fine part needs only the token's own keys, and
 * the mean's share needs only its tile's row of the coarse attention
 * (dO_c[i] from the tile's real rows). dq is fp64 [n_tok][D].
 */
int orc_dq_tokens(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const uint16_t *G,
                  const uint16_t *dOut, int32_t H, int32_t D, int32_t h, const int32_t *untile,
                  const int32_t *row_src, const int32_t *block_len, int32_t n_t, int32_t B,
                  const int32_t *off, const int32_t *lst, const float *qm, const float *km,
                  const float *vm, double scale, const int64_t *tokens, int64_t n_tok, double *dq)
{
    if (D > 256) return -1;
    int bad = 0;
#define X(A, t, d) ((double)bf16_to_float((A)[((int64_t)(t) * H + h) * D + (d)]))
#define GV(t, d) ((double)bf16_to_float(G[(int64_t)(t) * H * D + (int64_t)h * D + (d)]))
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t qi = 0; qi < n_tok; ++qi) {
        const int64_t t = tokens[qi];
        const int32_t i = untile[t] / B;
        double *res = dq + qi * D;
        /* coarse row i: Pc_ij, O_c[i], dO_c[i], Dc_i, then dqm_i */
        double *pc = (double *)malloc(sizeof(double) * (size_t)n_t);
        double zmax = -INFINITY, den = 0.0;
        for (int32_t j = 0; j < n_t; ++j) {
            double dot = 0.0;
            for (int32_t d = 0; d < D; ++d) dot += (double)qm[(int64_t)i * D + d] * (double)km[(int64_t)j * D + d];
            pc[j] = scale * dot;
            if (pc[j] > zmax) zmax = pc[j];
        }
        for (int32_t j = 0; j < n_t; ++j) {
            pc[j] = exp(pc[j] - zmax);
            den += pc[j];
        }
        double oc[256], doc[256], dqm[256];
        for (int32_t d = 0; d < D; ++d) oc[d] = doc[d] = dqm[d] = 0.0;
        for (int32_t j = 0; j < n_t; ++j) {
            pc[j] /= den;
            for (int32_t d = 0; d < D; ++d) oc[d] += pc[j] * (double)vm[(int64_t)j * D + d];
        }
        for (int32_t r = 0; r < B; ++r) {
            int32_t u = row_src[(int64_t)i * B + r];
            if (u < 0) continue;
            for (int32_t d = 0; d < D; ++d) doc[d] += X(dOut, u, d) * GV(u, d);
        }
        double Dc = 0.0;
        for (int32_t d = 0; d < D; ++d) Dc += doc[d] * oc[d];
        for (int32_t j = 0; j < n_t; ++j) {
            double dp = 0.0;
            for (int32_t d = 0; d < D; ++d) dp += doc[d] * (double)vm[(int64_t)j * D + d];
            double dz = pc[j] * (dp - Dc);
            for (int32_t d = 0; d < D; ++d) dqm[d] += scale * dz * (double)km[(int64_t)j * D + d];
        }
        free(pc);
        for (int32_t d = 0; d < D; ++d) res[d] = dqm[d] / (double)block_len[i];
        /* fine part over the token's own keys */
        int64_t nk = 0;
        for (int32_t a = off[i]; a < off[i + 1]; ++a) nk += block_len[lst[a]];
        if (nk == 0) {
            bad = 1;
            continue;
        }
        double *z = (double *)malloc(sizeof(double) * (size_t)nk);
        int32_t *u_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)nk);
        int64_t n = 0;
        zmax = -INFINITY;
        for (int32_t a = off[i]; a < off[i + 1]; ++a) {
            int32_t j = lst[a];
            for (int32_t rr = 0; rr < B; ++rr) {
                int32_t u = row_src[(int64_t)j * B + rr];
                if (u < 0) continue;
                double dot = 0.0;
                for (int32_t d = 0; d < D; ++d) dot += X(Q, t, d) * X(K, u, d);
                z[n] = scale * dot;
                u_of[n] = u;
                if (z[n] > zmax) zmax = z[n];
                ++n;
            }
        }
        den = 0.0;
        for (int64_t a = 0; a < n; ++a) {
            z[a] = exp(z[a] - zmax);
            den += z[a];
        }
        double o[256];
        for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
        for (int64_t a = 0; a < n; ++a) {
            z[a] /= den;
            for (int32_t d = 0; d < D; ++d) o[d] += z[a] * X(V, u_of[a], d);
        }
        double Dt = 0.0;
        for (int32_t d = 0; d < D; ++d) Dt += X(dOut, t, d) * o[d];
        for (int64_t a = 0; a < n; ++a) {
            double dp = 0.0;
            for (int32_t d = 0; d < D; ++d) dp += X(dOut, t, d) * X(V, u_of[a], d);
            double ds = z[a] * (dp - Dt);
            for (int32_t d = 0; d < D; ++d) res[d] += scale * ds * X(K, u_of[a], d);
        }
        free(z);
        free(u_of);
    }
#undef X
#undef GV
    return bad ? -1 : 0;
}

/* ----------------------------------------------------------- O8: combine -- */
/*
 * Layer output for individual (token, head) rows: out = O_fine + g * O_coarse
 * (elementwise), with g the gate projection of the token and O_coarse the
 * coarse output of the token's tile; computed in fp64 and rounded once to bf16.
 * (The gate is passed to the kernel as its coarse-gate input, [SnackOnAI]
 * snippet two; the combination itself is the specified one.)
 * All arrays are [n][D]; g_rows holds bf16 gate values.
 */
void orc_combine(const double *o_fine, const uint16_t *g_rows, const double *o_coarse, int64_t n,
                 int32_t D, uint16_t *out)
{
    for (int64_t i = 0; i < n * D; ++i)
        out[i] = orc_bf16_round(o_fine[i] + (double)bf16_to_float(g_rows[i]) * o_coarse[i]);
}

/* --------------------------------------------------- gate projection (a8) -- */
/*
 * g = x . W_gate^T for selected tokens, bias-free ([SnackOnAI] snippets two and
 * three: to_gate_compress is an nn.Linear without bias whose weight is
 * [heads*head_dim][hidden]); fp64 accumulation, one rounding to bf16.
 * x is bf16 [S][hidden]; W is bf16 [out_f][hidden]; g is bf16 [n_tok][out_f].
 */
void orc_gate_proj(const uint16_t *x, const uint16_t *W, int32_t hidden, int32_t out_f,
                   const int64_t *tokens, int64_t n_tok, uint16_t *g)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_tok; ++i) {
        const uint16_t *xr = x + tokens[i] * hidden;
        for (int32_t o = 0; o < out_f; ++o) {
            const uint16_t *w = W + (int64_t)o * hidden;
            double acc = 0.0;
            for (int32_t c = 0; c < hidden; ++c)
                acc += (double)bf16_to_float(xr[c]) * (double)bf16_to_float(w[c]);
            g[i * out_f + o] = orc_bf16_round(acc);
        }
    }
}

/* --------------------------------------------------- tile-pair fraction -- */
/*
 * Share of dense tile pairs that the sparse pass computes, as the pages count
 * it ([SnackOnAI] "It In Action", step three): each of n_v video query tiles
 * sees P prefix + k video key tiles, each of P prefix query tiles sees all
 * n_t tiles, out of n_t^2 pairs.
 */
double orc_tile_pair_fraction(int32_t P, int32_t n_v, int32_t k)
{
    double n_t = (double)P + (double)n_v;
    return ((double)n_v * ((double)P + (double)k) + (double)P * n_t) / (n_t * n_t);
}
