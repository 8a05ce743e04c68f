// Host side of libvsa: tile plan, plan validation, keep-count, workspace layout
// and the thread-local error state. No device code here.
//
// Tile plan: SnackOnAI analysis of ComfyUI-Ref2VA-VSA, "The Code, Annotated",
// snippet one (segment-pure prefix tiles, t-major video tiles, injectivity
// check) and "The Architecture, Unpacked".
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "common.h"

namespace vsa {

static thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

void clear_error() { g_last_error.clear(); }

namespace {

struct Geometry {
    int64_t B = 0, P = 0, prefix_rows = 0, nT = 0, nH = 0, nW = 0, n_v = 0, n_t = 0;
    int64_t S = 0, S_pad = 0;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int derive(const int64_t *seg, int32_t n_seg, const int32_t grid[3], const int32_t tile[3],
           Geometry *g)
{
    if (n_seg < 0 || (n_seg > 0 && seg == nullptr))
        return fail(VSA_ERR_ARG, "prefix segments: n=%d with %s pointer", n_seg,
                    seg ? "non-null" : "null");
    for (int a = 0; a < 3; ++a) {
        if (grid[a] <= 0) return fail(VSA_ERR_ARG, "grid[%d] = %d must be positive", a, grid[a]);
        if (tile[a] <= 0) return fail(VSA_ERR_ARG, "tile[%d] = %d must be positive", a, tile[a]);
    }
    g->B = int64_t(tile[0]) * tile[1] * tile[2];
    for (int32_t s = 0; s < n_seg; ++s) {
        if (seg[s] < 0) return fail(VSA_ERR_ARG, "prefix segment %d has negative length", s);
        g->P += ceil_div(seg[s], g->B);
        g->prefix_rows += seg[s];
    }
    g->nT = ceil_div(grid[0], tile[0]);
    g->nH = ceil_div(grid[1], tile[1]);
    g->nW = ceil_div(grid[2], tile[2]);
    g->n_v = g->nT * g->nH * g->nW;
    g->n_t = g->P + g->n_v;
    g->S = g->prefix_rows + int64_t(grid[0]) * grid[1] * grid[2];
    g->S_pad = g->n_t * g->B;
    if (g->S_pad >= (int64_t(1) << 31))
        return fail(VSA_ERR_ARG, "padded rows %lld do not fit int32 indices", (long long)g->S_pad);
    return VSA_OK;
}

void fill_info(const Geometry &g, const int32_t grid[3], const int32_t tile[3], vsa_plan_info *info)
{
    for (int a = 0; a < 3; ++a) {
        info->grid[a] = grid[a];
        info->tile[a] = tile[a];
    }
    info->tile_rows = int32_t(g.B);
    info->n_prefix_tiles = int32_t(g.P);
    info->n_video_tiles = int32_t(g.n_v);
    info->n_tiles = int32_t(g.n_t);
    info->rows_real = g.S;
    info->rows_padded = g.S_pad;
    info->prefix_rows = g.prefix_rows;
}

}  // namespace

int check_info(const vsa_plan_info *info)
{
    if (!info) return fail(VSA_ERR_ARG, "plan info is null");
    Geometry g;
    // Re-derive from the video fields; the prefix enters only through P and prefix_rows.
    for (int a = 0; a < 3; ++a)
        if (info->grid[a] <= 0 || info->tile[a] <= 0)
            return fail(VSA_ERR_ARG, "plan info: non-positive grid or tile");
    g.B = int64_t(info->tile[0]) * info->tile[1] * info->tile[2];
    g.n_v = ceil_div(info->grid[0], info->tile[0]) * ceil_div(info->grid[1], info->tile[1]) *
            ceil_div(info->grid[2], info->tile[2]);
    g.P = info->n_prefix_tiles;
    g.n_t = g.P + g.n_v;
    g.S = info->prefix_rows + int64_t(info->grid[0]) * info->grid[1] * info->grid[2];
    if (info->tile_rows != g.B || info->n_video_tiles != g.n_v || info->n_tiles != g.n_t ||
        info->rows_real != g.S || info->rows_padded != g.n_t * g.B || g.P < 0 ||
        info->prefix_rows < 0 || info->prefix_rows > g.P * g.B ||
        (g.P > 0 && info->prefix_rows < g.P))
        return fail(VSA_ERR_PLAN, "plan info fields are inconsistent");
    if (info->rows_padded >= (int64_t(1) << 31))
        return fail(VSA_ERR_ARG, "padded rows do not fit int32 indices");
    if (g.B != 64 && g.B != 128)
        return fail(VSA_ERR_UNSUPPORTED, "tile rows B = %lld; the device path supports 64 and 128",
                    (long long)g.B);
    return VSA_OK;
}

void compute_layout(const vsa_plan_info &info, int heads, int head_dim, int chunks, vsa_ws_layout *L)
{
    const size_t H = size_t(heads), D = size_t(head_dim);
    const size_t n_t = size_t(info.n_tiles);
    const size_t S_pad = size_t(info.rows_padded);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    L->k_tiled = take(H * S_pad * D * 2);
    L->v_tiled = take(H * S_pad * D * 2);
    L->q_mean = take(H * n_t * D * 4);
    L->k_mean = take(H * n_t * D * 4);
    L->v_mean = take(H * n_t * D * 4);
    // Coarse scores: [H][n_v][n_v] on the default path, [H][n_t][n_t] with
    // reference sparsity (every query tile against every key tile).
    L->scores = take(H * n_t * n_t * 4);
    const size_t items = H * n_t * size_t(info.tile_rows / 64);
    // INT8 fine pass: K codes in tile order (one byte per element) and one fp32
    // scale per 64-row block.
    L->k_i8 = take(H * S_pad * D);
    L->k_scale = take(items * 4);
    // Fine-pass chunk partials last: everything before them is independent of
    // the split count, so the coarse stage needs only that prefix.
    const size_t C = size_t(chunks);
    L->part_o = take(C > 1 ? items * C * 64 * D * 2 : 0);
    L->part_ml = take(C > 1 ? items * C * 128 * 4 : 0);
    L->total_bytes = off;
    L->split_chunks = int32_t(chunks);
}

}  // namespace vsa

using namespace vsa;

extern "C" {

const char *vsa_status_string(int status)
{
    switch (status) {
    case VSA_OK: return "ok";
    case VSA_ERR_ARG: return "invalid argument";
    case VSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case VSA_ERR_PLAN: return "inconsistent tile plan";
    case VSA_ERR_DEVICE: return "HIP device error";
    default: return "unknown status";
    }
}

const char *vsa_last_error(void) { return g_last_error.c_str(); }

int vsa_plan_tiles(const int64_t *seg, int32_t n_seg, int32_t grid_t, int32_t grid_h,
                   int32_t grid_w, int32_t tile_t, int32_t tile_h, int32_t tile_w,
                   vsa_plan_info *info, int32_t *untile, int32_t *row_src, int32_t *block_len)
{
    clear_error();
    if (!info) return fail(VSA_ERR_ARG, "info is null");
    const int32_t grid[3] = {grid_t, grid_h, grid_w};
    const int32_t tile[3] = {tile_t, tile_h, tile_w};
    Geometry g;
    if (int st = derive(seg, n_seg, grid, tile, &g)) return st;
    fill_info(g, grid, tile, info);
    const int given = (untile != nullptr) + (row_src != nullptr) + (block_len != nullptr);
    if (given == 0) return VSA_OK;
    if (given != 3) return fail(VSA_ERR_ARG, "pass all three plan arrays, or none");

    std::fill(row_src, row_src + g.S_pad, int32_t(-1));
    // Prefix: a new segment always opens a new tile; its last tile may be short.
    int64_t tile_id = 0, token = 0;
    for (int32_t s = 0; s < n_seg; ++s) {
        for (int64_t done = 0; done < seg[s]; done += g.B, ++tile_id) {
            const int64_t n = std::min<int64_t>(g.B, seg[s] - done);
            int32_t *rows = row_src + tile_id * g.B;
            for (int64_t r = 0; r < n; ++r, ++token) {
                rows[r] = int32_t(token);
                untile[token] = int32_t(tile_id * g.B + r);
            }
            block_len[tile_id] = int32_t(n);
        }
    }
    // Video: tiles in t-major order; each tile packs the in-grid part of its box.
    const int64_t T = grid_t, Hg = grid_h, Wg = grid_w;
    for (int64_t bt = 0; bt < g.nT; ++bt) {
        const int64_t t0 = bt * tile_t, et = std::min<int64_t>(tile_t, T - t0);
        for (int64_t bh = 0; bh < g.nH; ++bh) {
            const int64_t y0 = bh * tile_h, eh = std::min<int64_t>(tile_h, Hg - y0);
            for (int64_t bw = 0; bw < g.nW; ++bw, ++tile_id) {
                const int64_t x0 = bw * tile_w, ew = std::min<int64_t>(tile_w, Wg - x0);
                int64_t row = tile_id * g.B;
                for (int64_t dt = 0; dt < et; ++dt)
                    for (int64_t dy = 0; dy < eh; ++dy) {
                        int64_t tok = g.prefix_rows + ((t0 + dt) * Hg + (y0 + dy)) * Wg + x0;
                        for (int64_t dx = 0; dx < ew; ++dx, ++tok, ++row) {
                            row_src[row] = int32_t(tok);
                            untile[tok] = int32_t(row);
                        }
                    }
                block_len[tile_id] = int32_t(et * eh * ew);
            }
        }
    }
    return VSA_OK;
}

int vsa_plan_validate(const vsa_plan_info *info, const int64_t *seg, int32_t n_seg,
                      const int32_t *untile, const int32_t *row_src, const int32_t *block_len)
{
    clear_error();
    if (!info || !untile || !row_src || !block_len) return fail(VSA_ERR_ARG, "null argument");
    Geometry g;
    if (int st = derive(seg, n_seg, info->grid, info->tile, &g)) return st;
    vsa_plan_info want;
    fill_info(g, info->grid, info->tile, &want);
    if (std::memcmp(&want, info, sizeof want) != 0)
        return fail(VSA_ERR_PLAN, "plan info does not match the segments, grid and tile");
    // untile and row_src are mutually inverse (which makes untile injective).
    for (int64_t t = 0; t < g.S; ++t) {
        const int64_t r = untile[t];
        if (r < 0 || r >= g.S_pad || row_src[r] != t)
            return fail(VSA_ERR_PLAN, "untile map is not injective / not inverse at token %lld",
                        (long long)t);
    }
    int64_t real = 0;
    for (int64_t r = 0; r < g.S_pad; ++r) {
        if (row_src[r] == -1) continue;
        if (row_src[r] < 0 || row_src[r] >= g.S || untile[row_src[r]] != r)
            return fail(VSA_ERR_PLAN, "row_src entry %lld is not a token of this plan", (long long)r);
        ++real;
    }
    if (real != g.S) return fail(VSA_ERR_PLAN, "row_src holds %lld tokens, expected %lld",
                                 (long long)real, (long long)g.S);
    // Segment id of a token: prefix segments 0..n_seg-1, video = n_seg.
    std::vector<int64_t> seg_end(size_t(n_seg) + 1);
    int64_t acc = 0;
    for (int32_t s = 0; s < n_seg; ++s) seg_end[s] = (acc += seg[s]);
    seg_end[n_seg] = g.S;
    auto segment_of = [&](int64_t tok) {
        return int64_t(std::upper_bound(seg_end.begin(), seg_end.end(), tok) - seg_end.begin());
    };
    int64_t total = 0;
    for (int64_t tl = 0; tl < g.n_t; ++tl) {
        const int64_t n = block_len[tl];
        if (n < 1 || n > g.B) return fail(VSA_ERR_PLAN, "tile %lld has block_len %lld",
                                          (long long)tl, (long long)n);
        const int32_t *rows = row_src + tl * g.B;
        const int64_t sid = segment_of(rows[0]);
        for (int64_t r = 0; r < g.B; ++r) {
            if ((r < n) != (rows[r] >= 0))
                return fail(VSA_ERR_PLAN, "tile %lld: real rows are not packed first", (long long)tl);
            if (r < n && segment_of(rows[r]) != sid)
                return fail(VSA_ERR_PLAN, "tile %lld mixes two segments", (long long)tl);
        }
        if ((tl < g.P) != (sid < n_seg))
            return fail(VSA_ERR_PLAN, "tile %lld is on the wrong side of the prefix", (long long)tl);
        total += n;
    }
    if (total != g.S) return fail(VSA_ERR_PLAN, "block_len sums to %lld, expected %lld",
                                  (long long)total, (long long)g.S);
    return VSA_OK;
}

int vsa_keep_count(const vsa_plan_info *info, double sparsity, int64_t keep_k, int32_t *k_out)
{
    clear_error();
    if (!info || !k_out) return fail(VSA_ERR_ARG, "null argument");
    const int64_t n_v = info->n_video_tiles;
    if (n_v < 0) return fail(VSA_ERR_ARG, "negative video tile count");
    if (keep_k >= 0) {
        if (keep_k > n_v)
            return fail(VSA_ERR_ARG, "keep count %lld exceeds %lld video tiles", (long long)keep_k,
                        (long long)n_v);
        *k_out = int32_t(keep_k);
        return VSA_OK;
    }
    if (std::isnan(sparsity)) return fail(VSA_ERR_ARG, "sparsity is NaN");
    const double keep = std::min(1.0, std::max(0.0, 1.0 - sparsity));
    *k_out = int32_t(std::floor(keep * double(n_v) + 0.5));
    return VSA_OK;
}

int vsa_ref_keep_count(const vsa_plan_info *info, double ref_sparsity, int64_t ref_keep_k,
                       int32_t *k_out)
{
    clear_error();
    if (!info || !k_out) return fail(VSA_ERR_ARG, "null argument");
    const int64_t P = info->n_prefix_tiles;
    if (P < 0) return fail(VSA_ERR_ARG, "negative prefix tile count");
    if (ref_keep_k >= 0) {
        if (ref_keep_k > P)
            return fail(VSA_ERR_ARG, "reference keep count %lld exceeds %lld prefix tiles",
                        (long long)ref_keep_k, (long long)P);
        *k_out = int32_t(ref_keep_k);
        return VSA_OK;
    }
    if (std::isnan(ref_sparsity)) return fail(VSA_ERR_ARG, "reference sparsity is NaN");
    const double keep = std::min(1.0, std::max(0.0, 1.0 - ref_sparsity));
    *k_out = int32_t(std::floor(keep * double(P) + 0.5));
    return VSA_OK;
}

int vsa_tile_pair_fraction_ref(const vsa_plan_info *info, int32_t k_ref, int32_t k_gen,
                               double *fraction)
{
    clear_error();
    if (!info || !fraction) return fail(VSA_ERR_ARG, "null argument");
    if (k_ref < 0 || k_ref > info->n_prefix_tiles || k_gen < 0 || k_gen > info->n_video_tiles)
        return fail(VSA_ERR_ARG, "keep counts out of range");
    if (info->n_tiles <= 0) return fail(VSA_ERR_ARG, "empty plan");
    *fraction = (double(k_ref) + double(k_gen)) / double(info->n_tiles);
    return VSA_OK;
}

int vsa_tile_pair_fraction(const vsa_plan_info *info, int32_t k, double *fraction)
{
    clear_error();
    if (!info || !fraction) return fail(VSA_ERR_ARG, "null argument");
    if (k < 0 || k > info->n_video_tiles) return fail(VSA_ERR_ARG, "k out of range");
    const double P = info->n_prefix_tiles, nv = info->n_video_tiles, nt = info->n_tiles;
    if (nt <= 0) return fail(VSA_ERR_ARG, "empty plan");
    *fraction = (nv * (P + k) + P * nt) / (nt * nt);
    return VSA_OK;
}

int vsa_workspace_layout(const vsa_plan_info *info, int32_t heads, int32_t head_dim,
                         int32_t split_chunks, vsa_ws_layout *layout)
{
    clear_error();
    if (!layout) return fail(VSA_ERR_ARG, "layout is null");
    if (int st = check_info(info)) return st;
    if (heads <= 0) return fail(VSA_ERR_ARG, "heads = %d", heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(VSA_ERR_UNSUPPORTED, "head_dim = %d; supported: 64, 128", head_dim);
    int chunks = 0;
    if (int st = resolve_split(*info, head_dim, split_chunks, &chunks)) return st;
    compute_layout(*info, heads, head_dim, chunks, layout);
    return VSA_OK;
}

}  // extern "C"
