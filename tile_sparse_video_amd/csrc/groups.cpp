// Per-head tile shapes: one layer whose heads are split into groups, each with
// its own tile plan.
//
// Veda news item (comfyui-wiki.com), "How Veda works": tile shapes are chosen
// per layer and per head, so that heads that mix spatially and heads that mix
// temporally each get a tile that suits them within the same budget. A group
// here is a contiguous range of heads sharing one plan; its coarse stage, key
// selection and fine pass are exactly the single-plan path run on those heads
// of the shared q, k, v, gate and out tensors (rows of heads_total heads).
#include <cstdio>
#include <string>
#include <vector>

#include "common.h"

using namespace vsa;

namespace {

// Re-reports the error a callee just recorded, prefixed with the group index.
int wrap(int status, int group)
{
    const std::string msg = vsa_last_error();
    return fail(status, "vsa_layer_fwd_groups: group %d: %s", group, msg.c_str());
}

}  // namespace

extern "C" int vsa_layer_fwd_groups(const vsa_head_group *groups, int32_t n_groups, int32_t heads_total,
                                    int32_t head_dim, float scale, const void *q, const void *k,
                                    const void *v, const void *gate, void *out, void *stream)
{
    clear_error();
    if (!groups || n_groups <= 0) return fail(VSA_ERR_ARG, "vsa_layer_fwd_groups: no head groups");
    if (heads_total <= 0) return fail(VSA_ERR_ARG, "vsa_layer_fwd_groups: heads_total = %d", heads_total);
    if (!q || !k || !v || !gate || !out) return fail(VSA_ERR_ARG, "vsa_layer_fwd_groups: null device pointer");
    // Validate every group before anything is enqueued: head ranges in bounds and
    // disjoint, one token count for all plans, keep counts resolvable.
    std::vector<char> owner(static_cast<size_t>(heads_total), 0);
    int64_t tokens = -1;
    std::vector<int32_t> kk(static_cast<size_t>(n_groups)), kr(static_cast<size_t>(n_groups));
    for (int i = 0; i < n_groups; ++i) {
        const vsa_head_group &g = groups[i];
        if (!g.info) return fail(VSA_ERR_ARG, "vsa_layer_fwd_groups: group %d has no plan", i);
        if (int st = check_info(g.info)) return wrap(st, i);
        if (g.heads <= 0 || g.head_first < 0 || int64_t(g.head_first) + g.heads > heads_total)
            return fail(VSA_ERR_ARG, "vsa_layer_fwd_groups: group %d heads [%d, %d) outside [0, %d)", i,
                        g.head_first, g.head_first + g.heads, heads_total);
        for (int h = g.head_first; h < g.head_first + g.heads; ++h) {
            if (owner[size_t(h)])
                return fail(VSA_ERR_ARG, "vsa_layer_fwd_groups: head %d is in more than one group", h);
            owner[size_t(h)] = 1;
        }
        if (tokens >= 0 && g.info->rows_real != tokens)
            return fail(VSA_ERR_ARG, "vsa_layer_fwd_groups: group %d plans %lld tokens, group 0 %lld", i,
                        (long long)g.info->rows_real, (long long)tokens);
        tokens = g.info->rows_real;
        if (int st = vsa_keep_count(g.info, g.sparsity, g.keep_k, &kk[size_t(i)])) return wrap(st, i);
        kr[size_t(i)] = 0;
        if (g.ref)
            if (int st = vsa_ref_keep_count(g.info, g.ref_sparsity, g.ref_keep_k, &kr[size_t(i)]))
                return wrap(st, i);
        vsa_ws_layout L;
        if (int st = vsa_workspace_layout(g.info, g.heads, head_dim, g.split_chunks, &L)) return wrap(st, i);
        if (!g.row_src_dev || !g.block_len_dev || !g.workspace || !g.o_coarse_dev)
            return fail(VSA_ERR_ARG, "vsa_layer_fwd_groups: group %d: null device pointer", i);
        if ((g.ref ? kk[size_t(i)] + kr[size_t(i)] : kk[size_t(i)]) > 0 && !g.keep_idx_dev)
            return fail(VSA_ERR_ARG, "vsa_layer_fwd_groups: group %d: keep_idx is null", i);
        if (g.workspace_bytes < L.total_bytes || reinterpret_cast<uintptr_t>(g.workspace) % 256 != 0)
            return fail(VSA_ERR_ARG, "vsa_layer_fwd_groups: group %d: workspace of %zu bytes at %p; needs %zu, "
                        "256-byte aligned", i, g.workspace_bytes, g.workspace, L.total_bytes);
    }
    const size_t off = size_t(head_dim) * 2;  // bytes per head in a token row (bf16)
    for (int i = 0; i < n_groups; ++i) {
        const vsa_head_group &g = groups[i];
        const size_t first = size_t(g.head_first) * off;
        auto at = [&](const void *p) { return static_cast<const char *>(p) + first; };
        char name[64];
        std::snprintf(name, sizeof(name), "vsa_layer_fwd_groups[%d]", i);
        if (int st = coarse_impl(name, g.info, g.row_src_dev, g.block_len_dev, g.heads, heads_total, head_dim,
                                 g.ref != 0, g.sparsity, g.keep_k, g.ref_sparsity, g.ref_keep_k, scale,
                                 at(q), at(k), at(v), g.workspace, g.workspace_bytes, g.keep_idx_dev,
                                 g.o_coarse_dev, stream))
            return st;
        if (int st = fine_impl(name, g.info, g.row_src_dev, g.block_len_dev, g.heads, heads_total, head_dim,
                               g.ref != 0, g.int8 != 0, kk[size_t(i)], kr[size_t(i)], scale,
                               g.split_chunks, at(q), g.workspace, g.workspace_bytes, g.keep_idx_dev, g.o_coarse_dev, at(gate),
                               static_cast<char *>(out) + first, stream, nullptr, nullptr))
            return st;
    }
    return VSA_OK;
}
