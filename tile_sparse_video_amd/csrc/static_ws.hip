// A whole-layer entry point that allocates nothing: the workspace that
// vsa_coarse_topk and vsa_sparse_attn_fwd take from the caller lives here in a
// file-scope device array, for callers that cannot allocate device memory
// (code under graph capture, tight serving loops, harnesses that forbid it).
//
// The array is `scratch`, kStaticWorkspaceBytes long; every device the
// library runs on holds its own copy until the process ends. Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept in g_scratch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "common.h"

namespace vsa {
namespace {

constexpr size_t kStaticWorkspaceBytes = size_t(VSA_STATIC_WORKSPACE_BYTES);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];  // per device: the device address of `scratch`

// The current device's address of `scratch` (looked up on the first call on
// that device).
int scratch_on_current_device(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(VSA_ERR_DEVICE, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return fail(VSA_ERR_DEVICE, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(VSA_ERR_DEVICE, "hipGetSymbolAddress of the static workspace failed on device %d: %s",
                        dev, hipGetErrorString(e));
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return VSA_OK;
}

}  // namespace
}  // namespace vsa

using namespace vsa;

extern "C" int vsa_layer_fwd_static(const vsa_plan_info *info, const int32_t *row_src_dev,
                                    const int32_t *block_len_dev, int32_t heads, int32_t head_dim,
                                    double sparsity, int64_t keep_k, float scale, const void *q,
                                    const void *k, const void *v, const void *gate,
                                    int32_t *keep_idx_dev, float *o_coarse_dev, void *out,
                                    void *stream)
{
    clear_error();
    const char *name = "vsa_layer_fwd_static";
    if (int st = check_info(info)) return st;
    if (heads <= 0) return fail(VSA_ERR_ARG, "%s: heads = %d", name, heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(VSA_ERR_UNSUPPORTED, "%s: head_dim = %d; supported: 64, 128", name, head_dim);
    int32_t k_gen = 0;
    if (int st = vsa_keep_count(info, sparsity, keep_k, &k_gen)) return st;
    // Everything both stages check is checked here first, so a failed call
    // enqueues nothing.
    if (!row_src_dev || !block_len_dev || !q || !k || !v || !gate || !o_coarse_dev || !out)
        return fail(VSA_ERR_ARG, "%s: null device pointer", name);
    if (k_gen > 0 && !keep_idx_dev) return fail(VSA_ERR_ARG, "%s: keep_idx is null", name);
    if (info->n_prefix_tiles == 0 && k_gen == 0 && info->n_video_tiles > 0)
        return fail(VSA_ERR_ARG, "%s: empty key set: no prefix tiles and k = 0", name);
    if (!std::isfinite(scale)) return fail(VSA_ERR_ARG, "%s: scale is not finite", name);
    // The key lists are never split here, so the layout has no chunk partials.
    vsa_ws_layout L;
    compute_layout(*info, heads, head_dim, 1, &L);
    if (L.total_bytes > kStaticWorkspaceBytes)
        return fail(VSA_ERR_ARG, "%s: the layer needs a %zu-byte workspace; the static one holds %zu",
                    name, L.total_bytes, kStaticWorkspaceBytes);
    if (int st = check_device()) return st;
    void *ws = nullptr;
    if (int st = scratch_on_current_device(&ws)) return st;
    // Every region the two stages read is written first by the coarse stage
    // (tiled K/V with zero padding, means, scores), so nothing is cleared.
    if (int st = coarse_impl(name, info, row_src_dev, block_len_dev, heads, heads, head_dim, false, sparsity,
                             keep_k, 0.0, -1, scale, q, k, v, ws, kStaticWorkspaceBytes, keep_idx_dev,
                             o_coarse_dev, stream))
        return st;
    return fine_impl(name, info, row_src_dev, block_len_dev, heads, heads, head_dim, false, false, k_gen, 0,
                     scale, 1, q, ws, kStaticWorkspaceBytes, keep_idx_dev, o_coarse_dev, gate, out, stream,
                     nullptr, nullptr);
}
