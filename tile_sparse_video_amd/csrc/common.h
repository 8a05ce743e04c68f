// Internal helpers shared by the libvsa translation units (not part of the ABI).
#pragma once

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "vsa.h"

namespace vsa {

// Records a formatted message in the thread-local error slot and returns `status`.
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Re-derives every field of `info` from grid/tile/prefix fields and checks it is
// consistent and supported on the device path (B in {64,128}, S_pad < 2^31).
int check_info(const vsa_plan_info *info);

// Fills `layout` for a checked plan and a resolved split count (see vsa.h for
// the meaning of each region).
void compute_layout(const vsa_plan_info &info, int heads, int head_dim, int chunks, vsa_ws_layout *layout);
void compute_bwd_layout(const vsa_plan_info &info, int heads, int head_dim, int chunks, vsa_bwd_layout *layout);

// The automatic number of key chunks the fine pass splits each key list into
// (1 = no split): a function of the plan and head_dim only.
int auto_split_chunks(const vsa_plan_info &info, int head_dim);

// Resolves a caller's split request (0 = automatic, 1..kMaxSplit = that many
// chunks) into *chunks; VSA_ERR_ARG for anything else.
constexpr int kMaxSplit = 64;
int resolve_split(const vsa_plan_info &info, int head_dim, int32_t requested, int *chunks);

// Backward support: runs the fine pass with split key lists and a merge that
// writes the per-row log-sum-exp (log2 domain) and D_t = dout . O_fine
// ([H][S_pad], tile order). Returns VSA_ERR_UNSUPPORTED when the heads are
// too small to split (the caller then recomputes the statistics itself).
int fine_stats(const vsa_plan_info &info, const int32_t *row_src, const int32_t *block_len, int heads,
               int head_dim, int chunks, bool ref, int k, int k_ref, float scale, const void *q,
               const void *workspace, const int32_t *keep_idx, const void *dout, float *lse_out,
               float *dt_out, hipStream_t st);

// Checks that the current HIP device is a gfx950; caches the answer per device.
int check_device();

// Kernels whose launches vsa_timing_read can report.
enum KernelId {
    K_GATE_GEMM, K_GATHER_POOL, K_VIDEO_SCORES, K_COARSE_ATTN, K_TOPK, K_FINE_ATTN, K_MERGE,
    K_BWD_GATHER, K_BWD_PREP, K_BWD_COARSE, K_BWD_TLIST, K_BWD_DQ, K_BWD_DKDV, K_BWD_STATS,
    K_QUANT_K, K_QKV_PROJ,
    K_COUNT
};

// Scope guard around one launch: while timing is enabled for `stream` it
// records an event before the launch and one after it on that stream;
// otherwise it does nothing.
struct StreamTiming;
class KernelTimer {
  public:
    KernelTimer(KernelId id, hipStream_t stream);
    ~KernelTimer();
    KernelTimer(const KernelTimer &) = delete;
    KernelTimer &operator=(const KernelTimer &) = delete;

  private:
    hipStream_t stream_;
    StreamTiming *timing_;
    unsigned generation_;
    long slot_;
};

// Bodies of the coarse and fine entry points, also driven per head group by
// vsa_layer_fwd_groups. ld is the number of heads per token row of q, k, v,
// gate and out (>= heads); the pointers address the first head processed.
// fine_impl with lse_out and ofine_out set (a training forward) also writes,
// when the key lists are split, the per-row lse and fp32 O_fine ([H][S_pad]
// and [H][S_pad][D], tile order) for the backward.
int coarse_impl(const char *name, const vsa_plan_info *info, const int32_t *row_src_dev,
                const int32_t *block_len_dev, int heads, int ld, int head_dim, bool ref, double sparsity,
                int64_t keep_k, double ref_sparsity, int64_t ref_keep_k, float scale, const void *q,
                const void *k, const void *v, void *workspace, size_t workspace_bytes,
                int32_t *keep_idx_dev, float *o_coarse_dev, void *stream);
int fine_impl(const char *name, const vsa_plan_info *info, const int32_t *row_src_dev,
              const int32_t *block_len_dev, int heads, int ld, int head_dim, bool ref, bool i8, int k,
              int k_ref, float scale, int32_t split_req, const void *q, const void *workspace,
              size_t workspace_bytes,
              const int32_t *keep_idx_dev, const float *o_coarse_dev, const void *gate, void *out,
              void *stream, float *lse_out, float *ofine_out);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace vsa
