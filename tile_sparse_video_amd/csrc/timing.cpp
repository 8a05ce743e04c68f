// Per-kernel timing of this library's own launches (vsa_timing_enable /
// vsa_timing_read): each launch made while timing is on is bracketed by two HIP
// events recorded on the launch's own stream. Events are pooled and reused.
#include <hip/hip_runtime_api.h>

#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"

namespace vsa {
namespace {

const char *const kNames[K_COUNT] = {"gate_gemm",  "gather_pool", "video_scores", "coarse_attn",
                                     "topk",       "fine_attn",   "merge",        "bwd_gather",
                                     "bwd_prep",   "bwd_coarse",  "bwd_tlist",    "bwd_dq",
                                     "bwd_dkdv",   "bwd_stats",   "quant_k"};

struct Record {
    hipEvent_t start, stop;
    int kernel;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Record> g_pool;  // every event pair ever created (reused across enables)
size_t g_used = 0;           // records taken since the last enable

}  // namespace

KernelTimer::KernelTimer(KernelId id, hipStream_t stream) : stream_(stream), slot_(-1)
{
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on) return;
    if (g_used == g_pool.size()) {
        Record r{};
        if (hipEventCreate(&r.start) != hipSuccess) return;
        if (hipEventCreate(&r.stop) != hipSuccess) {
            (void)hipEventDestroy(r.start);
            return;
        }
        g_pool.push_back(r);
    }
    slot_ = long(g_used++);
    g_pool[slot_].kernel = id;
    (void)hipEventRecord(g_pool[slot_].start, stream_);
}

KernelTimer::~KernelTimer()
{
    if (slot_ < 0) return;
    std::lock_guard<std::mutex> lk(g_mu);
    (void)hipEventRecord(g_pool[slot_].stop, stream_);
}

}  // namespace vsa

using namespace vsa;

extern "C" int vsa_timing_enable(int32_t enable)
{
    clear_error();
    std::lock_guard<std::mutex> lk(g_mu);
    if (enable) g_used = 0;
    g_on = enable != 0;
    return VSA_OK;
}

extern "C" int vsa_timing_read(const char *kernel, int32_t *launches, double *total_ms)
{
    clear_error();
    if (!kernel || !launches || !total_ms) return fail(VSA_ERR_ARG, "null argument");
    int id = -1;
    for (int i = 0; i < K_COUNT; ++i)
        if (std::strcmp(kernel, kNames[i]) == 0) id = i;
    if (id < 0) return fail(VSA_ERR_ARG, "unknown kernel name '%s'", kernel);
    std::lock_guard<std::mutex> lk(g_mu);
    int32_t n = 0;
    double sum = 0.0;
    for (size_t i = 0; i < g_used; ++i) {
        if (g_pool[i].kernel != id) continue;
        float ms = 0.f;
        if (hipEventSynchronize(g_pool[i].stop) != hipSuccess ||
            hipEventElapsedTime(&ms, g_pool[i].start, g_pool[i].stop) != hipSuccess)
            return fail(VSA_ERR_DEVICE, "event query failed for a '%s' launch", kernel);
        ++n;
        sum += ms;
    }
    *launches = n;
    *total_ms = sum;
    return VSA_OK;
}
