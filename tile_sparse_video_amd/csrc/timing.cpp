// Per-kernel timing of this library's own launches (vsa_timing_enable /
// vsa_timing_read), kept per stream: each launch made on a stream whose timing
// is on is bracketed by two HIP events recorded on that stream. Callers on
// other streams are unaffected. Events are pooled per stream and reused.
#include <hip/hip_runtime_api.h>

#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <vector>

#include "common.h"

namespace vsa {

struct StreamTiming {
    struct Record {
        hipEvent_t start, stop;
        int kernel;
    };
    bool on = false;
    unsigned generation = 0;     // bumped by every enable; stale timers record nothing
    std::vector<Record> pool;    // every event pair created for this stream
    size_t used = 0;             // records taken since the last enable
};

namespace {

const char *const kNames[K_COUNT] = {"gate_gemm",  "gather_pool", "video_scores", "coarse_attn",
                                     "topk",       "fine_attn",   "merge",        "bwd_gather",
                                     "bwd_prep",   "bwd_coarse",  "bwd_tlist",    "bwd_dq",
                                     "bwd_dkdv",   "bwd_stats",   "quant_k",      "qkv_proj"};

std::mutex g_mu;
// One entry per stream that ever had timing enabled; entries are never removed,
// so a KernelTimer's pointer stays valid.
std::map<hipStream_t, std::unique_ptr<StreamTiming>> g_streams;

StreamTiming *find(hipStream_t s)
{
    auto it = g_streams.find(s);
    return it == g_streams.end() ? nullptr : it->second.get();
}

}  // namespace

KernelTimer::KernelTimer(KernelId id, hipStream_t stream)
    : stream_(stream), timing_(nullptr), generation_(0), slot_(-1)
{
    std::lock_guard<std::mutex> lk(g_mu);
    StreamTiming *t = find(stream);
    if (!t || !t->on) return;
    if (t->used == t->pool.size()) {
        StreamTiming::Record r{};
        if (hipEventCreate(&r.start) != hipSuccess) return;
        if (hipEventCreate(&r.stop) != hipSuccess) {
            (void)hipEventDestroy(r.start);
            return;
        }
        t->pool.push_back(r);
    }
    timing_ = t;
    generation_ = t->generation;
    slot_ = long(t->used++);
    t->pool[size_t(slot_)].kernel = id;
    (void)hipEventRecord(t->pool[size_t(slot_)].start, stream_);
}

KernelTimer::~KernelTimer()
{
    if (slot_ < 0) return;
    std::lock_guard<std::mutex> lk(g_mu);
    // A re-enable since the start event was recorded has dropped this record.
    if (timing_->generation != generation_) return;
    (void)hipEventRecord(timing_->pool[size_t(slot_)].stop, stream_);
}

}  // namespace vsa

using namespace vsa;

extern "C" int vsa_timing_enable(void *stream, int32_t enable)
{
    clear_error();
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lk(g_mu);
    StreamTiming *t = find(s);
    if (!t) {
        if (!enable) return VSA_OK;
        t = (g_streams[s] = std::make_unique<StreamTiming>()).get();
    }
    if (enable) {
        ++t->generation;
        t->used = 0;
    }
    t->on = enable != 0;
    return VSA_OK;
}

extern "C" int vsa_timing_read(void *stream, const char *kernel, int32_t *launches, double *total_ms)
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
    if (StreamTiming *t = find(static_cast<hipStream_t>(stream))) {
        for (size_t i = 0; i < t->used; ++i) {
            if (t->pool[i].kernel != id) continue;
            float ms = 0.f;
            if (hipEventSynchronize(t->pool[i].stop) != hipSuccess ||
                hipEventElapsedTime(&ms, t->pool[i].start, t->pool[i].stop) != hipSuccess)
                return fail(VSA_ERR_DEVICE, "event query failed for a '%s' launch", kernel);
            ++n;
            sum += ms;
        }
    }
    *launches = n;
    *total_ms = sum;
    return VSA_OK;
}
