// profile.cpp -- opt-in per-kernel timing with HIP events on the caller's stream.
//
// When enabled, the launchers bracket the named kernels with a pair of events
// recorded on the stream they launch on; mla_profile_read sums the elapsed
// times of the pairs recorded since the previous read. Events are created on
// first use and reused. Off by default: no event is ever recorded then.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "launch.hpp"

namespace mla {

namespace {

struct Pairs {
    std::vector<hipEvent_t> start, stop;
    size_t used = 0;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
Pairs g_pairs[PROF_KERNELS];
const char* const kNames[PROF_KERNELS] = {"kv_append", "indexer_scan", "topk_select", "decode",
                                             "decode_merge"};

}  // namespace

void prof_begin(ProfKernel k, hipStream_t s) {
    if (!g_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lock(g_mu);
    Pairs& p = g_pairs[k];
    if (p.used == p.start.size()) {
        hipEvent_t a, b;
        if (hipEventCreate(&a) != hipSuccess) return;
        if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return; }
        p.start.push_back(a);
        p.stop.push_back(b);
    }
    (void)hipEventRecord(p.start[p.used], s);
}

void prof_end(ProfKernel k, hipStream_t s) {
    if (!g_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lock(g_mu);
    Pairs& p = g_pairs[k];
    if (p.used < p.start.size()) {
        (void)hipEventRecord(p.stop[p.used], s);
        ++p.used;
    }
}

void prof_enable(bool on) { g_on.store(on); }

int prof_index(const char* name) {
    for (int i = 0; i < PROF_KERNELS; ++i)
        if (std::strcmp(name, kNames[i]) == 0) return i;
    return -1;
}

hipError_t prof_read(int k, int32_t* launches, double* total_ms) {
    std::lock_guard<std::mutex> lock(g_mu);
    Pairs& p = g_pairs[k];
    double sum = 0.0;
    for (size_t i = 0; i < p.used; ++i) {
        hipError_t e = hipEventSynchronize(p.stop[i]);
        if (e != hipSuccess) return e;
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, p.start[i], p.stop[i]);
        if (e != hipSuccess) return e;
        sum += ms;
    }
    *launches = (int32_t)p.used;
    *total_ms = sum;
    p.used = 0;
    return hipSuccess;
}

}  // namespace mla
