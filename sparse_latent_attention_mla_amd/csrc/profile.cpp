// profile.cpp -- opt-in per-kernel timing with HIP events on the caller's stream.
//
// When enabled, each launch of a timed kernel takes a fresh pair of events that
// the runtime stamps from that kernel's own dispatch (launch_kernel);
// mla_profile_read sums the elapsed times of the pairs taken since the previous
// read. Events are created on first use and reused. Off by default: no event is
// ever recorded then.
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

std::atomic<uint32_t> g_mask{0};      // bit k: time kernel k
std::mutex g_mu;
Pairs g_pairs[PROF_KERNELS];
const char* const kNames[PROF_KERNELS] = {"kv_append", "indexer_scan", "topk_select", "decode",
                                             "decode_merge"};

}  // namespace

ProfSlot prof_slot(ProfKernel k) {
    ProfSlot slot;
    if (!(g_mask.load(std::memory_order_relaxed) >> k & 1u)) return slot;
    std::lock_guard<std::mutex> lock(g_mu);
    Pairs& p = g_pairs[k];
    if (p.used == p.start.size()) {
        hipEvent_t a, b;
        if (hipEventCreate(&a) != hipSuccess) return slot;
        if (hipEventCreate(&b) != hipSuccess) {
            (void)hipEventDestroy(a);
            return slot;
        }
        p.start.push_back(a);
        p.stop.push_back(b);
    }
    slot.start = p.start[p.used];
    slot.stop = p.stop[p.used];
    ++p.used;
    return slot;
}

void prof_enable(uint32_t mask) { g_mask.store(mask & ((1u << PROF_KERNELS) - 1u)); }

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
