// options.cpp -- process-wide kernel-choice options (mla_set_option) and the
// record of the kernels the calling thread's last call launched (mla_last_kernels).
//
// The options only choose among kernels that compute the same result (for
// tuning and for tests that must reach a particular kernel); every default is
// the choice the library makes by itself.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <cxxabi.h>
#include <string>

#include "launch.hpp"

namespace mla {

namespace {

struct OptDef {
    const char* name;
    int64_t lo, hi;
};
// indexed by Opt; every option defaults to 0 ("the library decides")
const OptDef kOpts[OPT_COUNT] = {
    {"topk_path", 0, 2},          // 0 by size, 1 one workgroup per sequence, 2 many workgroups + final
    {"topk_final", 0, 1},         // 0 by workgroup count, 1 the 256-thread final of the many-workgroup path
    {"scan_queues", 0, 1},        // 1: the queue-fed 32x32 scan instead of the static partition
    {"scan_blocks", 0, 65536},    // target number of 4-wave scan workgroups (0: two per CU)
    {"decode_rows_per_split", 0, 256},   // selected rows per decode split (0: by shape; else 32 .. 256 (128 for
                                         // E2M1 and unpaired bf16 rows), a multiple of 32; a multiple of 64
                                         // for the paired bf16 decode)
};
std::atomic<int64_t> g_opt[OPT_COUNT];

constexpr int kMaxNoted = 64;
thread_local const void* t_launched[kMaxNoted];
thread_local int t_n = 0;
thread_local std::string t_names;

}  // namespace

int64_t option(Opt o) { return g_opt[o].load(std::memory_order_relaxed); }

int option_index(const char* name) {
    for (int i = 0; i < OPT_COUNT; ++i)
        if (std::strcmp(name, kOpts[i].name) == 0) return i;
    return -1;
}

bool option_set(int i, int64_t v) {
    if (i < 0 || i >= OPT_COUNT || v < kOpts[i].lo || v > kOpts[i].hi) return false;
    g_opt[i].store(v, std::memory_order_relaxed);
    return true;
}

thread_local bool t_group = false;                      // inside mla_csa2_group_step

void begin_call() {
    if (!t_group) t_n = 0;
}
void group_begin() {
    t_n = 0;
    t_group = true;
}
void group_end() { t_group = false; }

void note_launch(const void* f) {
    if (t_n < kMaxNoted) t_launched[t_n++] = f;
}

const char* launched_names() {
    t_names.clear();
    for (int i = 0; i < t_n; ++i) {
        const char* m = hipKernelNameRefByPtr(t_launched[i], nullptr);
        if (!m) m = "?";
        int st = 0;
        char* d = abi::__cxa_demangle(m, nullptr, nullptr, &st);
        if (i) t_names += ';';
        t_names += (st == 0 && d) ? d : m;
        std::free(d);
    }
    return t_names.c_str();
}

}  // namespace mla
