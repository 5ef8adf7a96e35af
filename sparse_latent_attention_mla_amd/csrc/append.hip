// append.hip -- quantise-append of a decode step's new entries.
//
// One workgroup per (new entry i, sequence b) runs append_load and append_store
// (append.hpp) back to back:
// the quantised main row and indexer key at row slots[b, i] and, for i == 0,
// the bf16 window entry at ring slot win_pos[b] mod W.
#include "append.hpp"

namespace mla {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_append(AppendArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kAppendLdsBytes];
    AppendStage<kThreads> st;
    append_load<kThreads>(a, blockIdx.x, blockIdx.y, st);
    append_store<kThreads>(a, blockIdx.x, blockIdx.y, st, lds);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
    int n_blocks_x = (a.main_cache || a.idx_cache) ? a.n_new : 0;
    if (a.win_ring && n_blocks_x < 1) n_blocks_x = 1;
    if (a.B == 0 || n_blocks_x == 0) return hipSuccess;
    const ProfSlot p = prof_slot(PROF_APPEND);
    return launch_kernel(k_append, dim3(n_blocks_x, a.B), dim3(kThreads), 0, stream, p.start, p.stop, a);
}

}  // namespace mla
