// Host-side head bucketing and work-list construction for per-head causal
// local-window attention.  Pure C++17: no HIP dependency, so it can be built
// and tested without a GPU.
#pragma once

#include <cstdint>
#include <vector>

namespace aah {

struct WorkItem {
  int32_t bh;    // b * H + h, or -1 for a padding slot
  int32_t tile;  // stationary row tile
  int32_t lo;    // first streamed tile (inclusive)
  int32_t hi;    // last streamed tile (exclusive)
};
static_assert(sizeof(WorkItem) == 16, "WorkItem must stay 16 bytes (one int4 load)");

// Effective window of a head: windows above T act as T.
inline int effective_window(int32_t w, int T) { return w > T ? T : w; }

// Exact in-window pairs of one head over length T: sum_{t=1}^{T} min(t, W).
inline int64_t pair_count(int T, int w) {
  const int64_t W = effective_window(w, T);
  return W * (W + 1) / 2 + (static_cast<int64_t>(T) - W) * W;
}

// Forward items: one per (b, h, query tile), with the key-tile range it needs.
std::vector<WorkItem> plan_forward(const int32_t* windows, int B, int H, int T,
                                   int q_tile, int kv_tile, int n_queues);

// Backward items: one per (b, h, key tile), with the query-tile range that sees it.
std::vector<WorkItem> plan_backward(const int32_t* windows, int B, int H, int T,
                                    int q_tile, int kv_tile, int n_queues);

}  // namespace aah
