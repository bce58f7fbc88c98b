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

// Effective sink size of a head (sink keys 0 .. S - 1 stay visible to every later
// query): only keys j <= T - 1 - W ever fall out of some row's window, so sinks
// past T - W change nothing, and a head whose window covers T has none.
inline int effective_sink(int32_t s, int32_t w, int T) {
  const int lim = T - effective_window(w, T);
  return s < 0 ? 0 : (s < lim ? s : lim);
}

// Sink key tiles a forward item visits before its window tiles [lo, hi): the
// tiles of keys 0 .. S - 1 that lie before lo.
inline int sink_tiles(int S, int lo, int kv_tile) {
  const int n = (S + kv_tile - 1) / kv_tile;
  return n < lo ? n : lo;
}

// Exact visible pairs of one head over length T: sum_{t=1}^{T} min(t, W), plus,
// with S sink keys, the sinks row t sees before its window: sum_t max(0, min(S, t - W)).
inline int64_t pair_count(int T, int w, int s = 0) {
  const int64_t W = effective_window(w, T);
  const int64_t S = effective_sink(s, w, T);
  const int64_t U = static_cast<int64_t>(T) - W;  // rows with keys before their window
  const int64_t sinks = U <= S ? U * (U + 1) / 2 : S * (S + 1) / 2 + (U - S) * S;
  return W * (W + 1) / 2 + U * W + sinks;
}

// Forward items: one per (b, h, query tile), with the key-tile range it needs.
// sinks: int32[H] or nullptr; an item's sink tiles are implied (sink_tiles).
std::vector<WorkItem> plan_forward(const int32_t* windows, const int32_t* sinks, int B, int H, int T,
                                   int q_tile, int kv_tile, int n_queues);

// Backward items: one per (b, h, key tile), with the query-tile range that sees it.
std::vector<WorkItem> plan_backward(const int32_t* windows, const int32_t* sinks, int B, int H, int T,
                                    int q_tile, int kv_tile, int n_queues);

}  // namespace aah
