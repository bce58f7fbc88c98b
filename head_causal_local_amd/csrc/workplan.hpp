// Host-side head bucketing and work-list construction for per-head causal
// local-window attention.  Pure C++17: no HIP dependency, so it can be built
// and tested without a GPU.
#pragma once

#include <cstdint>
#include <vector>

namespace aah {

struct WorkItem {
  int32_t bh;    // b * H + h (forward: query head; backward: b * H_kv + key/value head), or -1 for padding
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

// Query tiles [lo, hi) that see keys [k0, k1) of a query head with window w and
// effective sink S (every later query when the tile holds a sink key).
inline void query_range(int k0, int k1, int W, int S, int T, int q_tile, int* lo, int* hi) {
  const int last = k0 < S ? T - 1 : (k1 + W - 1 < T ? k1 + W - 1 : T) - 1;
  *lo = k0 / q_tile;
  *hi = last / q_tile + 1;
}

// Forward items: one per (b, h, query tile), with the key-tile range it needs.
// sinks: int32[H] or nullptr; an item's sink tiles are implied (sink_tiles).
// The H / H_kv query heads of a key/value group go to the same queue.
std::vector<WorkItem> plan_forward(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                                   int q_tile, int kv_tile, int n_queues);

// Forward items with long key ranges split into chunks (for launches with
// fewer items than the device holds workgroups).  Every item of more than
// chunk_tiles window tiles becomes ceil(n / chunk_tiles) items over
// consecutive sub-ranges of its tiles; each chunk writes its rows'
// unnormalised partial result to its own slot (slot[i] >= 0) and one merge
// record {bh, tile, first slot, number of chunks} per split item combines
// them.  Items of at most chunk_tiles tiles keep slot -1 and write O and LSE
// themselves.  Chunks are dealt to queues and ordered like plan_forward's
// items (longest first).  sinks: int32[H] or nullptr; an item's sink tiles are
// visited by its first chunk only (the one whose range starts at the window's
// first tile), and count in that chunk's cost.
struct SplitPlan {
  std::vector<WorkItem> items;
  std::vector<int32_t> slot;
  std::vector<WorkItem> merges;
  int n_slots = 0;
};
SplitPlan plan_forward_split(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                             int q_tile, int kv_tile, int n_queues, int chunk_tiles);

// Backward (key-stationary) items of plan_backward split along their query-tile
// ranges: an item whose steps (query tiles summed over the group's query
// heads, each over its own range from lo) exceed chunk_tiles becomes
// ceil(steps / chunk_tiles) chunks over consecutive sub-ranges [c_lo, c_hi) of
// [lo, hi) with near-equal steps, each running every head of the group over
// its part of the range (a head whose range ends before c_lo has none), with
// slots, and a merge record {bh, key tile, first slot, chunks} per split item.
SplitPlan plan_backward_split(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                              int q_tile, int kv_tile, int n_queues, int chunk_tiles);

// Backward items: one per (b, key/value head g, key tile); [lo, hi) spans the
// query tiles that see the keys in any of the group's query heads (each head's
// own range is query_range, starting at the same lo).
std::vector<WorkItem> plan_backward(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                                    int q_tile, int kv_tile, int n_queues);

}  // namespace aah
