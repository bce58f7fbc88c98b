// Work lists for per-head causal local-window attention.
//
// The pages bucket heads by their selected window and run each bucket
// ("Asymmetric Attention Heads", section 5.8 and Figure 1).  Here the buckets
// dissolve into one list of tile-level items: each item carries its own
// (batch, head) index, so bucket membership only changes how many tiles an
// item visits, and the output of every item lands directly at its head's slot.
// Tiles that lie wholly outside a head's window (section 5.8 mask; section 7.7
// describes the same block-level skipping for FlexAttention) are never listed.
// With sink keys ("Autonomy-of-Heads", section 5: a streaming head also keeps
// its first tokens), a forward item additionally visits the sink tiles before
// its window, and a backward item whose key tile holds a sink runs to the last
// query tile.
#include "workplan.hpp"

#include <algorithm>
#include <numeric>

namespace aah {
namespace {

int ceil_div(int a, int b) { return (a + b - 1) / b; }

struct Planned {
  WorkItem item;
  int cost;  // streamed tiles the item visits
};

// Deal the items of each head to n_queues queues (longest head first, each to
// the least-loaded queue), sort each queue by cost descending, and interleave
// the queues slot by slot.  Items arrive grouped by head in `per_head`.
std::vector<WorkItem> interleave(const std::vector<std::vector<Planned>>& per_head, int n_queues) {
  const int n_heads = static_cast<int>(per_head.size());
  std::vector<int64_t> head_cost(n_heads, 0);
  for (int i = 0; i < n_heads; ++i)
    for (const Planned& it : per_head[i]) head_cost[i] += it.cost;

  std::vector<int> order(n_heads);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return head_cost[a] > head_cost[b]; });

  std::vector<std::vector<Planned>> queues(n_queues);
  std::vector<int64_t> load(n_queues, 0);
  for (int hidx : order) {
    int best = 0;
    for (int qi = 1; qi < n_queues; ++qi)
      if (load[qi] < load[best]) best = qi;
    load[best] += head_cost[hidx];
    queues[best].insert(queues[best].end(), per_head[hidx].begin(), per_head[hidx].end());
  }
  size_t longest = 0;
  for (auto& q : queues) {
    std::stable_sort(q.begin(), q.end(), [](const Planned& a, const Planned& b) {
      if (a.cost != b.cost) return a.cost > b.cost;
      if (a.item.bh != b.item.bh) return a.item.bh < b.item.bh;
      return a.item.tile < b.item.tile;
    });
    longest = std::max(longest, q.size());
  }
  std::vector<WorkItem> out;
  out.reserve(longest * n_queues);
  for (size_t i = 0; i < longest; ++i)
    for (int qi = 0; qi < n_queues; ++qi)
      out.push_back(i < queues[qi].size() ? queues[qi][i].item : WorkItem{-1, 0, 0, 0});
  return out;
}

int head_sink(const int32_t* sinks, const int32_t* windows, int h, int T) {
  return sinks == nullptr ? 0 : effective_sink(sinks[h], windows[h], T);
}

}  // namespace

std::vector<WorkItem> plan_forward(const int32_t* windows, const int32_t* sinks, int B, int H, int T,
                                   int q_tile, int kv_tile, int n_queues) {
  const int n_qt = ceil_div(T, q_tile);
  std::vector<std::vector<Planned>> per_head(static_cast<size_t>(B) * H);
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      const int W = effective_window(windows[h], T);
      const int S = head_sink(sinks, windows, h, T);
      auto& list = per_head[static_cast<size_t>(b) * H + h];
      list.reserve(n_qt);
      for (int qt = 0; qt < n_qt; ++qt) {
        const int q0 = qt * q_tile;
        const int q1 = std::min(T, q0 + q_tile);
        const int key_first = std::max(0, q0 - W + 1);  // row q0's window start
        const int key_last = q1 - 1;                     // row q1-1's diagonal
        const WorkItem it{b * H + h, qt, key_first / kv_tile, key_last / kv_tile + 1};
        list.push_back(Planned{it, it.hi - it.lo + sink_tiles(S, it.lo, kv_tile)});
      }
    }
  }
  return interleave(per_head, n_queues);
}

std::vector<WorkItem> plan_backward(const int32_t* windows, const int32_t* sinks, int B, int H, int T,
                                    int q_tile, int kv_tile, int n_queues) {
  const int n_kt = ceil_div(T, kv_tile);
  std::vector<std::vector<Planned>> per_head(static_cast<size_t>(B) * H);
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      const int W = effective_window(windows[h], T);
      const int S = head_sink(sinks, windows, h, T);
      auto& list = per_head[static_cast<size_t>(b) * H + h];
      list.reserve(n_kt);
      for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * kv_tile;
        const int k1 = std::min(T, k0 + kv_tile);
        const int query_first = k0;  // key k0's own row
        // Last row that sees key k1-1, or every later row when the tile holds a sink key.
        const int query_last = k0 < S ? T - 1 : std::min(T, k1 + W - 1) - 1;
        const WorkItem it{b * H + h, kt, query_first / q_tile, query_last / q_tile + 1};
        list.push_back(Planned{it, it.hi - it.lo});
      }
    }
  }
  return interleave(per_head, n_queues);
}

}  // namespace aah
