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
// query tile.  With grouped key/value heads (G query heads per key/value head),
// the G heads' forward items share a queue (so their K/V tiles meet in one
// XCD's L2), and one backward item covers a key tile of the shared head for
// all G query heads, so dK and dV are summed in registers.
#include "workplan.hpp"

#include <algorithm>
#include <numeric>

namespace aah {
namespace {

int ceil_div(int a, int b) { return (a + b - 1) / b; }

struct Planned {
  WorkItem item;
  int cost;   // streamed tiles the item visits
  int32_t group;  // key/value group: items of one group share a queue and sort next to each other
  int32_t slot = -1;  // partial-result slot of a chunk of a split item, or -1
};

// Deal the items of each head to n_queues queues (longest head first, each to
// the least-loaded queue), sort each queue by cost descending, and interleave
// the queues slot by slot.  Items arrive grouped by head in `per_head`.
std::vector<WorkItem> interleave(const std::vector<std::vector<Planned>>& per_head, int n_queues,
                                 std::vector<int32_t>* slots = nullptr) {
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
    // Equal costs: group, then tile, then head, so that the query heads of one key/value group
    // visit the same tile back to back (with one head per group this is head, then tile).
    std::stable_sort(q.begin(), q.end(), [](const Planned& a, const Planned& b) {
      if (a.cost != b.cost) return a.cost > b.cost;
      if (a.group != b.group) return a.group < b.group;
      if (a.item.tile != b.item.tile) return a.item.tile < b.item.tile;
      return a.item.bh < b.item.bh;
    });
    longest = std::max(longest, q.size());
  }
  std::vector<WorkItem> out;
  out.reserve(longest * n_queues);
  if (slots != nullptr) slots->clear();
  for (size_t i = 0; i < longest; ++i)
    for (int qi = 0; qi < n_queues; ++qi) {
      const bool real = i < queues[qi].size();
      out.push_back(real ? queues[qi][i].item : WorkItem{-1, 0, 0, 0});
      if (slots != nullptr) slots->push_back(real ? queues[qi][i].slot : -1);
    }
  return out;
}

int head_sink(const int32_t* sinks, const int32_t* windows, int h, int T) {
  return sinks == nullptr ? 0 : effective_sink(sinks[h], windows[h], T);
}

}  // namespace

std::vector<WorkItem> plan_forward(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                                   int q_tile, int kv_tile, int n_queues) {
  const int n_qt = ceil_div(T, q_tile);
  const int G = H / H_kv;
  // One list per (b, key/value group): its G query heads' items, dealt to one queue together.
  std::vector<std::vector<Planned>> per_group(static_cast<size_t>(B) * H_kv);
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      const int W = effective_window(windows[h], T);
      const int S = head_sink(sinks, windows, h, T);
      const int32_t group = b * H_kv + h / G;
      auto& list = per_group[static_cast<size_t>(group)];
      for (int qt = 0; qt < n_qt; ++qt) {
        const int q0 = qt * q_tile;
        const int q1 = std::min(T, q0 + q_tile);
        const int key_first = std::max(0, q0 - W + 1);  // row q0's window start
        const int key_last = q1 - 1;                     // row q1-1's diagonal
        const WorkItem it{b * H + h, qt, key_first / kv_tile, key_last / kv_tile + 1};
        list.push_back(Planned{it, it.hi - it.lo + sink_tiles(S, it.lo, kv_tile), group});
      }
    }
  }
  return interleave(per_group, n_queues);
}

SplitPlan plan_forward_split(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                             int q_tile, int kv_tile, int n_queues, int chunk_tiles) {
  const int n_qt = ceil_div(T, q_tile);
  const int G = H / H_kv;
  SplitPlan plan;
  std::vector<std::vector<Planned>> per_group(static_cast<size_t>(B) * H_kv);
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      const int W = effective_window(windows[h], T);
      const int S = head_sink(sinks, windows, h, T);
      const int32_t group = b * H_kv + h / G;
      auto& list = per_group[static_cast<size_t>(group)];
      for (int qt = 0; qt < n_qt; ++qt) {
        const int q0 = qt * q_tile;
        const int q1 = std::min(T, q0 + q_tile);
        const int lo = std::max(0, q0 - W + 1) / kv_tile, hi = (q1 - 1) / kv_tile + 1;
        const int n = hi - lo;
        const int ns = sink_tiles(S, lo, kv_tile);  // visited by the item's first chunk only
        if (chunk_tiles < 1 || n <= chunk_tiles) {
          list.push_back(Planned{WorkItem{b * H + h, qt, lo, hi}, n + ns, group});
          continue;
        }
        const int n_chunks = ceil_div(n, chunk_tiles);
        plan.merges.push_back(WorkItem{b * H + h, qt, plan.n_slots, n_chunks});
        for (int c = 0; c < n_chunks; ++c) {
          // Near-equal chunks: the first n % n_chunks get one tile more.
          const int c_lo = lo + c * (n / n_chunks) + std::min(c, n % n_chunks);
          const int c_hi = c_lo + n / n_chunks + (c < n % n_chunks ? 1 : 0);
          list.push_back(
              Planned{WorkItem{b * H + h, qt, c_lo, c_hi}, c_hi - c_lo + (c == 0 ? ns : 0), group, plan.n_slots++});
        }
      }
    }
  }
  plan.items = interleave(per_group, n_queues, &plan.slot);
  return plan;
}

SplitPlan plan_backward_split(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                              int q_tile, int kv_tile, int n_queues, int chunk_tiles) {
  const int n_kt = ceil_div(T, kv_tile);
  const int G = H / H_kv;
  SplitPlan plan;
  std::vector<std::vector<Planned>> per_group(static_cast<size_t>(B) * H_kv);
  std::vector<int> hi_j(G);
  for (int b = 0; b < B; ++b) {
    for (int g = 0; g < H_kv; ++g) {
      const int32_t group = b * H_kv + g;
      auto& list = per_group[static_cast<size_t>(group)];
      for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * kv_tile, k1 = std::min(T, k0 + kv_tile);
        // The group's query heads share the first query tile; each ends at its own.  Steps: query tiles
        // summed over the heads.
        int lo = 0, hi = 0, n = 0;
        for (int j = 0; j < G; ++j) {
          const int h = g * G + j;
          query_range(k0, k1, effective_window(windows[h], T), head_sink(sinks, windows, h, T), T, q_tile, &lo,
                      &hi_j[j]);
          hi = std::max(hi, hi_j[j]);
          n += hi_j[j] - lo;
        }
        if (chunk_tiles < 1 || n <= chunk_tiles) {
          list.push_back(Planned{WorkItem{group, kt, lo, hi}, n, group});
          continue;
        }
        // Chunks are query-tile ranges [c_lo, c_hi) of [lo, hi), each running every head of the group over
        // its part of the range; the cuts fall where the steps before them first reach c n / n_chunks.
        const int n_chunks = ceil_div(n, chunk_tiles);
        plan.merges.push_back(WorkItem{group, kt, plan.n_slots, n_chunks});
        int c_lo = lo, steps = 0;  // steps of the tiles before c_lo
        for (int c = 0; c < n_chunks; ++c) {
          int c_hi = c_lo, c_steps = 0;
          const int64_t target = static_cast<int64_t>(c + 1) * n / n_chunks;
          while (c_hi < hi && (c == n_chunks - 1 || steps + c_steps < target || c_hi == c_lo)) {
            for (int j = 0; j < G; ++j) c_steps += c_hi < hi_j[j] ? 1 : 0;
            ++c_hi;
          }
          if (c_hi == c_lo) break;  // fewer distinct tiles than chunks (cannot happen with one head per group)
          list.push_back(Planned{WorkItem{group, kt, c_lo, c_hi}, c_steps, group, plan.n_slots++});
          steps += c_steps;
          c_lo = c_hi;
        }
        plan.merges.back().hi = plan.n_slots - plan.merges.back().lo;
      }
    }
  }
  plan.items = interleave(per_group, n_queues, &plan.slot);
  return plan;
}

std::vector<WorkItem> plan_backward(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                                    int q_tile, int kv_tile, int n_queues) {
  const int n_kt = ceil_div(T, kv_tile);
  const int G = H / H_kv;
  std::vector<std::vector<Planned>> per_group(static_cast<size_t>(B) * H_kv);
  for (int b = 0; b < B; ++b) {
    for (int g = 0; g < H_kv; ++g) {
      const int32_t group = b * H_kv + g;
      auto& list = per_group[static_cast<size_t>(group)];
      list.reserve(n_kt);
      for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * kv_tile;
        const int k1 = std::min(T, k0 + kv_tile);
        int lo = 0, hi = 0, cost = 0;
        for (int j = 0; j < G; ++j) {  // the group's query heads, each over its own range
          const int h = g * G + j;
          int lo_j = 0, hi_j = 0;
          query_range(k0, k1, effective_window(windows[h], T), head_sink(sinks, windows, h, T), T, q_tile, &lo_j,
                      &hi_j);
          lo = lo_j;
          hi = std::max(hi, hi_j);
          cost += hi_j - lo_j;
        }
        list.push_back(Planned{WorkItem{group, kt, lo, hi}, cost, group});
      }
    }
  }
  return interleave(per_group, n_queues);
}

}  // namespace aah
