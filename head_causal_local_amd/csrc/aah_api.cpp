// C ABI of the per-head causal local-window attention library: argument
// validation (always before the first HIP call), the device work-list cache,
// and kernel dispatch.  Contracts are documented in include/aah_attn.h.
#include "aah_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <tuple>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "plan_cache.hpp"
#include "workplan.hpp"

namespace {

using aah::WorkItem;

thread_local std::string g_detail;

aah_status fail(aah_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
aah_status fail(aah_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_detail = buf;
  return st;
}

aah_status hip_fail(hipError_t e, const char* what) {
  return fail(AAH_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool supported_d(int d) { return d == 32 || d == 64 || d == 128; }

#define AAH_TRY_INNER(expr)           \
  do {                                \
    const aah_status st_ = (expr);    \
    if (st_ != AAH_OK) return st_;    \
  } while (0)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

aah_status check_dims(int B, int H, int T, int d, aah_dtype dt);

aah_status check_windows(const int32_t* windows, const int32_t* sinks, int H) {
  if (windows == nullptr) return fail(AAH_ERR_INVALID_ARG, "windows is NULL");
  for (int h = 0; h < H; ++h)
    if (windows[h] < 1) return fail(AAH_ERR_INVALID_ARG, "windows[%d] = %d; every window must be >= 1", h, windows[h]);
  if (sinks != nullptr)
    for (int h = 0; h < H; ++h)
      if (sinks[h] < 0) return fail(AAH_ERR_INVALID_ARG, "sinks[%d] = %d; every sink size must be >= 0", h, sinks[h]);
  return AAH_OK;
}

aah_status check_kv_heads(int H, int H_kv) {
  if (H_kv < 1 || H_kv > H || H % H_kv != 0)
    return fail(AAH_ERR_INVALID_ARG, "H_kv = %d must divide H = %d (1 <= H_kv <= H)", H_kv, H);
  return AAH_OK;
}

// Shape checks shared by every entry point that takes windows (and sink sizes, may be NULL).
aah_status check_shape(const int32_t* windows, const int32_t* sinks, int B, int H, int T, int d, aah_dtype dt,
                       int H_kv = -1) {
  if (windows == nullptr) return fail(AAH_ERR_INVALID_ARG, "windows is NULL");
  AAH_TRY_INNER(check_dims(B, H, T, d, dt));
  AAH_TRY_INNER(check_kv_heads(H, H_kv < 0 ? H : H_kv));
  return check_windows(windows, sinks, H);
}

aah_status check_dims(int B, int H, int T, int d, aah_dtype dt) {
  if (B < 0 || H < 1 || T < 0)
    return fail(AAH_ERR_INVALID_ARG, "B, T must be >= 0 and H >= 1 (got B = %d, H = %d, T = %d)", B, H, T);
  if (static_cast<int64_t>(B) * H > INT32_MAX / 2)
    return fail(AAH_ERR_INVALID_ARG, "B * H = %lld is too large", static_cast<long long>(B) * H);
  if (T > (1 << 28)) return fail(AAH_ERR_INVALID_ARG, "T = %d is too large", T);
  if (d < 1) return fail(AAH_ERR_INVALID_ARG, "d must be >= 1 (got %d)", d);
  if (dt != AAH_BF16 && dt != AAH_F32) return fail(AAH_ERR_UNSUPPORTED, "unknown dtype %d", static_cast<int>(dt));
  if (!supported_d(d)) return fail(AAH_ERR_UNSUPPORTED, "head dim %d has no kernel (supported: 32, 64, 128)", d);
  // Kernels address one head's [T, d] slice with 32-bit buffer offsets.
  if (static_cast<int64_t>(T) * d * 4 >= (int64_t{1} << 31))
    return fail(AAH_ERR_UNSUPPORTED, "T * d = %lld is too large for one head slice", static_cast<long long>(T) * d);
  return AAH_OK;
}

// No batch entries or no tokens: nothing to compute.  Such a call checks its other arguments and returns
// AAH_OK without touching any tensor (they may be NULL: an empty tensor has no storage).
bool empty_problem(int B, int T) { return B == 0 || T == 0; }

aah_status check_tensor(const void* p, const char* name, size_t align) {
  if (p == nullptr) return fail(AAH_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(AAH_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return AAH_OK;
}

#define AAH_TRY(expr)                 \
  do {                                \
    const aah_status st_ = (expr);    \
    if (st_ != AAH_OK) return st_;    \
  } while (0)

// ------------------------------------------------------------------ device copies of work lists
//
// A work list reaches the device without synchronising it: its arrays are
// packed into a ring of pinned host memory (one per device, allocated on
// first use), a stream-ordered allocation (hipMallocAsync) receives them by
// hipMemcpyAsync on the caller's stream, and an event marks the copy's end.
// A later call on another stream waits for that event before its kernels read
// the list.  A list evicted from its cache is released by hipFreeAsync on the
// stream of the call that evicts it.  Lists larger than the ring (over a
// quarter of a million work items) take the old path: hipMalloc and a
// blocking hipMemcpy, and hipFree on release.

struct DeviceBlob {
  char* dev = nullptr;
  hipEvent_t ready = nullptr;   // recorded on `stream` after the copy
  hipStream_t stream = nullptr;
  bool async = true;            // allocated with hipMallocAsync (else hipMalloc)
};

constexpr size_t kStagingBytes = size_t{4} << 20;  // pinned staging ring per device

struct Staging {
  char* host = nullptr;
  size_t head = 0;
  struct Region {
    size_t begin, end;
    hipEvent_t done;  // recorded after the copy out of [begin, end)
  };
  std::vector<Region> inflight;
};

std::mutex g_mu;  // guards every cache and the staging rings
std::map<int, Staging> g_staging;

size_t round_up256(size_t x) { return (x + 255) / 256 * 256; }

bool stream_capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) return false;
  return st != hipStreamCaptureStatusNone;
}

// Copies parts[i] (host pointer, bytes) to one device allocation, part i at (*offsets)[i] (256-byte
// aligned), ordered on `stream`.  Called with g_mu held.
aah_status upload_blob(int dev, const std::vector<std::pair<const void*, size_t>>& parts, hipStream_t stream,
                       DeviceBlob* out, std::vector<size_t>* offsets) {
  size_t total = 0;
  offsets->clear();
  for (const auto& p : parts) {
    offsets->push_back(total);
    total += round_up256(std::max<size_t>(p.second, 1));
  }
  DeviceBlob b;
  b.stream = stream;
  hipError_t e = hipEventCreateWithFlags(&b.ready, hipEventDisableTiming);
  if (e != hipSuccess) return hip_fail(e, "hipEventCreate(work list)");
  auto fail_blob = [&](hipError_t err, const char* what) {
    if (b.dev != nullptr) (void)(b.async ? hipFreeAsync(b.dev, stream) : hipFree(b.dev));
    (void)hipEventDestroy(b.ready);
    return hip_fail(err, what);
  };
  if (total > kStagingBytes) {
    b.async = false;
    e = hipMalloc(reinterpret_cast<void**>(&b.dev), total);
    if (e != hipSuccess) return fail_blob(e, "hipMalloc(work list)");
    for (size_t i = 0; i < parts.size() && e == hipSuccess; ++i)
      e = hipMemcpy(b.dev + (*offsets)[i], parts[i].first, parts[i].second, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipEventRecord(b.ready, stream);
    if (e != hipSuccess) return fail_blob(e, "hipMemcpy(work list)");
    *out = b;
    return AAH_OK;
  }
  Staging& sg = g_staging[dev];
  if (sg.host == nullptr) {
    e = hipHostMalloc(reinterpret_cast<void**>(&sg.host), kStagingBytes, hipHostMallocDefault);
    if (e != hipSuccess) {
      sg.host = nullptr;
      return fail_blob(e, "hipHostMalloc(staging)");
    }
  }
  if (sg.head + total > kStagingBytes) sg.head = 0;
  const size_t begin = sg.head, end = begin + total;
  // Regions this one overlaps must have been copied out (in practice long ago).
  for (size_t i = 0; i < sg.inflight.size();) {
    const Staging::Region& r = sg.inflight[i];
    if (r.begin < end && begin < r.end) {
      e = hipEventSynchronize(r.done);
      (void)hipEventDestroy(r.done);
      if (e != hipSuccess) return fail_blob(e, "hipEventSynchronize(staging)");
      sg.inflight.erase(sg.inflight.begin() + static_cast<std::ptrdiff_t>(i));
    } else {
      ++i;
    }
  }
  for (size_t i = 0; i < parts.size(); ++i) std::memcpy(sg.host + begin + (*offsets)[i], parts[i].first, parts[i].second);
  hipEvent_t done = nullptr;
  e = hipEventCreateWithFlags(&done, hipEventDisableTiming);
  if (e != hipSuccess) return fail_blob(e, "hipEventCreate(staging)");
  e = hipMallocAsync(reinterpret_cast<void**>(&b.dev), total, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(b.dev, sg.host + begin, total, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipEventRecord(done, stream);
  if (e == hipSuccess) e = hipEventRecord(b.ready, stream);
  if (e != hipSuccess) {
    // Nothing may reuse the region before the device is done with it.
    (void)hipEventSynchronize(done);
    (void)hipEventDestroy(done);
    return fail_blob(e, "hipMallocAsync / hipMemcpyAsync(work list)");
  }
  sg.inflight.push_back(Staging::Region{begin, end, done});
  sg.head = end;
  *out = b;
  return AAH_OK;
}

// Releases a list evicted by a call on `stream` (in that stream's order).
void release_blob(DeviceBlob& b, hipStream_t stream) {
  if (b.dev != nullptr) (void)(b.async ? hipFreeAsync(b.dev, stream) : hipFree(b.dev));
  if (b.ready != nullptr) (void)hipEventDestroy(b.ready);
  b = DeviceBlob{};
}

// Before a call on `stream` uses a cached list: order it after the list's copy when that copy went out on
// another stream.  Under graph capture no wait on an outside event is recorded; the copy must be done.
aah_status order_after_upload(const DeviceBlob& b, hipStream_t stream, bool capturing) {
  if (b.stream == stream) return AAH_OK;
  if (capturing) {
    const hipError_t q = hipEventQuery(b.ready);
    if (q == hipSuccess) return AAH_OK;
    return fail(AAH_ERR_UNSUPPORTED,
                "the work list for these windows is still being copied on another stream; synchronise it before "
                "capturing a graph that uses it");
  }
  const hipError_t e = hipStreamWaitEvent(stream, b.ready, 0);
  return e == hipSuccess ? AAH_OK : hip_fail(e, "hipStreamWaitEvent(work list)");
}

// Looks key up in cache under g_mu: on a hit copies the entry to *out (pinning it when the stream is
// capturing a graph, which will refer to it for good) and returns true.  A miss during capture is an
// error (status in *st): building and uploading a list there would record the upload into the graph.
template <class V>
bool cache_lookup(aah::PlanLru<V>& cache, const std::vector<int64_t>& key, hipStream_t stream, bool capturing,
                  V* out, aah_status* st) {
  V* hit = cache.find(key);
  *st = AAH_OK;
  if (hit == nullptr) {
    if (capturing)
      *st = fail(AAH_ERR_UNSUPPORTED,
                 "no cached work list for these windows and shape: run the same call once outside graph capture");
    return capturing;
  }
  if (capturing) cache.pin(key);
  *st = order_after_upload(hit->blob, stream, capturing);
  if (*st == AAH_OK) *out = *hit;
  return true;
}

template <class V>
void cache_insert(aah::PlanLru<V>& cache, std::vector<int64_t> key, const V& value, hipStream_t stream) {
  for (V& old : cache.insert(std::move(key), value)) release_blob(old.blob, stream);
}

// Work lists kept per cache (forward / backward lists, split lists, decoding plans): enough for the
// layers of a model whose windows change at every control update, bounded for any run.
constexpr size_t kCacheCapacity = 64;

// ------------------------------------------------------------------ plan cache

struct DevicePlan {
  DeviceBlob blob;
  WorkItem* items = nullptr;
  int n_items = 0;
  int32_t* win = nullptr;   // effective windows int32[H], then effective sink sizes int32[H]
  const int32_t* sink = nullptr;  // win + H if some head has a sink, else NULL (the kernels without sinks)
};

enum PlanKind : int64_t { kPlanFwd = 0, kPlanBwd = 1 };

aah::PlanLru<DevicePlan> g_cache(kCacheCapacity);

constexpr int kQueues = 8;  // MI355X has eight XCDs; workgroups are placed round-robin over them

aah_status get_plan(PlanKind kind, const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                    int row_tile, int col_tile, hipStream_t stream, DevicePlan* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::vector<int32_t> win(2 * H);
  bool any_sink = false;
  for (int h = 0; h < H; ++h) {
    win[h] = aah::effective_window(windows[h], T);
    win[H + h] = sinks == nullptr ? 0 : aah::effective_sink(sinks[h], windows[h], T);
    any_sink = any_sink || win[H + h] > 0;
  }
  // Heads whose sinks change nothing plan (and run) exactly as without sinks.
  const int32_t* sink_arg = any_sink ? win.data() + H : nullptr;
  std::vector<int64_t> key = {kind, dev, B, H, H_kv, T, row_tile, col_tile, kQueues, any_sink ? 1 : 0};
  key.insert(key.end(), win.begin(), win.end());

  const bool capturing = stream_capturing(stream);
  std::lock_guard<std::mutex> lock(g_mu);
  aah_status st;
  if (cache_lookup(g_cache, key, stream, capturing, out, &st)) return st;
  // Forward: row tile = query rows per item, col tile = keys per step.
  // Backward: row tile = keys per item, col tile = query rows per step.
  const std::vector<WorkItem> items =
      kind == kPlanFwd ? aah::plan_forward(windows, sink_arg, B, H, H_kv, T, row_tile, col_tile, kQueues)
                       : aah::plan_backward(windows, sink_arg, B, H, H_kv, T, col_tile, row_tile, kQueues);

  DevicePlan p;
  p.n_items = static_cast<int>(items.size());
  std::vector<size_t> off;
  AAH_TRY_INNER(upload_blob(dev, {{items.data(), items.size() * sizeof(WorkItem)}, {win.data(), win.size() * sizeof(int32_t)}},
                            stream, &p.blob, &off));
  p.items = reinterpret_cast<WorkItem*>(p.blob.dev + off[0]);
  p.win = reinterpret_cast<int32_t*>(p.blob.dev + off[1]);
  p.sink = any_sink ? p.win + H : nullptr;
  cache_insert(g_cache, std::move(key), p, stream);
  *out = p;
  return AAH_OK;
}

void fwd_tiles(aah_dtype dt, int* row, int* col) {
  if (dt == AAH_BF16) {
    *row = aah::kFwdBf16RowTile;
    *col = aah::kFwdBf16ColTile;
  } else {
    *row = aah::kSimpleRowTile;
    *col = aah::kSimpleColTile;
  }
}

void bwd_tiles(aah_dtype dt, int* row, int* col) {
  if (dt == AAH_BF16) {
    *row = aah::kBwdBf16RowTile;
    *col = aah::kBwdBf16ColTile;
  } else {
    *row = aah::kSimpleRowTile;
    *col = aah::kSimpleColTile;
  }
}

// ------------------------------------------------------------------ split forward
//
// A bf16 forward whose longest items hold more key tiles than a resident
// workgroup's share of the whole launch (few items: one sequence, few heads; or
// items of very unequal length) takes the time of those items while the rest of
// the device idles.  Then every item longer than L key tiles is split into
// chunks of at most L tiles (plan_forward_split), L = max(kMinChunkTiles, total
// tiles / resident workgroups), so that no chunk exceeds that share; a merge
// launch combines each split item's chunks.  The chunks' partial results live in
// the caller's workspace (aah_attn_fwd_workspace_size).

// Does some head keep sink keys that change its mask (an effective sink size above 0)?
bool any_sink(const int32_t* windows, const int32_t* sinks, int H, int T) {
  if (sinks == nullptr) return false;
  for (int h = 0; h < H; ++h)
    if (aah::effective_sink(sinks[h], windows[h], T) > 0) return true;
  return false;
}

// Shortest chunk.  Each chunk adds a partial result (128 rows x (d + 2) fp32) that the merge reads back,
// so short chunks cost traffic; on the single layer B=1 H=16 T=4096 d=64 minimums of 8 / 12 / 16 / 24 / 32
// tiles measured 366 / 379 / 380 / 415 / 397 TFLOP/s.
constexpr int kMinChunkTiles = 24;

// Resident workgroups of the plain bf16 forward on the current device (occupancy query cached per device and d).
int resident_workgroups(int d) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::mutex mu;
  static std::map<std::pair<int, int>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto found = cache.find({dev, d});
  if (found != cache.end()) return found->second;
  const int n = aah::fwd_bf16_resident(d);
  if (n > 0) cache.emplace(std::make_pair(dev, d), n);
  return n;
}

// Chunk length for a bf16 forward (items cut along their window tiles; an item's sink tiles go with its first
// chunk and count in the total), or 0 when splitting does not apply.
int split_chunk_tiles(const int32_t* windows, const int32_t* sinks, int B, int H, int T, int d) {
  const int q_tile = aah::kFwdBf16RowTile, kv_tile = aah::kFwdBf16ColTile;
  const int n_qt = (T + q_tile - 1) / q_tile;
  const int64_t n_items = static_cast<int64_t>(B) * H * n_qt;
  const int resident = resident_workgroups(d);
  if (resident <= 0 || n_items == 0) return 0;
  int64_t total = 0;
  int longest = 0;
  for (int h = 0; h < H; ++h) {
    const int W = aah::effective_window(windows[h], T);
    const int S = sinks == nullptr ? 0 : aah::effective_sink(sinks[h], windows[h], T);
    for (int qt = 0; qt < n_qt; ++qt) {
      const int q0 = qt * q_tile, q1 = std::min(T, q0 + q_tile);
      const int lo = std::max(0, q0 - W + 1) / kv_tile;
      const int n = (q1 - 1) / kv_tile + 1 - lo;
      total += n + aah::sink_tiles(S, lo, kv_tile);
      longest = std::max(longest, n);
    }
  }
  total *= B;
  const int L = static_cast<int>(std::max<int64_t>(kMinChunkTiles, (total + resident - 1) / resident));
  return longest > L ? L : 0;
}

struct SplitDevicePlan {
  DeviceBlob blob;
  WorkItem* items = nullptr;
  int32_t* slots = nullptr;
  WorkItem* merges = nullptr;
  int32_t* win = nullptr;
  int32_t* sink = nullptr;  // effective sink sizes, or nullptr when no head has one
  int n_items = 0, n_merges = 0, n_slots = 0;
};
aah::PlanLru<SplitDevicePlan> g_split_cache(kCacheCapacity);

// Partial-result bytes of a split plan: accumulators, then (max, sum) pairs, each 256-byte aligned.
size_t split_acc_bytes(int n_slots, int d) {
  return round_up(static_cast<size_t>(n_slots) * aah::kFwdBf16RowTile * d * sizeof(float), 256);
}
size_t split_workspace(int n_slots, int d, bool diag = false) {
  return split_acc_bytes(n_slots, d) +
         round_up(static_cast<size_t>(n_slots) * aah::kFwdBf16RowTile * (diag ? aah::kMlDiag : 2) * sizeof(float),
                  256);
}

// Split plan with chunk length L (> 0), uploaded once per key.  kind 0: query-stationary items (forward,
// dQ); kind 1: key-stationary items (dK/dV).
aah_status get_split_plan(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T, int d, int L,
                          hipStream_t stream, SplitDevicePlan* out, int kind = 0) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  const bool has_sink = any_sink(windows, sinks, H, T);
  std::vector<int32_t> win(H), sink(H, 0);
  for (int h = 0; h < H; ++h) {
    win[h] = aah::effective_window(windows[h], T);
    if (has_sink) sink[h] = aah::effective_sink(sinks[h], windows[h], T);
  }
  std::vector<int64_t> key = {kind, dev, B, H, H_kv, T, d, L, has_sink ? 1 : 0};
  key.insert(key.end(), win.begin(), win.end());
  if (has_sink) key.insert(key.end(), sink.begin(), sink.end());
  const bool capturing = stream_capturing(stream);
  std::lock_guard<std::mutex> lock(g_mu);
  aah_status st;
  if (cache_lookup(g_split_cache, key, stream, capturing, out, &st)) return st;
  const aah::SplitPlan sp =
      kind == 0 ? aah::plan_forward_split(windows, sinks, B, H, H_kv, T, aah::kFwdBf16RowTile, aah::kFwdBf16ColTile,
                                          kQueues, L)
                : aah::plan_backward_split(windows, sinks, B, H, H_kv, T, aah::kBwdBf16ColTile, aah::kBwdBf16RowTile,
                                           kQueues, L);
  SplitDevicePlan p;
  p.n_items = static_cast<int>(sp.items.size());
  p.n_merges = static_cast<int>(sp.merges.size());
  p.n_slots = sp.n_slots;
  std::vector<size_t> off;
  AAH_TRY_INNER(upload_blob(dev,
                            {{sp.items.data(), sp.items.size() * sizeof(WorkItem)},
                             {sp.slot.data(), sp.slot.size() * sizeof(int32_t)},
                             {sp.merges.data(), sp.merges.size() * sizeof(WorkItem)},
                             {win.data(), win.size() * sizeof(int32_t)},
                             {sink.data(), sink.size() * sizeof(int32_t)}},
                            stream, &p.blob, &off));
  p.items = reinterpret_cast<WorkItem*>(p.blob.dev + off[0]);
  p.slots = reinterpret_cast<int32_t*>(p.blob.dev + off[1]);
  p.merges = reinterpret_cast<WorkItem*>(p.blob.dev + off[2]);
  p.win = reinterpret_cast<int32_t*>(p.blob.dev + off[3]);
  p.sink = has_sink ? reinterpret_cast<int32_t*>(p.blob.dev + off[4]) : nullptr;
  cache_insert(g_split_cache, std::move(key), p, stream);
  *out = p;
  return AAH_OK;
}

// Split backward: the same rule per kernel, with that kernel's residency and items (dQ: the forward's
// query items; dK/dV: key items over their query-tile ranges).
int resident_bwd(bool dkdv, int d) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::mutex mu;
  static std::map<std::tuple<int, int, int>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(dev, d, dkdv ? 1 : 0);
  auto found = cache.find(key);
  if (found != cache.end()) return found->second;
  const int n = dkdv ? aah::bwd_dkdv_resident(d) : aah::bwd_dq_resident(d);
  if (n > 0) cache.emplace(key, n);
  return n;
}

int chunk_len(const std::vector<int>& tiles, int resident) {
  if (resident <= 0 || tiles.empty()) return 0;
  int64_t total = 0;
  int longest = 0;
  for (int t : tiles) {
    total += t;
    longest = std::max(longest, t);
  }
  const int L = static_cast<int>(std::max<int64_t>(kMinChunkTiles, (total + resident - 1) / resident));
  return longest > L ? L : 0;
}

// Streamed tiles of every dQ item (query tile: its window's key tiles and the sink tiles before them) or
// dK/dV item (key tile of a key/value head: query tiles summed over the group's query heads).
std::vector<int> bwd_item_tiles(bool dkdv, const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv,
                                int T) {
  std::vector<int> tiles;
  const int rt = dkdv ? aah::kBwdBf16RowTile : aah::kFwdBf16RowTile;
  const int ct = dkdv ? aah::kBwdBf16ColTile : aah::kFwdBf16ColTile;
  const int n_rt = (T + rt - 1) / rt;
  const int G = H / H_kv;
  auto sink_of = [&](int h) { return sinks == nullptr ? 0 : aah::effective_sink(sinks[h], windows[h], T); };
  for (int b = 0; b < B; ++b) {
    if (dkdv) {
      for (int g = 0; g < H_kv; ++g)
        for (int t = 0; t < n_rt; ++t) {
          const int r0 = t * rt, r1 = std::min(T, r0 + rt);
          int steps = 0;
          for (int h = g * G; h < (g + 1) * G; ++h) {
            int lo = 0, hi = 0;
            aah::query_range(r0, r1, aah::effective_window(windows[h], T), sink_of(h), T, ct, &lo, &hi);
            steps += hi - lo;
          }
          tiles.push_back(steps);
        }
    } else {
      for (int h = 0; h < H; ++h) {
        const int W = aah::effective_window(windows[h], T);
        for (int t = 0; t < n_rt; ++t) {
          const int r0 = t * rt, r1 = std::min(T, r0 + rt);
          const int lo = std::max(0, r0 - W + 1) / ct;
          tiles.push_back((r1 - 1) / ct + 1 - lo + aah::sink_tiles(sink_of(h), lo, ct));
        }
      }
    }
  }
  return tiles;
}

struct BwdSplitLayout {
  SplitDevicePlan q, k;  // dQ and dK/dV split plans (n_slots = 0 when that kernel does not split)
  int q_L = 0, k_L = 0;
  size_t q_off = 0, k_off = 0, total = 0;  // byte offsets of the partials in the workspace, and its size
};

// Layout of a split backward's workspace: [nl2 | nD | dQ partials | dK/dV partials].  Returns false when
// splitting does not apply (dtype, enough items, or a failed plan upload).
bool bwd_split_layout(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T, int d,
                      aah_dtype dt, hipStream_t stream, BwdSplitLayout* lay) {
  if (dt != AAH_BF16) return false;
  lay->q_L = chunk_len(bwd_item_tiles(false, windows, sinks, B, H, H_kv, T), resident_bwd(false, d));
  lay->k_L = chunk_len(bwd_item_tiles(true, windows, sinks, B, H, H_kv, T), resident_bwd(true, d));
  if (lay->q_L == 0 && lay->k_L == 0) return false;
  if (lay->q_L > 0 && get_split_plan(windows, sinks, B, H, H_kv, T, d, lay->q_L, stream, &lay->q, 0) != AAH_OK)
    return false;
  if (lay->k_L > 0 && get_split_plan(windows, sinks, B, H, H_kv, T, d, lay->k_L, stream, &lay->k, 1) != AAH_OK)
    return false;
  const size_t rows = static_cast<size_t>(aah::kBwdBf16RowTile) * d * sizeof(float);
  lay->q_off = 2 * round_up(static_cast<size_t>(B) * H * T * sizeof(float), 256);
  lay->k_off = lay->q_off + round_up(static_cast<size_t>(lay->q_L > 0 ? lay->q.n_slots : 0) * rows, 256);
  lay->total = lay->k_off + round_up(static_cast<size_t>(lay->k_L > 0 ? lay->k.n_slots : 0) * 2 * rows, 256);
  return true;
}

// Workspace of the backward: nl2 = -lse log2(e) and nD = -D, fp32 [B,H,T]
// each, every array starting on a 256-byte boundary.
size_t bwd_array_bytes(int B, int H, int T) { return round_up(static_cast<size_t>(B) * H * T * sizeof(float), 256); }
size_t bwd_workspace(int B, int H, int T, int /*d*/, aah_dtype /*dt*/) { return 2 * bwd_array_bytes(B, H, T); }
const float* ws_nl2(const void* ws) { return static_cast<const float*>(ws); }
const float* ws_nd(const void* ws, int B, int H, int T) {
  return reinterpret_cast<const float*>(static_cast<const char*>(ws) + bwd_array_bytes(B, H, T));
}

aah_status check_workspace(const void* workspace, size_t workspace_bytes, int B, int H, int T, int d, aah_dtype dt) {
  const size_t need = bwd_workspace(B, H, T, d, dt);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(AAH_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace == nullptr ? 0 : workspace_bytes,
                need);
  if (!aligned(workspace, 256)) return fail(AAH_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  return AAH_OK;
}

// ------------------------------------------------------------------ decode plans

struct DecodePlan {
  DeviceBlob blob;
  aah::DecodeChunk* chunks = nullptr;
  // kv_off[H_kv], kv_sink[H_kv], kv_ring[H_kv], kv_first[H_kv + 1], q_cap[H], q_sink[H]
  int32_t* tables = nullptr;
  std::vector<int32_t> host_sink, host_ring;
  int n_chunks = 0;
  int rows = 0;
  int H = 0, H_kv = 0;
  aah::DecodePlanView view() const {
    const int32_t* t = tables;
    return aah::DecodePlanView{chunks,         n_chunks,         t,    t + H_kv, t + 2 * H_kv, t + 3 * H_kv,
                               t + 4 * H_kv + 1, t + 4 * H_kv + 1 + H, rows, H, H_kv, host_sink.data(),
                               host_ring.data()};
  }
};

aah::PlanLru<DecodePlan> g_decode_cache(kCacheCapacity);

// Per query head: C_h = min(W_h, T_max) and the effective sink min(S_h, T_max - C_h) (sinks past it are
// always inside the window); per key/value head: the largest of each over its query heads.
struct DecodeShape {
  std::vector<int64_t> cap, sink;  // per query head
  std::vector<int64_t> ring, ksink;  // per key/value head
  int64_t rows = 0, chunks = 0;
};

DecodeShape decode_shape(const int32_t* windows, const int32_t* sinks, int H, int H_kv, int T_max) {
  DecodeShape s;
  const int G = H / H_kv;
  s.cap.resize(H);
  s.sink.resize(H);
  s.ring.assign(H_kv, 0);
  s.ksink.assign(H_kv, 0);
  for (int h = 0; h < H; ++h) {
    s.cap[h] = std::min<int64_t>(windows[h], T_max);
    const int64_t sk = sinks == nullptr ? 0 : sinks[h];
    s.sink[h] = std::max<int64_t>(0, std::min<int64_t>(sk, T_max - s.cap[h]));
    s.ring[h / G] = std::max(s.ring[h / G], s.cap[h]);
    s.ksink[h / G] = std::max(s.ksink[h / G], s.sink[h]);
  }
  const int cr = aah::decode_chunk_rows(H, H_kv);
  for (int g = 0; g < H_kv; ++g) {
    s.rows += s.ksink[g] + s.ring[g];
    s.chunks += (s.ksink[g] + s.ring[g] + cr - 1) / cr;
  }
  return s;
}

// Rows R of one batch entry's cache; -1 if it does not fit in int32.
int64_t decode_rows(const int32_t* windows, const int32_t* sinks, int H, int H_kv, int T_max) {
  const int64_t r = decode_shape(windows, sinks, H, H_kv, T_max).rows;
  return r > INT32_MAX ? -1 : r;
}

aah_status get_decode_plan(const int32_t* windows, const int32_t* sinks, int H, int H_kv, int T_max,
                           hipStream_t stream, DecodePlan* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  const DecodeShape sh = decode_shape(windows, sinks, H, H_kv, T_max);
  std::vector<int64_t> key = {dev, H, H_kv, T_max};
  key.insert(key.end(), sh.cap.begin(), sh.cap.end());
  key.insert(key.end(), sh.sink.begin(), sh.sink.end());
  const bool capturing = stream_capturing(stream);
  std::lock_guard<std::mutex> lock(g_mu);
  aah_status st;
  if (cache_lookup(g_decode_cache, key, stream, capturing, out, &st)) return st;
  DecodePlan p;
  p.H = H;
  p.H_kv = H_kv;
  std::vector<int32_t> tables(4 * H_kv + 1 + 2 * H);
  std::vector<aah::DecodeChunk> chunks;
  int32_t off = 0;
  const int G = H / H_kv;
  const int cr = aah::decode_chunk_rows(H, H_kv);
  for (int g = 0; g < H_kv; ++g) {
    const int32_t n = static_cast<int32_t>(sh.ksink[g] + sh.ring[g]);
    const int32_t first = static_cast<int32_t>(chunks.size());
    const int32_t count = (n + cr - 1) / cr;
    int64_t cap_s = INT64_MAX;
    for (int j = 0; j < G; ++j)
      if (sh.sink[g * G + j] > 0) cap_s = std::min(cap_s, sh.cap[g * G + j]);
    if (cap_s == INT64_MAX) cap_s = 1;  // no query head of g has sink keys (then S_g = 0): any positive value
    tables[g] = off;
    tables[H_kv + g] = static_cast<int32_t>(sh.ksink[g]);
    tables[2 * H_kv + g] = static_cast<int32_t>(sh.ring[g]);
    tables[3 * H_kv + g] = first;
    for (int32_t r0 = 0; r0 < n; r0 += cr)
      chunks.push_back(aah::DecodeChunk{g, r0, static_cast<int32_t>(sh.ksink[g]), static_cast<int32_t>(sh.ring[g]), off,
                                        first, count, static_cast<int32_t>(cap_s)});
    off += n;
  }
  tables[4 * H_kv] = static_cast<int32_t>(chunks.size());
  for (int h = 0; h < H; ++h) {
    tables[4 * H_kv + 1 + h] = static_cast<int32_t>(sh.cap[h]);
    tables[4 * H_kv + 1 + H + h] = static_cast<int32_t>(sh.sink[h]);
  }
  p.rows = off;
  p.n_chunks = static_cast<int>(chunks.size());
  p.host_sink.assign(tables.begin() + H_kv, tables.begin() + 2 * H_kv);
  p.host_ring.assign(tables.begin() + 2 * H_kv, tables.begin() + 3 * H_kv);
  std::vector<size_t> at;
  AAH_TRY_INNER(upload_blob(dev,
                            {{chunks.data(), chunks.size() * sizeof(aah::DecodeChunk)},
                             {tables.data(), tables.size() * sizeof(int32_t)}},
                            stream, &p.blob, &at));
  p.chunks = reinterpret_cast<aah::DecodeChunk*>(p.blob.dev + at[0]);
  p.tables = reinterpret_cast<int32_t*>(p.blob.dev + at[1]);
  cache_insert(g_decode_cache, std::move(key), p, stream);
  *out = std::move(p);
  return AAH_OK;
}

// Decode workspace: B*H_kv int32 merge counters (256-byte rounded), then the partials: one per
// (batch entry, chunk, query head of the chunk's group).
size_t decode_counter_bytes(int B, int H_kv) { return round_up(static_cast<size_t>(B) * H_kv * sizeof(int32_t), 256); }
size_t decode_workspace(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T_max, int d) {
  const DecodeShape sh = decode_shape(windows, sinks, H, H_kv, T_max);
  return decode_counter_bytes(B, H_kv) +
         round_up(static_cast<size_t>(B) * sh.chunks * (H / H_kv) * (2 + d) * sizeof(float), 256);
}

// Checks shared by the decode entry points (bf16 only; T_max plays the role of T).
aah_status check_decode(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T_max, int d,
                        aah_dtype dt) {
  AAH_TRY_INNER(check_shape(windows, sinks, B, H, T_max, d, dt, H_kv));
  if (T_max < 1) return fail(AAH_ERR_INVALID_ARG, "T_max must be >= 1 (got %d)", T_max);
  if (dt != AAH_BF16) return fail(AAH_ERR_UNSUPPORTED, "decoding runs on bf16 caches only");
  const int64_t rows = decode_rows(windows, sinks, H, H_kv, T_max);
  if (rows < 0) return fail(AAH_ERR_UNSUPPORTED, "cache rows per batch entry exceed 2^31");
  // The decode and cache-fill launches put B (and B * H_kv) on the second grid dimension.
  if (static_cast<int64_t>(B) * H_kv > 65535)
    return fail(AAH_ERR_UNSUPPORTED, "B * H_kv = %lld exceeds 65535", static_cast<long long>(B) * H_kv);
  if (static_cast<int64_t>(B) * rows * d >= (int64_t{1} << 40)) return fail(AAH_ERR_UNSUPPORTED, "cache too large");
  // The kernel reads a batch entry's query rows and a key/value head's region (under 2 T_max rows, so
  // under 2^31 bytes by check_dims) through 32-bit buffer offsets.
  if (static_cast<int64_t>(H) * d * 2 >= (int64_t{1} << 31))
    return fail(AAH_ERR_UNSUPPORTED, "H * d = %lld is too large for one step's query rows",
                static_cast<long long>(H) * d);
  return AAH_OK;
}

aah_status plan_to_host(PlanKind kind, const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv,
                        int T, int q_tile, int kv_tile, int n_queues, aah_work_item* items, int64_t capacity,
                        int64_t* n_items) {
  if (n_items == nullptr) return fail(AAH_ERR_INVALID_ARG, "n_items is NULL");
  if (windows == nullptr) return fail(AAH_ERR_INVALID_ARG, "windows is NULL");
  if (B < 1 || H < 1 || T < 1) return fail(AAH_ERR_INVALID_ARG, "B, H, T must be >= 1");
  if (q_tile < 1 || kv_tile < 1 || n_queues < 1) return fail(AAH_ERR_INVALID_ARG, "tiles and n_queues must be >= 1");
  AAH_TRY_INNER(check_kv_heads(H, H_kv));
  AAH_TRY_INNER(check_windows(windows, sinks, H));
  const std::vector<WorkItem> v = kind == kPlanFwd
                                      ? aah::plan_forward(windows, sinks, B, H, H_kv, T, q_tile, kv_tile, n_queues)
                                      : aah::plan_backward(windows, sinks, B, H, H_kv, T, q_tile, kv_tile, n_queues);
  *n_items = static_cast<int64_t>(v.size());
  if (capacity < static_cast<int64_t>(v.size()))
    return fail(AAH_ERR_INVALID_ARG, "capacity %lld < %zu items", static_cast<long long>(capacity), v.size());
  if (items == nullptr) return fail(AAH_ERR_INVALID_ARG, "items is NULL");
  static_assert(sizeof(aah_work_item) == sizeof(WorkItem), "ABI work item layout");
  std::memcpy(items, v.data(), v.size() * sizeof(WorkItem));
  return AAH_OK;
}

}  // namespace

extern "C" {

int aah_abi_version(void) { return AAH_ABI_VERSION; }

const char* aah_status_string(aah_status status) {
  switch (status) {
    case AAH_OK: return "AAH_OK";
    case AAH_ERR_INVALID_ARG: return "AAH_ERR_INVALID_ARG";
    case AAH_ERR_UNSUPPORTED: return "AAH_ERR_UNSUPPORTED";
    case AAH_ERR_WORKSPACE: return "AAH_ERR_WORKSPACE";
    case AAH_ERR_HIP: return "AAH_ERR_HIP";
  }
  return "AAH_ERR_UNKNOWN";
}

const char* aah_last_error_detail(void) { return g_detail.c_str(); }

size_t aah_attn_workspace_size(int B, int H, int T, int d, aah_dtype dt, int is_bwd) {
  if (B < 1 || H < 1 || T < 1 || !supported_d(d) || (dt != AAH_BF16 && dt != AAH_F32)) return 0;
  return is_bwd ? bwd_workspace(B, H, T, d, dt) : 0;
}

// Forward split workspace (with the diagnostics' larger per-row partials when diag is set).
size_t fwd_split_workspace_size(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T, int d,
                                aah_dtype dt, bool diag) {
  if (dt != AAH_BF16 || check_shape(windows, sinks, B, H, T, d, dt, H_kv) != AAH_OK) return 0;
  g_detail.clear();
  if (empty_problem(B, T)) return 0;
  const int L = split_chunk_tiles(windows, sinks, B, H, T, d);
  if (L == 0) return 0;
  SplitDevicePlan sp;
  if (get_split_plan(windows, sinks, B, H, H_kv, T, d, L, nullptr, &sp) != AAH_OK) return 0;
  return split_workspace(sp.n_slots, d, diag);
}

size_t aah_attn_fwd_workspace_size(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                                   int d, aah_dtype dt) {
  return fwd_split_workspace_size(windows, sinks, B, H, H_kv, T, d, dt, false);
}

size_t aah_attn_fwd_diag_workspace_size(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                                        int d, aah_dtype dt) {
  return fwd_split_workspace_size(windows, sinks, B, H, H_kv, T, d, dt, true);
}

size_t aah_attn_bwd_split_workspace_size(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv,
                                         int T, int d, aah_dtype dt) {
  if (dt != AAH_BF16 || check_shape(windows, sinks, B, H, T, d, dt, H_kv) != AAH_OK) return 0;
  g_detail.clear();
  if (empty_problem(B, T)) return 0;
  BwdSplitLayout lay;
  return bwd_split_layout(windows, sinks, B, H, H_kv, T, d, dt, nullptr, &lay) ? lay.total : 0;
}

aah_status aah_tile_shape(aah_dtype dt, int d, int is_bwd, int* row_tile, int* col_tile) {
  if (row_tile == nullptr || col_tile == nullptr) return fail(AAH_ERR_INVALID_ARG, "NULL output pointer");
  if (dt != AAH_BF16 && dt != AAH_F32) return fail(AAH_ERR_UNSUPPORTED, "unknown dtype %d", static_cast<int>(dt));
  if (!supported_d(d)) return fail(AAH_ERR_UNSUPPORTED, "head dim %d has no kernel", d);
  if (is_bwd)
    bwd_tiles(dt, row_tile, col_tile);
  else
    fwd_tiles(dt, row_tile, col_tile);
  return AAH_OK;
}

}  // extern "C"

namespace {

// Forward, with the per-row diagnostics when ent / onorm are set (both or neither).
aah_status fwd_impl(const void* q, const void* k, const void* v, const int32_t* windows, const int32_t* sinks, int B,
                    int H, int H_kv, int T, int d, aah_dtype dt, float scale, void* o, float* lse, float* ent,
                    float* onorm, void* workspace, size_t workspace_bytes, aah_stream_t stream) {
  AAH_TRY(check_shape(windows, sinks, B, H, T, d, dt, H_kv));
  if (!std::isfinite(scale) || scale == 0.0f) return fail(AAH_ERR_INVALID_ARG, "scale must be finite and nonzero");
  if (empty_problem(B, T)) return AAH_OK;
  AAH_TRY(check_tensor(q, "q", 16));
  AAH_TRY(check_tensor(k, "k", 16));
  AAH_TRY(check_tensor(v, "v", 16));
  AAH_TRY(check_tensor(o, "o", 16));
  AAH_TRY(check_tensor(lse, "lse", 4));
  // An optional workspace, when given, follows the same alignment rule as every other workspace, whether or
  // not this launch would split (checked here, before any HIP call).
  if (workspace != nullptr && !aligned(workspace, 256))
    return fail(AAH_ERR_INVALID_ARG, "workspace is not 256-byte aligned");

  int row = 0, col = 0;
  fwd_tiles(dt, &row, &col);
  DevicePlan plan;
  const aah::AttnShape s{B, H, T, d, scale, H_kv};
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  // Split launch: bf16 and a workspace large enough for the partials (larger with the diagnostics).
  const int L = dt == AAH_BF16 && workspace != nullptr ? split_chunk_tiles(windows, sinks, B, H, T, d) : 0;
  if (L > 0) {
    SplitDevicePlan sp;
    AAH_TRY(get_split_plan(windows, sinks, B, H, H_kv, T, d, L, st, &sp));
    if (workspace_bytes >= split_workspace(sp.n_slots, d, ent != nullptr)) {
      float* part_acc = static_cast<float*>(workspace);
      float* part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + split_acc_bytes(sp.n_slots, d));
      const aah::FwdSplit split{sp.slots, sp.merges, sp.n_merges, part_acc, part_ml};
      e = aah::launch_fwd_bf16(q, k, v, o, lse, ent, onorm, sp.items, sp.n_items, sp.win, sp.sink, s, &split, st);
      if (e != hipSuccess) return hip_fail(e, "split forward launch");
      return AAH_OK;
    }
  }
  AAH_TRY(get_plan(kPlanFwd, windows, sinks, B, H, H_kv, T, row, col, st, &plan));
  if (dt == AAH_BF16)
    e = aah::launch_fwd_bf16(q, k, v, o, lse, ent, onorm, plan.items, plan.n_items, plan.win, plan.sink, s, nullptr,
                             st);
  else
    e = aah::launch_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                            static_cast<const float*>(v), static_cast<float*>(o), lse, ent, onorm, plan.items,
                            plan.n_items, plan.win, plan.sink, s, st);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return AAH_OK;
}

size_t features_workspace(int B, int H, int T, int d) {
  // Q/K/V partials (count, mean, M2, sum |x|) and the row sums (entropy, norm) per (b, h, chunk).
  return round_up(static_cast<size_t>(3 * 4 + 2) * H * B * aah::feature_chunks(T, d) * sizeof(double), 256);
}

}  // namespace

extern "C" {

aah_status aah_attn_fwd(const void* q, const void* k, const void* v, const int32_t* windows, const int32_t* sinks,
                        int B, int H, int H_kv, int T, int d, aah_dtype dt, float scale, void* o, float* lse,
                        void* workspace, size_t workspace_bytes, aah_stream_t stream) {
  g_detail.clear();
  return fwd_impl(q, k, v, windows, sinks, B, H, H_kv, T, d, dt, scale, o, lse, nullptr, nullptr, workspace,
                  workspace_bytes, stream);
}

aah_status aah_attn_fwd_diag(const void* q, const void* k, const void* v, const int32_t* windows,
                             const int32_t* sinks, int B, int H, int H_kv, int T, int d, aah_dtype dt, float scale,
                             void* o, float* lse, float* row_entropy, float* row_onorm, void* workspace,
                             size_t workspace_bytes, aah_stream_t stream) {
  g_detail.clear();
  if (!empty_problem(B, T)) {
    AAH_TRY(check_tensor(row_entropy, "row_entropy", 4));
    AAH_TRY(check_tensor(row_onorm, "row_onorm", 4));
  }
  return fwd_impl(q, k, v, windows, sinks, B, H, H_kv, T, d, dt, scale, o, lse, row_entropy, row_onorm, workspace,
                  workspace_bytes, stream);
}

size_t aah_head_features_workspace_size(int B, int H, int T, int d) {
  if (B < 1 || H < 1 || T < 1 || !supported_d(d)) return 0;
  return features_workspace(B, H, T, d);
}

aah_status aah_head_features(const void* q, const void* k, const void* v, const float* row_entropy,
                             const float* row_onorm, const int32_t* windows, int B, int H, int H_kv, int T, int d,
                             aah_dtype dt, float alpha, int init, float* features, float* features_ema,
                             void* workspace, size_t workspace_bytes, aah_stream_t stream) {
  g_detail.clear();
  AAH_TRY(check_shape(windows, nullptr, B, H, T, d, dt, H_kv));
  // The statistics are means over tokens: they need at least one.
  if (empty_problem(B, T)) return fail(AAH_ERR_INVALID_ARG, "head features need B, T >= 1 (got %d, %d)", B, T);
  AAH_TRY(check_tensor(q, "q", 16));
  AAH_TRY(check_tensor(k, "k", 16));
  AAH_TRY(check_tensor(v, "v", 16));
  if ((row_entropy == nullptr) != (row_onorm == nullptr))
    return fail(AAH_ERR_INVALID_ARG, "row_entropy and row_onorm must both be given or both be NULL");
  if (row_entropy != nullptr) {
    AAH_TRY(check_tensor(row_entropy, "row_entropy", 4));
    AAH_TRY(check_tensor(row_onorm, "row_onorm", 4));
  }
  if (features == nullptr && features_ema == nullptr)
    return fail(AAH_ERR_INVALID_ARG, "features and features_ema are both NULL: nothing to write");
  if (features != nullptr) AAH_TRY(check_tensor(features, "features", 4));
  if (features_ema != nullptr) AAH_TRY(check_tensor(features_ema, "features_ema", 4));
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(AAH_ERR_INVALID_ARG, "alpha must be in [0, 1]");
  const size_t need = features_workspace(B, H, T, d);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(AAH_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace == nullptr ? 0 : workspace_bytes,
                need);
  if (!aligned(workspace, 256)) return fail(AAH_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (static_cast<int64_t>(B) * H * aah::feature_chunks(T, d) > INT32_MAX)
    return fail(AAH_ERR_UNSUPPORTED, "too many statistics workgroups");
  // The effective windows (usage = min(W, T) / T, with diagnostic rows) come from the cached forward work list's table.
  int row = 0, col = 0;
  fwd_tiles(dt, &row, &col);
  DevicePlan plan;
  AAH_TRY(get_plan(kPlanFwd, windows, nullptr, B, H, H_kv, T, row, col, static_cast<hipStream_t>(stream), &plan));
  const hipError_t e = aah::launch_head_features(q, k, v, dt == AAH_BF16, row_entropy, row_onorm, plan.win, B, H,
                                                 H_kv, T, d, alpha, init != 0, features, features_ema,
                                                 static_cast<double*>(workspace), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "head features launch");
  return AAH_OK;
}

aah_status aah_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const int32_t* windows,
                             const int32_t* sinks, int B, int H, int H_kv, int T, int d, aah_dtype dt, float scale,
                             void* dk, void* dv, void* workspace, size_t workspace_bytes,
                             aah_stream_t stream) {
  g_detail.clear();
  AAH_TRY(check_shape(windows, sinks, B, H, T, d, dt, H_kv));
  if (!std::isfinite(scale) || scale == 0.0f) return fail(AAH_ERR_INVALID_ARG, "scale must be finite and nonzero");
  if (empty_problem(B, T)) return AAH_OK;
  AAH_TRY(check_tensor(q, "q", 16));
  AAH_TRY(check_tensor(k, "k", 16));
  AAH_TRY(check_tensor(v, "v", 16));
  AAH_TRY(check_tensor(dout, "dout", 16));
  AAH_TRY(check_tensor(dk, "dk", 16));
  AAH_TRY(check_tensor(dv, "dv", 16));
  AAH_TRY(check_workspace(workspace, workspace_bytes, B, H, T, d, dt));
  const aah::AttnShape s{B, H, T, d, scale, H_kv};
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float* nl2 = ws_nl2(workspace);
  const float* nd = ws_nd(workspace, B, H, T);
  int row = 0, col = 0;
  bwd_tiles(dt, &row, &col);
  BwdSplitLayout lay;
  if (bwd_split_layout(windows, sinks, B, H, H_kv, T, d, dt, st, &lay) && lay.k_L > 0 && workspace_bytes >= lay.total) {
    const aah::BwdSplit split{lay.k.slots, lay.k.merges, lay.k.n_merges,
                              reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.k_off)};
    const hipError_t e = aah::launch_bwd_dkdv_bf16_split(q, k, v, dout, nl2, nd, dk, dv, lay.k.items, lay.k.n_items,
                                                         lay.k.win, lay.k.sink, s, split, st);
    if (e != hipSuccess) return hip_fail(e, "split dK/dV launch");
    return AAH_OK;
  }
  DevicePlan plan;
  AAH_TRY(get_plan(kPlanBwd, windows, sinks, B, H, H_kv, T, row, col, st, &plan));
  hipError_t e;
  if (dt == AAH_BF16)
    e = aah::launch_bwd_dkdv_bf16(q, k, v, dout, nl2, nd, dk, dv, plan.items, plan.n_items, plan.win, plan.sink, s,
                                  st);
  else
    e = aah::launch_bwd_dkdv_simple(static_cast<const float*>(q), static_cast<const float*>(k),
                                    static_cast<const float*>(v), static_cast<const float*>(dout), nl2, nd,
                                    static_cast<float*>(dk), static_cast<float*>(dv), plan.items, plan.n_items,
                                    plan.win, plan.sink, s, st);
  if (e != hipSuccess) return hip_fail(e, "dK/dV launch");
  return AAH_OK;
}

aah_status aah_attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv,
                           int T, int d, aah_dtype dt, float scale, void* dq, void* workspace,
                           size_t workspace_bytes, aah_stream_t stream) {
  g_detail.clear();
  AAH_TRY(check_shape(windows, sinks, B, H, T, d, dt, H_kv));
  if (!std::isfinite(scale) || scale == 0.0f) return fail(AAH_ERR_INVALID_ARG, "scale must be finite and nonzero");
  if (empty_problem(B, T)) return AAH_OK;
  AAH_TRY(check_tensor(q, "q", 16));
  AAH_TRY(check_tensor(k, "k", 16));
  AAH_TRY(check_tensor(v, "v", 16));
  AAH_TRY(check_tensor(o, "o", 16));
  AAH_TRY(check_tensor(dout, "dout", 16));
  AAH_TRY(check_tensor(lse, "lse", 4));
  AAH_TRY(check_tensor(dq, "dq", 16));
  AAH_TRY(check_workspace(workspace, workspace_bytes, B, H, T, d, dt));
  const aah::AttnShape s{B, H, T, d, scale, H_kv};
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* nl2 = const_cast<float*>(ws_nl2(workspace));
  float* nd = const_cast<float*>(ws_nd(workspace, B, H, T));
  int row = 0, col = 0;
  fwd_tiles(dt, &row, &col);  // dQ walks the forward's (query tile, key tiles) items
  BwdSplitLayout lay;
  if (bwd_split_layout(windows, sinks, B, H, H_kv, T, d, dt, st, &lay) && lay.q_L > 0 && workspace_bytes >= lay.total) {
    const aah::BwdSplit split{lay.q.slots, lay.q.merges, lay.q.n_merges,
                              reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.q_off)};
    const hipError_t e = aah::launch_bwd_dq_bf16_split(q, k, v, o, dout, lse, nl2, nd, dq, lay.q.items,
                                                       lay.q.n_items, lay.q.win, lay.q.sink, s, split, st);
    if (e != hipSuccess) return hip_fail(e, "split dQ launch");
    return AAH_OK;
  }
  DevicePlan plan;
  AAH_TRY(get_plan(kPlanFwd, windows, sinks, B, H, H_kv, T, row, col, st, &plan));
  hipError_t e;
  if (dt == AAH_BF16) {
    // One kernel: D and the workspace rows come out of the dQ kernel's prologue.
    e = aah::launch_bwd_dq_bf16(q, k, v, o, dout, lse, nl2, nd, dq, plan.items, plan.n_items, plan.win, plan.sink,
                                s, st);
  } else {
    e = aah::launch_bwd_preprocess(o, dout, lse, false, nl2, nd, s, st);
    if (e == hipSuccess)
      e = aah::launch_bwd_dq_simple(static_cast<const float*>(q), static_cast<const float*>(k),
                                    static_cast<const float*>(v), static_cast<const float*>(dout), nl2, nd,
                                    static_cast<float*>(dq), plan.items, plan.n_items, plan.win, plan.sink, s, st);
  }
  if (e != hipSuccess) return hip_fail(e, "dQ launch");
  return AAH_OK;
}

aah_status aah_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                        int d, aah_dtype dt, float scale, void* dq, void* dk, void* dv, void* workspace,
                        size_t workspace_bytes, aah_stream_t stream) {
  g_detail.clear();
  // Validate everything up front so that no step runs unless all of them can.
  AAH_TRY(check_shape(windows, sinks, B, H, T, d, dt, H_kv));
  if (!std::isfinite(scale) || scale == 0.0f) return fail(AAH_ERR_INVALID_ARG, "scale must be finite and nonzero");
  if (empty_problem(B, T)) return AAH_OK;
  AAH_TRY(check_tensor(q, "q", 16));
  AAH_TRY(check_tensor(k, "k", 16));
  AAH_TRY(check_tensor(v, "v", 16));
  AAH_TRY(check_tensor(o, "o", 16));
  AAH_TRY(check_tensor(dout, "dout", 16));
  AAH_TRY(check_tensor(lse, "lse", 4));
  AAH_TRY(check_tensor(dq, "dq", 16));
  AAH_TRY(check_tensor(dk, "dk", 16));
  AAH_TRY(check_tensor(dv, "dv", 16));
  AAH_TRY(check_workspace(workspace, workspace_bytes, B, H, T, d, dt));
  AAH_TRY(aah_attn_bwd_dq(q, k, v, o, dout, lse, windows, sinks, B, H, H_kv, T, d, dt, scale, dq, workspace,
                          workspace_bytes, stream));
  return aah_attn_bwd_dkdv(q, k, v, dout, windows, sinks, B, H, H_kv, T, d, dt, scale, dk, dv, workspace,
                           workspace_bytes, stream);
}

int64_t aah_kv_cache_rows(const int32_t* windows, const int32_t* sinks, int H, int H_kv, int T_max) {
  g_detail.clear();
  if (windows == nullptr || H < 1 || T_max < 1 || H_kv < 1 || H_kv > H || H % H_kv != 0) return -1;
  for (int h = 0; h < H; ++h)
    if (windows[h] < 1 || (sinks != nullptr && sinks[h] < 0)) return -1;
  return decode_rows(windows, sinks, H, H_kv, T_max);
}

size_t aah_attn_decode_workspace_size(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv,
                                      int T_max, int d, aah_dtype dt) {
  if (windows == nullptr || B < 1 || H < 1 || T_max < 1 || !supported_d(d) || dt != AAH_BF16) return 0;
  if (H_kv < 1 || H_kv > H || H % H_kv != 0) return 0;
  for (int h = 0; h < H; ++h)
    if (windows[h] < 1 || (sinks != nullptr && sinks[h] < 0)) return 0;
  return decode_workspace(windows, sinks, B, H, H_kv, T_max, d);
}

aah_status aah_kv_cache_fill(const void* k, const void* v, const int32_t* windows, const int32_t* sinks, int B, int H,
                             int H_kv, int T, int T_max, int d, aah_dtype dt, void* kcache, void* vcache,
                             aah_stream_t stream) {
  g_detail.clear();
  AAH_TRY(check_decode(windows, sinks, B, H, H_kv, T_max, d, dt));
  if (T < 0 || T > T_max) return fail(AAH_ERR_INVALID_ARG, "prefill length T = %d must be in [0, T_max = %d]", T, T_max);
  if (empty_problem(B, T)) return AAH_OK;
  AAH_TRY(check_tensor(k, "k", 16));
  AAH_TRY(check_tensor(v, "v", 16));
  AAH_TRY(check_tensor(kcache, "kcache", 16));
  AAH_TRY(check_tensor(vcache, "vcache", 16));
  DecodePlan plan;
  AAH_TRY(get_decode_plan(windows, sinks, H, H_kv, T_max, static_cast<hipStream_t>(stream), &plan));
  const hipError_t e =
      aah::launch_cache_fill_bf16(k, v, kcache, vcache, plan.view(), B, T, d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cache fill launch");
  return AAH_OK;
}

aah_status aah_attn_decode(const void* q, const void* k_new, const void* v_new, void* kcache, void* vcache,
                           const int32_t* pos, const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv,
                           int T_max, int d, aah_dtype dt, float scale, void* o, float* lse, void* workspace,
                           size_t workspace_bytes, aah_stream_t stream) {
  g_detail.clear();
  AAH_TRY(check_decode(windows, sinks, B, H, H_kv, T_max, d, dt));
  if (!std::isfinite(scale) || scale == 0.0f) return fail(AAH_ERR_INVALID_ARG, "scale must be finite and nonzero");
  if (B == 0) return AAH_OK;  // no sequences: nothing to decode
  AAH_TRY(check_tensor(q, "q", 16));
  AAH_TRY(check_tensor(k_new, "k_new", 16));
  AAH_TRY(check_tensor(v_new, "v_new", 16));
  AAH_TRY(check_tensor(kcache, "kcache", 16));
  AAH_TRY(check_tensor(vcache, "vcache", 16));
  AAH_TRY(check_tensor(pos, "pos", 4));
  AAH_TRY(check_tensor(o, "o", 16));
  AAH_TRY(check_tensor(lse, "lse", 4));
  const size_t need = decode_workspace(windows, sinks, B, H, H_kv, T_max, d);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(AAH_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace == nullptr ? 0 : workspace_bytes,
                need);
  if (!aligned(workspace, 256)) return fail(AAH_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  DecodePlan plan;
  AAH_TRY(get_decode_plan(windows, sinks, H, H_kv, T_max, static_cast<hipStream_t>(stream), &plan));
  const hipError_t e = aah::launch_decode_bf16(
      q, k_new, v_new, kcache, vcache, pos, plan.view(), B, T_max, d, scale, o, lse,
      static_cast<int32_t*>(workspace),
      reinterpret_cast<float*>(static_cast<char*>(workspace) + decode_counter_bytes(B, H_kv)),
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return AAH_OK;
}

aah_status aah_attn_decode_noalloc(const void* q, const void* k_new, const void* v_new, void* kcache, void* vcache,
                                   const int32_t* pos, const int32_t* windows, const int32_t* sinks, int B, int H,
                                   int H_kv, int T_max, int d, aah_dtype dt, float scale, void* o, float* lse,
                                   aah_stream_t stream) {
  g_detail.clear();
  // The same checks as aah_attn_decode, on fixed-size tables: nothing here allocates (host or device).
  if (windows == nullptr) return fail(AAH_ERR_INVALID_ARG, "windows is NULL");
  AAH_TRY(check_dims(B, H, T_max, d, dt));
  if (T_max < 1) return fail(AAH_ERR_INVALID_ARG, "T_max must be >= 1 (got %d)", T_max);
  AAH_TRY(check_kv_heads(H, H_kv));
  AAH_TRY(check_windows(windows, sinks, H));
  if (dt != AAH_BF16) return fail(AAH_ERR_UNSUPPORTED, "decoding runs on bf16 caches only");
  if (H > aah::kNoAllocMaxHeads)
    return fail(AAH_ERR_UNSUPPORTED, "H = %d: the allocation-free decode takes at most %d query heads", H,
                aah::kNoAllocMaxHeads);
  if (static_cast<int64_t>(B) * H_kv > 65535)
    return fail(AAH_ERR_UNSUPPORTED, "B * H_kv = %lld exceeds 65535", static_cast<long long>(B) * H_kv);
  if (!std::isfinite(scale) || scale == 0.0f) return fail(AAH_ERR_INVALID_ARG, "scale must be finite and nonzero");
  if (B == 0) return AAH_OK;  // no sequences: nothing to decode
  AAH_TRY(check_tensor(q, "q", 16));
  AAH_TRY(check_tensor(k_new, "k_new", 16));
  AAH_TRY(check_tensor(v_new, "v_new", 16));
  AAH_TRY(check_tensor(kcache, "kcache", 16));
  AAH_TRY(check_tensor(vcache, "vcache", 16));
  AAH_TRY(check_tensor(pos, "pos", 4));
  AAH_TRY(check_tensor(o, "o", 16));
  AAH_TRY(check_tensor(lse, "lse", 4));
  // Per query head C_h and effective sink, per key/value head ring and sink rows (as decode_shape).
  aah::NoAllocHeads heads;
  const int G = H / H_kv;
  const int cr = aah::decode_chunk_rows(H, H_kv);
  int64_t rows = 0, chunks = 0;
  for (int g = 0; g < H_kv; ++g) {
    int64_t ring = 0, ksink = 0;
    for (int j = 0; j < G; ++j) {
      const int h = g * G + j;
      const int64_t cap = std::min<int64_t>(windows[h], T_max);
      const int64_t sk = std::max<int64_t>(0, std::min<int64_t>(sinks == nullptr ? 0 : sinks[h], T_max - cap));
      heads.cap[h] = static_cast<int32_t>(cap);
      heads.sink[h] = static_cast<int32_t>(sk);
      ring = std::max(ring, cap);
      ksink = std::max(ksink, sk);
    }
    rows += ksink + ring;
    chunks += (ksink + ring + cr - 1) / cr;
  }
  if (rows > INT32_MAX) return fail(AAH_ERR_UNSUPPORTED, "cache rows per batch entry exceed 2^31");
  if (static_cast<int64_t>(B) * rows * d >= (int64_t{1} << 40)) return fail(AAH_ERR_UNSUPPORTED, "cache too large");
  const aah::NoAllocLayout lay = aah::noalloc_layout(B, H, H_kv, d, chunks);
  if (lay.total > aah::kNoAllocScratchBytes)
    return fail(AAH_ERR_UNSUPPORTED,
                "this step needs %zu bytes of scratch (counters, plan, partials); the library holds %zu per device: "
                "use aah_attn_decode with a workspace",
                lay.total, aah::kNoAllocScratchBytes);
  const hipError_t e = aah::launch_decode_noalloc_bf16(
      q, k_new, v_new, kcache, vcache, pos, heads, H, H_kv, static_cast<int>(chunks), static_cast<int>(rows), B, T_max,
      d, scale, o, lse, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "allocation-free decode launch");
  return AAH_OK;
}

aah_status aah_plan_fwd(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T, int q_tile,
                        int kv_tile, int n_queues, aah_work_item* items, int64_t capacity, int64_t* n_items) {
  g_detail.clear();
  return plan_to_host(kPlanFwd, windows, sinks, B, H, H_kv, T, q_tile, kv_tile, n_queues, items, capacity, n_items);
}

aah_status aah_plan_bwd(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T, int q_tile,
                        int kv_tile, int n_queues, aah_work_item* items, int64_t capacity, int64_t* n_items) {
  g_detail.clear();
  return plan_to_host(kPlanBwd, windows, sinks, B, H, H_kv, T, q_tile, kv_tile, n_queues, items, capacity, n_items);
}

aah_status aah_window_stats(const int32_t* windows, const int32_t* sinks, int H, int T, int64_t* pairs_per_batch,
                            double* acr) {
  g_detail.clear();
  if (windows == nullptr || pairs_per_batch == nullptr || acr == nullptr)
    return fail(AAH_ERR_INVALID_ARG, "NULL pointer argument");
  if (H < 1 || T < 1) return fail(AAH_ERR_INVALID_ARG, "H and T must be >= 1");
  AAH_TRY(check_windows(windows, sinks, H));
  int64_t pairs = 0;
  double cover = 0.0;
  for (int h = 0; h < H; ++h) {
    pairs += aah::pair_count(T, windows[h], sinks == nullptr ? 0 : sinks[h]);
    cover += static_cast<double>(aah::effective_window(windows[h], T)) / T;
  }
  *pairs_per_batch = pairs;
  *acr = cover / H;
  return AAH_OK;
}

namespace {
// Copies a split plan to the caller's arrays (the capacities checked after the counts are stored).
aah_status split_to_host(const aah::SplitPlan& sp, aah_work_item* items, int32_t* slots, int64_t capacity,
                         int64_t* n_items, aah_work_item* merges, int64_t merge_capacity, int64_t* n_merges) {
  *n_items = static_cast<int64_t>(sp.items.size());
  *n_merges = static_cast<int64_t>(sp.merges.size());
  if (capacity < *n_items || merge_capacity < *n_merges)
    return fail(AAH_ERR_INVALID_ARG, "capacity %lld / %lld < %lld items / %lld merge records",
                static_cast<long long>(capacity), static_cast<long long>(merge_capacity),
                static_cast<long long>(*n_items), static_cast<long long>(*n_merges));
  if ((*n_items > 0 && (items == nullptr || slots == nullptr)) || (*n_merges > 0 && merges == nullptr))
    return fail(AAH_ERR_INVALID_ARG, "output array is NULL");
  std::memcpy(items, sp.items.data(), sp.items.size() * sizeof(WorkItem));
  std::memcpy(slots, sp.slot.data(), sp.slot.size() * sizeof(int32_t));
  if (!sp.merges.empty()) std::memcpy(merges, sp.merges.data(), sp.merges.size() * sizeof(WorkItem));
  return AAH_OK;
}
}  // namespace

aah_status aah_plan_bwd_split(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                              int q_tile, int kv_tile, int n_queues, int chunk_tiles, aah_work_item* items,
                              int32_t* slots, int64_t capacity, int64_t* n_items, aah_work_item* merges,
                              int64_t merge_capacity, int64_t* n_merges) {
  g_detail.clear();
  if (n_items == nullptr || n_merges == nullptr) return fail(AAH_ERR_INVALID_ARG, "n_items / n_merges is NULL");
  if (windows == nullptr) return fail(AAH_ERR_INVALID_ARG, "windows is NULL");
  if (B < 1 || H < 1 || T < 1) return fail(AAH_ERR_INVALID_ARG, "B, H, T must be >= 1");
  if (q_tile < 1 || kv_tile < 1 || n_queues < 1 || chunk_tiles < 1)
    return fail(AAH_ERR_INVALID_ARG, "tiles, n_queues and chunk_tiles must be >= 1");
  AAH_TRY(check_kv_heads(H, H_kv));
  AAH_TRY(check_windows(windows, sinks, H));
  return split_to_host(
      aah::plan_backward_split(windows, sinks, B, H, H_kv, T, q_tile, kv_tile, n_queues, chunk_tiles), items, slots,
      capacity, n_items, merges, merge_capacity, n_merges);
}

aah_status aah_plan_fwd_split(const int32_t* windows, const int32_t* sinks, int B, int H, int H_kv, int T,
                              int q_tile, int kv_tile, int n_queues, int chunk_tiles, aah_work_item* items,
                              int32_t* slots, int64_t capacity, int64_t* n_items, aah_work_item* merges,
                              int64_t merge_capacity, int64_t* n_merges) {
  g_detail.clear();
  if (n_items == nullptr || n_merges == nullptr) return fail(AAH_ERR_INVALID_ARG, "n_items / n_merges is NULL");
  if (windows == nullptr) return fail(AAH_ERR_INVALID_ARG, "windows is NULL");
  if (B < 1 || H < 1 || T < 1) return fail(AAH_ERR_INVALID_ARG, "B, H, T must be >= 1");
  if (q_tile < 1 || kv_tile < 1 || n_queues < 1 || chunk_tiles < 1)
    return fail(AAH_ERR_INVALID_ARG, "tiles, n_queues and chunk_tiles must be >= 1");
  AAH_TRY(check_kv_heads(H, H_kv));
  AAH_TRY(check_windows(windows, sinks, H));
  return split_to_host(
      aah::plan_forward_split(windows, sinks, B, H, H_kv, T, q_tile, kv_tile, n_queues, chunk_tiles), items, slots,
      capacity, n_items, merges, merge_capacity, n_merges);
}

void aah_cache_clear(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  // hipFree synchronises the device: nothing still queued can be using the lists afterwards.
  auto drop = [](DeviceBlob& b) {
    if (b.dev != nullptr) (void)hipFree(b.dev);
    if (b.ready != nullptr) (void)hipEventDestroy(b.ready);
    b = DeviceBlob{};
  };
  for (auto& p : g_cache.clear()) drop(p.blob);
  for (auto& p : g_split_cache.clear()) drop(p.blob);
  for (auto& p : g_decode_cache.clear()) drop(p.blob);
  for (auto& kv : g_staging) {
    for (auto& r : kv.second.inflight) {
      (void)hipEventSynchronize(r.done);
      (void)hipEventDestroy(r.done);
    }
    kv.second.inflight.clear();
    kv.second.head = 0;
  }
}

int64_t aah_cache_entries(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  return static_cast<int64_t>(g_cache.size() + g_split_cache.size() + g_decode_cache.size());
}

}  // extern "C"
