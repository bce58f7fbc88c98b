// Launch wrappers of the HIP kernels (defined in the .hip files).  Every
// wrapper only enqueues on `stream` and returns the launch status; argument
// checking has already happened in the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "workplan.hpp"

namespace aah {

// Tile shapes (rows of the stationary operand per item, rows of the streamed
// operand per step).  The planner is called with exactly these.
constexpr int kFwdBf16RowTile = 128;  // 4 waves x 32 query rows
constexpr int kFwdBf16ColTile = 64;   // keys per LDS stage
constexpr int kBwdBf16RowTile = 128;  // 4 waves x 32 keys per item
constexpr int kBwdBf16ColTile = 64;   // queries per step
constexpr int kSimpleRowTile = 64;    // one wave, one row per lane
constexpr int kSimpleColTile = 64;

// win_eff: effective window per head (int32[H], device).  sink_eff: effective
// sink size per head (int32[H], device; keys 0 .. S - 1 stay visible to every
// later query), or nullptr when no head has one -- then the kernels without
// sink handling run.

struct AttnShape {
  int B, H, T, d;
  float scale;          // softmax scale applied to q . k
  int H_kv;             // key/value heads; query head h reads head h / (H / H_kv)
};

// log2(n) when n is a power of two, else -1: the kernels split a (batch, head) index with a shift and a
// mask instead of a division when the head counts allow it.
inline int log2_exact(int n) {
  int l = 0;
  while (l < 30 && (1 << l) < n) ++l;
  return (1 << l) == n ? l : -1;
}

// bf16 forward on MFMA (d in {32, 64, 128}).  ent / onorm: nullptr, or fp32
// [B,H,T] outputs of each row's attention entropy and output-row norm (both set
// or both null).
// Split forward (plan_forward_split): slots[i] is item i's partial slot or -1;
// a chunk writes its rows' fp32 accumulator to part_acc [slot][128][d] and
// (max in the log2 domain, row sum) to part_ml [slot][128][2] -- with the
// diagnostics, (max, row sum, sum of weights times offsets, unused) to
// part_ml [slot][128][kMlDiag]; after the forward, one merge workgroup group
// per record in merges combines them into O and LSE (and the diagnostics).
constexpr int kMlDiag = 4;
struct FwdSplit {
  const int32_t* slots;
  const WorkItem* merges;
  int n_merges;
  float* part_acc;
  float* part_ml;
};

// split: nullptr, or the split plan's device arrays and the partial buffers.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, float* ent,
                           float* onorm, const WorkItem* items, int n_items, const int32_t* win_eff,
                           const int32_t* sink_eff, const AttnShape& s, const FwdSplit* split, hipStream_t stream);

// Workgroups of the plain bf16 forward the current device holds at once, or 0 if the query fails.
int fwd_bf16_resident(int d);

// Scalar forward for fp32 (d in {32, 64, 128}); ent / onorm as for bf16.
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, float* ent,
                          float* onorm, const WorkItem* items, int n_items, const int32_t* win_eff,
                          const int32_t* sink_eff, const AttnShape& s, hipStream_t stream);

// Per row: nd = -(dO . O) and nl2 = -lse log2(e), in fp32.  is_bf16 selects the
// element type of o / dout.
hipError_t launch_bwd_preprocess(const void* o, const void* dout, const float* lse, bool is_bf16, float* nl2,
                                 float* nd, const AttnShape& s, hipStream_t stream);

// bf16 backward on MFMA, no atomics.  dK, dV: items from the backward
// planner (kBwdBf16RowTile keys of one key/value head per item, kBwdBf16ColTile
// queries per step, over every query head of the group).
hipError_t launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const void* dout, const float* nl2,
                                const float* nd, void* dk, void* dv, const WorkItem* items, int n_items,
                                const int32_t* win_eff, const int32_t* sink_eff, const AttnShape& s, hipStream_t stream);

// dQ: items from the forward planner (kFwdBf16RowTile queries, kFwdBf16ColTile keys per step).
// Also writes, for every row, nl2 = -lse log2(e) and nd = -(dO . O), which
// launch_bwd_dkdv_bf16 reads: it must run first.
hipError_t launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, float* nl2, float* nd, void* dq, const WorkItem* items, int n_items,
                              const int32_t* win_eff, const int32_t* sink_eff, const AttnShape& s, hipStream_t stream);

// Split backward (plan_forward_split items for dQ, plan_backward_split items
// for dK/dV; sink_eff and grouped heads as for the unsplit launches): slots[i]
// is item i's partial slot or -1.  A dQ chunk leaves its fp32 dQ sum (before
// the scale) in part [slot][128][d]; a dK/dV chunk its dK and dV sums (over
// the group's query heads) in part [slot][2][128][d]; a merge launch per
// kernel adds each split item's chunks and writes bf16.
struct BwdSplit {
  const int32_t* slots;
  const WorkItem* merges;
  int n_merges;
  float* part;
};
hipError_t launch_bwd_dkdv_bf16_split(const void* q, const void* k, const void* v, const void* dout, const float* nl2,
                                      const float* nd, void* dk, void* dv, const WorkItem* items, int n_items,
                                      const int32_t* win_eff, const int32_t* sink_eff, const AttnShape& s,
                                      const BwdSplit& split, hipStream_t stream);
hipError_t launch_bwd_dq_bf16_split(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                    const float* lse, float* nl2, float* nd, void* dq, const WorkItem* items,
                                    int n_items, const int32_t* win_eff, const int32_t* sink_eff,
                                    const AttnShape& s, const BwdSplit& split, hipStream_t stream);
// Workgroups of the plain bf16 dQ / dK,dV kernels the current device holds at once (0 if the query fails).
int bwd_dq_resident(int d);
int bwd_dkdv_resident(int d);

// Scalar backward for fp32: dQ one query row per lane over the forward work
// list; dK/dV one key row per lane over the backward work list.
hipError_t launch_bwd_dq_simple(const float* q, const float* k, const float* v, const float* dout,
                                const float* nl2, const float* nd, float* dq, const WorkItem* items,
                                int n_items, const int32_t* win_eff, const int32_t* sink_eff, const AttnShape& s, hipStream_t stream);
hipError_t launch_bwd_dkdv_simple(const float* q, const float* k, const float* v, const float* dout,
                                  const float* nl2, const float* nd, float* dk, float* dv,
                                  const WorkItem* items, int n_items, const int32_t* win_eff, const int32_t* sink_eff,
                                  const AttnShape& s, hipStream_t stream);

// ---- per-head controller features
constexpr int kNumFeatures = 9;      // [mu|q|, sigma q, mu|k|, sigma k, mu|v|, sigma v, entropy, out norm, usage]
constexpr int kFeatureSpan = 32768;  // elements of one (b, h) slice per statistics workgroup

// Statistics workgroups per (b, h) slice of T * d elements.
inline int feature_chunks(int T, int d) {
  const int64_t n = static_cast<int64_t>(T) * d;
  return static_cast<int>((n + kFeatureSpan - 1) / kFeatureSpan);
}

// Writes features [H, 9] (if non-null) and updates ema [H, 9] (if non-null;
// ema = x when init) from q [B,H,T,d], k, v [B,H_kv,T,d] (bf16 or fp32) and the
// per-row entropy / output norm [B,H,T] (nullptr: those features are 0).  partials:
// (3 * 4 + 2) * H * B * feature_chunks(T, d) doubles of scratch.
hipError_t launch_head_features(const void* q, const void* k, const void* v, bool is_bf16, const float* ent,
                                const float* onorm, const int32_t* win_eff, int B, int H, int H_kv, int T, int d,
                                float alpha, bool init, float* features, float* ema, double* partials,
                                hipStream_t stream);

// ---- decoding over per-head trimmed K/V caches (bf16)
constexpr int kDecodeRows = 256;  // cache rows per decode workgroup (4 waves of 64 rows)
constexpr int kDecodeRowsGrouped = 512;  // ... with grouped key/value heads (8 waves of 64 rows)
// Rows per decode workgroup: a grouped step forms every query head of the group from each loaded row, so
// it has more work per byte and takes longer chunks (fewer partials per head to merge).
inline int decode_chunk_rows(int H, int H_kv) { return H_kv < H ? kDecodeRowsGrouped : kDecodeRows; }

// One decode workgroup's share: local rows [row0, row0 + decode_chunk_rows) of one
// key/value head's region (its sink rows, then its ring rows), with what the
// workgroup needs of its key/value head before it can address its rows, so
// that one 32-byte scalar load precedes the row loads.
struct DecodeChunk {
  int32_t kvhead;  // g
  int32_t row0;
  int32_t sink;    // S_g sink rows
  int32_t ring;    // R_g ring rows
  int32_t off;     // first row of g's region in a batch entry's cache
  int32_t first;   // g's first chunk
  int32_t count;   // g's chunks
  int32_t cap_s;   // smallest C_h among g's query heads with sink keys (any positive value if none)
};
static_assert(sizeof(DecodeChunk) == 32, "DecodeChunk layout");

// Device tables of one (windows, sinks, H, H_kv, T_max) combination.  Key/value
// head g owns kv_sink[g] sink rows then kv_ring[g] ring rows from row
// kv_off[g]; its chunks are [kv_first[g], kv_first[g + 1]).  Query head h has
// window q_cap[h] = min(W_h, T_max) and effective sink q_sink[h].
struct DecodePlanView {
  const DecodeChunk* chunks;
  int n_chunks;
  const int32_t* kv_off;
  const int32_t* kv_sink;
  const int32_t* kv_ring;
  const int32_t* kv_first;
  const int32_t* q_cap;
  const int32_t* q_sink;
  int rows;  // R = sum over key/value heads of sink + ring rows
  int H, H_kv;
  const int32_t* host_kv_sink;  // host copies of kv_sink / kv_ring
  const int32_t* host_kv_ring;
};

// Writes k_new / v_new [B,H_kv,d] into the rows of position pos[b] (device
// int32[B], clamped to [0, T_max)) and o [B,H,d] / lse [B,H] of that token.
// counters: int32[B*H_kv], zero on entry and left zero; partials: B * n_chunks *
// (H / H_kv) * (2 + d) floats.
hipError_t launch_decode_bf16(const void* q, const void* knew, const void* vnew, void* kcache, void* vcache,
                              const int32_t* pos, const DecodePlanView& plan, int B, int T_max, int d, float scale,
                              void* o, float* lse, int32_t* counters, float* partials, hipStream_t stream);

// Copies the positions each region keeps of a prefill k, v [B,H_kv,T,d].
hipError_t launch_cache_fill_bf16(const void* k, const void* v, void* kcache, void* vcache,
                                  const DecodePlanView& plan, int B, int T, int d, hipStream_t stream);

// ---- decoding with no caller workspace (counters, plan tables and partials in a library-held device array)
constexpr int kNoAllocMaxHeads = 256;                     // query heads (the per-head table travels by value)
constexpr size_t kNoAllocScratchBytes = size_t{8} << 20;  // bytes of that array on each device

// Per query head: C_h = min(W_h, T_max) and the effective sink min(S_h, T_max - C_h), passed to the
// planning kernel as a kernel argument.
struct NoAllocHeads {
  int32_t cap[kNoAllocMaxHeads];
  int32_t sink[kNoAllocMaxHeads];
};

// Byte offsets of the scratch regions of one call: merge counters (at 0), plan tables, decode chunks,
// partials, and the bytes used in all.
struct NoAllocLayout {
  size_t tables, chunks, partials, total;
};
inline NoAllocLayout noalloc_layout(int B, int H, int H_kv, int d, int64_t n_chunks) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  NoAllocLayout l;
  l.tables = up(static_cast<size_t>(B) * H_kv * sizeof(int32_t));
  l.chunks = l.tables + up(static_cast<size_t>(4 * H_kv + 1 + 2 * H) * sizeof(int32_t));
  l.partials = l.chunks + up(static_cast<size_t>(n_chunks) * sizeof(DecodeChunk));
  l.total = l.partials + static_cast<size_t>(B) * n_chunks * (H / H_kv) * (2 + d) * sizeof(float);
  return l;
}

// One decoding step as launch_decode_bf16, with the plan built on the device from `heads` (one small
// kernel that also clears the counters) and every buffer in the library's scratch array.  The caller
// has checked the arguments and that noalloc_layout(...).total <= kNoAllocScratchBytes; n_chunks and
// rows are the decode plan's chunk and cache-row counts for these heads.
hipError_t launch_decode_noalloc_bf16(const void* q, const void* knew, const void* vnew, void* kcache, void* vcache,
                                      const int32_t* pos, const NoAllocHeads& heads, int H, int H_kv, int n_chunks,
                                      int rows, int B, int T_max, int d, float scale, void* o, float* lse,
                                      hipStream_t stream);

}  // namespace aah
