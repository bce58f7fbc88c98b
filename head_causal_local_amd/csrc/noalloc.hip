// One decoding step that allocates nothing, for callers that cannot allocate
// device memory at the point of the call: code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc.
//
// It runs the decode kernel of decode.hip unchanged.  Where aah_attn_decode
// takes its merge counters and partial results from the caller's workspace and
// its plan tables from the library's cache of uploaded plans, this path keeps
// all three in `scratch`, one fixed device array per GPU that the library holds
// until the process ends.  A small planning kernel rebuilds the tables from the
// per-head windows (passed by value, as a kernel argument) and clears the
// counters on every call, so no host memory is read after the call returns and
// a captured graph replays the whole step.  Every call on one GPU shares its
// array: calls that overlap on one GPU race.
#include <mutex>

#include "device_common.hpp"
#include "kernels.hpp"

namespace aah {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch array: looked up once per device, with that device current
// (each GPU holds its own copy of the array at its own address; the host-side name is not an address).
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

constexpr int kPlanThreads = 256;

// The decode plan of aah_attn_decode's cache, computed on the device: per key/value head g (query heads
// g G .. g G + G - 1) the ring R_g = max C_h and sink rows S_g = max effective sink, its first row
// off_g = sum over g' < g of (S_g' + R_g'), its first chunk, and one chunk record per cr rows of
// its region (carrying those per-head values, as the host plan's records do).  Tables: kv_off[H_kv],
// kv_sink[H_kv], kv_ring[H_kv], kv_first[H_kv + 1], q_cap[H], q_sink[H].  Also sets the B * H_kv merge
// counters to zero (each decode call leaves them zero, but nothing else clears this array).  One workgroup.
__global__ __launch_bounds__(kPlanThreads) void noalloc_plan_kernel(NoAllocHeads heads, int H, int H_kv, int B,
                                                                   int32_t* __restrict__ counters,
                                                                   int32_t* __restrict__ tables,
                                                                   DecodeChunk* __restrict__ chunks) {
  __shared__ int32_t s_ring[kNoAllocMaxHeads], s_sink[kNoAllocMaxHeads], s_caps[kNoAllocMaxHeads];
  __shared__ int32_t s_off[kNoAllocMaxHeads + 1], s_first[kNoAllocMaxHeads + 1];
  const int tid = threadIdx.x;
  const int G = H / H_kv;
  const int cr = H_kv < H ? kDecodeRowsGrouped : kDecodeRows;  // rows per chunk, as decode_chunk_rows
  for (int i = tid; i < B * H_kv; i += kPlanThreads) counters[i] = 0;
  for (int h = tid; h < H; h += kPlanThreads) {
    tables[4 * H_kv + 1 + h] = heads.cap[h];
    tables[4 * H_kv + 1 + H + h] = heads.sink[h];
  }
  for (int g = tid; g < H_kv; g += kPlanThreads) {
    int ring = 0, sink = 0, cap_s = INT32_MAX;
    for (int j = 0; j < G; ++j) {
      ring = max(ring, heads.cap[g * G + j]);
      sink = max(sink, heads.sink[g * G + j]);
      if (heads.sink[g * G + j] > 0) cap_s = min(cap_s, heads.cap[g * G + j]);
    }
    s_ring[g] = ring;
    s_sink[g] = sink;
    s_caps[g] = cap_s == INT32_MAX ? 1 : cap_s;
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0, first = 0;
    for (int g = 0; g < H_kv; ++g) {
      s_off[g] = off;
      s_first[g] = first;
      const int n = s_sink[g] + s_ring[g];
      off += n;
      first += (n + cr - 1) / cr;
    }
    s_off[H_kv] = off;
    s_first[H_kv] = first;
  }
  __syncthreads();
  for (int g = tid; g < H_kv; g += kPlanThreads) {
    tables[g] = s_off[g];
    tables[H_kv + g] = s_sink[g];
    tables[2 * H_kv + g] = s_ring[g];
    tables[3 * H_kv + g] = s_first[g];
  }
  if (tid == 0) tables[4 * H_kv] = s_first[H_kv];
  for (int g = 0; g < H_kv; ++g) {
    const int n_g = s_first[g + 1] - s_first[g];
    for (int c = tid; c < n_g; c += kPlanThreads)
      chunks[s_first[g] + c] = DecodeChunk{g, c * cr, s_sink[g], s_ring[g], s_off[g], s_first[g], n_g, s_caps[g]};
  }
}

}  // namespace

hipError_t launch_decode_noalloc_bf16(const void* q, const void* knew, const void* vnew, void* kcache, void* vcache,
                                      const int32_t* pos, const NoAllocHeads& heads, int H, int H_kv, int n_chunks,
                                      int rows, int B, int T_max, int d, float scale, void* o, float* lse,
                                      hipStream_t stream) {
  void* base = nullptr;
  hipError_t e = scratch_ptr(&base);
  if (e != hipSuccess) return e;
  const NoAllocLayout lay = noalloc_layout(B, H, H_kv, d, n_chunks);
  if (lay.total > kNoAllocScratchBytes) return hipErrorInvalidValue;  // the caller checks this first
  char* p = static_cast<char*>(base);
  int32_t* counters = reinterpret_cast<int32_t*>(p);
  int32_t* tables = reinterpret_cast<int32_t*>(p + lay.tables);
  DecodeChunk* chunks = reinterpret_cast<DecodeChunk*>(p + lay.chunks);
  float* partials = reinterpret_cast<float*>(p + lay.partials);
  hipLaunchKernelGGL(noalloc_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, heads, H, H_kv, B, counters, tables,
                     chunks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int32_t* t = tables;
  const DecodePlanView view{chunks, n_chunks, t, t + H_kv, t + 2 * H_kv, t + 3 * H_kv, t + 4 * H_kv + 1,
                            t + 4 * H_kv + 1 + H, rows, H, H_kv, nullptr, nullptr};
  return launch_decode_bf16(q, knew, vnew, kcache, vcache, pos, view, B, T_max, d, scale, o, lse, counters, partials,
                            stream);
}

}  // namespace aah
