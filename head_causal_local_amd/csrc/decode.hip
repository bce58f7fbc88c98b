// Decoding over per-head trimmed K/V caches (bf16, gfx950).
//
// Operation: one decoding step of "Asymmetric Attention Heads" section 5.8 --
// the newest token at position p of head h (window W_h, maximum context
// T_max) attends to positions max(0, p - C_h + 1) .. p, C_h = min(W_h, T_max).
// Per-head caches keep exactly those keys: head h owns C_h rows of K and of V
// and position t lives in row off_h + (t mod C_h) (AAH Table 6 runs inference
// with per-head windows; "Autonomy-of-Heads" section 5 bounds a streaming
// head's decode-time cache by its window).  Softmax does not depend on the
// order of its keys, so the step attends to the valid rows of the ring as they
// lie, with no position mask: rows 0 .. min(p + 1, C_h) - 1 of the head.
//
// The step reads every cached K and V row once, so it is bound by HBM
// bandwidth, not by arithmetic (d = 64: 256 bytes per row for about 4 d flops).
// Kernels:
//   decode_kernel -- one workgroup = kDecodeRows rows of one (b, h) ring; each
//     wave takes 64 rows.  Lane = row for the scores (its K row is one contiguous
//     2 d-byte read; q . k with v_dot2_f32_bf16 on bf16 pairs); lanes =
//     dimension slices for P V (two rows per load instruction, so each
//     instruction reads 2 x 2 d contiguous bytes).  Both the K and the V loads
//     are issued before the first wait, so a workgroup pays one HBM round trip.
//     The new token's K / V come from k_new / v_new and are stored into their
//     ring row by the one lane that owns it, so no separate append launch and
//     no ordering between workgroups is needed.  The waves merge (max,
//     sum, weighted values) in LDS and the workgroup writes one unnormalised
//     partial; the last workgroup of a (b, h) to finish (a per-(b, h) counter
//     in the workspace, reset by that workgroup) merges the head's partials
//     with log-sum-exp rescaling and writes o (bf16) and lse (fp32).
//   cache_fill_kernel -- copies the positions each ring keeps out of a prefill
//     [B, H, T, d] into the cache layout.
#include <cmath>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace aah {
namespace {

using namespace dev;

constexpr int kRowsPerWave = 64;
constexpr int kDecodeWaves = kDecodeRows / kRowsPerWave;
constexpr int kDecodeThreads = 64 * kDecodeWaves;
static_assert(kDecodeWaves * kRowsPerWave == kDecodeRows && kDecodeWaves <= 4, "chunk size");

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Device-coherent (all XCDs) store and load of one float.
__device__ inline void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ Knew, const bf16* __restrict__ Vnew,
    bf16* __restrict__ Kc, bf16* __restrict__ Vc, const int32_t* __restrict__ pos,
    const DecodeChunk* __restrict__ chunks, const int32_t* __restrict__ head_off, const int32_t* __restrict__ head_cap,
    const int32_t* __restrict__ head_first, int H, int R, int T_max, float c, int32_t* __restrict__ counters,
    float* __restrict__ part, int n_chunks, bf16* __restrict__ O, float* __restrict__ LSE) {
  constexpr int kDL = D / 32;  // value dimensions per lane in P V
  constexpr int kPairs = kRowsPerWave / 2;
  using vec_t = typename std::conditional<kDL == 1, bf16,
                                          typename std::conditional<kDL == 2, bf16x2, bf16x4>::type>::type;
  __shared__ float sm_m[kDecodeWaves], sm_l[kDecodeWaves];
  __shared__ float sm_o[kDecodeWaves][D];
  __shared__ int sm_last;

  const int ch = blockIdx.x, b = blockIdx.y;
  const DecodeChunk ck = chunks[ch];
  const int h = ck.head;
  const int C = head_cap[h];
  const int p = min(max(pos[b], 0), T_max - 1);
  const int n_valid = min(p + 1, C);
  const int new_slot = p % C;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const bf16* qrow = Q + bh * D;
  const bf16* knew = Knew + bh * D;
  const bf16* vnew = Vnew + bh * D;
  const size_t ring = (static_cast<size_t>(b) * R + head_off[h]) * D;  // first element of this head's ring
  bf16* kring = Kc + ring;
  bf16* vring = Vc + ring;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hl = lane >> 5, j = lane & 31;
  const int w0 = ck.slot0 + wave * kRowsPerWave;  // first ring row of this wave

  // ---- all loads first: this lane's K row (scores) and its V slices of the wave's rows (P V)
  const int slot = w0 + lane;
  const bool valid = slot < n_valid;
  bf16x8 kr[D / 8];
  if (valid) {
    const bf16* krow = slot == new_slot ? knew : kring + static_cast<size_t>(slot) * D;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) kr[i] = *reinterpret_cast<const bf16x8*>(krow + 8 * i);
  }
  vec_t vr[kPairs];
#pragma unroll
  for (int r = 0; r < kPairs; ++r) {
    const int sk = w0 + 2 * r + hl;
    if (sk < n_valid) {
      const bf16* vrow = sk == new_slot ? vnew : vring + static_cast<size_t>(sk) * D;
      vr[r] = *reinterpret_cast<const vec_t*>(vrow + kDL * j);
    } else {
      vr[r] = vec_t{};
    }
  }

  // ---- scores: lane = ring row
  float s = -INFINITY;
  if (valid) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qrow + 8 * i);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 a = {kr[i][e], kr[i][e + 1]};
        const bf16x2 q2 = {qv[e], qv[e + 1]};
        if (e & 2)
          s1 = __builtin_amdgcn_fdot2_f32_bf16(a, q2, s1, false);
        else
          s0 = __builtin_amdgcn_fdot2_f32_bf16(a, q2, s0, false);
      }
    }
    s = (s0 + s1) * c;
    if (slot == new_slot) {  // the new token's row enters its ring slot
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        *reinterpret_cast<bf16x8*>(kring + static_cast<size_t>(slot) * D + 8 * i) = kr[i];
        *reinterpret_cast<bf16x8*>(vring + static_cast<size_t>(slot) * D + 8 * i) =
            *reinterpret_cast<const bf16x8*>(vnew + 8 * i);
      }
    }
  }
  const float m_w = wave_max(s);
  const float pw = (valid && m_w != -INFINITY) ? __builtin_amdgcn_exp2f(s - m_w) : 0.f;
  const float l_w = wave_sum(pw);

  // ---- P V: lanes (hl, j) take rows 2 r + hl of the wave and dimensions kDL j .. kDL j + kDL - 1
  float acc[kDL];
#pragma unroll
  for (int x = 0; x < kDL; ++x) acc[x] = 0.f;
#pragma unroll
  for (int r = 0; r < kPairs; ++r) {
    const float pk = __shfl(pw, 2 * r + hl);  // 0 for rows past n_valid, whose slices are zero too
    if constexpr (kDL == 1) {
      acc[0] = fmaf(pk, static_cast<float>(vr[r]), acc[0]);
    } else {
#pragma unroll
      for (int x = 0; x < kDL; ++x) acc[x] = fmaf(pk, static_cast<float>(vr[r][x]), acc[x]);
    }
  }
  // Even and odd rows: lanes j and j + 32 hold the same dimensions.
#pragma unroll
  for (int x = 0; x < kDL; ++x) acc[x] += __shfl_xor(acc[x], 32);

  // ---- merge the waves in LDS: one partial per workgroup
  if (lane == 0) {
    sm_m[wave] = m_w;
    sm_l[wave] = l_w;
  }
  if (hl == 0) {
#pragma unroll
    for (int x = 0; x < kDL; ++x) sm_o[wave][kDL * j + x] = acc[x];
  }
  __syncthreads();
  const int c0 = head_first[h], c1 = head_first[h + 1];
  float* pbase = part + static_cast<size_t>(b) * n_chunks * (2 + D);
  if (wave == 0) {
    float m = sm_m[0];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) m = fmaxf(m, sm_m[w]);
    float f[kDecodeWaves];
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) f[w] = sm_m[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm_m[w] - m);
    // The workgroups of one (b, h) may run on different XCDs, whose L2 caches are not coherent
    // with each other: partials go out with device-coherent stores, the counter is a
    // device-scope atomic issued once those stores have completed, and the merging workgroup
    // reads the partials with device-coherent loads.  (Release / acquire fences would write back
    // and invalidate whole L2 caches instead.)
    float* out = pbase + static_cast<size_t>(ch) * (2 + D);
    if (lane == 0) {
      coherent_store(out, m);
      float lsum = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) lsum = fmaf(f[w], sm_l[w], lsum);
      coherent_store(out + 1, lsum);
    }
    for (int d = lane; d < D; d += 64) {
      float od = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) od = fmaf(f[w], sm_o[w][d], od);
      coherent_store(out + 2 + d, od);
    }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) {
      const int done = __hip_atomic_fetch_add(&counters[bh], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm_last = done == c1 - c0 - 1;
    }
  }
  __syncthreads();
  if (!sm_last || wave != 0) return;
  if (lane == 0) __hip_atomic_store(&counters[bh], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next call
  float m = -INFINITY;
  for (int cc = c0; cc < c1; ++cc) m = fmaxf(m, coherent_load(pbase + static_cast<size_t>(cc) * (2 + D)));
  float l = 0.f;
  float o[(D + 63) / 64];
#pragma unroll
  for (int x = 0; x < (D + 63) / 64; ++x) o[x] = 0.f;
  for (int cc = c0; cc < c1; ++cc) {
    const float* pc = pbase + static_cast<size_t>(cc) * (2 + D);
    const float mc = coherent_load(pc);
    const float fc = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - m);
    l = fmaf(fc, coherent_load(pc + 1), l);
#pragma unroll
    for (int x = 0; x < (D + 63) / 64; ++x)
      if (lane + 64 * x < D) o[x] = fmaf(fc, coherent_load(pc + 2 + lane + 64 * x), o[x]);
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int x = 0; x < (D + 63) / 64; ++x)
    if (lane + 64 * x < D) O[bh * D + lane + 64 * x] = static_cast<bf16>(o[x] * inv);
  if (lane == 0) LSE[bh] = (m + log2f(l)) * kLn2;
}

// One thread per 16-byte piece of a kept row: (b, h, kept position, piece).
template <int D>
__global__ __launch_bounds__(256) void cache_fill_kernel(const bf16* __restrict__ K, const bf16* __restrict__ V,
                                                         bf16* __restrict__ Kc, bf16* __restrict__ Vc,
                                                         const int32_t* __restrict__ head_off,
                                                         const int32_t* __restrict__ head_cap, int H, int T, int R) {
  constexpr int kPieces = D / 8;
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh % H;
  const int C = head_cap[h];
  const int kept = min(C, T);
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= kept * kPieces) return;
  const int t = T - kept + idx / kPieces;  // position
  const int piece = idx % kPieces;
  const size_t src = (static_cast<size_t>(bh) * T + t) * D + 8 * piece;
  const size_t dst = (static_cast<size_t>(b) * R + head_off[h] + t % C) * D + 8 * piece;
  *reinterpret_cast<bf16x8*>(Kc + dst) = *reinterpret_cast<const bf16x8*>(K + src);
  *reinterpret_cast<bf16x8*>(Vc + dst) = *reinterpret_cast<const bf16x8*>(V + src);
}

template <int D>
hipError_t decode_d(const void* q, const void* knew, const void* vnew, void* kc, void* vc, const int32_t* pos,
                    const DecodePlanView& pl, int B, int H, int T_max, float scale, void* o, float* lse,
                    int32_t* counters, float* part, hipStream_t stream) {
  const float c = scale * kLog2e;
  hipLaunchKernelGGL(decode_kernel<D>, dim3(pl.n_chunks, B), dim3(kDecodeThreads), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(knew), static_cast<const bf16*>(vnew),
                     static_cast<bf16*>(kc), static_cast<bf16*>(vc), pos, pl.chunks, pl.head_off, pl.head_cap,
                     pl.head_first, H, pl.rows, T_max, c, counters, part, pl.n_chunks, static_cast<bf16*>(o), lse);
  return hipGetLastError();
}

template <int D>
hipError_t fill_d(const void* k, const void* v, void* kc, void* vc, const DecodePlanView& pl, int B, int H, int T,
                  hipStream_t stream) {
  int max_kept = 0;
  for (int h = 0; h < H; ++h) max_kept = max(max_kept, min(pl.host_cap[h], T));
  const int pieces = max_kept * (D / 8);
  hipLaunchKernelGGL(cache_fill_kernel<D>, dim3((pieces + 255) / 256, B * H), dim3(256), 0, stream,
                     static_cast<const bf16*>(k), static_cast<const bf16*>(v), static_cast<bf16*>(kc),
                     static_cast<bf16*>(vc), pl.head_off, pl.head_cap, H, T, pl.rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const void* q, const void* knew, const void* vnew, void* kcache, void* vcache,
                              const int32_t* pos, const DecodePlanView& plan, int B, int H, int T_max, int d,
                              float scale, void* o, float* lse, int32_t* counters, float* partials,
                              hipStream_t stream) {
  switch (d) {
    case 32:
      return decode_d<32>(q, knew, vnew, kcache, vcache, pos, plan, B, H, T_max, scale, o, lse, counters, partials,
                          stream);
    case 64:
      return decode_d<64>(q, knew, vnew, kcache, vcache, pos, plan, B, H, T_max, scale, o, lse, counters, partials,
                          stream);
    case 128:
      return decode_d<128>(q, knew, vnew, kcache, vcache, pos, plan, B, H, T_max, scale, o, lse, counters, partials,
                           stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_cache_fill_bf16(const void* k, const void* v, void* kcache, void* vcache,
                                  const DecodePlanView& plan, int B, int H, int T, int d, hipStream_t stream) {
  switch (d) {
    case 32: return fill_d<32>(k, v, kcache, vcache, plan, B, H, T, stream);
    case 64: return fill_d<64>(k, v, kcache, vcache, plan, B, H, T, stream);
    case 128: return fill_d<128>(k, v, kcache, vcache, plan, B, H, T, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace aah
