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
//   decode_partial_kernel -- one workgroup = 256 rows of one (b, h) ring; each
//     wave takes 64 rows.  Lane = row for the scores (its K row is one
//     contiguous 2 d-byte read; q . k with v_dot2_f32_bf16 on bf16 pairs);
//     then lanes = dimension pairs for P V (two rows per load instruction, so
//     each instruction reads 2 x 2 d contiguous bytes).  The new token's K / V
//     come from k_new / v_new and are stored into their ring row by the one
//     lane that owns it, so no separate append launch and no ordering between
//     workgroups is needed.  The four waves merge (max, sum, weighted values)
//     in LDS and the workgroup writes one unnormalised partial.
//   decode_combine_kernel -- one wave per (b, h) merges the head's partials
//     (log-sum-exp rescaling) and writes o (bf16) and lse (fp32).
//   cache_fill_kernel -- copies the positions each ring keeps out of a prefill
//     [B, H, T, d] into the cache layout.
#include <cmath>

#include "device_common.hpp"
#include "kernels.hpp"

namespace aah {
namespace {

using namespace dev;

constexpr int kRowsPerWave = 64;
constexpr int kDecodeThreads = 256;
static_assert(kDecodeRows == kRowsPerWave * kDecodeThreads / 64, "chunk size");

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_partial_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ Knew, const bf16* __restrict__ Vnew,
    bf16* __restrict__ Kc, bf16* __restrict__ Vc, const int32_t* __restrict__ pos,
    const DecodeChunk* __restrict__ chunks, const int32_t* __restrict__ head_off, const int32_t* __restrict__ head_cap,
    int H, int R, int T_max, float c, float* __restrict__ part, int n_chunks) {
  constexpr int kDL = D / 32;  // value dimensions per lane in P V
  __shared__ float sm_m[4], sm_l[4];
  __shared__ float sm_o[4][D];

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
  const int w0 = ck.slot0 + wave * kRowsPerWave;  // first ring row of this wave

  // ---- scores: lane = ring row
  const int slot = w0 + lane;
  const bool valid = slot < n_valid;
  float s = -INFINITY;
  if (valid) {
    const bf16* krow = slot == new_slot ? knew : kring + static_cast<size_t>(slot) * D;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(krow + 8 * i);
      const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qrow + 8 * i);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 a = {kv[e], kv[e + 1]};
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
        *reinterpret_cast<bf16x8*>(kring + static_cast<size_t>(slot) * D + 8 * i) =
            *reinterpret_cast<const bf16x8*>(knew + 8 * i);
        *reinterpret_cast<bf16x8*>(vring + static_cast<size_t>(slot) * D + 8 * i) =
            *reinterpret_cast<const bf16x8*>(vnew + 8 * i);
      }
    }
  }
  const float m_w = wave_max(s);
  const float pw = (valid && m_w != -INFINITY) ? __builtin_amdgcn_exp2f(s - m_w) : 0.f;
  const float l_w = wave_sum(pw);

  // ---- P V: lanes (hl, j) take rows 2 r + hl of the wave and dimensions kDL j .. kDL j + kDL - 1
  const int hl = lane >> 5, j = lane & 31;
  float acc[kDL];
#pragma unroll
  for (int x = 0; x < kDL; ++x) acc[x] = 0.f;
#pragma unroll 8
  for (int r = 0; r < kRowsPerWave / 2; ++r) {
    const int k = 2 * r + hl;
    const float pk = __shfl(pw, k);
    const int sk = w0 + k;
    if (sk < n_valid) {
      const bf16* vrow = sk == new_slot ? vnew : vring + static_cast<size_t>(sk) * D;
      if constexpr (kDL == 1) {
        acc[0] = fmaf(pk, static_cast<float>(vrow[j]), acc[0]);
      } else if constexpr (kDL == 2) {
        const bf16x2 v2 = *reinterpret_cast<const bf16x2*>(vrow + 2 * j);
        acc[0] = fmaf(pk, static_cast<float>(v2[0]), acc[0]);
        acc[1] = fmaf(pk, static_cast<float>(v2[1]), acc[1]);
      } else {
        const bf16x4 v4 = *reinterpret_cast<const bf16x4*>(vrow + 4 * j);
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[x] = fmaf(pk, static_cast<float>(v4[x]), acc[x]);
      }
    }
  }
  // Even and odd rows: lanes j and j + 32 hold the same dimensions.
#pragma unroll
  for (int x = 0; x < kDL; ++x) acc[x] += __shfl_xor(acc[x], 32);

  // ---- merge the four waves in LDS, then one partial per workgroup
  if (lane == 0) {
    sm_m[wave] = m_w;
    sm_l[wave] = l_w;
  }
  if (hl == 0) {
#pragma unroll
    for (int x = 0; x < kDL; ++x) sm_o[wave][kDL * j + x] = acc[x];
  }
  __syncthreads();
  if (wave != 0) return;
  float m = fmaxf(fmaxf(sm_m[0], sm_m[1]), fmaxf(sm_m[2], sm_m[3]));
  float f[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) f[w] = sm_m[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm_m[w] - m);
  float* out = part + (static_cast<size_t>(b) * n_chunks + ch) * (2 + D);
  if (lane == 0) {
    out[0] = m;
    out[1] = f[0] * sm_l[0] + f[1] * sm_l[1] + f[2] * sm_l[2] + f[3] * sm_l[3];
  }
  for (int d = lane; d < D; d += 64)
    out[2 + d] = f[0] * sm_o[0][d] + f[1] * sm_o[1][d] + f[2] * sm_o[2][d] + f[3] * sm_o[3][d];
}

template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ part,
                                                            const int32_t* __restrict__ head_first, int H,
                                                            int n_chunks, bf16* __restrict__ O,
                                                            float* __restrict__ LSE) {
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int c0 = head_first[h], c1 = head_first[h + 1];
  const float* base = part + static_cast<size_t>(b) * n_chunks * (2 + D);
  float m = -INFINITY;
  for (int ch = c0; ch < c1; ++ch) m = fmaxf(m, base[static_cast<size_t>(ch) * (2 + D)]);
  float l = 0.f;
  float o[(D + 63) / 64];
#pragma unroll
  for (int x = 0; x < (D + 63) / 64; ++x) o[x] = 0.f;
  for (int ch = c0; ch < c1; ++ch) {
    const float* pc = base + static_cast<size_t>(ch) * (2 + D);
    const float f = pc[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pc[0] - m);
    l = fmaf(f, pc[1], l);
#pragma unroll
    for (int x = 0; x < (D + 63) / 64; ++x)
      if (lane + 64 * x < D) o[x] = fmaf(f, pc[2 + lane + 64 * x], o[x]);
  }
  const size_t bh = static_cast<size_t>(b) * H + h;
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
                    float* part, hipStream_t stream) {
  const float c = scale * kLog2e;
  hipLaunchKernelGGL(decode_partial_kernel<D>, dim3(pl.n_chunks, B), dim3(kDecodeThreads), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(knew), static_cast<const bf16*>(vnew),
                     static_cast<bf16*>(kc), static_cast<bf16*>(vc), pos, pl.chunks, pl.head_off, pl.head_cap, H,
                     pl.rows, T_max, c, part, pl.n_chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(H, B), dim3(64), 0, stream, part, pl.head_first, H,
                     pl.n_chunks, static_cast<bf16*>(o), lse);
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
                              float scale, void* o, float* lse, float* partials, hipStream_t stream) {
  switch (d) {
    case 32: return decode_d<32>(q, knew, vnew, kcache, vcache, pos, plan, B, H, T_max, scale, o, lse, partials, stream);
    case 64: return decode_d<64>(q, knew, vnew, kcache, vcache, pos, plan, B, H, T_max, scale, o, lse, partials, stream);
    case 128:
      return decode_d<128>(q, knew, vnew, kcache, vcache, pos, plan, B, H, T_max, scale, o, lse, partials, stream);
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
