// Per-head controller features of "Asymmetric Attention Heads" section 5.3
// (Head features and EMA smoothing), on the device:
//   x_h = [mu(|q_h|), sigma(q_h), mu(|k_h|), sigma(k_h), mu(|v_h|), sigma(v_h), e_h, n_h, rho_h]
// with the Q/K/V entries reduced over batch, sequence and head dimension of head
// h (mean of the absolute activations; population standard deviation), e_h and
// n_h the means over batch and rows of the per-row attention entropy and output
// norm that a diagnostic forward pass wrote, rho_h = min(W_h, T) / T, and the
// smoothing xbar = alpha xbar + (1 - alpha) x (xbar = x at the first update).
//
// Two launches, deterministic (fixed reduction order, no atomics):
//   qkv_stats_kernel: one workgroup per 32768-element span of one (b, h) slice
//     of Q, K or V (grid y picks the tensor).  The slice is contiguous in the
//     [B, H, T, d] layout, so each lane streams 16-byte vectors.  Lanes keep
//     fp32 sums of x - x0 and (x - x0)^2 about their own first element x0 (no
//     cancellation when the mean is large against the spread) and of |x|; the
//     workgroup merges them pairwise in fp64 (count, mean, M2) and writes one
//     partial.  HBM-bound: every element is read once.
//   features_kernel: one workgroup per head merges the head's partials in a
//     fixed order, averages the entropy and norm rows, and writes x_h and the
//     smoothed features.
#include <cmath>

#include "kernels.hpp"

namespace aah {
namespace {

typedef __bf16 bf16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
static_assert(kFeatureSpan % 8 == 0, "span must hold whole 16-byte vectors");

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return static_cast<float>(x); }

struct Mom {
  double n, mean, m2, abs_sum;
};

// Pairwise merge of two (count, mean, M2) summaries (the parallel form of the
// running-variance update).
__device__ inline Mom merge(const Mom& a, const Mom& b) {
  const double n = a.n + b.n;
  if (n == 0.0) return a;
  const double delta = b.mean - a.mean;
  Mom r;
  r.n = n;
  r.mean = a.mean + delta * (b.n / n);
  r.m2 = a.m2 + b.m2 + delta * delta * (a.n * b.n / n);
  r.abs_sum = a.abs_sum + b.abs_sum;
  return r;
}

template <typename E>
__global__ __launch_bounds__(kThreads) void qkv_stats_kernel(const E* __restrict__ Q, const E* __restrict__ K,
                                                             const E* __restrict__ V, int64_t slice, int chunks,
                                                             double* __restrict__ partials, int H, int B) {
  constexpr int kPer = 16 / sizeof(E);  // elements per 16-byte vector
  __shared__ Mom sm[kThreads];
  const int bh = blockIdx.x / chunks, chunk = blockIdx.x % chunks;
  const int tensor = blockIdx.y;
  const E* src = (tensor == 0 ? Q : tensor == 1 ? K : V) + static_cast<int64_t>(bh) * slice +
                 static_cast<int64_t>(chunk) * kFeatureSpan;
  const int64_t left = slice - static_cast<int64_t>(chunk) * kFeatureSpan;
  const int n_vec = static_cast<int>((left < kFeatureSpan ? left : kFeatureSpan) / kPer);

  float x0 = 0.f, s1 = 0.f, s2 = 0.f, sa = 0.f;
  int cnt = 0;
  if (static_cast<int>(threadIdx.x) < n_vec) x0 = to_f32(src[threadIdx.x * kPer]);
  for (int vi = threadIdx.x; vi < n_vec; vi += kThreads) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(vi) * kPer);
    const E* e = reinterpret_cast<const E*>(&raw);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const float x = to_f32(e[i]);
      const float y = x - x0;
      s1 += y;
      s2 = fmaf(y, y, s2);
      sa += fabsf(x);
    }
    cnt += kPer;
  }
  Mom m{static_cast<double>(cnt), 0.0, 0.0, static_cast<double>(sa)};
  if (cnt > 0) {
    const double d1 = s1, n = cnt;
    m.mean = static_cast<double>(x0) + d1 / n;
    m.m2 = fmax(static_cast<double>(s2) - d1 * d1 / n, 0.0);
  }
  sm[threadIdx.x] = m;
  __syncthreads();
  for (int stride = kThreads / 2; stride > 0; stride >>= 1) {
    if (static_cast<int>(threadIdx.x) < stride) sm[threadIdx.x] = merge(sm[threadIdx.x], sm[threadIdx.x + stride]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int b = bh / H, h = bh % H;
    double* out = partials + ((static_cast<int64_t>(tensor) * H + h) * B + b) * chunks * 4 + chunk * 4;
    out[0] = sm[0].n;
    out[1] = sm[0].mean;
    out[2] = sm[0].m2;
    out[3] = sm[0].abs_sum;
  }
}

__global__ __launch_bounds__(kThreads) void features_kernel(const double* __restrict__ partials, int chunks,
                                                            const float* __restrict__ ENT,
                                                            const float* __restrict__ ONORM,
                                                            const int32_t* __restrict__ win_eff, int B, int H,
                                                            int T, float alpha, int init,
                                                            float* __restrict__ features,
                                                            float* __restrict__ ema) {
  __shared__ double se[kThreads], sn[kThreads];
  const int h = blockIdx.x;
  double e = 0.0, n = 0.0;
  if (ENT != nullptr) {
    for (int b = 0; b < B; ++b) {
      const int64_t row0 = (static_cast<int64_t>(b) * H + h) * T;
      for (int t = threadIdx.x; t < T; t += kThreads) {
        e += ENT[row0 + t];
        n += ONORM[row0 + t];
      }
    }
  }
  se[threadIdx.x] = e;
  sn[threadIdx.x] = n;
  __syncthreads();
  for (int stride = kThreads / 2; stride > 0; stride >>= 1) {
    if (static_cast<int>(threadIdx.x) < stride) {
      se[threadIdx.x] += se[threadIdx.x + stride];
      sn[threadIdx.x] += sn[threadIdx.x + stride];
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  double x[kNumFeatures];
  for (int tensor = 0; tensor < 3; ++tensor) {
    const double* p = partials + (static_cast<int64_t>(tensor) * H + h) * B * chunks * 4;
    Mom m{0.0, 0.0, 0.0, 0.0};
    for (int i = 0; i < B * chunks; ++i) m = merge(m, Mom{p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]});
    x[2 * tensor] = m.abs_sum / m.n;
    x[2 * tensor + 1] = sqrt(m.m2 / m.n);
  }
  const double rows = static_cast<double>(B) * T;
  x[6] = se[0] / rows;
  x[7] = sn[0] / rows;
  x[8] = static_cast<double>(win_eff[h]) / T;
  for (int i = 0; i < kNumFeatures; ++i) {
    if (features != nullptr) features[h * kNumFeatures + i] = static_cast<float>(x[i]);
    if (ema != nullptr) {
      const double prev = ema[h * kNumFeatures + i];
      ema[h * kNumFeatures + i] = static_cast<float>(init ? x[i] : alpha * prev + (1.0 - alpha) * x[i]);
    }
  }
}

}  // namespace

hipError_t launch_head_features(const void* q, const void* k, const void* v, bool is_bf16, const float* ent,
                                const float* onorm, const int32_t* win_eff, int B, int H, int T, int d,
                                float alpha, bool init, float* features, float* ema, double* partials,
                                hipStream_t stream) {
  const int64_t slice = static_cast<int64_t>(T) * d;
  const int chunks = feature_chunks(T, d);
  const dim3 grid(static_cast<unsigned>(B * H * chunks), 3);
  if (is_bf16)
    hipLaunchKernelGGL(qkv_stats_kernel<bf16>, grid, dim3(kThreads), 0, stream, static_cast<const bf16*>(q),
                       static_cast<const bf16*>(k), static_cast<const bf16*>(v), slice, chunks, partials, H, B);
  else
    hipLaunchKernelGGL(qkv_stats_kernel<float>, grid, dim3(kThreads), 0, stream, static_cast<const float*>(q),
                       static_cast<const float*>(k), static_cast<const float*>(v), slice, chunks, partials, H, B);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(features_kernel, dim3(H), dim3(kThreads), 0, stream, partials, chunks, ent, onorm, win_eff, B,
                     H, T, alpha, init ? 1 : 0, features, ema);
  return hipGetLastError();
}

}  // namespace aah
