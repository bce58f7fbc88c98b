// Per-head controller features of "Asymmetric Attention Heads" section 5.3
// (Head features and EMA smoothing), on the device:
//   x_h = [mu(|q_h|), sigma(q_h), mu(|k_h|), sigma(k_h), mu(|v_h|), sigma(v_h), e_h, n_h, rho_h]
// with the Q/K/V entries reduced over batch, sequence and head dimension of head
// h (mean of the absolute activations; population standard deviation), e_h and
// n_h the means over batch and rows of the per-row attention entropy and output
// norm that a diagnostic forward pass wrote, rho_h = min(W_h, T) / T the window
// usage of that pass (all three 0 when there are no such rows: missing
// previous-attention diagnostics start at zero), and the smoothing
// xbar = alpha xbar + (1 - alpha) x (xbar = x at the first update).
//
// Two launches, deterministic (fixed reduction order, no atomics):
//   qkv_stats_kernel: one workgroup per 32768-element span of one (b, h) slice
//     of Q, K or V (grid y = 0, 1, 2 picks the tensor).  The slice is
//     contiguous in the [B, H, T, d] layout, so each lane streams 16-byte
//     vectors, four loads in flight.  Lanes keep fp32 sums of x - x0 and
//     (x - x0)^2 about their own first element x0 (no cancellation when the
//     mean is large against the spread) and of |x|; the workgroup merges them
//     pairwise in fp64 (count, mean, M2) and writes one partial.  Grid y = 3
//     sums the matching 1/chunks of the (b, h) entropy and norm rows.
//     HBM-bound: every element is read once.
//   features_kernel: one wave per head merges the head's partials (lanes take
//     strided shares, then a fixed tree over the lanes) and writes x_h and the
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

// Grid y = 3: sums of the entropy and norm rows [r0, r1) of one (b, h), r0..r1 its chunk-th share.
__device__ void row_sums(const float* __restrict__ ENT, const float* __restrict__ ONORM, int bh, int chunk,
                         int chunks, int T, double* __restrict__ out) {
  __shared__ double se[kThreads], sn[kThreads];
  const int per = (T + chunks - 1) / chunks;
  const int r0 = chunk * per, r1 = min(T, r0 + per);
  const int64_t base = static_cast<int64_t>(bh) * T;
  double e = 0.0, n = 0.0;
  for (int r = r0 + threadIdx.x; r < r1; r += kThreads) {
    e += ENT[base + r];
    n += ONORM[base + r];
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
  if (threadIdx.x == 0) {
    out[0] = se[0];
    out[1] = sn[0];
  }
}

template <typename E>
__global__ __launch_bounds__(kThreads) void qkv_stats_kernel(const E* __restrict__ Q, const E* __restrict__ K,
                                                             const E* __restrict__ V,
                                                             const float* __restrict__ ENT,
                                                             const float* __restrict__ ONORM, int T,
                                                             int64_t slice, int chunks,
                                                             double* __restrict__ partials,
                                                             double* __restrict__ row_partials, int H, int H_kv,
                                                             int B) {
  constexpr int kPer = 16 / sizeof(E);  // elements per 16-byte vector
  constexpr int kUnroll = 4;            // vectors in flight per lane
  __shared__ Mom sm[kThreads];
  const int bh = blockIdx.x / chunks, chunk = blockIdx.x % chunks;
  const int tensor = blockIdx.y;
  // K and V have H_kv heads per batch entry: workgroups past B H_kv slices have nothing to do.
  if ((tensor == 1 || tensor == 2) && bh >= B * H_kv) return;
  const int Ht = (tensor == 1 || tensor == 2) ? H_kv : H;  // heads of this tensor
  if (tensor == 3) {  // uniform over the workgroup
    const int b = bh / H, h = bh % H;
    row_sums(ENT, ONORM, bh, chunk, chunks, T, row_partials + ((static_cast<int64_t>(h) * B + b) * chunks + chunk) * 2);
    return;
  }
  const E* src = (tensor == 0 ? Q : tensor == 1 ? K : V) + static_cast<int64_t>(bh) * slice +
                 static_cast<int64_t>(chunk) * kFeatureSpan;
  const int64_t left = slice - static_cast<int64_t>(chunk) * kFeatureSpan;
  const int n_vec = static_cast<int>((left < kFeatureSpan ? left : kFeatureSpan) / kPer);

  float x0 = 0.f, s1 = 0.f, s2 = 0.f, sa = 0.f;
  int cnt = 0;
  if (static_cast<int>(threadIdx.x) < n_vec) x0 = to_f32(src[threadIdx.x * kPer]);
  auto take = [&](const u32x4& raw) __attribute__((always_inline)) {
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
  };
  int vi = threadIdx.x;
  for (; vi + (kUnroll - 1) * kThreads < n_vec; vi += kUnroll * kThreads) {
    u32x4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      raw[u] = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(vi + u * kThreads) * kPer);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) take(raw[u]);
  }
  for (; vi < n_vec; vi += kThreads) take(*reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(vi) * kPer));
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
    const int b = bh / Ht, h = bh % Ht;
    double* out = partials + ((static_cast<int64_t>(tensor) * H + h) * B + b) * chunks * 4 + chunk * 4;
    out[0] = sm[0].n;
    out[1] = sm[0].mean;
    out[2] = sm[0].m2;
    out[3] = sm[0].abs_sum;
  }
}

__global__ __launch_bounds__(64) void features_kernel(const double* __restrict__ partials,
                                                      const double* __restrict__ row_partials, int chunks,
                                                      bool have_rows, const int32_t* __restrict__ win_eff, int B,
                                                      int H, int H_kv, int T, float alpha, int init,
                                                      float* __restrict__ features, float* __restrict__ ema) {
  __shared__ Mom sm[3][64];
  __shared__ double sr[2][64];
  __shared__ double sx[kNumFeatures];
  const int h = blockIdx.x;
  const int lane = threadIdx.x;
  const int n = B * chunks;  // partials per head and tensor
  // Lane i < 9 owns feature i of this head; its previous smoothed value is fetched now so that the
  // load's latency overlaps the merges.
  const bool owner = lane < kNumFeatures;
  const float prev = (owner && ema != nullptr && !init) ? ema[h * kNumFeatures + lane] : 0.f;
  const int w_h = win_eff[h];
  // Lane i merges partials i, i + 64, ... of every tensor (all loads of a round issued together), then a
  // fixed tree over the lanes.
  Mom m[3] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
  double e = 0.0, nr = 0.0;
  for (int i = lane; i < n; i += 64) {
    Mom in[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int hh = t == 0 ? h : h / (H / H_kv);  // K and V: the query head's key/value head
      const double* p = partials + ((static_cast<int64_t>(t) * H + hh) * n + i) * 4;
      in[t] = Mom{p[0], p[1], p[2], p[3]};
    }
    if (have_rows) {
      const double* p = row_partials + (static_cast<int64_t>(h) * n + i) * 2;
      e += p[0];
      nr += p[1];
    }
#pragma unroll
    for (int t = 0; t < 3; ++t) m[t] = merge(m[t], in[t]);
  }
#pragma unroll
  for (int t = 0; t < 3; ++t) sm[t][lane] = m[t];
  sr[0][lane] = e;
  sr[1][lane] = nr;
  __syncthreads();
  for (int stride = 32; stride > 0; stride >>= 1) {
    if (lane < stride) {
#pragma unroll
      for (int t = 0; t < 3; ++t) sm[t][lane] = merge(sm[t][lane], sm[t][lane + stride]);
      sr[0][lane] += sr[0][lane + stride];
      sr[1][lane] += sr[1][lane + stride];
    }
    __syncthreads();
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      sx[2 * t] = sm[t][0].abs_sum / sm[t][0].n;
      sx[2 * t + 1] = sqrt(sm[t][0].m2 / sm[t][0].n);
    }
    const double rows = static_cast<double>(B) * T;
    sx[6] = sr[0][0] / rows;
    sx[7] = sr[1][0] / rows;
    // Usage belongs to the stored statistics like e_h and n_h: zero when there are none (section 5.3),
    // else the share of the context the window of the forward that produced them covers.
    sx[8] = have_rows ? static_cast<double>(w_h) / T : 0.0;
  }
  __syncthreads();
  if (!owner) return;
  const double x = sx[lane];
  if (features != nullptr) features[h * kNumFeatures + lane] = static_cast<float>(x);
  if (ema != nullptr)
    ema[h * kNumFeatures + lane] = static_cast<float>(init ? x : alpha * static_cast<double>(prev) + (1.0 - alpha) * x);
}

}  // namespace

hipError_t launch_head_features(const void* q, const void* k, const void* v, bool is_bf16, const float* ent,
                                const float* onorm, const int32_t* win_eff, int B, int H, int H_kv, int T, int d,
                                float alpha, bool init, float* features, float* ema, double* partials,
                                hipStream_t stream) {
  const int64_t slice = static_cast<int64_t>(T) * d;
  const int chunks = feature_chunks(T, d);
  const bool rows = ent != nullptr;
  double* row_partials = partials + static_cast<int64_t>(3) * H * B * chunks * 4;
  const dim3 grid(static_cast<unsigned>(B * H * chunks), rows ? 4 : 3);
  if (is_bf16)
    hipLaunchKernelGGL(qkv_stats_kernel<bf16>, grid, dim3(kThreads), 0, stream, static_cast<const bf16*>(q),
                       static_cast<const bf16*>(k), static_cast<const bf16*>(v), ent, onorm, T, slice, chunks,
                       partials, row_partials, H, H_kv, B);
  else
    hipLaunchKernelGGL(qkv_stats_kernel<float>, grid, dim3(kThreads), 0, stream, static_cast<const float*>(q),
                       static_cast<const float*>(k), static_cast<const float*>(v), ent, onorm, T, slice, chunks,
                       partials, row_partials, H, H_kv, B);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(features_kernel, dim3(H), dim3(64), 0, stream, partials, row_partials, chunks, rows, win_eff,
                     B, H, H_kv, T, alpha, init ? 1 : 0, features, ema);
  return hipGetLastError();
}

}  // namespace aah
