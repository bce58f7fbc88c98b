// Scalar (VALU) kernels of per-head causal local-window attention:
//   * the fp32 forward (exact fp32 arithmetic, one query row per lane);
//   * the backward preprocess D_i = sum_c dO_ic O_ic (stored as -D_i, next to
//     -lse_i / scale);
//   * the fp32 backward: dQ one query row per lane, dK/dV one key row per lane.
//
// Operation: "Asymmetric Attention Heads" section 5.8 -- key j is visible to
// query i iff i - W < j <= i; A = softmax(scale Q K^T + M_W), Y = A V.  The
// backward gradients are those of sum(Y * dO):
//   P_ij = exp(scale q_i.k_j - lse_i),  dP_ij = dO_i.v_j,  D_i = sum_j P_ij dP_ij,
//   dS_ij = P_ij (dP_ij - D_i),  dQ_i = scale sum_j dS_ij k_j,
//   dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i.
// D_i is computed as dO_i . O_i, which equals sum_j P_ij dP_ij because O_i = sum_j P_ij v_j.
// With S sink keys per head ("Autonomy-of-Heads", section 5) key j is also
// visible to every query i >= j when j < S; items then visit the sink tiles
// before their window tiles (forward and dQ), and dK/dV items of sink keys
// run to the last query tile (the planner's range).
// With ENT / ONORM set, the fp32 forward also writes each row's attention
// entropy -sum_j p_j ln p_j and the Euclidean norm of its output row
// ("Asymmetric Attention Heads" section 5.3 diagnostics): entropy =
// ln 2 (log2 l - a / l) with a = sum_j w_j (s_j - m), kept against the running
// max like l.
#include <cmath>

#include "kernels.hpp"

namespace aah {
namespace {

typedef __bf16 bf16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = kSimpleRowTile;  // rows per item = lanes per workgroup
constexpr int kCols = kSimpleColTile;  // streamed rows per LDS stage
constexpr int kChunk = 16;             // keys scored per inner pass
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return static_cast<float>(x); }

// Key j visible to query i: causal, and inside the window of W or a sink (j < S).
__device__ inline bool visible(int i, int j, int W, int S) { return j <= i && (j > i - W || j < S); }

// Sink tiles an item visits before its window tiles [lo, hi).
__device__ inline int n_sink_tiles(int S, int lo) { return min((S + kCols - 1) / kCols, lo); }

// First element of the key/value head read by query head bh = b H + h: b H_kv + h / (H / H_kv).
__device__ inline size_t kv_base(int bh, int H, int H_kv, int T, int D) {
  return (static_cast<size_t>(bh / H) * H_kv + (bh % H) / (H / H_kv)) * T * D;
}
template <typename E> __device__ inline E from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }

// Copy rows [r0, r0 + kCols) of a [T, D] tensor into an fp32 LDS tile; rows past T are zero.
template <typename E, int D>
__device__ inline void stage_rows(float* dst, const E* src, int r0, int T) {
  for (int e = threadIdx.x; e < kCols * D; e += blockDim.x) {
    const int row = r0 + e / D;
    dst[e] = row < T ? to_f32(src[static_cast<size_t>(row) * D + e % D]) : 0.f;
  }
}

// ---------------------------------------------------------------- fp32 forward

template <int D>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, float* __restrict__ ENT, float* __restrict__ ONORM,
    const WorkItem* __restrict__ items, const int32_t* __restrict__ win_eff, const int32_t* __restrict__ sink_eff,
    int H, int H_kv, int T, float c) {
  __shared__ float ks[kCols * D];
  __shared__ float vs[kCols * D];
  const WorkItem it = items[blockIdx.x];
  if (it.bh < 0) return;
  const int W = win_eff[it.bh % H];
  const int S = sink_eff == nullptr ? 0 : sink_eff[it.bh % H];
  const int ns = n_sink_tiles(S, it.lo);
  const size_t base = static_cast<size_t>(it.bh) * T * D;
  const size_t kvbase = kv_base(it.bh, H, H_kv, T, D);
  const int qi = it.tile * kRows + threadIdx.x;
  const bool row_ok = qi < T;

  float qr[D], acc[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    qr[x] = row_ok ? Q[base + static_cast<size_t>(qi) * D + x] : 0.f;
    acc[x] = 0.f;
  }
  float m = -INFINITY, l = 0.f;  // log2-domain running max and running sum
  float a = 0.f;                 // sum of the weights times their offsets from the max (entropy)
  const bool diag = ENT != nullptr;

  for (int v = 0; v < ns + it.hi - it.lo; ++v) {
    const int k0 = (v < ns ? v : v - ns + it.lo) * kCols;
    __syncthreads();
    stage_rows<float, D>(ks, K + kvbase, k0, T);
    stage_rows<float, D>(vs, V + kvbase, k0, T);
    __syncthreads();
    for (int j0 = 0; j0 < kCols; j0 += kChunk) {
      float s[kChunk];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const int key = k0 + j0 + j;
        float dot = 0.f;
#pragma unroll
        for (int x = 0; x < D; ++x) dot = fmaf(qr[x], ks[(j0 + j) * D + x], dot);
        const bool ok = visible(qi, key, W, S) && key < T;
        s[j] = ok ? dot * c : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float m_new = fmaxf(m, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m - m_use);
      if (diag) a = m == -INFINITY ? 0.f : alpha * fmaf(m - m_use, l, a);
      l *= alpha;
#pragma unroll
      for (int x = 0; x < D; ++x) acc[x] *= alpha;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const float p = exp2f(s[j] - m_use);
        if (diag && p > 0.f) a = fmaf(p, s[j] - m_use, a);
        l += p;
#pragma unroll
        for (int x = 0; x < D; ++x) acc[x] = fmaf(p, vs[(j0 + j) * D + x], acc[x]);
      }
      m = m_new;
    }
  }
  if (!row_ok) return;
  const float inv = 1.f / l;
  float sq = 0.f;
#pragma unroll
  for (int x = 0; x < D; ++x) {
    O[base + static_cast<size_t>(qi) * D + x] = acc[x] * inv;
    sq = fmaf(acc[x] * inv, acc[x] * inv, sq);
  }
  const size_t row = static_cast<size_t>(it.bh) * T + qi;
  LSE[row] = (m + log2f(l)) * kLn2;
  if (diag) {
    ENT[row] = (log2f(l) - a * inv) * kLn2;
    ONORM[row] = sqrtf(sq);
  }
}

// ---------------------------------------------------------------- backward preprocess

// Each thread reduces one 16-byte chunk of a row; the D/E lanes of a row then
// combine with xor-shuffles (E = elements per chunk).  Writes, per row,
// nl2 = -lse log2(e) and nD = -(dO . O): a weight is exp2(scale log2(e) s + nl2)
// and dS = p * (dp + nD), where s = q . k and dp = dO . v are unscaled.
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const E* __restrict__ O, const E* __restrict__ dO,
                                                      const float* __restrict__ LSE, float* __restrict__ NL2,
                                                      float* __restrict__ ND, int64_t rows) {
  constexpr int kPer = 16 / sizeof(E);
  constexpr int kLanesPerRow = D / kPer;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t row = t / kLanesPerRow;
  const int part = static_cast<int>(t % kLanesPerRow);
  float sum = 0.f;
  if (row < rows) {
    const u32x4 ov = *reinterpret_cast<const u32x4*>(O + row * D + part * kPer);
    const u32x4 gv = *reinterpret_cast<const u32x4*>(dO + row * D + part * kPer);
    const E* oe = reinterpret_cast<const E*>(&ov);
    const E* ge = reinterpret_cast<const E*>(&gv);
#pragma unroll
    for (int x = 0; x < kPer; ++x) sum = fmaf(to_f32(oe[x]), to_f32(ge[x]), sum);
  }
#pragma unroll
  for (int off = kLanesPerRow / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (row < rows && part == 0) {
    ND[row] = -sum;
    NL2[row] = -LSE[row] * kLog2e;
  }
}

// ---------------------------------------------------------------- simple backward

// dQ: one query row per lane, over the forward work list (query tile, key tiles).
template <typename E, int D>
__global__ __launch_bounds__(kRows) void bwd_dq_simple_kernel(
    const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
    const E* __restrict__ dO, const float* __restrict__ NL2, const float* __restrict__ ND,
    E* __restrict__ dQ, const WorkItem* __restrict__ items, const int32_t* __restrict__ win_eff,
    const int32_t* __restrict__ sink_eff, int H, int H_kv, int T, float scale) {
  __shared__ float ks[kCols * D];
  __shared__ float vs[kCols * D];
  const WorkItem it = items[blockIdx.x];
  if (it.bh < 0) return;
  const int W = win_eff[it.bh % H];
  const int S = sink_eff == nullptr ? 0 : sink_eff[it.bh % H];
  const int ns = n_sink_tiles(S, it.lo);
  const size_t base = static_cast<size_t>(it.bh) * T * D;
  const size_t kvbase = kv_base(it.bh, H, H_kv, T, D);
  const int qi = it.tile * kRows + threadIdx.x;
  const bool row_ok = qi < T;
  const float c = scale * kLog2e;

  float qr[D], gr[D], dq[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    qr[x] = row_ok ? to_f32(Q[base + static_cast<size_t>(qi) * D + x]) : 0.f;
    gr[x] = row_ok ? to_f32(dO[base + static_cast<size_t>(qi) * D + x]) : 0.f;
    dq[x] = 0.f;
  }
  const float cl = row_ok ? NL2[static_cast<size_t>(it.bh) * T + qi] : 0.f;  // -lse * log2(e)
  const float nD = row_ok ? ND[static_cast<size_t>(it.bh) * T + qi] : 0.f;

  for (int v = 0; v < ns + it.hi - it.lo; ++v) {
    const int k0 = (v < ns ? v : v - ns + it.lo) * kCols;
    __syncthreads();
    stage_rows<E, D>(ks, K + kvbase, k0, T);
    stage_rows<E, D>(vs, V + kvbase, k0, T);
    __syncthreads();
    for (int j = 0; j < kCols; ++j) {
      const int key = k0 + j;
      if (!(visible(qi, key, W, S) && key < T)) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int x = 0; x < D; ++x) {
        s = fmaf(qr[x], ks[j * D + x], s);
        dp = fmaf(gr[x], vs[j * D + x], dp);
      }
      const float p = exp2f(fmaf(s, c, cl));
      const float ds = p * (dp + nD);
#pragma unroll
      for (int x = 0; x < D; ++x) dq[x] = fmaf(ds, ks[j * D + x], dq[x]);
    }
  }
  if (!row_ok) return;
#pragma unroll
  for (int x = 0; x < D; ++x) dQ[base + static_cast<size_t>(qi) * D + x] = from_f32<E>(dq[x] * scale);
}

// dK, dV: one key row per lane, over the backward work list: it.bh = b H_kv + g
// is a key/value head, whose G = H / H_kv query heads are walked one after
// another, each over the query tiles that see this key tile.
template <typename E, int D>
__global__ __launch_bounds__(kRows) void bwd_dkdv_simple_kernel(
    const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
    const E* __restrict__ dO, const float* __restrict__ NL2, const float* __restrict__ ND,
    E* __restrict__ dK, E* __restrict__ dV, const WorkItem* __restrict__ items,
    const int32_t* __restrict__ win_eff, const int32_t* __restrict__ sink_eff, int H, int H_kv, int T,
    float scale) {
  __shared__ float qs[kCols * D];
  __shared__ float gs[kCols * D];
  __shared__ float ls[kCols];
  __shared__ float ds_[kCols];
  const WorkItem it = items[blockIdx.x];
  if (it.bh < 0) return;
  const int G = H / H_kv;
  const int qh0 = (it.bh / H_kv) * H + (it.bh % H_kv) * G;  // first query head of the group (b H + h)
  const size_t base = static_cast<size_t>(it.bh) * T * D;   // K, V, dK, dV
  const int kj = it.tile * kRows + threadIdx.x;
  const bool row_ok = kj < T;
  const float c = scale * kLog2e;

  float kr[D], vr[D], dk[D], dv[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    kr[x] = row_ok ? to_f32(K[base + static_cast<size_t>(kj) * D + x]) : 0.f;
    vr[x] = row_ok ? to_f32(V[base + static_cast<size_t>(kj) * D + x]) : 0.f;
    dk[x] = 0.f;
    dv[x] = 0.f;
  }
  const int k0 = it.tile * kRows, k1 = min(T, k0 + kRows);
  for (int j = 0; j < G; ++j) {
    const int h = (qh0 + j) % H;
    const int W = win_eff[h];
    const int S = sink_eff == nullptr ? 0 : sink_eff[h];
    // The query tiles that see keys [k0, k1) in this head (the planner's per-head range).
    const int hi = (k0 < S ? T - 1 : min(T, k1 + W - 1) - 1) / kCols + 1;
    const size_t qbase = static_cast<size_t>(qh0 + j) * T * D;
    const size_t rbase = static_cast<size_t>(qh0 + j) * T;
    for (int qt = it.lo; qt < hi; ++qt) {
      const int q0 = qt * kCols;
      __syncthreads();
      stage_rows<E, D>(qs, Q + qbase, q0, T);
      stage_rows<E, D>(gs, dO + qbase, q0, T);
      for (int e = threadIdx.x; e < kCols; e += blockDim.x) {
        const int row = q0 + e;
        ls[e] = row < T ? NL2[rbase + row] : 0.f;  // -lse * log2(e)
        ds_[e] = row < T ? ND[rbase + row] : 0.f;
      }
      __syncthreads();
      for (int i = 0; i < kCols; ++i) {
        const int qrow = q0 + i;
        if (!(visible(qrow, kj, W, S) && qrow < T && row_ok)) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int x = 0; x < D; ++x) {
          s = fmaf(qs[i * D + x], kr[x], s);
          dp = fmaf(gs[i * D + x], vr[x], dp);
        }
        const float p = exp2f(fmaf(s, c, ls[i]));
        const float dsv = p * (dp + ds_[i]);
#pragma unroll
        for (int x = 0; x < D; ++x) {
          dv[x] = fmaf(p, gs[i * D + x], dv[x]);
          dk[x] = fmaf(dsv, qs[i * D + x], dk[x]);
        }
      }
    }
  }
  if (!row_ok) return;
#pragma unroll
  for (int x = 0; x < D; ++x) {
    dK[base + static_cast<size_t>(kj) * D + x] = from_f32<E>(dk[x] * scale);
    dV[base + static_cast<size_t>(kj) * D + x] = from_f32<E>(dv[x]);
  }
}

template <int D>
hipError_t fwd_f32_d(const float* q, const float* k, const float* v, float* o, float* lse, float* ent,
                     float* onorm, const WorkItem* items, int n_items, const int32_t* win_eff,
                     const int32_t* sink_eff, const AttnShape& s, hipStream_t stream) {
  hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3(n_items), dim3(kRows), 0, stream, q, k, v, o, lse, ent, onorm, items,
                     win_eff, sink_eff, s.H, s.H_kv, s.T, s.scale * kLog2e);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t pre_d(const void* o, const void* dout, const float* lse, float* nl2, float* nd, const AttnShape& s,
                 hipStream_t stream) {
  constexpr int kLanesPerRow = D / (16 / sizeof(E));
  const int64_t rows = static_cast<int64_t>(s.B) * s.H * s.T;
  const int64_t threads = rows * kLanesPerRow;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((bwd_pre_kernel<E, D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<const E*>(o), static_cast<const E*>(dout), lse, nl2, nd, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, float* ent,
                          float* onorm, const WorkItem* items, int n_items, const int32_t* win_eff,
                          const int32_t* sink_eff, const AttnShape& s, hipStream_t stream) {
  switch (s.d) {
    case 32: return fwd_f32_d<32>(q, k, v, o, lse, ent, onorm, items, n_items, win_eff, sink_eff, s, stream);
    case 64: return fwd_f32_d<64>(q, k, v, o, lse, ent, onorm, items, n_items, win_eff, sink_eff, s, stream);
    case 128: return fwd_f32_d<128>(q, k, v, o, lse, ent, onorm, items, n_items, win_eff, sink_eff, s, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_preprocess(const void* o, const void* dout, const float* lse, bool is_bf16, float* nl2,
                                 float* nd, const AttnShape& s, hipStream_t stream) {
  switch (s.d) {
    case 32: return is_bf16 ? pre_d<bf16, 32>(o, dout, lse, nl2, nd, s, stream)
                            : pre_d<float, 32>(o, dout, lse, nl2, nd, s, stream);
    case 64: return is_bf16 ? pre_d<bf16, 64>(o, dout, lse, nl2, nd, s, stream)
                            : pre_d<float, 64>(o, dout, lse, nl2, nd, s, stream);
    case 128: return is_bf16 ? pre_d<bf16, 128>(o, dout, lse, nl2, nd, s, stream)
                             : pre_d<float, 128>(o, dout, lse, nl2, nd, s, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dq_simple(const float* q, const float* k, const float* v, const float* dout, const float* nl2,
                                const float* nd, float* dq, const WorkItem* items, int n_items, const int32_t* win_eff,
                                const int32_t* sink_eff, const AttnShape& s, hipStream_t stream) {
#define AAH_DQ(DD)                                                                                                \
  hipLaunchKernelGGL((bwd_dq_simple_kernel<float, DD>), dim3(n_items), dim3(kRows), 0, stream, q, k, v, dout, nl2, \
                     nd, dq, items, win_eff, sink_eff, s.H, s.H_kv, s.T, s.scale)
  switch (s.d) {
    case 32: AAH_DQ(32); break;
    case 64: AAH_DQ(64); break;
    case 128: AAH_DQ(128); break;
    default: return hipErrorInvalidValue;
  }
#undef AAH_DQ
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_simple(const float* q, const float* k, const float* v, const float* dout,
                                  const float* nl2, const float* nd, float* dk, float* dv, const WorkItem* items,
                                  int n_items, const int32_t* win_eff, const int32_t* sink_eff, const AttnShape& s,
                                  hipStream_t stream) {
#define AAH_DKDV(DD)                                                                                            \
  hipLaunchKernelGGL((bwd_dkdv_simple_kernel<float, DD>), dim3(n_items), dim3(kRows), 0, stream, q, k, v, dout, \
                     nl2, nd, dk, dv, items, win_eff, sink_eff, s.H, s.H_kv, s.T, s.scale)
  switch (s.d) {
    case 32: AAH_DKDV(32); break;
    case 64: AAH_DKDV(64); break;
    case 128: AAH_DKDV(128); break;
    default: return hipErrorInvalidValue;
  }
#undef AAH_DKDV
  return hipGetLastError();
}

}  // namespace aah
