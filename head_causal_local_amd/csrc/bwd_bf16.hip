// bf16 backward kernels of per-head causal local-window attention for gfx950.
//
// Gradients of sum(O * dO) for A = softmax(scale Q K^T + M_W), O = A V
// ("Asymmetric Attention Heads" section 5.8 mask: key j visible to query i iff
// i - W < j <= i), given the forward's per-row log-sum-exp:
//   P = exp(scale Q K^T - lse),  dP = dO V^T,  dS = P * (dP - D),  D_i = dO_i . O_i,
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
//
// Two kernels, no atomics, every output written exactly once:
//
// bwd_dkdv_kernel -- one item = 128 keys of one head (4 waves x 32 keys) and
//   the 64-query steps that can see them.  K and V rows stay in registers, dK
//   and dV accumulate in registers.  Per step (Q, dO, lse, D double-buffered
//   in LDS): S = Q K^T and dP = dO V^T with M = queries, N = the wave's keys,
//   so P and dS come out with one key per lane and are directly the B operand
//   of dV^T += dO^T P and dK^T += Q^T dS (M = d, N = keys, K = queries); the
//   A operands are read transposed from the row-major Q / dO tiles.
//
// bwd_dq_kernel -- one item = 128 queries of one head (4 waves x 32 queries)
//   and the 64-key tiles of their windows (the forward's work list).  Q and dO
//   rows stay in registers; K and V tiles are double-buffered in LDS.  Per
//   tile: S^T = K Q^T and dP^T = V dO^T with M = keys, N = the wave's queries,
//   so P^T and dS^T come out with one query per lane and are directly the B
//   operand of dQ^T += K^T dS^T, whose A operand is read transposed from the
//   row-major K tile.
//
// Recomputing S and dP in both kernels costs 4 d flops per in-window pair on
// top of the 10 d of a fused backward; in exchange dQ needs no fp32
// accumulator in HBM and no atomics (which this device resolves in memory,
// not in L2), and every gradient is deterministic.
//
// In both kernels a wave skips the MFMAs of a step none of its rows/keys can
// see, and only steps that touch a window edge or the diagonal evaluate the
// mask.  Rows and keys past T read as zero through bounds-checked buffer
// loads and are never stored.
#include <cmath>

#include "device_common.hpp"
#include "kernels.hpp"

namespace aah {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStat = 32 * kWaves;   // stationary rows per item (keys for dK/dV, queries for dQ)
constexpr int kStep = 64;            // streamed rows per step
static_assert(kStat == kBwdBf16RowTile && kStep == kBwdBf16ColTile, "planner tile mismatch (dK/dV)");
static_assert(kStat == kFwdBf16RowTile && kStep == kFwdBf16ColTile, "planner tile mismatch (dQ)");

template <int D>
struct Cfg {
  static constexpr int kStride = D + 8;              // LDS row stride (elements): 16-byte pad
  static constexpr int kTile = kStep * kStride;      // one streamed tile
  static constexpr int kSteps = D / 16;              // MFMA k-steps over d
  static constexpr int kBlocks = D / 32;             // 32-wide blocks over d
  static constexpr int kChunkPerRow = D / 8;         // 16-byte chunks per row
  static constexpr int kChunks = kStep * kChunkPerRow / kThreads;  // per thread per tile
  static constexpr size_t kBytes = 2u * 2u * kTile * sizeof(bf16) + 2u * 2u * kStep * sizeof(float);
  static_assert(kChunks >= 1, "tile too small for the thread count");
};

// ---------------------------------------------------------------- dK, dV

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16* __restrict__ dK, bf16* __restrict__ dV, const WorkItem* __restrict__ items,
    const int32_t* __restrict__ win_eff, int H, int T, float scale) {
  using C = Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];
  float* const rowf = reinterpret_cast<float*>(smem + 2 * 2 * C::kTile);  // [buf][lse2 | scale*D][kStep]

  const WorkItem it = items[blockIdx.x];
  if (it.bh < 0) return;
  const int W = win_eff[it.bh % H];
  const size_t base = static_cast<size_t>(it.bh) * T * D;
  const size_t rbase = static_cast<size_t>(it.bh) * T;
  const float c = scale * kLog2e;
  const uint32_t slice = static_cast<uint32_t>(T) * D * sizeof(bf16);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + base, slice);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(dO + base, slice);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(LSE + rbase, static_cast<uint32_t>(T) * sizeof(float));
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(Dv + rbase, static_cast<uint32_t>(T) * sizeof(float));

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5, ln = lane & 31;
  const int g = lane >> 4, s16 = lane & 15;
  const int k0w = it.tile * kStat + 32 * wave;  // first key of this wave
  const int key = k0w + ln;                      // this lane's key (column of S)

  // K and V rows (B operands of S = Q K^T and dP = dO V^T): lane holds dims 16 st + 8 hl + 0..7.
  bf16x8 kf[C::kSteps], vf[C::kSteps];
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + base, slice);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + base, slice);
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) {
      const uint32_t off = (static_cast<uint32_t>(key) * D + 16 * st + 8 * hl) * sizeof(bf16);
      kf[st] = __builtin_bit_cast(bf16x8, load16(rk, off));
      vf[st] = __builtin_bit_cast(bf16x8, load16(rv, off));
    }
  }

  u32x4 stq[C::kChunks], stg[C::kChunks];
  float st_l = 0.f, st_d = 0.f;
  auto load_step = [&](int qt) {
    const int q0 = qt * kStep;
#pragma unroll
    for (int i = 0; i < C::kChunks; ++i) {
      const int cidx = tid + kThreads * i;
      const uint32_t off = (static_cast<uint32_t>(q0 + cidx / C::kChunkPerRow) * D + (cidx % C::kChunkPerRow) * 8) *
                           sizeof(bf16);
      stq[i] = load16(rq, off);
      stg[i] = load16(rg, off);
    }
    if (tid < kStep) {
      // Rows past T read lse = D = 0; their Q and dO are zero, so they add nothing.
      st_l = load_f32(rl, static_cast<uint32_t>(q0 + tid) * sizeof(float)) * kLog2e;
      st_d = load_f32(rd, static_cast<uint32_t>(q0 + tid) * sizeof(float)) * scale;
    }
  };
  auto store_step = [&](int buf) {
    bf16* qs = smem + buf * 2 * C::kTile;
    bf16* gs = qs + C::kTile;
#pragma unroll
    for (int i = 0; i < C::kChunks; ++i) {
      const int cidx = tid + kThreads * i;
      const int off = (cidx / C::kChunkPerRow) * C::kStride + (cidx % C::kChunkPerRow) * 8;
      *reinterpret_cast<u32x4*>(qs + off) = stq[i];
      *reinterpret_cast<u32x4*>(gs + off) = stg[i];
    }
    if (tid < kStep) {
      rowf[buf * 2 * kStep + tid] = st_l;
      rowf[buf * 2 * kStep + kStep + tid] = st_d;
    }
  };

  f32x16 dk[C::kBlocks], dv[C::kBlocks];
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b) {
    dk[b] = f32x16{};
    dv[b] = f32x16{};
  }
  // Transposed reads in the slot order of the P / dS registers (second read 8 rows down).
  const int tr_off = (4 * hl + (s16 >> 2)) * C::kStride + 16 * (g & 1) + 4 * (s16 & 3);

  load_step(it.lo);
  store_step(0);
  __syncthreads();

  for (int qt = it.lo; qt < it.hi; ++qt) {
    const int buf = (qt - it.lo) & 1;
    const bool has_next = qt + 1 < it.hi;
    if (has_next) load_step(qt + 1);
    const int q0 = qt * kStep;

    // Can any query of this step see any key of this wave?
    if (k0w <= q0 + kStep - 1 && k0w + 31 > q0 - W && k0w < T) {
      const bf16* qs = smem + buf * 2 * C::kTile;
      const bf16* gs = qs + C::kTile;
      const float* lse2 = rowf + buf * 2 * kStep;
      const float* sD = lse2 + kStep;
      f32x16 s[2], dp[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16{};
        dp[mb] = f32x16{};
#pragma unroll
        for (int st = 0; st < C::kSteps; ++st) {
          const int off = (32 * mb + ln) * C::kStride + 16 * st + 8 * hl;
          s[mb] = mfma(*reinterpret_cast<const bf16x8*>(qs + off), kf[st], s[mb]);
          dp[mb] = mfma(*reinterpret_cast<const bf16x8*>(gs + off), vf[st], dp[mb]);
        }
      }
      // Register r of block mb holds query q0 + 32 mb + 8 (r/4) + 4 hl + r%4.
      const bool interior = (k0w + 31 <= q0) && (k0w > q0 + kStep - 1 - W);
      bf16x8 pf[4], df[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r0 = 32 * mb + 8 * i + 4 * hl;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + r0);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(sD + r0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * i + j;
            float sv = s[mb][r];
            if (!interior && static_cast<unsigned>(q0 + r0 + j - key) >= static_cast<unsigned>(W)) sv = -INFINITY;
            const float p = __builtin_amdgcn_exp2f(fmaf(sv, c, -l4[j]));
            const float ds = p * fmaf(dp[mb][r], scale, -d4[j]);
            const int st = 2 * mb + (i >> 1);
            const int e = 4 * (i & 1) + j;
            pf[st][e] = static_cast<bf16>(p);
            df[st][e] = static_cast<bf16>(ds);
          }
        }
      // dV^T += dO^T P,  dK^T += Q^T dS   (K = the step's 64 queries in 4 MFMA steps).
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int b = 0; b < C::kBlocks; ++b) {
          const int off = 16 * st * C::kStride + 32 * b + tr_off;
          dv[b] = mfma(read_tr(gs + off, 8 * C::kStride), pf[st], dv[b]);
          dk[b] = mfma(read_tr(qs + off, 8 * C::kStride), df[st], dk[b]);
        }
    }

    if (has_next) store_step(buf ^ 1);
    __syncthreads();
  }

  if (key >= T) return;
  bf16* dkrow = dK + base + static_cast<size_t>(key) * D;
  bf16* dvrow = dV + base + static_cast<size_t>(key) * D;
  // dK^T / dV^T block b, register r: dim 32 b + 8 (r/4) + 4 hl + r%4 of this lane's key.
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = 32 * b + 8 * i + 4 * hl;
      store_bf16x4(dkrow + col, dk[b][4 * i], dk[b][4 * i + 1], dk[b][4 * i + 2], dk[b][4 * i + 3]);
      store_bf16x4(dvrow + col, dv[b][4 * i], dv[b][4 * i + 1], dv[b][4 * i + 2], dv[b][4 * i + 3]);
    }
}

// ---------------------------------------------------------------- dQ

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16* __restrict__ dQ, const WorkItem* __restrict__ items, const int32_t* __restrict__ win_eff, int H,
    int T, float scale) {
  using C = Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];

  const WorkItem it = items[blockIdx.x];
  if (it.bh < 0) return;
  const int W = win_eff[it.bh % H];
  const size_t base = static_cast<size_t>(it.bh) * T * D;
  const size_t rbase = static_cast<size_t>(it.bh) * T;
  const float c = scale * kLog2e;
  const uint32_t slice = static_cast<uint32_t>(T) * D * sizeof(bf16);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + base, slice);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + base, slice);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5, ln = lane & 31;
  const int g = lane >> 4, s16 = lane & 15;
  const int q0w = it.tile * kStat + 32 * wave;   // first query of this wave
  const int qi = q0w + ln;                        // this lane's query (column of S^T)
  const bool wave_active = q0w < T;
  const int wave_key_lo = q0w - W + 1;
  const int wave_key_hi = min(q0w + 31, T - 1);

  // Q and dO rows of this lane's query (B operands of S^T = K Q^T and dP^T = V dO^T).
  bf16x8 qf[C::kSteps], gf[C::kSteps];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + base, slice);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(dO + base, slice);
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) {
      const uint32_t off = (static_cast<uint32_t>(qi) * D + 16 * st + 8 * hl) * sizeof(bf16);
      qf[st] = __builtin_bit_cast(bf16x8, load16(rq, off));
      gf[st] = __builtin_bit_cast(bf16x8, load16(rg, off));
    }
  }
  const bool row_ok = qi < T;
  const float lse2 = row_ok ? LSE[rbase + qi] * kLog2e : 0.f;
  const float sD = row_ok ? Dv[rbase + qi] * scale : 0.f;

  u32x4 stk[C::kChunks], stv[C::kChunks];
  auto load_tile = [&](int kt) {
    const int k0 = kt * kStep;
#pragma unroll
    for (int i = 0; i < C::kChunks; ++i) {
      const int cidx = tid + kThreads * i;
      const uint32_t off = (static_cast<uint32_t>(k0 + cidx / C::kChunkPerRow) * D + (cidx % C::kChunkPerRow) * 8) *
                           sizeof(bf16);
      stk[i] = load16(rk, off);
      stv[i] = load16(rv, off);
    }
  };
  auto store_tile = [&](int buf) {
    bf16* ks = smem + buf * 2 * C::kTile;
    bf16* vs = ks + C::kTile;
#pragma unroll
    for (int i = 0; i < C::kChunks; ++i) {
      const int cidx = tid + kThreads * i;
      const int off = (cidx / C::kChunkPerRow) * C::kStride + (cidx % C::kChunkPerRow) * 8;
      *reinterpret_cast<u32x4*>(ks + off) = stk[i];
      *reinterpret_cast<u32x4*>(vs + off) = stv[i];
    }
  };

  f32x16 acc[C::kBlocks];
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b) acc[b] = f32x16{};
  const int tr_off = (4 * hl + (s16 >> 2)) * C::kStride + 16 * (g & 1) + 4 * (s16 & 3);

  load_tile(it.lo);
  store_tile(0);
  __syncthreads();

  for (int kt = it.lo; kt < it.hi; ++kt) {
    const int buf = (kt - it.lo) & 1;
    const bool has_next = kt + 1 < it.hi;
    if (has_next) load_tile(kt + 1);
    const int k0 = kt * kStep;

    if (wave_active && k0 <= wave_key_hi && k0 + kStep - 1 >= wave_key_lo) {
      const bf16* ks = smem + buf * 2 * C::kTile;
      const bf16* vs = ks + C::kTile;
      f32x16 s[2], dp[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16{};
        dp[mb] = f32x16{};
#pragma unroll
        for (int st = 0; st < C::kSteps; ++st) {
          const int off = (32 * mb + ln) * C::kStride + 16 * st + 8 * hl;
          s[mb] = mfma(*reinterpret_cast<const bf16x8*>(ks + off), qf[st], s[mb]);
          dp[mb] = mfma(*reinterpret_cast<const bf16x8*>(vs + off), gf[st], dp[mb]);
        }
      }
      // Register r of block mb holds key k0 + 32 mb + 8 (r/4) + 4 hl + r%4.  Keys past T
      // fail qi - key >= 0 for every stored row.
      const bool interior = (k0 + kStep - 1 <= q0w) && (k0 >= q0w + 31 - W + 1);
      const int rel = qi - k0 - 4 * hl;
      bf16x8 df[4];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int mb = st >> 1, r = 8 * (st & 1) + e;
          float sv = s[mb][r];
          if (!interior && static_cast<unsigned>(rel - (32 * mb + 8 * (r >> 2) + (r & 3))) >= static_cast<unsigned>(W))
            sv = -INFINITY;
          const float p = __builtin_amdgcn_exp2f(fmaf(sv, c, -lse2));
          df[st][e] = static_cast<bf16>(p * fmaf(dp[mb][r], scale, -sD));
        }
      // dQ^T += K^T dS^T  (K = the tile's 64 keys in 4 MFMA steps, slot order of the dS registers).
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int b = 0; b < C::kBlocks; ++b)
          acc[b] = mfma(read_tr(ks + 16 * st * C::kStride + 32 * b + tr_off, 8 * C::kStride), df[st], acc[b]);
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!row_ok) return;
  bf16* dqrow = dQ + base + static_cast<size_t>(qi) * D;
  // dQ^T block b, register r: dim 32 b + 8 (r/4) + 4 hl + r%4 of this lane's query.
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      store_bf16x4(dqrow + 32 * b + 8 * i + 4 * hl, acc[b][4 * i], acc[b][4 * i + 1], acc[b][4 * i + 2],
                   acc[b][4 * i + 3]);
}

template <typename Kernel>
hipError_t allow_smem(Kernel* k, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(bytes));
}

template <int D>
hipError_t dkdv_d(const void* q, const void* k, const void* v, const void* dout, const float* lse, const float* Dv,
                  void* dk, void* dv, const WorkItem* items, int n_items, const int32_t* win_eff,
                  const AttnShape& s, hipStream_t stream) {
  const size_t smem = Cfg<D>::kBytes;
  hipError_t e = allow_smem(&bwd_dkdv_kernel<D>, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(n_items), dim3(kThreads), smem, stream, static_cast<const bf16*>(q),
                     static_cast<const bf16*>(k), static_cast<const bf16*>(v), static_cast<const bf16*>(dout), lse, Dv,
                     static_cast<bf16*>(dk), static_cast<bf16*>(dv), items, win_eff, s.H, s.T, s.scale);
  return hipGetLastError();
}

template <int D>
hipError_t dq_d(const void* q, const void* k, const void* v, const void* dout, const float* lse, const float* Dv,
                void* dq, const WorkItem* items, int n_items, const int32_t* win_eff, const AttnShape& s,
                hipStream_t stream) {
  const size_t smem = Cfg<D>::kBytes;
  hipError_t e = allow_smem(&bwd_dq_kernel<D>, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(n_items), dim3(kThreads), smem, stream, static_cast<const bf16*>(q),
                     static_cast<const bf16*>(k), static_cast<const bf16*>(v), static_cast<const bf16*>(dout), lse, Dv,
                     static_cast<bf16*>(dq), items, win_eff, s.H, s.T, s.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                const float* D, void* dk, void* dv, const WorkItem* items, int n_items,
                                const int32_t* win_eff, const AttnShape& s, hipStream_t stream) {
  switch (s.d) {
    case 32: return dkdv_d<32>(q, k, v, dout, lse, D, dk, dv, items, n_items, win_eff, s, stream);
    case 64: return dkdv_d<64>(q, k, v, dout, lse, D, dk, dv, items, n_items, win_eff, s, stream);
    case 128: return dkdv_d<128>(q, k, v, dout, lse, D, dk, dv, items, n_items, win_eff, s, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                              const float* D, void* dq, const WorkItem* items, int n_items, const int32_t* win_eff,
                              const AttnShape& s, hipStream_t stream) {
  switch (s.d) {
    case 32: return dq_d<32>(q, k, v, dout, lse, D, dq, items, n_items, win_eff, s, stream);
    case 64: return dq_d<64>(q, k, v, dout, lse, D, dq, items, n_items, win_eff, s, stream);
    case 128: return dq_d<128>(q, k, v, dout, lse, D, dq, items, n_items, win_eff, s, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace aah
