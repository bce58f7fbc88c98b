// bf16 backward kernels of per-head causal local-window attention for gfx950.
//
// Gradients of sum(O * dO) for A = softmax(scale Q K^T + M_W), O = A V
// ("Asymmetric Attention Heads" section 5.8 mask: key j visible to query i iff
// i - W < j <= i), with the forward's per-row log-sum-exp:
//   P = exp(scale Q K^T - lse),  dP = dO V^T,  dS = P * (dP - D),  D_i = dO_i . O_i,
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
//
// One workgroup = one work item = 128 keys of one head (4 waves x 32 keys)
// and the contiguous range of 64-query tiles that can see them (tiles wholly
// outside the window are never listed).  K and V stay in registers / LDS for
// the whole item; dK and dV accumulate in registers and are written once.
// Per 64-query step (Q, dO, lse, D double-buffered in LDS):
//   * S = Q K^T and dP = dO V^T on v_mfma_f32_32x32x16_bf16 with M = queries,
//     N = the wave's 32 keys, so that P and dS come out with one key per lane
//     and directly form the B operand of
//   * dV^T += dO^T P and dK^T += Q^T dS (M = d, N = keys, K = queries), whose
//     A operands are read transposed from the row-major Q / dO tiles with
//     ds_read_b64_tr_b16;
//   * dS (bf16, scale folded in) is written to LDS as [key][query]; after a
//     barrier each wave computes one 32x32 block of dQ = dS K over all 128
//     keys and adds it to an fp32 accumulator with coalesced atomics (lanes
//     0..31 cover 32 consecutive dims of one row).
// A wave whose 32 keys no query of the step can see skips its MFMAs and
// writes zeros into its part of dS.
#include <cmath>

#include "kernels.hpp"

namespace aah {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define AAH_LDS __attribute__((address_space(3)))

constexpr int kWaves = 4;
constexpr int kKeys = 32 * kWaves;  // keys per item
constexpr int kQ = 64;              // queries per step
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
static_assert(kKeys == kBwdBf16RowTile && kQ == kBwdBf16ColTile, "planner tile mismatch");

template <int D>
struct Cfg {
  static constexpr int kStride = D + 8;    // row stride (elements) of K, Q, dO tiles: 16-byte pad
  static constexpr int kDsStride = kQ + 8; // row stride of the dS [key][query] tile
  static constexpr int kSteps = D / 16;    // MFMA k-steps over d
  static constexpr int kBlocks = D / 32;   // 32-wide blocks over d
  static constexpr int kOffK = 0;                           // [kKeys][kStride]
  static constexpr int kOffQ = kOffK + kKeys * kStride;     // 2 x [kQ][kStride]
  static constexpr int kOffG = kOffQ + 2 * kQ * kStride;    // 2 x [kQ][kStride]   (dO)
  static constexpr int kOffS = kOffG + 2 * kQ * kStride;    // [kKeys][kDsStride]  (dS)
  static constexpr int kElems = kOffS + kKeys * kDsStride;  // bf16 elements; fp32 row data follows
  static constexpr size_t kBytes = kElems * sizeof(bf16) + 2 * 2 * kQ * sizeof(float);
  static constexpr int kChunkPerRow = D / 8;
  static constexpr int kQChunks = kQ * kChunkPerRow / kThreads;   // 16-byte chunks per thread per tile
  static constexpr int kKChunks = kKeys * kChunkPerRow / kThreads;
  static_assert(kQChunks >= 1 && kKChunks >= 1, "tile too small for the thread count");
  static_assert((kElems * sizeof(bf16)) % 16 == 0, "fp32 area must stay 16-byte aligned");
};

// Two transposing LDS reads: rows [r, r+4) and [r+gap, r+gap+4) of the
// addressed 4-column chunk (see the 16-lane group semantics of ds_read_b64_tr_b16).
__device__ inline bf16x8 read_tr(const bf16* p, int gap_elems) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AAH_LDS s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AAH_LDS s16x4*)(p + gap_elems));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16* __restrict__ dK, bf16* __restrict__ dV, float* __restrict__ dq_acc,
    const WorkItem* __restrict__ items, const int32_t* __restrict__ win_eff, int H, int T, float scale) {
  using C = Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];
  bf16* const Ks = smem + C::kOffK;
  bf16* const dSs = smem + C::kOffS;
  float* const rowf = reinterpret_cast<float*>(smem + C::kElems);  // [2][2][kQ]: lse2, scale*D

  const WorkItem it = items[blockIdx.x];
  if (it.bh < 0) return;
  const int W = win_eff[it.bh % H];
  const size_t base = static_cast<size_t>(it.bh) * T * D;
  const size_t rbase = static_cast<size_t>(it.bh) * T;
  const float c = scale * kLog2e;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5, ln = lane & 31;
  const int g = lane >> 4, s16 = lane & 15;
  const int k0 = it.tile * kKeys;
  const int k0w = k0 + 32 * wave;  // first key of this wave
  const int key = k0w + ln;        // this lane's key (column of S)
  const bool key_ok = key < T;

  // K and V fragments (B operands of S = Q K^T, dP = dO V^T): lane holds row `key`, dims 16 st + 8 hl + 0..7.
  bf16x8 kf[C::kSteps], vf[C::kSteps];
#pragma unroll
  for (int st = 0; st < C::kSteps; ++st) {
    if (key_ok) {
      kf[st] = *reinterpret_cast<const bf16x8*>(K + base + static_cast<size_t>(key) * D + 16 * st + 8 * hl);
      vf[st] = *reinterpret_cast<const bf16x8*>(V + base + static_cast<size_t>(key) * D + 16 * st + 8 * hl);
    } else {
      kf[st] = bf16x8{};
      vf[st] = bf16x8{};
    }
  }
  // K tile in LDS (B operand of dQ = dS K, read transposed).
#pragma unroll
  for (int i = 0; i < C::kKChunks; ++i) {
    const int cidx = tid + kThreads * i;
    const int row = cidx / C::kChunkPerRow;
    const int col = (cidx % C::kChunkPerRow) * 8;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (k0 + row < T) v = *reinterpret_cast<const u32x4*>(K + base + static_cast<size_t>(k0 + row) * D + col);
    *reinterpret_cast<u32x4*>(Ks + row * C::kStride + col) = v;
  }

  // Staging of one query step: Q and dO rows, lse * log2(e) and scale * D.
  u32x4 stq[C::kQChunks], stg[C::kQChunks];
  float st_l = 0.f, st_d = 0.f;
  auto load_step = [&](int qt) {
    const int q0 = qt * kQ;
#pragma unroll
    for (int i = 0; i < C::kQChunks; ++i) {
      const int cidx = tid + kThreads * i;
      const int row = q0 + cidx / C::kChunkPerRow;
      const int col = (cidx % C::kChunkPerRow) * 8;
      if (row < T) {
        stq[i] = *reinterpret_cast<const u32x4*>(Q + base + static_cast<size_t>(row) * D + col);
        stg[i] = *reinterpret_cast<const u32x4*>(dO + base + static_cast<size_t>(row) * D + col);
      } else {
        stq[i] = u32x4{0u, 0u, 0u, 0u};
        stg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < kQ) {
      const int row = q0 + tid;
      st_l = row < T ? LSE[rbase + row] * kLog2e : 0.f;
      st_d = row < T ? Dv[rbase + row] * scale : 0.f;
    }
  };
  auto store_step = [&](int buf) {
    bf16* qs = smem + C::kOffQ + buf * kQ * C::kStride;
    bf16* gs = smem + C::kOffG + buf * kQ * C::kStride;
#pragma unroll
    for (int i = 0; i < C::kQChunks; ++i) {
      const int cidx = tid + kThreads * i;
      const int row = cidx / C::kChunkPerRow;
      const int col = (cidx % C::kChunkPerRow) * 8;
      *reinterpret_cast<u32x4*>(qs + row * C::kStride + col) = stq[i];
      *reinterpret_cast<u32x4*>(gs + row * C::kStride + col) = stg[i];
    }
    if (tid < kQ) {
      rowf[buf * 2 * kQ + tid] = st_l;
      rowf[buf * 2 * kQ + kQ + tid] = st_d;
    }
  };

  f32x16 dk[C::kBlocks], dv[C::kBlocks];
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b) {
    dk[b] = f32x16{};
    dv[b] = f32x16{};
  }

  // Lane-constant offsets of the transposed reads.
  const int tr_col = 16 * (g & 1) + 4 * (s16 & 3);
  const int tr_row_pv = 4 * hl + (s16 >> 2);   // slot order of P / dS registers (second read at +8)
  const int tr_row_dq = 8 * hl + (s16 >> 2);   // natural key order (second read at +4)

  load_step(it.lo);
  store_step(0);
  __syncthreads();

  for (int qt = it.lo; qt < it.hi; ++qt) {
    const int buf = (qt - it.lo) & 1;
    const bool has_next = qt + 1 < it.hi;
    if (has_next) load_step(qt + 1);
    const int q0 = qt * kQ;
    const bf16* qs = smem + C::kOffQ + buf * kQ * C::kStride;
    const bf16* gs = smem + C::kOffG + buf * kQ * C::kStride;
    const float* lse2 = rowf + buf * 2 * kQ;
    const float* sD = lse2 + kQ;

    // Can any query of this step see any key of this wave?
    const bool visible = (k0w <= q0 + kQ - 1) && (k0w + 31 > q0 - W) && (k0w < T);
    if (visible) {
      f32x16 s[2], dp[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16{};
        dp[mb] = f32x16{};
#pragma unroll
        for (int st = 0; st < C::kSteps; ++st) {
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qs + (32 * mb + ln) * C::kStride + 16 * st + 8 * hl);
          const bf16x8 ag = *reinterpret_cast<const bf16x8*>(gs + (32 * mb + ln) * C::kStride + 16 * st + 8 * hl);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[st], s[mb], 0, 0, 0);
          dp[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, vf[st], dp[mb], 0, 0, 0);
        }
      }
      const bool interior = (k0w + 31 <= q0) && (k0w > q0 + kQ - 1 - W) && (q0 + kQ - 1 < T);
      // P and dS (scale folded in).  Register r of block mb is query 32 mb + 8 (r/4) + 4 hl + r%4.
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
            float p = __builtin_amdgcn_exp2f(fmaf(s[mb][r], c, -l4[j]));
            if (!interior) {
              const int qrow = q0 + r0 + j;
              const bool ok = key <= qrow && key > qrow - W && qrow < T && key_ok;
              if (!ok) p = 0.f;
            }
            const float ds = p * fmaf(dp[mb][r], scale, -d4[j]);
            const int st = 2 * mb + (i >> 1);
            const int e = 4 * (i & 1) + j;
            pf[st][e] = static_cast<bf16>(p);
            df[st][e] = static_cast<bf16>(ds);
          }
        }
      // dV^T += dO^T P, dK^T += Q^T dS  (M = d, N = keys, K = 64 queries in 4 steps).
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int b = 0; b < C::kBlocks; ++b) {
          const int off = (16 * st + tr_row_pv) * C::kStride + 32 * b + tr_col;
          const bf16x8 ag = read_tr(gs + off, 8 * C::kStride);
          const bf16x8 aq = read_tr(qs + off, 8 * C::kStride);
          dv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, pf[st], dv[b], 0, 0, 0);
          dk[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, df[st], dk[b], 0, 0, 0);
        }
      // dS to LDS as [key][query]: 4 consecutive queries per 8-byte write.
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int mb = st >> 1, i = 2 * (st & 1) + half;
          bf16x4 v4;
#pragma unroll
          for (int j = 0; j < 4; ++j) v4[j] = df[st][4 * half + j];
          *reinterpret_cast<u32x2*>(dSs + (32 * wave + ln) * C::kDsStride + 32 * mb + 8 * i + 4 * hl) =
              __builtin_bit_cast(u32x2, v4);
        }
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x2*>(dSs + (32 * wave + ln) * C::kDsStride + 32 * mb + 8 * i + 4 * hl) =
              u32x2{0u, 0u};
    }
    __syncthreads();

    // dQ (64 queries x D dims = 2 * kBlocks blocks of 32x32) += dS K over the item's 128 keys.
    constexpr int kDqBlocks = 2 * C::kBlocks;
    constexpr int kPerWave = kDqBlocks >= kWaves ? kDqBlocks / kWaves : 1;
    constexpr int kKeySplit = kDqBlocks >= kWaves ? 1 : kWaves / kDqBlocks;  // waves sharing one block
    constexpr int kStepsPerWave = (kKeys / 16) / kKeySplit;
#pragma unroll
    for (int pb = 0; pb < kPerWave; ++pb) {
      const int blk = kDqBlocks >= kWaves ? wave * kPerWave + pb : wave % kDqBlocks;
      const int ks0 = kDqBlocks >= kWaves ? 0 : (wave / kDqBlocks) * kStepsPerWave;
      const int mb = blk & 1, nb = blk >> 1;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int st = ks0; st < ks0 + kStepsPerWave; ++st) {
        const int row = 16 * st + tr_row_dq;
        const bf16x8 a = read_tr(dSs + row * C::kDsStride + 32 * mb + tr_col, 4 * C::kDsStride);
        const bf16x8 bk = read_tr(Ks + row * C::kStride + 32 * nb + tr_col, 4 * C::kStride);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bk, acc, 0, 0, 0);
      }
      // acc register r: query 32 mb + 8 (r/4) + 4 hl + r%4, dim 32 nb + ln.
      float* dst = dq_acc + base + 32 * nb + ln;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = q0 + 32 * mb + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (qrow < T) unsafeAtomicAdd(dst + static_cast<size_t>(qrow) * D, acc[r]);
      }
    }

    if (has_next) store_step(buf ^ 1);
    __syncthreads();
  }

  if (!key_ok) return;
  bf16* dkrow = dK + base + static_cast<size_t>(key) * D;
  bf16* dvrow = dV + base + static_cast<size_t>(key) * D;
  // dK^T / dV^T block b, register r: dim 32 b + 8 (r/4) + 4 hl + r%4 of key `key`.
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 k4, v4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        k4[j] = static_cast<bf16>(dk[b][4 * i + j]);
        v4[j] = static_cast<bf16>(dv[b][4 * i + j]);
      }
      *reinterpret_cast<u32x2*>(dkrow + 32 * b + 8 * i + 4 * hl) = __builtin_bit_cast(u32x2, k4);
      *reinterpret_cast<u32x2*>(dvrow + 32 * b + 8 * i + 4 * hl) = __builtin_bit_cast(u32x2, v4);
    }
}

// dQ = bf16(dq_acc); 8 elements per thread.
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc, bf16* __restrict__ dq,
                                                         int64_t n8) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(acc + 8 * t);
  const f32x4 b = *reinterpret_cast<const f32x4*>(acc + 8 * t + 4);
  bf16x8 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[j] = static_cast<bf16>(a[j]);
    o[4 + j] = static_cast<bf16>(b[j]);
  }
  *reinterpret_cast<bf16x8*>(dq + 8 * t) = o;
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                    const float* Dv, void* dk, void* dv, float* dq_acc, const WorkItem* items, int n_items,
                    const int32_t* win_eff, const AttnShape& s, hipStream_t stream) {
  const size_t smem = Cfg<D>::kBytes;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_bf16_kernel<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_bf16_kernel<D>, dim3(n_items), dim3(kThreads), smem, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                     static_cast<const bf16*>(dout), lse, Dv, static_cast<bf16*>(dk), static_cast<bf16*>(dv),
                     dq_acc, items, win_eff, s.H, s.T, s.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                           const float* D, void* dk, void* dv, float* dq_acc, const WorkItem* items, int n_items,
                           const int32_t* win_eff, const AttnShape& s, hipStream_t stream) {
  switch (s.d) {
    case 32: return launch_d<32>(q, k, v, dout, lse, D, dk, dv, dq_acc, items, n_items, win_eff, s, stream);
    case 64: return launch_d<64>(q, k, v, dout, lse, D, dk, dv, dq_acc, items, n_items, win_eff, s, stream);
    case 128: return launch_d<128>(q, k, v, dout, lse, D, dk, dv, dq_acc, items, n_items, win_eff, s, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dq_convert(const float* dq_acc, void* dq, const AttnShape& s, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(s.B) * s.H * s.T * s.d;
  const int64_t n8 = n / 8;  // d is a multiple of 32
  const int64_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL(dq_convert_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, dq_acc,
                     static_cast<bf16*>(dq), n8);
  return hipGetLastError();
}

}  // namespace aah
