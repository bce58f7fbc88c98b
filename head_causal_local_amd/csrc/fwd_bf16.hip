// bf16 forward kernel of per-head causal local-window attention for gfx950.
//
// Operation: "Asymmetric Attention Heads" section 5.8 -- for each (b, h) with
// window W, A = softmax(scale * Q K^T + M_W), Y = A V, where M_W keeps key j
// for query i iff i - W < j <= i.  Also writes the per-row natural
// log-sum-exp of the scaled scores, used by the backward pass.
//
// One workgroup = one work item = 128 query rows of one head (4 waves x 32
// rows) and the contiguous range of 64-key tiles the planner listed for them;
// tiles wholly outside the window are never visited, and inside a workgroup
// each wave also skips the tiles that none of its own 32 rows can see.
//
// Data flow per 64-key tile:
//   * K and V tiles are copied row-major from HBM to LDS with 16-byte loads
//     (double-buffered: the next tile's loads are in flight while the current
//     one is used).
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (M = keys, N = queries, K = d).
//     The output layout gives lane l the query (l mod 32) and 16 keys per
//     32-key block, so the row max / row sum of the online softmax are
//     in-lane reductions plus one permlane32 swap between the half-waves.
//   * P^T (bf16) stays in registers and is the B operand of O^T += V^T P^T
//     (M = d, N = queries, K = keys).  The MFMA k-slots are mapped to keys in
//     the order the S^T output already holds them, and the V^T operand is
//     read from the row-major V tile with ds_read_b64_tr_b16, which hands each
//     lane four consecutive rows of one column.
//   * The online softmax runs in the log2 domain: exp2(s * scale * log2 e - m).
// Only tiles that touch a window edge, the diagonal or the end of the
// sequence evaluate the mask.  The running max is updated lazily: the O
// accumulators are rescaled only when some row's tile max exceeds its running
// max by more than kLazyTau (log2 units), so P never exceeds 2^kLazyTau and
// most tiles skip the rescale.  Row sums accumulate the fp32 P before its
// rounding to bf16, so the log-sum-exp carries no bf16 quantization.
// Global loads go through buffer resources whose range is the head's [T, d]
// slice, so rows past T read as zero without branches.
#include <cmath>

#include "device_common.hpp"
#include "kernels.hpp"

namespace aah {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kRows = 32 * kWaves;  // query rows per item
constexpr int kKeys = 64;           // keys per LDS stage
constexpr int kThreads = 64 * kWaves;
constexpr float kLazyTau = 8.0f;    // rescale threshold in log2 units (P <= 256)
static_assert(kRows == kFwdBf16RowTile && kKeys == kFwdBf16ColTile, "planner tile mismatch");

template <int D>
struct Cfg {
  static constexpr int kStride = D + 8;               // LDS row stride (elements): 16-byte pad
  static constexpr int kTileElems = kKeys * kStride;  // one K or V stage
  static constexpr int kChunkPerRow = D / 8;          // 16-byte chunks per row
  static constexpr int kChunksPerThread = kKeys * kChunkPerRow / kThreads;
  static constexpr int kSteps = D / 16;               // MFMA k-steps over d for S^T
  static constexpr int kBlocks = D / 32;              // 32-row blocks of O^T
  static constexpr size_t kSmemBytes = 2u * 2u * kTileElems * sizeof(bf16);
  static_assert(kChunksPerThread >= 1, "tile too small for the thread count");
};

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, const WorkItem* __restrict__ items,
    const int32_t* __restrict__ win_eff, int H, int T, float c) {
  using C = Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];

  const WorkItem it = items[blockIdx.x];
  if (it.bh < 0) return;  // padding slot (uniform over the workgroup)
  const int W = win_eff[it.bh % H];
  const size_t base = static_cast<size_t>(it.bh) * T * D;
  const bf16* Qh = Q + base;
  const bf16* Kh = K + base;
  const bf16* Vh = V + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5, ln = lane & 31;
  const int q0w = it.tile * kRows + wave * 32;  // first query row of this wave
  const int qi = q0w + ln;                      // this lane's query row
  const bool row_ok = qi < T;
  const bool wave_active = q0w < T;
  const int wave_key_lo = q0w - W + 1;          // first key any row of the wave sees (may be < 0)
  const int wave_key_hi = min(q0w + 31, T - 1); // last key any row of the wave sees

  // Q^T fragments (B operand of S^T = K Q^T): lane holds q[qi][16 s + 8 hl + 0..7].
  const uint32_t slice_bytes = static_cast<uint32_t>(T) * D * sizeof(bf16);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qh, slice_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh, slice_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh, slice_bytes);
  bf16x8 qf[C::kSteps];
#pragma unroll
  for (int s = 0; s < C::kSteps; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, load16(rq, (static_cast<uint32_t>(qi) * D + 16 * s + 8 * hl) * sizeof(bf16)));

  f32x16 acc[C::kBlocks];
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b) acc[b] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled scores (log2 domain)
  float l_run = 0.f;        // this half-wave's running sum of exp2(. - m_run)

  // Staging registers for one K and one V tile.
  u32x4 stk[C::kChunksPerThread], stv[C::kChunksPerThread];
  auto load_tile = [&](int kt) {
    const int k0 = kt * kKeys;
#pragma unroll
    for (int i = 0; i < C::kChunksPerThread; ++i) {
      const int cidx = tid + kThreads * i;
      const int row = cidx / C::kChunkPerRow;
      const int col = (cidx % C::kChunkPerRow) * 8;
      // Keys past T read as zero (masked in S, and 0 * 0 in P V).
      const uint32_t off = (static_cast<uint32_t>(k0 + row) * D + col) * sizeof(bf16);
      stk[i] = load16(rk, off);
      stv[i] = load16(rv, off);
    }
  };
  auto store_tile = [&](int buf) {
    bf16* kb = smem + buf * 2 * C::kTileElems;
    bf16* vb = kb + C::kTileElems;
#pragma unroll
    for (int i = 0; i < C::kChunksPerThread; ++i) {
      const int cidx = tid + kThreads * i;
      const int row = cidx / C::kChunkPerRow;
      const int col = (cidx % C::kChunkPerRow) * 8;
      *reinterpret_cast<u32x4*>(kb + row * C::kStride + col) = stk[i];
      *reinterpret_cast<u32x4*>(vb + row * C::kStride + col) = stv[i];
    }
  };

  // Lane-constant parts of the LDS addresses.
  const int g = lane >> 4, s16 = lane & 15;
  const int vt_row = 4 * hl + (s16 >> 2);       // + 16 * step
  const int vt_col = 16 * (g & 1) + 4 * (s16 & 3);  // + 32 * block

  load_tile(it.lo);
  store_tile(0);
  __syncthreads();

  for (int kt = it.lo; kt < it.hi; ++kt) {
    const int buf = (kt - it.lo) & 1;
    const bool has_next = kt + 1 < it.hi;
    if (has_next) load_tile(kt + 1);

    const int k0 = kt * kKeys;
    const bool needed = wave_active && k0 <= wave_key_hi && k0 + kKeys - 1 >= wave_key_lo;
    if (needed) {
      const bf16* kb = smem + buf * 2 * C::kTileElems;
      const bf16* vb = kb + C::kTileElems;

      // S^T for the 64 keys of the tile (two 32-key blocks) and this wave's 32 queries.
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16{};
#pragma unroll
        for (int st = 0; st < C::kSteps; ++st) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + (32 * mb + ln) * C::kStride + 16 * st + 8 * hl);
          s[mb] = mfma(a, qf[st], s[mb]);
        }
      }

      // Mask only when some (row, key) pair of the wave x tile lies outside a
      // window.  Key j is visible to row qi iff 0 <= qi - j < W; keys past T
      // fail qi - j >= 0 for every stored row, and rows past T are never stored.
      const bool interior = (k0 + kKeys - 1 <= q0w) && (k0 >= q0w + 31 - W + 1);
      if (!interior) {
        const int rel = qi - k0 - 4 * hl;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int dist = rel - (32 * mb + 8 * (r >> 2) + (r & 3));
            if (static_cast<unsigned>(dist) >= static_cast<unsigned>(W)) s[mb][r] = -INFINITY;
          }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
      const float m_tile = half_swap_max(mx) * c;
      // Lazy rescale: only when some row's max grew by more than kLazyTau.
      if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kLazyTau) != 0) {
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < C::kBlocks; ++b) acc[b] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;  // row with nothing visible yet

      // P^T fragments for the four 16-key MFMA steps.  Step st takes registers
      // 8*(st&1) .. 8*(st&1)+7 of block st>>1, i.e. keys 16 st + 8 (e/4) + 4 hl + e%4.
      bf16x8 pf[4];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[st >> 1][8 * (st & 1) + e], c, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[st >> 1][8 * (st & 1) + e + 1], c, -m_use));
          l_run += p0;
          l_run += p1;
          pf[st][e] = static_cast<bf16>(p0);
          pf[st][e + 1] = static_cast<bf16>(p1);
        }

      // O^T += V^T P^T.
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int b = 0; b < C::kBlocks; ++b) {
          const bf16x8 a = read_tr(vb + (16 * st + vt_row) * C::kStride + 32 * b + vt_col, 8 * C::kStride);
          acc[b] = mfma(a, pf[st], acc[b]);
        }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;
  const float l_tot = half_swap_sum(l_run);
  if (!row_ok) return;
  const float inv = 1.f / l_tot;
  bf16* Orow = O + base + static_cast<size_t>(qi) * D;
  // O^T block b, register r holds dim 32 b + 8 (r/4) + 4 hl + r%4 of query qi.
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      store_bf16x4(Orow + 32 * b + 8 * i + 4 * hl, acc[b][4 * i] * inv, acc[b][4 * i + 1] * inv,
                   acc[b][4 * i + 2] * inv, acc[b][4 * i + 3] * inv);
  if (hl == 0) LSE[static_cast<size_t>(it.bh) * T + qi] = (m_run + log2f(l_tot)) * kLn2;
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, float* lse,
                    const WorkItem* items, int n_items, const int32_t* win_eff,
                    const AttnShape& s, hipStream_t stream) {
  const size_t smem = Cfg<D>::kSmemBytes;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_bf16_kernel<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
  }
  const float c = s.scale * 1.4426950408889634f;  // scale * log2(e)
  hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3(n_items), dim3(kThreads), smem, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                     static_cast<bf16*>(o), lse, items, win_eff, s.H, s.T, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const WorkItem* items, int n_items, const int32_t* win_eff,
                           const AttnShape& s, hipStream_t stream) {
  switch (s.d) {
    case 32: return launch_d<32>(q, k, v, o, lse, items, n_items, win_eff, s, stream);
    case 64: return launch_d<64>(q, k, v, o, lse, items, n_items, win_eff, s, stream);
    case 128: return launch_d<128>(q, k, v, o, lse, items, n_items, win_eff, s, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace aah
