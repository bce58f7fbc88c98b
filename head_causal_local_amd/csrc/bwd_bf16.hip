// bf16 backward kernels of per-head causal local-window attention for gfx950.
//
// Gradients of sum(O * dO) for A = softmax(scale Q K^T + M_W), O = A V
// ("Asymmetric Attention Heads" section 5.8 mask: key j visible to query i iff
// i - W < j <= i), given the forward's per-row log-sum-exp:
//   P = exp(scale Q K^T - lse),  dP = dO V^T,  dS = P * (dP - D),  D_i = dO_i . O_i,
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
// The query-stationary kernel runs first: from each of its query rows it forms
// D = dO . O and leaves nl2 = -lse log2(e) and nD = -D in the workspace, which
// the key-stationary kernel then reads.  Each kernel keeps its stationary operand of S (K rows in the
// key-stationary kernel, Q rows in the query-stationary one) in registers
// premultiplied by c = scale log2(e) and rounded to bf16, and starts the S and
// dP MFMA chains from nl2 and nD instead of zero.  So c s - lse log2(e) and
// dP - D come straight out of the matrix cores: a weight is exp2(acc) and
// dS = p * (dP - D) is one multiply.  The rounding of the premultiplied operand
// moves each exponent by at most 2^-8 sum_i |c q_i k_i|, a relative change of
// the weight of the same order as its own rounding to bf16 for the dV / dK /
// dQ products.  The softmax scale of dK and dQ is applied once, when they are
// stored.
//
// Two kernels, no atomics, every output written exactly once:
//
// bwd_dkdv_kernel -- one item = 128 keys of one head (4 waves x 32 keys) and
//   the 64-query steps that can see them.  K and V rows stay in registers, dK
//   and dV accumulate in registers.  Per step the Q and dO tiles and the
//   step's nl2 / nD rows are copied HBM -> LDS (three-stage ring).  For each
//   32-query block S = Q K^T and dP = dO V^T with M = queries, so P and dS come
//   out with one key per lane and are directly the B operand of
//   dV^T += dO^T P and dK^T += Q^T dS (M = d, N = keys, K = queries); the A
//   operands are read transposed from the row-major Q / dO tiles.
//
// bwd_dq_kernel -- one item = 128 queries of one head (4 waves x 32 queries)
//   and the 64-key tiles of their windows (the forward's work list).  Q and dO
//   rows stay in registers (the O rows are read once, for D); K and V tiles
//   come through the same kind of LDS ring.  For each 32-key block S^T = K Q^T and dP^T = V dO^T with M = keys,
//   so P^T and dS^T come out with one query per lane and are directly the B
//   operand of dQ^T += K^T dS^T, whose A operand is read transposed from the
//   row-major K tile.
//
// Recomputing S and dP in both kernels costs 4 d flops per in-window pair on
// top of the 10 d of a fused backward; in exchange dQ needs no fp32
// accumulator in HBM and no atomics (which this device resolves in memory,
// not in L2), and every gradient is deterministic.
//
// Grouped key/value heads (G query heads share one K/V head): the dQ kernel
// reads the K / V tiles of its query head's group; a dK/dV item holds one key
// tile of the shared head and walks the group's G query heads one after
// another, each over its own query-tile range, so the group's contributions to
// dK and dV add up in registers (still no atomics).
//
// Both kernels skip 32-row blocks that no row of the wave sees and mask only
// blocks that cross the diagonal or the window's trailing edge.  Tiles are
// row-major with the XOR chunk swizzle of the forward kernel.  Rows past T
// read as zero (bounded buffer resources) and contribute nothing.
//
// Sink keys ("Autonomy-of-Heads", section 5): with S sinks, key j is visible
// to query i iff j <= i and (i - W < j or j < S).  The SINK instantiations
// spare keys below S from the trailing-edge mask and never skip their blocks;
// the dQ kernel walks the sink tiles before its window tiles (as the forward
// does), and a dK/dV item holding a sink key runs over every later query tile
// (its planner range says so).  Without sinks the SINK = false code runs.
#include <cmath>
#include <type_traits>

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
  static constexpr int kNC = D / 8;                     // 16-byte chunks per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = kStep * kRowBytes;  // one streamed tile
  static constexpr int kDmaPerWave = kNC / kWaves;      // 1 KiB copies per wave per tensor per step
  static constexpr int kSteps = D / 16;                 // MFMA k-steps over d
  static constexpr int kBlocks = D / 32;                // 32-wide blocks over d
  static_assert(kDmaPerWave >= 1 && kDmaPerWave * kWaves == kNC, "tile / wave split");
};

// Row offset (within a 32-row block, before the 4 hl lane offset) held by MFMA output register r.
__device__ constexpr int reg_row(int r) { return 8 * (r >> 2) + (r & 3); }

// Lane-constant LDS offsets shared by both kernels, for a row-major swizzled tile:
//   rd(st): MFMA A operand read with ds_read_b128 -- row ln, logical chunk 2 st + hl;
//   tr(half, b): ds_read_b64_tr_b16 of row 4 hl + s16 / 4 + 8 half (+ 16 step),
//           columns 32 b + 16 (g & 1) + 4 (s16 & 3) .. + 3 (the swizzle depends on
//           the row modulo 16, so each half has its own offset).
// Up to d = 64 every offset is kept in a register.  At d = 128 that would be
// 16 registers, which the dK/dV kernel cannot spare (it needs two waves per
// SIMD in 256), so only bases are kept: with the swizzle an XOR of the chunk
// index, rd(st) = base + 32 (st ^ z1) and tr(half, b) = base_half + 64 (b ^ zh),
// one v_xad_u32 per use.
// (The copy offsets, dma_off below, are recomputed per copy: cheap, and they
// would otherwise hold registers through the whole loop.)
template <int D>
struct Offsets {
  using C = Cfg<D>;
  static constexpr bool kCompact = D >= 128;
  uint32_t rd_[kCompact ? 1 : C::kSteps];
  uint32_t tr_[2][kCompact ? 1 : C::kBlocks];
  uint32_t rdx = 0, trx[2] = {0, 0};  // compact form: the XOR masks, pre-shifted
  __device__ Offsets(int /*wave*/, int lane) {
    constexpr int NC = C::kNC;
    const int hl = lane >> 5, ln = lane & 31, g = lane >> 4, s16 = lane & 15;
    if constexpr (kCompact) {
      const int z = swz<NC>(ln);
      rd_[0] = static_cast<uint32_t>(ln * C::kRowBytes + 16 * (hl ^ (z & 1)));
      rdx = static_cast<uint32_t>((z >> 1) << 5);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int trow = 4 * hl + (s16 >> 2) + 8 * half;
        const int zt = swz<NC>(trow);
        const int c0 = 2 * (g & 1) + ((s16 & 3) >> 1);
        tr_[half][0] = static_cast<uint32_t>(trow * C::kRowBytes + 16 * (c0 ^ (zt & 3)) + 8 * (s16 & 1));
        trx[half] = static_cast<uint32_t>((zt >> 2) << 6);
      }
    } else {
#pragma unroll
      for (int st = 0; st < C::kSteps; ++st)
        rd_[st] = static_cast<uint32_t>(ln * C::kRowBytes + (((2 * st + hl) ^ swz<NC>(ln)) * 16));
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int b = 0; b < C::kBlocks; ++b) {
          const int trow = 4 * hl + (s16 >> 2) + 8 * half;
          const int col = 32 * b + 16 * (g & 1) + 4 * (s16 & 3);
          tr_[half][b] =
              static_cast<uint32_t>(trow * C::kRowBytes + (((col >> 3) ^ swz<NC>(trow)) * 16) + (col & 7) * 2);
        }
    }
  }
  __device__ __forceinline__ uint32_t rd(int st) const {
    if constexpr (kCompact) return ((static_cast<uint32_t>(st) << 5) ^ rdx) + rd_[0];
    else return rd_[st];
  }
  __device__ __forceinline__ uint32_t tr(int half, int b) const {
    if constexpr (kCompact) return ((static_cast<uint32_t>(b) << 6) ^ trx[half]) + tr_[half][0];
    else return tr_[half][b];
  }
};

// Source offset of this lane's chunk in the wave's j-th 1 KiB copy of a tile:
// tile chunk P = (wave * kDmaPerWave + j) * 64 + lane is row P / NC at stored
// chunk P % NC, which holds logical chunk (P % NC) ^ swz(row).
template <int D>
__device__ __forceinline__ uint32_t dma_off(int wave, int lane, int j) {
  using C = Cfg<D>;
  constexpr int NC = C::kNC;
  const int P = (wave * C::kDmaPerWave + j) * 64 + lane;
  const int row = P / NC;
  return static_cast<uint32_t>(row * C::kRowBytes + (((P % NC) ^ swz<NC>(row)) * 16));
}

// Copy rows [r0, r0 + 64) of one head's [T, D] tensor into a swizzled LDS tile
// (this wave's share); rows past T arrive as zeros.
template <int D>
__device__ __forceinline__ void copy_tile(const bf16* head, int r0, int T, char* dst, int wave, int lane) {
  using C = Cfg<D>;
  const i32x4 r = rsrc_words(head + static_cast<size_t>(r0) * D, static_cast<uint32_t>(T - r0) * C::kRowBytes);
#pragma unroll
  for (int j = 0; j < C::kDmaPerWave; ++j)
    dma16(r, dst + (wave * C::kDmaPerWave + j) * 1024, dma_off<D>(wave, lane, j));
}

// ---------------------------------------------------------------- dK, dV

// Query tiles [lo, hi) of one query head (window W, effective sink S) that see
// keys [k0, k1): the planner's per-head range (query_range in workplan.hpp).
__device__ __forceinline__ int query_hi(int k0, int k1, int W, int S, int T) {
  const int last = k0 < S ? T - 1 : min(T, k1 + W - 1) - 1;
  return last / kStep + 1;
}

// Scalar walk over the steps of a key/value item: query head j of the group,
// query tile qt of that head's range [lo, hi), its window and sink.
struct StepCursor {
  int j, qt, hi, W, S;
};

template <int D, bool SINK, bool GQA>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 3 : 2)))
void bwd_dkdv_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                     const bf16* __restrict__ dO, const float* __restrict__ NL2, const float* __restrict__ ND,
                     bf16* __restrict__ dK, bf16* __restrict__ dV, const WorkItem* __restrict__ items,
                     const int32_t* __restrict__ win_eff, const int32_t* __restrict__ sink_eff, int H, int H_kv,
                     int T, float scale, const int32_t* __restrict__ slots, float* __restrict__ part) {
  using C = Cfg<D>;
  // Ring of stages = {Q tile, dO tile, nl2 row, nD row}: three (copies two steps ahead) up to d = 64; at
  // d = 128 a stage is 33 KiB and two stages let two workgroups share a CU (with at most 256 registers
  // per lane, two waves per SIMD).
  constexpr int kStage = 2 * C::kTileBytes + 2 * kStep * 4;
  constexpr int kStages = D >= 128 ? 2 : 3;
  constexpr int kStagePitch = (kStage + 1023) / 1024 * 1024;  // every stage starts 1 KiB aligned
  __shared__ __attribute__((aligned(1024))) char ring[kStages][kStagePitch];
  constexpr int kG = C::kTileBytes, kL = 2 * C::kTileBytes, kDd = kL + kStep * 4;  // offsets in a stage

  const WorkItem it = items[blockIdx.x];
  if (it.bh < 0) return;
  // Without grouping it.bh = b * H + h indexes Q, K and V alike.  With grouping it.bh = b * H_kv + g
  // indexes K / V / dK / dV, and the item walks the group's query heads g G .. g G + G - 1.
  const int G = GQA ? H / H_kv : 1;
  const int qh0 = GQA ? (it.bh / H_kv) * H + (it.bh % H_kv) * G : it.bh;  // first query head (b H + h)
  const int W = win_eff[qh0 % H];
  const int S = SINK ? sink_eff[qh0 % H] : 0;  // keys 0 .. S - 1 are sinks
  const size_t base = static_cast<size_t>(it.bh) * T * D;  // K, V, dK, dV (and Q, dO without grouping)
  const size_t rbase = static_cast<size_t>(it.bh) * T;
  const float c = scale * kLog2e;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ln = lane & 31;
  const int k0w = it.tile * kStat + 32 * wave;  // first key of this wave
  const int key = k0w + ln;                      // this lane's key (column of S)
  const bool wave_active = k0w < T;
  const Offsets<D> off(wave, lane);

  bf16x8 kf[C::kSteps], vf[C::kSteps];
  // At d = 128 the last two K fragments and the last V fragment of each lane wait in LDS between their
  // uses (12 KiB), which keeps the kernel within 256 registers per lane without spilling to memory.
  constexpr int kStash = D >= 128 ? 1 : 0;
  __shared__ __attribute__((aligned(16))) bf16x8 stash[3][kStash ? kThreads : 1];

  // Stage fill: Q and dO tiles (every wave its share), nl2 row (wave 0), nD row (wave 1) of the query
  // head whose rows start at qb (elements) and rb (rows).
  auto fill_rows = [&](size_t qb, size_t rb, int qt, char* st) __attribute__((always_inline)) {
    const int q0 = qt * kStep;
    copy_tile<D>(Q + qb, q0, T, st, wave, lane);
    copy_tile<D>(dO + qb, q0, T, st + kG, wave, lane);
    if (wave < 2) {
      const float* src = (wave == 0 ? NL2 : ND) + rb + q0;
      dma4(rsrc_words(src, static_cast<uint32_t>(T - q0) * 4), st + (wave == 0 ? kL : kDd),
           static_cast<uint32_t>(lane) * 4);
    }
  };
  auto fill = [&](int qt, char* st) __attribute__((always_inline)) { fill_rows(base, rbase, qt, st); };
  constexpr int kFill = 2 * C::kDmaPerWave;  // copies per wave per fill, plus one for waves 0 and 1
  auto wait_barrier = [&](bool keep_next) __attribute__((always_inline)) {
    if (keep_next) {
      if (wave < 2)
        wait_vm_barrier(kFill + 1);
      else
        wait_vm_barrier(kFill);
    } else {
      wait_vm_barrier(0);
    }
  };

  f32x16 dk[C::kBlocks], dv[C::kBlocks];
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b) {
    dk[b] = f32x16{};
    dv[b] = f32x16{};
  }

  // c s - lse log2(e) and dP - D of 32-query block mb of the stage in st: the
  // chains start from the step's nl2 and nD rows.
  auto scores = [&](const char* st, int mb, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
    const char* qs = st;
    const char* gs = st + kG;
    // Registers 4 i .. 4 i + 3 hold queries 32 mb + 8 i + 4 hl + 0..3 of the step.
    const float* nl = reinterpret_cast<const float*>(st + kL) + 32 * mb + 4 * hl;
    const float* nd = reinterpret_cast<const float*>(st + kDd) + 32 * mb + 4 * hl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(nl + 8 * i);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(nd + 8 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[4 * i + j] = l4[j];
        dp[4 * i + j] = d4[j];
      }
    }
#pragma unroll
    for (int k = 0; k < C::kSteps; ++k) {
      // stash[0]: K fragment kSteps - 1, stash[1]: K fragment kSteps - 2, stash[2]: V fragment kSteps - 1.
      const bf16x8 kb = kStash && k >= C::kSteps - 2 ? stash[C::kSteps - 1 - k][tid] : kf[k];
      const bf16x8 vb = kStash && k == C::kSteps - 1 ? stash[2][tid] : vf[k];
      s = mfma(*reinterpret_cast<const bf16x8*>(qs + 32 * mb * C::kRowBytes + off.rd(k)), kb, s);
      dp = mfma(*reinterpret_cast<const bf16x8*>(gs + 32 * mb * C::kRowBytes + off.rd(k)), vb, dp);
    }
  };
  // P and dS (bf16 B operands; step h takes registers 8 h .. 8 h + 7).
  auto weights = [&](const f32x16& s, const f32x16& dp, bf16x8* pf, bf16x8* df) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(s[r]);
      pf[r >> 3][r & 7] = static_cast<bf16>(p);
      df[r >> 3][r & 7] = static_cast<bf16>(p * dp[r]);
    }
  };
  // dV^T += dO^T P,  dK^T += Q^T dS over block mb's two 16-query steps.
  auto accumulate = [&](const char* st, int mb, const bf16x8* pf, const bf16x8* df) __attribute__((always_inline)) {
    const char* qs = st;
    const char* gs = st + kG;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row0 = (32 * mb + 16 * h) * C::kRowBytes;
#pragma unroll
      for (int b = 0; b < C::kBlocks; ++b) {
        dv[b] = mfma(read_tr(gs + row0 + off.tr(0, b), gs + row0 + off.tr(1, b)), pf[h], dv[b]);
        dk[b] = mfma(read_tr(qs + row0 + off.tr(0, b), qs + row0 + off.tr(1, b)), df[h], dk[b]);
      }
    }
  };

  // One 64-query step, block by block.  Query i sees key j iff 0 <= i - j < W
  // (or j < S and i >= j); the wave's keys are [k0w, k0w + 32).  Blocks no key
  // sees are skipped; only blocks crossing the diagonal or the window's
  // trailing edge are masked.  W and S are those of the step's query head.
  auto do_step = [&](const char* st, int q0, int W, int S) __attribute__((always_inline)) {
    const bool wave_sink = SINK && k0w < S;  // every later query sees some key of this wave
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int qb = q0 + 32 * mb;
      if (!(wave_active && qb < T && qb + 31 >= k0w && (qb <= k0w + 30 + W || wave_sink))) continue;
      f32x16 s, dp;
      scores(st, mb, s, dp);
      // Register r holds query qb + 4 hl + reg_row(r); i - j = reg_row(r) - lim.
      const int lim = key - qb - 4 * hl;
      if (qb < k0w + 31) {  // some query precedes some key
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = reg_row(r) < lim ? -INFINITY : s[r];
      }
      if (qb + 31 >= k0w + W && (!SINK || k0w + 31 >= S)) {  // some query is W or more past some non-sink key
        // A sink key (key < S) is never past the edge: reg_row(r) < 32 <= hi.
        const int hi = SINK && key < S ? 32 : lim + W;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = reg_row(r) >= hi ? -INFINITY : s[r];
      }
      bf16x8 pf[2], df[2];
      weights(s, dp, pf, df);
      accumulate(st, mb, pf, df);
    }
  };

  // Grouped heads: the item's steps are the group's query heads one after another, each over its own
  // query-tile range (all starting at it.lo), cut at it.hi; two cursors follow the step being filled (two
  // ahead) and the step being computed.  A chunk of a split item (query tiles [it.lo, it.hi) of the
  // group's union range) skips the heads whose range ends before it.lo.
  const int k0 = it.tile * kStat, k1 = min(T, k0 + kStat);
  auto set_head = [&](StepCursor& cu, int j) __attribute__((always_inline)) {
    for (;; ++j) {
      cu.j = j;
      cu.qt = it.lo;
      cu.W = win_eff[(qh0 + j) % H];
      cu.S = SINK ? sink_eff[(qh0 + j) % H] : 0;
      cu.hi = min(it.hi, query_hi(k0, k1, cu.W, cu.S, T));
      if (cu.hi > it.lo || j + 1 >= G) break;
    }
  };
  auto advance = [&](StepCursor& cu) __attribute__((always_inline)) {
    if (++cu.qt == cu.hi && cu.j + 1 < G) set_head(cu, cu.j + 1);
  };
  StepCursor dc{0, it.lo, it.hi, W, S}, fc{0, it.lo, it.hi, W, S};
  int n_steps = it.hi - it.lo;
  if constexpr (GQA) {
    set_head(dc, 0);
    n_steps = 0;
    for (int j = 0; j < G; ++j)
      n_steps += max(0, min(it.hi, query_hi(k0, k1, win_eff[(qh0 + j) % H], SINK ? sink_eff[(qh0 + j) % H] : 0, T)) -
                            it.lo);
    fc = dc;
  }
  auto fill_cursor = [&](const StepCursor& cu, char* st) __attribute__((always_inline)) {
    const size_t qh = static_cast<size_t>(qh0 + cu.j);
    fill_rows(qh * T * D, qh * T, cu.qt, st);
  };

  // Ring: step v uses stage v % kStages and fills the stage of step v + kStages - 1, which held step v - 1:
  // the barrier that ended step v - 1 saw every wave finish with it.  A step ends once the next step's
  // copies have landed (each wave waits for its own, then the barrier); with three stages the copies
  // issued in this step may stay in flight.
  //
  // Skewed waves (three stages, one query head, an item that starts at its diagonal tile): waves 2 and 3
  // hold keys 64 .. 127 of the item, which no query of its first tile sees and which see the queries of
  // one more tile at the end than waves 0 and 1 do.  So at step v waves 0 and 1 take tile lo + v and waves
  // 2 and 3 tile lo + v + 1 (both resident: the ring holds three stages), and the item needs one step
  // fewer: 9 instead of 10 at a 512-key window.  The price: every copy issued in a step is waited for at
  // its end (waves 2 and 3 use it in the next step).
  constexpr int kAhead = kStages - 1;
  const bool skew = kStages == 3 && !GQA && it.lo * kStep == k0;
  const int sk = skew && wave >= 2 ? 1 : 0;  // tile offset of this wave (uniform)
  int n_plain = it.hi - it.lo;
  if (skew) {
    // The last tile waves 0 and 1 need, and then the steps the skewed walk takes.
    const int hi01 = min(it.hi, query_hi(k0, min(T, k0 + kStat / 2), W, S, T));
    n_plain = max(hi01 - it.lo, it.hi - it.lo - 1);
  }
  // SK: this wave takes the next tile (waves 2 and 3); each wave pair runs its own copy of the loop, so
  // that every LDS address keeps a compile-time stage (the pairs meet at the same barriers).
  auto step_skew = [&](auto sk_t, int v, const char* cur, const char* nxt1, char* nxtf)
                       __attribute__((always_inline)) {
    constexpr bool SK = decltype(sk_t)::value;
    const int qt = it.lo + v;
    const bool more = qt + kAhead < it.hi;
    if (more) fill(qt + kAhead, nxtf);
    if constexpr (SK) {
      if (qt + 1 < it.hi) do_step(nxt1, (qt + 1) * kStep, W, S);
    } else {
      do_step(cur, qt * kStep, W, S);
    }
    if (v + 1 >= n_plain) return true;
    wait_barrier(false);
    return false;
  };
  auto loop_skew = [&](auto sk_t) __attribute__((always_inline)) {
    for (int v = 0;; v += 3) {
      if (step_skew(sk_t, v, ring[0], ring[1], ring[2])) break;
      if (step_skew(sk_t, v + 1, ring[1], ring[2], ring[0])) break;
      if (step_skew(sk_t, v + 2, ring[2], ring[0], ring[1])) break;
    }
  };
  auto step = [&](int v, const char* cur, char* nxtf) __attribute__((always_inline)) {
    if constexpr (GQA) {
      const bool more = v + kAhead < n_steps;
      if (more) {
        fill_cursor(fc, nxtf);
        advance(fc);
      }
      do_step(cur, dc.qt * kStep, dc.W, dc.S);
      advance(dc);
      if (v + 1 >= n_steps) return true;
      wait_barrier(kStages == 3 && more);
      return false;
    } else {
      const int qt = it.lo + v;
      const bool more = qt + kAhead < it.hi;
      if (more) fill(qt + kAhead, nxtf);
      do_step(cur, qt * kStep, W, S);
      if (qt + 1 >= it.hi) return true;
      wait_barrier(kStages == 3 && more);
      return false;
    }
  };
  // Prologue: the first kStages - 1 stages' copies and the K / V row loads all
  // go out before the first wait, so their latencies overlap.
  if constexpr (GQA) {
    fill_cursor(fc, ring[0]);
    advance(fc);
    if (kStages == 3 && n_steps > 1) {
      fill_cursor(fc, ring[1]);
      advance(fc);
    }
  } else {
    fill(it.lo, ring[0]);
    if (kStages == 3 && it.lo + 1 < it.hi) fill(it.lo + 1, ring[1]);
  }
  // K and V rows (B operands of S = Q K^T and dP = dO V^T): lane holds dims
  // 16 st + 8 hl + 0..7; K premultiplied by c.
  {
    const uint32_t slice = static_cast<uint32_t>(T) * C::kRowBytes;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + base, slice);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + base, slice);
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) {
      const uint32_t o = static_cast<uint32_t>(key) * C::kRowBytes + (16 * st + 8 * hl) * 2;
      kf[st] = __builtin_bit_cast(bf16x8, load16(rk, o));
      vf[st] = __builtin_bit_cast(bf16x8, load16(rv, o));
    }
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) kf[st] = scale_bf16x8(kf[st], c);
    // Consume the rows here: the compiler's wait for them (which also covers
    // the copies above) then sits before the loop, not inside it.
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) __asm__ volatile("" ::"v"(kf[st]), "v"(vf[st]));
    if constexpr (kStash) {
      stash[0][tid] = kf[C::kSteps - 1];
      stash[1][tid] = kf[C::kSteps - 2];
      stash[2][tid] = vf[C::kSteps - 1];
    }
  }
  wait_vm_barrier(0);
  if constexpr (kStages == 3) {
    if (skew) {
      if (sk)
        loop_skew(std::true_type{});
      else
        loop_skew(std::false_type{});
    } else {
      for (int v = 0;; v += 3) {
        if (step(v, ring[0], ring[2])) break;
        if (step(v + 1, ring[1], ring[0])) break;
        if (step(v + 2, ring[2], ring[1])) break;
      }
    }
  } else {
    for (int v = 0;; v += 2) {
      if (step(v, ring[0], ring[1])) break;
      if (step(v + 1, ring[1], ring[0])) break;
    }
  }

  if (key >= T) return;
  if (slots != nullptr && slots[blockIdx.x] >= 0) {
    // A chunk of a split item: its fp32 dK (before the softmax scale) and dV sums over its query tiles.
    const size_t prow = static_cast<size_t>(slots[blockIdx.x]) * 2 * kStat + 32 * wave + ln;
#pragma unroll
    for (int b = 0; b < C::kBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = 32 * b + 8 * i + 4 * hl;
        *reinterpret_cast<f32x4*>(part + prow * D + col) = f32x4{dk[b][4 * i], dk[b][4 * i + 1], dk[b][4 * i + 2],
                                                                 dk[b][4 * i + 3]};
        *reinterpret_cast<f32x4*>(part + (prow + kStat) * D + col) =
            f32x4{dv[b][4 * i], dv[b][4 * i + 1], dv[b][4 * i + 2], dv[b][4 * i + 3]};
      }
    return;
  }
  bf16* dkrow = dK + base + static_cast<size_t>(key) * D;
  bf16* dvrow = dV + base + static_cast<size_t>(key) * D;
  // dK^T / dV^T block b, register r: dim 32 b + 8 (r/4) + 4 hl + r%4 of this lane's key.
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = 32 * b + 8 * i + 4 * hl;
      store_bf16x4(dkrow + col, dk[b][4 * i] * scale, dk[b][4 * i + 1] * scale, dk[b][4 * i + 2] * scale,
                   dk[b][4 * i + 3] * scale);
      store_bf16x4(dvrow + col, dv[b][4 * i], dv[b][4 * i + 1], dv[b][4 * i + 2], dv[b][4 * i + 3]);
    }
}

// ---------------------------------------------------------------- dQ

template <int D, bool SINK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 3 : 1)))
void bwd_dq_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                   const bf16* __restrict__ O, const bf16* __restrict__ dO, const float* __restrict__ LSE,
                   float* __restrict__ NL2, float* __restrict__ ND, bf16* __restrict__ dQ,
                   const WorkItem* __restrict__ items, const int32_t* __restrict__ win_eff,
                   const int32_t* __restrict__ sink_eff, int H, int H_kv, int T, float scale,
                   const int32_t* __restrict__ slots, float* __restrict__ part) {
  using C = Cfg<D>;
  constexpr int kStage = 2 * C::kTileBytes;  // {K tile, V tile}
  // Three stages (copies two steps ahead) up to d = 64; at d = 128 a stage is 32 KiB and two stages let
  // two workgroups share a CU's LDS (the registers allow two waves per SIMD).
  constexpr int kStages = D >= 128 ? 2 : 3;
  __shared__ __attribute__((aligned(1024))) char ring[kStages][kStage];

  const WorkItem it = items[blockIdx.x];
  if (it.bh < 0) return;
  const int W = win_eff[it.bh % H];
  const int S = SINK ? sink_eff[it.bh % H] : 0;  // keys 0 .. S - 1 are sinks
  // Tiles in visiting order: the sink tiles before the window's first tile, then it.lo .. it.hi - 1.  Only
  // the first chunk of a split item (the one that starts at the window's first tile, as every unsplit item
  // does) visits the sink tiles.
  int ns = 0;
  if constexpr (SINK) {
    if (it.lo * kStep <= max(0, it.tile * kStat - W + 1)) ns = min((S + kStep - 1) / kStep, it.lo);
  }
  const int n_tiles = ns + it.hi - it.lo;
  auto tile_at = [&](int v) __attribute__((always_inline)) { return SINK && v < ns ? v : v - ns + it.lo; };
  const size_t base = static_cast<size_t>(it.bh) * T * D;
  const size_t rbase = static_cast<size_t>(it.bh) * T;
  const float c = scale * kLog2e;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ln = lane & 31;
  const int q0w = it.tile * kStat + 32 * wave;   // first query of this wave
  const int qi = q0w + ln;                        // this lane's query (column of S^T)
  const bool wave_active = q0w < T;
  const int wave_key_lo = q0w - W + 1;
  const int wave_key_hi = min(q0w + 31, T - 1);
  const Offsets<D> off(wave, lane);

  // K / V tiles of this query head's key/value head, h / (H / H_kv).
  const size_t kvbase = (static_cast<size_t>(it.bh / H) * H_kv + (it.bh % H) / (H / H_kv)) * T * D;
  auto fill = [&](int kt, char* st) __attribute__((always_inline)) {
    const int k0 = kt * kStep;
    copy_tile<D>(K + kvbase, k0, T, st, wave, lane);
    copy_tile<D>(V + kvbase, k0, T, st + C::kTileBytes, wave, lane);
  };
  constexpr int kFill = 2 * C::kDmaPerWave;

  // Prologue: the copies of the first kStages - 1 tiles go out before the row loads below, so that
  // their latencies overlap.
  fill(tile_at(0), ring[0]);
  if (kStages == 3 && 1 < n_tiles) fill(tile_at(1), ring[1]);

  // Q (premultiplied by c) and dO rows of this lane's query: the B operands of
  // S^T = K Q^T and dP^T = V dO^T.  Lanes ln and ln + 32 hold the two halves
  // of the row (dims 16 st + 8 hl + 0..7).
  bf16x8 qf[C::kSteps], gf[C::kSteps];
  float cl = 0.f, nD = 0.f;  // -lse log2(e) and -D of this lane's query
  {
    const uint32_t slice = static_cast<uint32_t>(T) * C::kRowBytes;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + base, slice);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(dO + base, slice);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + base, slice);
    bf16x8 of[C::kSteps];
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) {
      const uint32_t o = static_cast<uint32_t>(qi) * C::kRowBytes + (16 * st + 8 * hl) * 2;
      qf[st] = __builtin_bit_cast(bf16x8, load16(rq, o));
      gf[st] = __builtin_bit_cast(bf16x8, load16(rg, o));
      of[st] = __builtin_bit_cast(bf16x8, load16(ro, o));
    }
    const float lse = load_f32(make_rsrc(LSE + rbase, static_cast<uint32_t>(T) * 4), static_cast<uint32_t>(qi) * 4);
    // D = dO . O over this lane's half row, then over both halves.
    float dh = 0.f;
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 a = {gf[st][e], gf[st][e + 1]};
        const bf16x2 b = {of[st][e], of[st][e + 1]};
        dh = __builtin_amdgcn_fdot2_f32_bf16(a, b, dh, false);
      }
    nD = -half_swap_sum(dh);
    cl = -lse * kLog2e;
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) qf[st] = scale_bf16x8(qf[st], c);
    // Consume the rows here: the compiler's wait for them (which also covers
    // the copies above) then sits before the loop, not inside it.
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) __asm__ volatile("" ::"v"(qf[st]), "v"(gf[st]));
    __asm__ volatile("" ::"v"(cl), "v"(nD));
  }
  // The start values of the S^T and dP^T chains: -lse log2(e) and -D of this
  // lane's query in every register.
  f32x16 cl16, nd16;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    cl16[r] = cl;
    nd16[r] = nD;
  }

  f32x16 acc[C::kBlocks];
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b) acc[b] = f32x16{};

  // One 32-key block [kb, kb + 32) of the stage in st.
  auto do_block = [&](const char* st, int kb, int mb) __attribute__((always_inline)) {
    if constexpr (SINK) {
      if (!(wave_active && kb <= wave_key_hi && (kb + 31 >= wave_key_lo || kb < S))) return;
    } else {
      if (!(wave_active && kb <= wave_key_hi && kb + 31 >= wave_key_lo)) return;
    }
    const char* ks = st;
    const char* vs = st + C::kTileBytes;
    f32x16 s = cl16, dp = nd16;
#pragma unroll
    for (int k = 0; k < C::kSteps; ++k) {
      s = mfma(*reinterpret_cast<const bf16x8*>(ks + 32 * mb * C::kRowBytes + off.rd(k)), qf[k], s);
      dp = mfma(*reinterpret_cast<const bf16x8*>(vs + 32 * mb * C::kRowBytes + off.rd(k)), gf[k], dp);
    }
    // Register r holds key kb + 4 hl + reg_row(r), visible iff lim - W < reg_row(r) <= lim
    // (or reg_row(r) < sl, a sink, with reg_row(r) <= lim).
    const int lim = qi - kb - 4 * hl;
    if (kb + 31 > q0w) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = reg_row(r) > lim ? -INFINITY : s[r];
    }
    if (SINK ? kb < q0w + 32 - W && kb + 31 >= S : kb < q0w + 32 - W) {
      const int lo = lim - W;
      const int sl = S - kb - 4 * hl;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = reg_row(r) <= lo && (!SINK || reg_row(r) >= sl) ? -INFINITY : s[r];
    }
    bf16x8 df[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(s[r]);
      df[r >> 3][r & 7] = static_cast<bf16>(p * dp[r]);
    }
    // dQ^T += K^T dS^T over the block's two 16-key steps (slot order of the dS registers).
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row0 = (32 * mb + 16 * h) * C::kRowBytes;
#pragma unroll
      for (int b = 0; b < C::kBlocks; ++b)
        acc[b] = mfma(read_tr(ks + row0 + off.tr(0, b), ks + row0 + off.tr(1, b)), df[h], acc[b]);
    }
  };

  // Ring: the v-th tile visited uses stage v % kStages and fills the stage of tile v + kStages - 1, which
  // held tile v - 1: the barrier that ended step v - 1 saw every wave finish with it.  A step ends
  // once the next tile's copies have landed (each wave waits for its own, then the barrier); with
  // three stages the copies issued in this step may stay in flight.
  auto step = [&](int v, const char* cur, char* nxtf) __attribute__((always_inline)) {
    const bool more = v + kStages - 1 < n_tiles;
    if (more) fill(tile_at(v + kStages - 1), nxtf);
    const int k0 = tile_at(v) * kStep;
    do_block(cur, k0, 0);
    do_block(cur, k0 + 32, 1);
    if (v + 1 >= n_tiles) return true;
    if (kStages == 3 && more)
      wait_vm_barrier(kFill);
    else
      wait_vm_barrier(0);
    return false;
  };
  wait_vm_barrier(0);
  if constexpr (kStages == 3) {
    for (int v = 0;; v += 3) {
      if (step(v, ring[0], ring[2])) break;
      if (step(v + 1, ring[1], ring[0])) break;
      if (step(v + 2, ring[2], ring[1])) break;
    }
  } else {
    for (int v = 0;; v += 2) {
      if (step(v, ring[0], ring[1])) break;
      if (step(v + 1, ring[1], ring[0])) break;
    }
  }

  if (qi >= T) return;
  // The rows the key-stationary kernel starts its chains from (stored here,
  // after the loop, so that no store is outstanding while the loop counts its
  // copies).
  if (hl == 0) {
    NL2[rbase + qi] = cl;
    ND[rbase + qi] = nD;
  }
  if (slots != nullptr && slots[blockIdx.x] >= 0) {
    // A chunk of a split item: its fp32 dQ sum (before the softmax scale) over its key tiles.
    float* prow = part + (static_cast<size_t>(slots[blockIdx.x]) * kStat + q0w - it.tile * kStat + ln) * D;
#pragma unroll
    for (int b = 0; b < C::kBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(prow + 32 * b + 8 * i + 4 * hl) =
            f32x4{acc[b][4 * i], acc[b][4 * i + 1], acc[b][4 * i + 2], acc[b][4 * i + 3]};
    return;
  }
  bf16* dqrow = dQ + base + static_cast<size_t>(qi) * D;
  // dQ^T block b, register r: dim 32 b + 8 (r/4) + 4 hl + r%4 of this lane's query.
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      store_bf16x4(dqrow + 32 * b + 8 * i + 4 * hl, acc[b][4 * i] * scale, acc[b][4 * i + 1] * scale,
                   acc[b][4 * i + 2] * scale, acc[b][4 * i + 3] * scale);
}

// Sums the chunks of each split item (record {bh, tile, first slot, chunks}):
// out0 = f0 * sum_c part[c][0] and, for dK / dV, out1 = sum_c part[c][1], each
// [128 rows][D] in fp32, rounded to bf16.  D / 4 threads per row, four dims each;
// chunks are added in order, so the result is deterministic.
template <int D, int NOUT>
__global__ __launch_bounds__(256) void bwd_merge_kernel(const WorkItem* __restrict__ merges,
                                                        const float* __restrict__ part, bf16* __restrict__ out0,
                                                        bf16* __restrict__ out1, float f0, int T) {
  constexpr int kPerRow = D / 4;
  constexpr int kRowsPerWg = 256 / kPerRow;
  const WorkItem mg = merges[blockIdx.x];
  const int r = blockIdx.y * kRowsPerWg + static_cast<int>(threadIdx.x) / kPerRow;
  const int dq = (static_cast<int>(threadIdx.x) % kPerRow) * 4;
  const int row = mg.tile * kStat + r;
  if (r >= kStat || row >= T) return;
  f32x4 a0 = f32x4{}, a1 = f32x4{};
  for (int ch = 0; ch < mg.hi; ++ch) {
    const size_t base = (static_cast<size_t>(mg.lo + ch) * NOUT * kStat + r) * D + dq;
    a0 += *reinterpret_cast<const f32x4*>(part + base);
    if constexpr (NOUT == 2) a1 += *reinterpret_cast<const f32x4*>(part + base + static_cast<size_t>(kStat) * D);
  }
  const size_t o = (static_cast<size_t>(mg.bh) * T + row) * D + dq;
  store_bf16x4(out0 + o, a0[0] * f0, a0[1] * f0, a0[2] * f0, a0[3] * f0);
  if constexpr (NOUT == 2) store_bf16x4(out1 + o, a1[0], a1[1], a1[2], a1[3]);
}

template <int D, bool SINK, bool GQA>
hipError_t dkdv_d(const void* q, const void* k, const void* v, const void* dout, const float* nl2, const float* nd,
                  void* dk, void* dv, const WorkItem* items, int n_items, const int32_t* win_eff,
                  const int32_t* sink_eff, const AttnShape& s, hipStream_t stream, const BwdSplit* split = nullptr) {
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, SINK, GQA>), dim3(n_items), dim3(kThreads), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                     static_cast<const bf16*>(dout), nl2, nd, static_cast<bf16*>(dk), static_cast<bf16*>(dv), items,
                     win_eff, sink_eff, s.H, s.H_kv, s.T, s.scale, split != nullptr ? split->slots : nullptr,
                     split != nullptr ? split->part : nullptr);
  return hipGetLastError();
}

template <int D, bool SINK>
hipError_t dq_d(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                float* nl2, float* nd, void* dq, const WorkItem* items, int n_items, const int32_t* win_eff,
                const int32_t* sink_eff, const AttnShape& s, hipStream_t stream, const BwdSplit* split = nullptr) {
  hipLaunchKernelGGL((bwd_dq_kernel<D, SINK>), dim3(n_items), dim3(kThreads), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                     static_cast<const bf16*>(o), static_cast<const bf16*>(dout), lse, nl2, nd,
                     static_cast<bf16*>(dq), items, win_eff, sink_eff, s.H, s.H_kv, s.T, s.scale,
                     split != nullptr ? split->slots : nullptr, split != nullptr ? split->part : nullptr);
  return hipGetLastError();
}

template <int D>
hipError_t dkdv_s(const void* q, const void* k, const void* v, const void* dout, const float* nl2, const float* nd,
                  void* dk, void* dv, const WorkItem* items, int n_items, const int32_t* win_eff,
                  const int32_t* sink_eff, const AttnShape& s, hipStream_t stream) {
  const bool sink = sink_eff != nullptr, gqa = s.H_kv != s.H;
  if (sink && gqa)
    return dkdv_d<D, true, true>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, stream);
  if (sink)
    return dkdv_d<D, true, false>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, stream);
  if (gqa)
    return dkdv_d<D, false, true>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, stream);
  return dkdv_d<D, false, false>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, stream);
}

template <int D>
hipError_t dq_s(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                float* nl2, float* nd, void* dq, const WorkItem* items, int n_items, const int32_t* win_eff,
                const int32_t* sink_eff, const AttnShape& s, hipStream_t stream) {
  return sink_eff != nullptr
             ? dq_d<D, true>(q, k, v, o, dout, lse, nl2, nd, dq, items, n_items, win_eff, sink_eff, s, stream)
             : dq_d<D, false>(q, k, v, o, dout, lse, nl2, nd, dq, items, n_items, win_eff, sink_eff, s, stream);
}

template <int D>
hipError_t dkdv_split_d(const void* q, const void* k, const void* v, const void* dout, const float* nl2, const float* nd,
                        void* dk, void* dv, const WorkItem* items, int n_items, const int32_t* win_eff,
                        const int32_t* sink_eff, const AttnShape& s, const BwdSplit& split, hipStream_t stream) {
  const bool sink = sink_eff != nullptr, gqa = s.H_kv != s.H;
  const BwdSplit* sp = &split;
  hipError_t e;
  if (sink && gqa)
    e = dkdv_d<D, true, true>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, stream, sp);
  else if (sink)
    e = dkdv_d<D, true, false>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, stream, sp);
  else if (gqa)
    e = dkdv_d<D, false, true>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, stream, sp);
  else
    e = dkdv_d<D, false, false>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, stream, sp);
  if (e != hipSuccess || split.n_merges == 0) return e;
  hipLaunchKernelGGL((bwd_merge_kernel<D, 2>), dim3(split.n_merges, kStat / (256 / (D / 4))), dim3(256), 0, stream,
                     split.merges, split.part, static_cast<bf16*>(dk), static_cast<bf16*>(dv), s.scale, s.T);
  return hipGetLastError();
}

template <int D>
hipError_t dq_split_d(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      float* nl2, float* nd, void* dq, const WorkItem* items, int n_items, const int32_t* win_eff,
                      const int32_t* sink_eff, const AttnShape& s, const BwdSplit& split, hipStream_t stream) {
  const hipError_t e =
      sink_eff != nullptr
          ? dq_d<D, true>(q, k, v, o, dout, lse, nl2, nd, dq, items, n_items, win_eff, sink_eff, s, stream, &split)
          : dq_d<D, false>(q, k, v, o, dout, lse, nl2, nd, dq, items, n_items, win_eff, nullptr, s, stream, &split);
  if (e != hipSuccess || split.n_merges == 0) return e;
  hipLaunchKernelGGL((bwd_merge_kernel<D, 1>), dim3(split.n_merges, kStat / (256 / (D / 4))), dim3(256), 0, stream,
                     split.merges, split.part, static_cast<bf16*>(dq), nullptr, s.scale, s.T);
  return hipGetLastError();
}

template <typename Fn>
int resident_of(Fn fn) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), kThreads, 0) !=
      hipSuccess)
    return 0;
  return per_cu * cus;
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16_split(const void* q, const void* k, const void* v, const void* dout, const float* nl2,
                                      const float* nd, void* dk, void* dv, const WorkItem* items, int n_items,
                                      const int32_t* win_eff, const int32_t* sink_eff, const AttnShape& s,
                                      const BwdSplit& split, hipStream_t stream) {
  switch (s.d) {
    case 32:
      return dkdv_split_d<32>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, split, stream);
    case 64:
      return dkdv_split_d<64>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, split, stream);
    case 128:
      return dkdv_split_d<128>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, split, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dq_bf16_split(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                    const float* lse, float* nl2, float* nd, void* dq, const WorkItem* items,
                                    int n_items, const int32_t* win_eff, const int32_t* sink_eff,
                                    const AttnShape& s, const BwdSplit& split, hipStream_t stream) {
  switch (s.d) {
    case 32:
      return dq_split_d<32>(q, k, v, o, dout, lse, nl2, nd, dq, items, n_items, win_eff, sink_eff, s, split, stream);
    case 64:
      return dq_split_d<64>(q, k, v, o, dout, lse, nl2, nd, dq, items, n_items, win_eff, sink_eff, s, split, stream);
    case 128:
      return dq_split_d<128>(q, k, v, o, dout, lse, nl2, nd, dq, items, n_items, win_eff, sink_eff, s, split,
                             stream);
    default: return hipErrorInvalidValue;
  }
}

int bwd_dq_resident(int d) {
  switch (d) {
    case 32: return resident_of(&bwd_dq_kernel<32, false>);
    case 64: return resident_of(&bwd_dq_kernel<64, false>);
    case 128: return resident_of(&bwd_dq_kernel<128, false>);
    default: return 0;
  }
}

int bwd_dkdv_resident(int d) {
  switch (d) {
    case 32: return resident_of(&bwd_dkdv_kernel<32, false, false>);
    case 64: return resident_of(&bwd_dkdv_kernel<64, false, false>);
    case 128: return resident_of(&bwd_dkdv_kernel<128, false, false>);
    default: return 0;
  }
}

hipError_t launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const void* dout, const float* nl2,
                                const float* nd, void* dk, void* dv, const WorkItem* items, int n_items,
                                const int32_t* win_eff, const int32_t* sink_eff, const AttnShape& s,
                                hipStream_t stream) {
  switch (s.d) {
    case 32: return dkdv_s<32>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, stream);
    case 64: return dkdv_s<64>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, stream);
    case 128: return dkdv_s<128>(q, k, v, dout, nl2, nd, dk, dv, items, n_items, win_eff, sink_eff, s, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, float* nl2, float* nd, void* dq, const WorkItem* items, int n_items,
                              const int32_t* win_eff, const int32_t* sink_eff, const AttnShape& s,
                              hipStream_t stream) {
  switch (s.d) {
    case 32: return dq_s<32>(q, k, v, o, dout, lse, nl2, nd, dq, items, n_items, win_eff, sink_eff, s, stream);
    case 64: return dq_s<64>(q, k, v, o, dout, lse, nl2, nd, dq, items, n_items, win_eff, sink_eff, s, stream);
    case 128: return dq_s<128>(q, k, v, o, dout, lse, nl2, nd, dq, items, n_items, win_eff, sink_eff, s, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace aah
