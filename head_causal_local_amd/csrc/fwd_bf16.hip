// bf16 forward kernel of per-head causal local-window attention for gfx950.
//
// Operation: "Asymmetric Attention Heads" section 5.8 -- for each (b, h) with
// window W, A = softmax(scale * Q K^T + M_W), Y = A V, where M_W keeps key j
// for query i iff i - W < j <= i.  Also writes the per-row natural
// log-sum-exp of the scaled scores, used by the backward pass.
//
// One workgroup = one work item = 128 query rows of one head (4 waves x 32
// rows) and the contiguous range of 64-key tiles the planner listed for them
// (with grouped key/value heads the tiles come from the group's K/V head; the
// planner sends a group's query heads to the same XCD, so they meet in its L2);
// tiles wholly outside the window are never visited.  Each wave walks the
// keys in 32-key blocks and classifies each block against its own 32 rows:
// blocks no row sees are skipped (no MFMA, no exp), blocks every row sees in
// full run without a mask, and only the (at most two) partial blocks per
// wave -- the diagonal and the window's trailing edge -- apply a one-sided
// mask.
//
// Data flow per LDS stage (64 keys in two stages at d <= 64; 32 keys in three
// stages at d = 128):
//   * K and V tiles go from HBM straight into LDS (buffer_load ... lds, no
//     register staging) through a ring: the next stages' copies are in flight
//     while the current one is used.  Tiles are row-major with an XOR swizzle
//     of their 16-byte chunks so that both read patterns below are free of
//     bank conflicts.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (M = keys, N = queries, K = d).
//     The output layout gives lane l the query (l mod 32) and 16 keys per
//     32-key block, so all softmax bookkeeping is in-lane, plus one
//     permlane32 swap between the half-waves when a row max is needed.
//   * P^T (bf16) stays in registers and is the B operand of O^T += V^T P^T
//     (M = d, N = queries, K = keys).  The MFMA k-slots are mapped to keys in
//     the order the S^T output already holds them, and the V^T operand is
//     read from the row-major V tile with ds_read_b64_tr_b16, which hands each
//     lane four consecutive rows of one column.
//
// Softmax (log2 domain, p = exp2(s * scale * log2 e - m)).  The reference m of
// a row is the exact running max at its last refresh.  A block's weights are
// first formed against the current reference, packed to bf16 and summed with
// v_dot2 (so the row sum adds exactly the weights used in P V).  A lane's
// partial sum bounds each of its weights, so only if some partial sum exceeds
// 2^10 (or some row of the wave has no reference yet) is the block redone:
// the wave exchanges the half-row maxima, rescales O and the row sum, moves
// the reference and forms the weights again.  Hence every p is <= 2^10 and
// some p of every row was >= 1 when its reference was set, so row sums never
// underflow.
// Global loads go through buffer resources whose range ends at the head's
// last row, so rows past T read as zero without branches.
//
// Sink keys ("Autonomy-of-Heads", section 5: a streaming head keeps its first
// S tokens besides its recent window).  Key j is then visible to query i iff
// j <= i and (i - W < j or j < S).  The SINK instantiation walks the sink
// tiles before the item's first window tile (keys there precede every row's
// window, so only j < S decides), then the window tiles as usual; its
// trailing-edge mask spares keys below S, and blocks of sink keys are never
// skipped.  Without sinks the SINK = false instantiation runs, unchanged.
//
// Diagnostics ("Asymmetric Attention Heads" section 5.3: the controller's head
// features include the attention entropy and the output norm).  The DIAG
// instantiation also writes, per query row, the entropy -sum_j p_j ln p_j of
// its attention weights and the Euclidean norm of its output row, from values
// the kernel already has: with w_j the bf16 weights that enter the row sum l
// and x_j = s_j c - m their log2 offsets from the reference m, the entropy is
// ln 2 (log2 l - sum_j w_j x_j / l).  The sum follows the reference like l does
// (when m moves up by delta, a becomes alpha (a - delta l), alpha = 2^-delta).  Using the rounded
// weights for both sums makes the result the cross entropy of the normalised
// rounded weights against the exact ones, within 2^-7 H + 2^-8 of the exact H.
//
// Split launches (few work items for the device): an item may be one chunk of
// a longer item's key range.  Such a chunk ends by leaving, per row, its
// unnormalised accumulator, its reference m and its row sum in a slot of the
// caller's workspace; fwd_merge_kernel then rescales the chunks of each split
// item to a common reference and writes O and LSE.
#include <cmath>

#include "device_common.hpp"
#include "kernels.hpp"

namespace aah {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kRows = 32 * kWaves;  // query rows per item
constexpr int kPlanKeys = 64;       // keys per tile of the planner's ranges
constexpr int kThreads = 64 * kWaves;
constexpr float kThresh = 1024.0f;  // lazy-rescale bound on every weight p (2^10)
static_assert(kRows == kFwdBf16RowTile && kPlanKeys == kFwdBf16ColTile, "planner tile mismatch");

template <int D>
struct Cfg {
  static constexpr int kNC = D / 8;                 // 16-byte chunks per row
  static constexpr int kRowBytes = D * 2;
  // Keys per LDS stage and stages in the ring.  At d = 128 a stage holds 32 keys and the ring three
  // stages (copies issued two steps ahead): 48 KiB instead of 64, so a CU holds three workgroups, not
  // two (grouped d = 128 layer: forward 292 -> 274 us).  At d <= 64 LDS is no tighter than registers
  // with 64-key stages and two of them (32 KiB at d = 64: four workgroups per CU); 32-key stages there
  // measured 2.5 % slower (twice the barriers per key, and a fifth workgroup per CU bought nothing).
  static constexpr int kKT = D >= 128 ? 32 : 64;
  static constexpr int kNS = D >= 128 ? 3 : 2;
  static constexpr int kTileBytes = kKT * kRowBytes;              // one K or V stage
  static constexpr int kDmaPerWave = kKT * kNC / (64 * kWaves);  // 1 KiB DMA instructions per wave per tensor per stage
  static constexpr int kSteps = D / 16;             // MFMA k-steps over d for S^T
  static constexpr int kBlocks = D / 32;            // 32-row blocks of O^T
  // Resident waves per SIMD the register allocation is sized for.
  static constexpr int kWavesPerSimd = D <= 64 ? 4 : 1;
  static_assert(kDmaPerWave >= 1 && kDmaPerWave * 64 * kWaves == kKT * kNC, "tile / wave split");
  static_assert(kPlanKeys % kKT == 0, "stages subdivide the planner's tiles");
};

// Key offset (within its 32-key block, before the 4 hl lane offset) held by S^T register r.
__device__ constexpr int reg_key(int r) { return 8 * (r >> 2) + (r & 3); }

template <int D, bool SINK, bool DIAG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Cfg<D>::kWavesPerSimd)))
void fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                     bf16* __restrict__ O, float* __restrict__ LSE, float* __restrict__ ENT,
                     float* __restrict__ ONORM, const WorkItem* __restrict__ items,
                     const int32_t* __restrict__ win_eff, const int32_t* __restrict__ sink_eff, int H, int H_kv,
                     int T, float c, const int32_t* __restrict__ slots, float* __restrict__ part_acc,
                     float* __restrict__ part_ml, int h_shift, int g_shift) {
  using C = Cfg<D>;
  constexpr int NC = C::kNC;
  constexpr int KT = C::kKT;
  constexpr int kSub = kPlanKeys / KT;  // stages per planner tile
  // Ring slot i: K tile at lds + 2 i kTileBytes, its V tile right after it.
  __shared__ __attribute__((aligned(1024))) char lds[C::kNS * 2 * C::kTileBytes];

  const WorkItem it = items[blockIdx.x];
  // The kernel arguments the prologue needs are read here, so that their loads go out with the
  // item's rather than one scalar round trip after the padding test.
  __asm__ volatile("" ::"s"(H), "s"(H_kv), "s"(T), "s"(Q), "s"(K), "s"(V), "s"(slots), "s"(win_eff), "s"(h_shift),
                   "s"(g_shift));
  if (it.bh < 0) return;  // padding slot (uniform over the workgroup)
  // Head h = bh mod H of batch entry bh / H, and its key/value head h / G (G = H / H_kv): shifts and masks
  // when H (and G) are powers of two (h_shift, g_shift >= 0), else divisions.
  const int hq = h_shift >= 0 ? it.bh & ((1 << h_shift) - 1) : it.bh % H;
  const int bq = h_shift >= 0 ? it.bh >> h_shift : it.bh / H;
  const int hkv = g_shift >= 0 ? hq >> g_shift : hq / (H / H_kv);
  // A chunk of a split item leaves its rows' partial result in its slot instead of O and LSE.
  const int slot = slots != nullptr ? slots[blockIdx.x] : -1;
  // The window (and sink size) come from a table indexed by the item's head.  Where the first
  // copies do not depend on them (64-key stages, no sinks) that load is issued after those copies,
  // so that waiting for it (scalar loads complete in any order) does not hold them back.
  constexpr bool kLateW = kSub == 1 && !SINK;
  int W = 0;
  if constexpr (!kLateW) W = win_eff[hq];
  const int S = SINK ? sink_eff[hq] : 0;  // keys 0 .. S - 1 are sinks
  // Stages (KT keys each) in visiting order: sink stages 0 .. ns - 1 (those before the window's first
  // stage), then the window's stages w_lo .. w_hi - 1 -- the planner's tiles [lo, hi) trimmed to the keys
  // [q0 - W + 1, q1 - 1] the item's rows see.
  const int q0i = it.tile * kRows, q1i = min(T, q0i + kRows);
  const int w_lo = kSub == 1 ? it.lo : max(it.lo * kSub, max(0, q0i - W + 1) / KT);
  const int w_hi = kSub == 1 ? it.hi : min(it.hi * kSub, (q1i - 1) / KT + 1);
  // Only the first chunk of a split item (the one that starts at the window's first tile, as every unsplit
  // item does) visits the sink stages.
  const int ns = SINK && it.lo * kPlanKeys <= max(0, q0i - W + 1) ? min((S + KT - 1) / KT, w_lo) : 0;
  const int n_tiles = ns + w_hi - w_lo;
  auto tile_at = [&](int v) __attribute__((always_inline)) { return SINK && v < ns ? v : v - ns + w_lo; };
  const size_t base = static_cast<size_t>(it.bh) * T * D;
  const size_t kvbase = (static_cast<size_t>(bq) * H_kv + hkv) * T * D;
  const bf16* Qh = Q + base;
  const bf16* Kh = K + kvbase;
  const bf16* Vh = V + kvbase;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index is uniform across the wave: keep it (and everything derived
  // from it) in scalar registers so block decisions compile to scalar branches.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ln = lane & 31;
  const int q0w = it.tile * kRows + wave * 32;  // first query row of this wave
  const int qi = q0w + ln;                      // this lane's query row
  const bool row_ok = qi < T;
  const bool wave_active = q0w < T;
  int wave_key_lo = q0w - W + 1;                // first key any row of the wave sees (may be < 0; set again
                                                // below where W is read late)
  const int wave_key_hi = min(q0w + 31, T - 1); // last key any row of the wave sees

  bf16x8 qf[C::kSteps];  // Q^T fragments (B operand of S^T = K Q^T), loaded in the prologue below
  f32x16 acc[C::kBlocks];
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b) acc[b] = f32x16{};
  float m_run = -INFINITY;  // reference max of this lane's row (log2 domain)
  float m_use = 0.f;        // m_run, or 0 while the row has seen no visible key (then every p is 0)
  float l_run = 0.f;        // this half-wave's running sum of the bf16 weights
  float a_run = 0.f;        // DIAG: this half-wave's sum of those weights times their offsets x = s c - m_run
  bool ready = false;       // every row of the wave has a reference

  // DMA sources: instruction j of this wave fills tile chunks P = (wave * kDmaPerWave + j) * 64 + lane,
  // i.e. row P / NC at stored chunk P % NC, which holds logical chunk (P % NC) ^ swz(row).
  uint32_t dma_off[C::kDmaPerWave];
#pragma unroll
  for (int j = 0; j < C::kDmaPerWave; ++j) {
    const int P = (wave * C::kDmaPerWave + j) * 64 + lane;
    const int row = P / NC;
    dma_off[j] = static_cast<uint32_t>(row * C::kRowBytes + (((P % NC) ^ swz<NC>(row)) * 16));
  }
  auto issue_tile = [&](int kt, char* kdst, char* vdst) __attribute__((always_inline)) {
    const int k0 = kt * KT;
    // Resources start at the tile's first row and end at row T: keys past T read as zero.
    const uint32_t left = static_cast<uint32_t>(T - k0) * C::kRowBytes;
    const i32x4 rk = rsrc_words(Kh + static_cast<size_t>(k0) * D, left);
    const i32x4 rv = rsrc_words(Vh + static_cast<size_t>(k0) * D, left);
#pragma unroll
    for (int j = 0; j < C::kDmaPerWave; ++j) {
      const int off = (wave * C::kDmaPerWave + j) * 1024;
      dma16(rk, kdst + off, dma_off[j]);
      dma16(rv, vdst + off, dma_off[j]);
    }
  };

  // Lane-constant LDS read offsets.  K (A operand of S^T): row 32 mb + ln, logical chunk 2 st + hl.
  uint32_t k_off[C::kSteps];
#pragma unroll
  for (int st = 0; st < C::kSteps; ++st)
    k_off[st] = static_cast<uint32_t>(ln * C::kRowBytes + (((2 * st + hl) ^ swz<NC>(ln)) * 16));
  // V^T (A operand of O^T += V^T P^T) by ds_read_b64_tr_b16: lane (g, s16) addresses
  // row 16 st + 4 hl + s16 / 4 and that row + 8, columns 32 b + 16 (g & 1) + 4 (s16 & 3) .. + 3.
  // The swizzle depends on the row modulo 16, so the +16 st offset is common to both reads.
  const int g = lane >> 4, s16 = lane & 15;
  uint32_t v_off[2][C::kBlocks];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int b = 0; b < C::kBlocks; ++b) {
      const int vrow = 4 * hl + (s16 >> 2) + 8 * half;
      const int col = 32 * b + 16 * (g & 1) + 4 * (s16 & 3);
      v_off[half][b] =
          static_cast<uint32_t>(vrow * C::kRowBytes + (((col >> 3) ^ swz<NC>(vrow)) * 16) + (col & 7) * 2);
    }
  const bf16x2 ones = {static_cast<bf16>(1.f), static_cast<bf16>(1.f)};

  // One 32-key block [kb, kb + 32) of the tile held in (kt_lds, vt_lds), for this wave.
  auto do_block = [&](const char* kt_lds, const char* vt_lds, int kb, int mb) __attribute__((always_inline)) {
    if constexpr (SINK) {
      if (!(wave_active && kb <= wave_key_hi && (kb + 31 >= wave_key_lo || kb < S))) return;  // no row sees it
    } else {
      if (!(wave_active && kb <= wave_key_hi && kb + 31 >= wave_key_lo)) return;  // no row sees it
    }
    const bool mh = kb + 31 > q0w;       // some key may be after some row (diagonal)
    // Some non-sink key may precede some row's window (trailing edge).
    const bool ml = SINK ? kb < q0w + 32 - W && kb + 31 >= S : kb < q0w + 32 - W;
    const int lim = qi - kb - 4 * hl;    // register r's key is visible iff lim - W < reg_key(r) <= lim
    const int sl = S - kb - 4 * hl;      // ... or reg_key(r) < sl (a sink), with reg_key(r) <= lim

    auto compute_s = [&]() __attribute__((always_inline)) {
      f32x16 s = f32x16{};
#pragma unroll
      for (int st = 0; st < C::kSteps; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt_lds + 32 * mb * C::kRowBytes + k_off[st]);
        s = mfma(a, qf[st], s);
      }
      if (mh) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (reg_key(r) > lim) s[r] = -INFINITY;
      }
      if (ml) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (reg_key(r) <= lim - W && (!SINK || reg_key(r) >= sl)) s[r] = -INFINITY;
      }
      return s;
    };

    const f32x16 s = compute_s();

    // P^T fragments of the block's two 16-key MFMA steps: step h takes registers
    // 8 h .. 8 h + 7, i.e. keys kb + 16 h + 8 (e / 4) + 4 hl + e % 4 for e = 0 .. 7.
    // part = this lane's sum of exactly the bf16 weights that enter P V.
    bf16x8 pf[2];
    float part;
    float apart = 0.f;  // DIAG: sum of the lane's weights times their offsets
    auto make_p = [&]() __attribute__((always_inline)) {
      float pa = 0.f, pb = 0.f, ea = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          bf16x2 pp;
          const float x0 = fmaf(s[8 * h + e], c, -m_use);
          const float x1 = fmaf(s[8 * h + e + 1], c, -m_use);
          pp[0] = static_cast<bf16>(__builtin_amdgcn_exp2f(x0));
          pp[1] = static_cast<bf16>(__builtin_amdgcn_exp2f(x1));
          if (e & 2)
            pb = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, pb, false);
          else
            pa = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, pa, false);
          if constexpr (DIAG) {
            // A masked score gives x = -inf with weight 0: clamp x (exp2 of anything below -150
            // is 0 in fp32 anyway) so that the product stays 0.
            ea = fmaf(static_cast<float>(pp[0]), fmaxf(x0, -256.f), ea);
            ea = fmaf(static_cast<float>(pp[1]), fmaxf(x1, -256.f), ea);
          }
          pf[h][e] = pp[0];
          pf[h][e + 1] = pp[1];
        }
      part = pa + pb;
      if constexpr (DIAG) apart = ea;
    };

    // Lazy reference: the weights are formed against the current reference
    // first; since a lane's partial sum bounds each of its weights, the block is
    // redone against a refreshed reference only if some partial sum exceeds
    // 2^kTau (or some row of the wave has no reference yet).
    bool refresh = !ready;
    if (ready) {
      make_p();
      refresh = __builtin_amdgcn_ballot_w64(part > kThresh) != 0;
    }
    if (refresh) {
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      const float m_new = fmaxf(m_run, half_swap_max(mx) * c);
      // Only rows that held a finite reference rescale their sums when it moves up: a row whose
      // reference is still -inf has seen no visible key, so its sums are exactly 0.  On a wave's first
      // block no row has one, and the rescaling is skipped.
      const bool rescale = m_new > m_run && m_run != -INFINITY;
      if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
        const float alpha = rescale ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        if constexpr (DIAG) a_run = rescale ? alpha * fmaf(m_run - m_new, l_run, a_run) : a_run;
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < C::kBlocks; ++b) acc[b] *= alpha;
      }
      if (m_new > m_run) {
        m_run = m_new;
        m_use = m_new;
      }
      ready = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) == 0;
      make_p();
    }
    l_run += part;
    if constexpr (DIAG) a_run += apart;

    // O^T += V^T P^T over the block's two 16-key steps.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row0 = 32 * mb + 16 * h;
#pragma unroll
      for (int b = 0; b < C::kBlocks; ++b) {
        const char* p = vt_lds + row0 * C::kRowBytes;
        acc[b] = mfma(read_tr(p + v_off[0][b], p + v_off[1][b]), pf[h], acc[b]);
      }
    }
  };

  auto do_tile = [&](const char* kt_lds, const char* vt_lds, int kt) __attribute__((always_inline)) {
    const int k0 = kt * KT;
#pragma unroll
    for (int mb = 0; mb < KT / 32; ++mb) do_block(kt_lds, vt_lds, k0 + 32 * mb, mb);
  };
  auto kst = [&](int i) __attribute__((always_inline)) { return lds + 2 * i * C::kTileBytes; };
  auto vst = [&](int i) __attribute__((always_inline)) { return lds + (2 * i + 1) * C::kTileBytes; };

  // Ring of kNS slots: the v-th stage visited lives in slot v % kNS.  A step
  // issues the copies of stage v + kNS - 1 into the slot every wave finished
  // reading before the barrier that ended the previous step, computes stage v,
  // then waits until its own copies of stage v + 1 have landed (those of later
  // stages may still be in flight) and meets the other waves at the barrier.
  // Returns true after the last stage.
  constexpr int kFill = 2 * C::kDmaPerWave;  // copies per wave per stage
  auto step = [&](int v, int cur, int nxt) __attribute__((always_inline)) {
    const bool fill = v + C::kNS - 1 < n_tiles;
    if (fill) issue_tile(tile_at(v + C::kNS - 1), kst(nxt), vst(nxt));
    do_tile(kst(cur), vst(cur), tile_at(v));
    if (v + 1 >= n_tiles) return true;  // nothing left to wait for; the workgroup is done with LDS
    if (C::kNS == 3 && fill)
      wait_vm_barrier(kFill);
    else
      wait_vm_barrier(0);
    return false;
  };

  // Prologue: the first stage's copies go out before the Q rows are loaded, so
  // that the two round trips overlap; waiting for the rows (which the compiler
  // does where they are consumed, in issue order) then also covers the copies.
  issue_tile(tile_at(0), kst(0), vst(0));
  // Q^T fragments: lane holds q[qi][16 s + 8 hl + 0..7].
  {
    const uint32_t slice_bytes = static_cast<uint32_t>(T) * C::kRowBytes;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qh, slice_bytes);
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, load16(rq, static_cast<uint32_t>(qi) * C::kRowBytes + (16 * s + 8 * hl) * 2));
    if constexpr (kLateW) {
      W = win_eff[hq];
      wave_key_lo = q0w - W + 1;
    }
    // Consume the fragments here, so that the compiler waits for these loads now
    // rather than at their first use inside the loop, where its wait would also
    // cover the LDS copies in flight.
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) __asm__ volatile("" ::"v"(qf[s]));
  }
  if (C::kNS == 3 && n_tiles > 1) {
    issue_tile(tile_at(1), kst(1), vst(1));
    wait_vm_barrier(kFill);
  } else {
    wait_vm_barrier(0);
  }
  if constexpr (C::kNS == 3) {
    for (int v = 0;; v += 3) {
      if (step(v, 0, 2)) break;
      if (step(v + 1, 1, 0)) break;
      if (step(v + 2, 2, 1)) break;
    }
  } else {
    for (int v = 0;; v += 2) {
      if (step(v, 0, 1)) break;
      if (step(v + 1, 1, 0)) break;
    }
  }

  if (!wave_active) return;
  const float l_tot = half_swap_sum(l_run);
  float a_tot = 0.f, sq_tot = 0.f;
  if constexpr (DIAG) {
    a_tot = half_swap_sum(a_run);
    float sq = 0.f;  // this lane's share of |O row|^2 (before the division by l)
#pragma unroll
    for (int b = 0; b < C::kBlocks; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) sq = fmaf(acc[b][r], acc[b][r], sq);
    sq_tot = half_swap_sum(sq);
  }
  if (!row_ok) return;
  if (slot >= 0) {
    // Unnormalised partial of row qi over this chunk's keys: acc (fp32, [d]), then (m, l) with m in
    // the log2 domain (-inf and l = 0 if the row saw none of them); DIAG adds a = sum p x, the weights
    // times their offsets x = s c - m (0 for such a row).
    const size_t prow = static_cast<size_t>(slot) * kRows + wave * 32 + ln;
    float* arow = part_acc + prow * D;
#pragma unroll
    for (int b = 0; b < C::kBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(arow + 32 * b + 8 * i + 4 * hl) =
            f32x4{acc[b][4 * i], acc[b][4 * i + 1], acc[b][4 * i + 2], acc[b][4 * i + 3]};
    if constexpr (DIAG) {
      if (hl == 0)
        *reinterpret_cast<f32x4*>(part_ml + prow * kMlDiag) = f32x4{m_run, l_tot, a_tot, 0.f};
    } else {
      if (hl == 0)
        *reinterpret_cast<u32x2*>(part_ml + prow * 2) = u32x2{__float_as_uint(m_run), __float_as_uint(l_tot)};
    }
    return;
  }
  const float inv = __builtin_amdgcn_rcpf(l_tot);  // l_tot >= 1: the key that set the reference weighs 1
  bf16* Orow = O + base + static_cast<size_t>(qi) * D;
  // O^T block b, register r holds dim 32 b + 8 (r/4) + 4 hl + r%4 of query qi.
#pragma unroll
  for (int b = 0; b < C::kBlocks; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      store_bf16x4(Orow + 32 * b + 8 * i + 4 * hl, acc[b][4 * i] * inv, acc[b][4 * i + 1] * inv,
                   acc[b][4 * i + 2] * inv, acc[b][4 * i + 3] * inv);
  if (hl == 0) {
    const size_t row = static_cast<size_t>(it.bh) * T + qi;
    LSE[row] = (m_run + log2f(l_tot)) * kLn2;
    if constexpr (DIAG) {
      ENT[row] = (log2f(l_tot) - a_tot * inv) * kLn2;
      ONORM[row] = sqrtf(sq_tot) * inv;
    }
  }
}

// Combines the chunks of each split item: with (acc_c, m_c, l_c) the partials
// of row i over chunk c and M = max_c m_c, O_i = sum_c 2^(m_c - M) acc_c /
// sum_c 2^(m_c - M) l_c and LSE_i = (M + log2 sum_c 2^(m_c - M) l_c) ln 2.
// DIAG: the chunks' weighted offsets a_c, taken to the common reference M,
// add up to A = sum_c 2^(m_c - M) (a_c + (m_c - M) l_c) (chunks the row did not
// see count 0), so the entropy is (log2 L - A / L) ln 2 as in an unsplit row,
// and the output norm is |sum_c 2^(m_c - M) acc_c| / L (the D / 4 threads of a
// row, consecutive lanes of one wave, add their squares by lane swaps).
// Workgroup (merge record, row group); D / 4 threads per row, four dims each.
template <int D, bool DIAG>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const WorkItem* __restrict__ merges,
                                                        const float* __restrict__ part_acc,
                                                        const float* __restrict__ part_ml, bf16* __restrict__ O,
                                                        float* __restrict__ LSE, float* __restrict__ ENT,
                                                        float* __restrict__ ONORM, int T) {
  constexpr int kPerRow = D / 4;
  constexpr int kRowsPerWg = 256 / kPerRow;
  constexpr int kMl = DIAG ? kMlDiag : 2;  // floats per row of part_ml
  const WorkItem mg = merges[blockIdx.x];  // {bh, tile, first slot, chunks}
  const int r = blockIdx.y * kRowsPerWg + static_cast<int>(threadIdx.x) / kPerRow;
  const int dq = (static_cast<int>(threadIdx.x) % kPerRow) * 4;
  const int row = mg.tile * kRows + r;
  // Rows past T leave together with the rest of their kPerRow-thread group, so the DIAG lane swaps
  // below only ever combine lanes that are all present.
  if (r >= kRows || row >= T) return;
  float M = -INFINITY;
  for (int ch = 0; ch < mg.hi; ++ch) M = fmaxf(M, part_ml[(static_cast<size_t>(mg.lo + ch) * kRows + r) * kMl]);
  float L = 0.f, A = 0.f;
  f32x4 a = f32x4{};
  for (int ch = 0; ch < mg.hi; ++ch) {
    const size_t prow = static_cast<size_t>(mg.lo + ch) * kRows + r;
    const float m_c = part_ml[prow * kMl];
    const float w = __builtin_amdgcn_exp2f(m_c - M);  // 0 for a chunk the row did not see
    L = fmaf(w, part_ml[prow * kMl + 1], L);
    if constexpr (DIAG) {
      if (m_c != -INFINITY) A = fmaf(w, fmaf(m_c - M, part_ml[prow * kMl + 1], part_ml[prow * kMl + 2]), A);
    }
    const f32x4 x = *reinterpret_cast<const f32x4*>(part_acc + prow * D + dq);
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = fmaf(w, x[j], a[j]);
  }
  const float inv = 1.f / L;
  store_bf16x4(O + (static_cast<size_t>(mg.bh) * T + row) * D + dq, a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
  const size_t orow = static_cast<size_t>(mg.bh) * T + row;
  if constexpr (DIAG) {
    float sq = a[0] * a[0] + a[1] * a[1] + a[2] * a[2] + a[3] * a[3];
#pragma unroll
    for (int o = 1; o < kPerRow; o <<= 1) sq += __shfl_xor(sq, o);
    if (dq == 0) {
      ENT[orow] = (log2f(L) - A * inv) * kLn2;
      ONORM[orow] = sqrtf(sq) * inv;
    }
  }
  if (dq == 0) LSE[orow] = (M + log2f(L)) * kLn2;
}

template <int D, bool SINK, bool DIAG>
void launch_k(const void* q, const void* k, const void* v, void* o, float* lse, float* ent, float* onorm,
              const WorkItem* items, int n_items, const int32_t* win_eff, const int32_t* sink_eff,
              const AttnShape& s, const FwdSplit* split, hipStream_t stream) {
  const float c = s.scale * 1.4426950408889634f;  // scale * log2(e)
  hipLaunchKernelGGL((fwd_bf16_kernel<D, SINK, DIAG>), dim3(n_items), dim3(kThreads), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                     static_cast<bf16*>(o), lse, ent, onorm, items, win_eff, sink_eff, s.H, s.H_kv, s.T, c,
                     split != nullptr ? split->slots : nullptr, split != nullptr ? split->part_acc : nullptr,
                     split != nullptr ? split->part_ml : nullptr, log2_exact(s.H), log2_exact(s.H / s.H_kv));
  if (split != nullptr && split->n_merges > 0)
    hipLaunchKernelGGL((fwd_merge_kernel<D, DIAG>), dim3(split->n_merges, kRows / (256 / (D / 4))), dim3(256), 0,
                       stream, split->merges, split->part_acc, split->part_ml, static_cast<bf16*>(o), lse, ent, onorm,
                       s.T);
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, float* lse, float* ent, float* onorm,
                    const WorkItem* items, int n_items, const int32_t* win_eff, const int32_t* sink_eff,
                    const AttnShape& s, const FwdSplit* split, hipStream_t stream) {
  const bool sink = sink_eff != nullptr, diag = ent != nullptr;
  if (sink && diag)
    launch_k<D, true, true>(q, k, v, o, lse, ent, onorm, items, n_items, win_eff, sink_eff, s, split, stream);
  else if (sink)
    launch_k<D, true, false>(q, k, v, o, lse, ent, onorm, items, n_items, win_eff, sink_eff, s, split, stream);
  else if (diag)
    launch_k<D, false, true>(q, k, v, o, lse, ent, onorm, items, n_items, win_eff, sink_eff, s, split, stream);
  else
    launch_k<D, false, false>(q, k, v, o, lse, ent, onorm, items, n_items, win_eff, sink_eff, s, split, stream);
  return hipGetLastError();
}

}  // namespace

int fwd_bf16_resident(int d) {
  const void* fn = nullptr;
  switch (d) {
    case 32: fn = reinterpret_cast<const void*>(&fwd_bf16_kernel<32, false, false>); break;
    case 64: fn = reinterpret_cast<const void*>(&fwd_bf16_kernel<64, false, false>); break;
    case 128: fn = reinterpret_cast<const void*>(&fwd_bf16_kernel<128, false, false>); break;
    default: return 0;
  }
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess) return 0;
  return per_cu * cus;
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, float* ent,
                           float* onorm, const WorkItem* items, int n_items, const int32_t* win_eff,
                           const int32_t* sink_eff, const AttnShape& s, const FwdSplit* split, hipStream_t stream) {
  switch (s.d) {
    case 32: return launch_d<32>(q, k, v, o, lse, ent, onorm, items, n_items, win_eff, sink_eff, s, split, stream);
    case 64: return launch_d<64>(q, k, v, o, lse, ent, onorm, items, n_items, win_eff, sink_eff, s, split, stream);
    case 128: return launch_d<128>(q, k, v, o, lse, ent, onorm, items, n_items, win_eff, sink_eff, s, split, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace aah
