// Decoding over per-head trimmed K/V caches (bf16, gfx950).
//
// Operation: one decoding step of "Asymmetric Attention Heads" section 5.8 --
// the newest token at position p of query head h (window W_h, maximum context
// T_max) attends to positions max(0, p - C_h + 1) .. p, C_h = min(W_h, T_max),
// and, for a streaming head ("Autonomy-of-Heads" section 5: sink tokens plus a
// recent window), to its sink positions 0 .. S_h - 1 as well.  With grouped
// key/value heads (G = H / H_kv query heads per key/value head), head h reads
// key/value head h / G.
//
// Cache: key/value head g keeps S_g sink rows (position j in row j) and a ring
// of R_g rows (position t in row S_g + t mod R_g), R_g and S_g the largest
// window and sink its query heads need; heads are back to back.  A query head
// attends to the ring rows younger than its window and to the sink rows that
// lie before its window, so no position counts twice; softmax does not depend
// on the order of its keys, so rows are used where they lie.
//
// The step reads every needed K and V row once (the G query heads of a group
// share the loads), so it is bound by HBM bandwidth, not by arithmetic.
// Kernels:
//   decode_kernel -- one workgroup = kDecodeRows rows of one key/value head's
//     region (kDecodeRowsGrouped with grouped heads, whose rows serve G query
//     heads each, so that fewer partials per head are left to merge); each
//     wave takes 64 rows.  Lane = row for the scores (its K row is
//     one contiguous 2 d-byte read; q . k with v_dot2_f32_bf16 on bf16 pairs);
//     for P V each lane takes 16 bytes (8 dimensions) of d / 8 rows, so every
//     V load instruction reads 512 / d whole rows.  The query rows, K and V
//     are all requested, through buffer resources whose range check turns the
//     rows no head needs into zeros, before the first wait and with no branch
//     among them, so a workgroup pays one HBM round trip.  The new token's
//     K / V come from k_new / v_new and are stored into their rows by the
//     lanes that hold them, so no separate append launch and no ordering
//     between workgroups is needed.  For each query
//     head of the group in turn the waves merge (max, sum, weighted values) in
//     LDS and the workgroup writes one unnormalised partial; the last
//     workgroup of a (b, g) to finish (a per-(b, g) counter in the workspace,
//     reset by that workgroup) merges each head's partials with log-sum-exp
//     rescaling and writes o (bf16) and lse (fp32).
//   cache_fill_kernel -- copies the positions each region keeps out of a
//     prefill [B, H_kv, T, d] into the cache layout.
#include <cmath>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace aah {
namespace {

using namespace dev;

constexpr int kRowsPerWave = 64;
// Waves per workgroup: kDecodeRows (kDecodeRowsGrouped with grouped heads) rows, 64 per wave.
template <bool GROUPED>
constexpr int decode_waves() { return (GROUPED ? kDecodeRowsGrouped : kDecodeRows) / kRowsPerWave; }
static_assert(decode_waves<false>() * kRowsPerWave == kDecodeRows &&
                  decode_waves<true>() * kRowsPerWave == kDecodeRowsGrouped && decode_waves<true>() <= 8,
              "chunk size");

// Lane x from lane l ^ 1, l ^ 2 (quad permutations) or rotated by 4 / 8 within its 16-lane row (DPP).
template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor4 = 0x124, kDppRor8 = 0x128;

// Wave-wide max and sum without LDS traffic: within quads, across the quads of each 16-lane row by
// rotations, then the 16- and 32-lane swaps.
__device__ inline float wave_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppRor4>(x));
  x = fmaxf(x, dpp<kDppRor8>(x));
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Device-coherent (all XCDs) store and load of one float.
__device__ inline void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum over the lanes l, l + LR, l + 2 LR, ... of a wave (LR in {4, 8, 16}: the lanes holding the same
// P V dimensions), with no LDS traffic: rotations within each 16-lane row, then the 16- and 32-lane swaps.
template <int LR>
__device__ inline float group_sum(float x) {
  if constexpr (LR <= 4) x += dpp<kDppRor4>(x);
  if constexpr (LR <= 8) x += dpp<kDppRor8>(x);
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

__device__ inline float wave_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  return group_sum<4>(x);
}

// Local rows of key/value head g's region: rows [0, S_g) are sinks (row j holds position j), rows
// [S_g, S_g + R_g) the ring (row S_g + r holds the newest position t <= p with t mod R_g = r, whose
// age p - t is (p mod R_g) - r, plus R_g if negative).  Query head h (window C_h, effective sink
// S_h) attends at position p to
//   ring rows of age below C_h and no older than the sequence (age <= p), and
//   sink rows j < min(S_h, p - C_h + 1): sinks that lie before its window, so no position counts twice.
// Every test below is a compare against per-workgroup scalars: the row's age needs no division.
__device__ __forceinline__ int ring_age(int local, int S_g, int R_g, int pr) {
  const int a = pr - (local - S_g);
  return a < 0 ? a + R_g : a;
}

template <int D, bool GROUPED>
__global__ __launch_bounds__(64 * decode_waves<GROUPED>()) void decode_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ Knew, const bf16* __restrict__ Vnew,
    bf16* __restrict__ Kc, bf16* __restrict__ Vc, const int32_t* __restrict__ pos,
    const DecodeChunk* __restrict__ chunks, const int32_t* __restrict__ q_cap, const int32_t* __restrict__ q_sink,
    int H, int H_kv, int R, int T_max, float c, int32_t* __restrict__ counters,
    float* __restrict__ part, int n_chunks, bf16* __restrict__ O, float* __restrict__ LSE) {
  constexpr int kDecodeWaves = decode_waves<GROUPED>();
  // Per-wave partials of up to kGB query heads at a time, merged across the waves after one barrier (a
  // round's query rows, kGB * D / 8 pieces of 16 bytes, are read by one wave's lanes).
  constexpr int kGB = GROUPED ? (kDecodeWaves < 512 / D ? kDecodeWaves : 512 / D) : 1;
  __shared__ float sm_m[kGB][kDecodeWaves], sm_l[kGB][kDecodeWaves];
  __shared__ float sm_o[kGB][kDecodeWaves][D];
  __shared__ __attribute__((aligned(16))) bf16 sm_q[kDecodeWaves][kGB * D];  // one copy per wave
  __shared__ u32x4 sm_knew[D / 8];
  __shared__ __attribute__((aligned(16))) float sm_p[kDecodeWaves][kRowsPerWave];  // one head's weights, per wave
  __shared__ int sm_last;

  const int ch = blockIdx.x, b = blockIdx.y;
  // The position and the chunk record (everything the row addresses need) are independent scalar loads:
  // both are issued before either is waited for.
  const int pos_b = pos[b];
  const DecodeChunk ck = chunks[ch];
  __asm__ volatile("" ::"s"(pos_b), "s"(ck.kvhead));
  const int g = ck.kvhead;
  const int G = GROUPED ? H / H_kv : 1;  // query heads per key/value head (one: plain heads)
  const int S_g = ck.sink, R_g = ck.ring;
  const int p = min(max(pos_b, 0), T_max - 1);
  const int pr = p % R_g;
  const int new_ring = S_g + pr;            // local row of the new token in the ring
  const int new_sink = p < S_g ? p : -1;     // and of its sink copy
  // Sink rows below sink_lim may be attended by some query head of the group: head h attends to the sink
  // rows j < min(S_h, p - C_h + 1), and S_h <= S_g, C_h >= cap_s for every head with sinks (S_g = 0 if none).
  // Exact with one query head per group; with several it may also load rows no head attends to, which
  // are positions already written (j <= p) and get zero weight.
  const int sink_lim = max(0, min(S_g, p - ck.cap_s + 1));
  const size_t bg = static_cast<size_t>(b) * H_kv + g;
  const bf16* knew = Knew + bg * D;
  const bf16* vnew = Vnew + bg * D;
  const size_t region = (static_cast<size_t>(b) * R + ck.off) * D;  // first element of head g's rows
  bf16* kreg = Kc + region;
  bf16* vreg = Vc + region;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int w0 = ck.row0 + wave * kRowsPerWave;  // first local row of this wave

  // The rows some query head of the group attends to form two runs: sink rows [0, sink_lim) and ring
  // rows [S_g, S_g + ring_live).  The widest window is R_g, so only the age <= p test thins the ring,
  // and while p < R_g the ring rows no older than p are exactly its first p + 1.
  const int ring_live = min(p + 1, R_g);
  auto needed_any = [&](int r) __attribute__((always_inline)) {
    return (static_cast<unsigned>(r) < static_cast<unsigned>(sink_lim)) |
           (static_cast<unsigned>(r - S_g) < static_cast<unsigned>(ring_live));
  };
  const int row = w0 + lane;
  const bool any = needed_any(row);
  const bool is_sink = row < S_g;
  const int age = ring_age(row, S_g, R_g, pr);

  // ---- all loads first, with no branch among them, so that a workgroup pays one round trip for its rows.
  // K: lane = row, its whole row.  V: lane (rg, dg) takes dimensions 8 dg .. 8 dg + 7 of rows rg + kRG i
  // (kLR lanes per row, so each load instruction reads kRG whole rows).  Both come through buffer
  // resources over the region's rows: a row no query head attends to, and each row of the new token, is
  // addressed past the range and reads as zero (a zero weight then never meets stale bits); the new
  // token's K and V come from k_new / v_new below.
  constexpr int kLR = D / 8;                // lanes per V row, 16 bytes each
  constexpr int kRG = 64 / kLR;             // rows per V load instruction
  constexpr int kVL = kRowsPerWave / kRG;   // V loads per lane
  constexpr uint32_t kPast = 0x80000000u;   // past any region (regions are under 2 T_max rows, < 2^31 bytes)
  const uint32_t region_bytes = static_cast<uint32_t>(S_g + R_g) * D * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kreg, region_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vreg, region_bytes);
  // Query rows of the current round of (at most kGB) query heads go through LDS, every lane then reading
  // the same bytes (a broadcast): each wave's first nb D / 8 lanes read 16 bytes each into the wave's
  // own copy (so no barrier: one wave's LDS accesses are in order), issued before the rows so that they
  // arrive first.  (No branch around any load: a value defined on one side of a branch makes the
  // compiler wait for it at the join, before the loads after it are issued.)
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + static_cast<size_t>(b) * H * D, static_cast<uint32_t>(H) * D * 2);
  auto q_piece = [&](int jb) __attribute__((always_inline)) {
    const int nb = GROUPED ? min(kGB, G - jb) : 1;
    const bool has = lane < nb * (D / 8);  // other lanes read past the range (no access)
    return load16(rq, has ? static_cast<uint32_t>((g * G + jb) * D + 8 * lane) * 2 : kPast);
  };
  u32x4 qpiece = q_piece(0);
  const bool owns_new = row == new_ring || row == new_sink;
  const uint32_t koff = (any & !owns_new) ? static_cast<uint32_t>(row) * D * 2 : kPast;
  bf16x8 kr[D / 8];
#pragma unroll
  for (int i = 0; i < D / 8; ++i) kr[i] = __builtin_bit_cast(bf16x8, load16(rk, koff + 16 * i));
  const int dg = lane % kLR, rg = lane / kLR;
  bf16x8 vr[kVL];
#pragma unroll
  for (int i = 0; i < kVL; ++i) {
    const int vrow = w0 + rg + kRG * i;
    const bool use = needed_any(vrow) & (vrow != new_ring);  // (the new token's sink copy is never attended)
    vr[i] = __builtin_bit_cast(bf16x8, load16(rv, use ? static_cast<uint32_t>(vrow) * D * 2 + 16 * dg : kPast));
  }
  // The wave holding a row of the new token (its ring row and, while p < S_g, its sink row) takes that
  // row's K and V from k_new / v_new and stores them into the cache; no workgroup reads either row from
  // memory during this step (the sink copy is first attended once the window has moved past it).
  const bool wave_new = static_cast<unsigned>(new_ring - w0) < static_cast<unsigned>(kRowsPerWave) ||
                        static_cast<unsigned>(new_sink - w0) < static_cast<unsigned>(kRowsPerWave);
  if (wave_new) {
    // Vector loads, past the range where not needed (in scalar registers the rows would crowd out the
    // addressing state): lanes 0 .. D / 8 - 1 read k_new, which goes to the owning lanes through LDS
    // (one wave's LDS accesses are in order), and every lane reads v_new's 16 bytes at its dimensions.
    const __amdgpu_buffer_rsrc_t rkn = make_rsrc(knew, D * 2), rvn = make_rsrc(vnew, D * 2);
    const u32x4 kpiece = load16(rkn, lane < D / 8 ? 16u * lane : kPast);
    const bf16x8 vslice = __builtin_bit_cast(bf16x8, load16(rvn, 16 * dg));
    if (lane < D / 8) sm_knew[lane] = kpiece;  // two waves of a workgroup may both write: the same bytes
    if (owns_new) {
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        kr[i] = __builtin_bit_cast(bf16x8, sm_knew[i]);
        *reinterpret_cast<bf16x8*>(kreg + static_cast<size_t>(row) * D + 8 * i) = kr[i];
      }
    }
    if (rg == 0) {  // lanes 0 .. D / 8 - 1 hold the new V row between them
      if (static_cast<unsigned>(new_ring - w0) < static_cast<unsigned>(kRowsPerWave))
        *reinterpret_cast<bf16x8*>(vreg + static_cast<size_t>(new_ring) * D + 8 * dg) = vslice;
      if (static_cast<unsigned>(new_sink - w0) < static_cast<unsigned>(kRowsPerWave))
        *reinterpret_cast<bf16x8*>(vreg + static_cast<size_t>(new_sink) * D + 8 * dg) = vslice;
    }
#pragma unroll
    for (int i = 0; i < kVL; ++i)
      if (w0 + rg + kRG * i == new_ring) vr[i] = vslice;
  }

  // Grouped heads: V regrouped for v_dot2_f32_bf16, dword x of vpk[j] holding dimension x of this lane's
  // rows 2 j and 2 j + 1, so each of the G heads' P V takes one dot2 per dimension and row pair with no
  // conversions (one head alone does not repay the regrouping).
  uint32_t vpk[kVL / 2][8];
#pragma unroll
  for (int j = 0; j < (GROUPED ? kVL / 2 : 0); ++j) {
    const u32x4 a = __builtin_bit_cast(u32x4, vr[2 * j]), bb = __builtin_bit_cast(u32x4, vr[2 * j + 1]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      vpk[j][2 * k] = __builtin_amdgcn_perm(bb[k], a[k], 0x05040100u);      // low halves: dimension 2 k
      vpk[j][2 * k + 1] = __builtin_amdgcn_perm(bb[k], a[k], 0x07060302u);  // high halves: dimension 2 k + 1
    }
  }

  const int c0 = ck.first, c1 = ck.first + ck.count;
  float* pbase = part + static_cast<size_t>(b) * n_chunks * G * (2 + D);
  // ---- the group's query heads in rounds of kGB: each wave forms every head's scores, softmax partial
  // and P V over its rows into LDS; after one barrier wave w merges head w of the round across the waves
  // and writes the workgroup's partial.
  for (int jb = 0; jb < G; jb += kGB) {
    const int nb = GROUPED ? min(kGB, G - jb) : 1;
    if (jb > 0) qpiece = q_piece(jb);
    if (lane < nb * (D / 8)) *reinterpret_cast<u32x4*>(sm_q[wave] + 8 * lane) = qpiece;
    for (int u = 0; u < nb; ++u) {
      const int jh = jb + u;
      const int h = g * G + jh;
      const int C_h = q_cap[h];
      const bool valid = is_sink ? row < min(q_sink[h], p - C_h + 1)
                                 : static_cast<unsigned>(row - S_g) < static_cast<unsigned>(ring_live) && age < C_h;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        const bf16x8 qv = *reinterpret_cast<const bf16x8*>(sm_q[wave] + u * D + 8 * i);
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
      const float s = valid ? (s0 + s1) * c : -INFINITY;
      const float m_w = wave_max(s);
      const float pw = (valid && m_w != -INFINITY) ? __builtin_amdgcn_exp2f(s - m_w) : 0.f;
      const float l_w = wave_sum(pw);  // exact fp32 row sum, so the log-sum-exp stays fp32-accurate

      // P V: lane (rg, dg) sums its kVL rows for its 8 dimensions, then the kRG row groups of the wave
      // that hold the same dimensions (lanes dg, dg + kLR, ...) add up theirs.
      float acc[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[x] = 0.f;
      // The weights reach the P V lanes through the wave's LDS row: lane r writes its weight at
      // (r mod kRG) kVL + r / kRG, so lane (rg, dg) reads its kVL weights (rows rg + kRG i, 0 for rows
      // this head does not attend to) as consecutive floats.  One wave's LDS accesses are in order.
      sm_p[wave][(lane % kRG) * kVL + lane / kRG] = pw;
      float pk[kVL];
#pragma unroll
      for (int i = 0; i < kVL; i += 4) *reinterpret_cast<f32x4*>(pk + i) = *reinterpret_cast<const f32x4*>(&sm_p[wave][rg * kVL + i]);
      if constexpr (GROUPED) {
#pragma unroll
        for (int j = 0; j < kVL / 2; ++j) {
          // P V multiplies bf16-rounded weights (relative error 2^-9 each, so |o| moves by at most
          // 2^-9 max |v|, below the output's own bf16 rounding)
          const bf16x2 pp = {static_cast<bf16>(pk[2 * j]), static_cast<bf16>(pk[2 * j + 1])};
#pragma unroll
          for (int x = 0; x < 8; ++x)
            acc[x] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, vpk[j][x]), pp, acc[x], false);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kVL; ++i)
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[x] = fmaf(pk[i], static_cast<float>(vr[i][x]), acc[x]);
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[x] = group_sum<kLR>(acc[x]);

      if (lane == 0) {
        sm_m[u][wave] = m_w;
        sm_l[u][wave] = l_w;
      }
      if (rg == 0) {
#pragma unroll
        for (int x = 0; x < 8; ++x) sm_o[u][wave][8 * dg + x] = acc[x];
      }
    }
    __syncthreads();
    if (wave < nb) {
      const int u = wave, jh = jb + wave;
      float m = sm_m[u][0];
#pragma unroll
      for (int w = 1; w < kDecodeWaves; ++w) m = fmaxf(m, sm_m[u][w]);
      float f[kDecodeWaves];
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w)
        f[w] = sm_m[u][w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm_m[u][w] - m);
      // The workgroups of one (b, g) may run on different XCDs, whose L2 caches are not coherent
      // with each other: partials go out with device-coherent stores, the counter is a
      // device-scope atomic issued once those stores have completed, and the merging workgroup
      // reads the partials with device-coherent loads.  (Release / acquire fences would write back
      // and invalidate whole L2 caches instead.)
      //
      // Why this handoff is ordered, in the terms of the AMDGPU memory model (LLVM's AMDGPUUsage,
      // the GFX942 / gfx950 code sequences): an agent-scope atomic load, store or RMW is a plain
      // global memory instruction with the sc1 cache-policy bit, so a store writes through the
      // XCD's L2 to the device-coherent level and a load or RMW is served from that level, never
      // from a stale L2 line.  On this target stores are counted by vmcnt, and vmcnt reaches 0
      // only once each store is acknowledged at the scope its policy names; the writer waits for
      // vmcnt(0) (and, with several storing waves, a barrier after each wave's own wait) before
      // the counter RMW is issued.  That is the release sequence of the model without its
      // buffer_wbl2, which only writes back lines of earlier non-coherent stores; every access to
      // a partial here is agent-scope.  On the reading side the merge's loads depend on the RMW's
      // returned value (branch on sm_last after a barrier), so they issue after the RMW has
      // completed and see every partial whose writer incremented the counter before it; the
      // acquire sequence's buffer_inv is again only for later non-coherent loads.
      float* out = pbase + (static_cast<size_t>(ch) * G + jh) * (2 + D);
      if (lane == 0) {
        coherent_store(out, m);
        float lsum = 0.f;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) lsum = fmaf(f[w], sm_l[u][w], lsum);
        coherent_store(out + 1, lsum);
      }
      for (int d = lane; d < D; d += 64) {
        float od = 0.f;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) od = fmaf(f[w], sm_o[u][w][d], od);
        coherent_store(out + 2 + d, od);
      }
    }
    if (jb + kGB < G) __syncthreads();  // the next round reuses the LDS buffers
  }
  if constexpr (GROUPED) {
    // Several waves stored partials: each waits for its own stores, then the barrier orders them
    // before the counter.
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  if (wave == 0) {
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) {
      const int done = __hip_atomic_fetch_add(&counters[bg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm_last = done == c1 - c0 - 1;
    }
  }
  __syncthreads();
  if (!sm_last) return;
  if (tid == 0) __hip_atomic_store(&counters[bg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next call
  // The last workgroup of (b, g) merges every chunk's partial of each query head: wave w takes heads
  // w, w + kDecodeWaves, ...  One pass with running rescaling (as in online softmax): chunks go in
  // batches of kMergeBatch whose loads (every lane reads each chunk's max and sum, and its own value
  // dimensions) all leave before the first is used, so a step with up to kMergeBatch chunks per head
  // pays one round trip for the merge.  Some chunk holds the new token's row, which every head
  // attends to, so the final max is finite and the sum positive.
  constexpr int kX = (D + 63) / 64;
  constexpr int kMergeBatch = 16;
  const int nc = c1 - c0;
  for (int jh = wave; jh < G; jh += kDecodeWaves) {
    const size_t bh = static_cast<size_t>(b) * H + g * G + jh;
    float m = -INFINITY, l = 0.f, o[kX];
#pragma unroll
    for (int x = 0; x < kX; ++x) o[x] = 0.f;
    for (int base = 0; base < nc; base += kMergeBatch) {
      float mu[kMergeBatch], lu[kMergeBatch], vu[kMergeBatch][kX];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const int cc = c0 + min(base + u, nc - 1);  // slots past the last chunk re-read it and are dropped
        const float* pc = pbase + (static_cast<size_t>(cc) * G + jh) * (2 + D);
        mu[u] = coherent_load(pc);
        lu[u] = coherent_load(pc + 1);
#pragma unroll
        for (int x = 0; x < kX; ++x) vu[u][x] = lane + 64 * x < D ? coherent_load(pc + 2 + lane + 64 * x) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const float mc = base + u < nc ? mu[u] : -INFINITY;
        const float mn = fmaxf(m, mc);
        const float a = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        const float f = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - mn);
        l = fmaf(f, lu[u], l * a);
#pragma unroll
        for (int x = 0; x < kX; ++x) o[x] = fmaf(f, vu[u][x], o[x] * a);
        m = mn;
      }
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int x = 0; x < kX; ++x)
      if (lane + 64 * x < D) O[bh * D + lane + 64 * x] = static_cast<bf16>(o[x] * inv);
    if (lane == 0) LSE[bh] = (m + log2f(l)) * kLn2;
  }
}

// One thread per 16-byte piece of a kept row: (b, g, kept row, piece).  Kept rows of key/value head g:
// positions 0 .. min(S_g, T) - 1 into the sink rows, then the last min(R_g, T) positions into the ring.
template <int D>
__global__ __launch_bounds__(256) void cache_fill_kernel(const bf16* __restrict__ K, const bf16* __restrict__ V,
                                                         bf16* __restrict__ Kc, bf16* __restrict__ Vc,
                                                         const int32_t* __restrict__ kv_off,
                                                         const int32_t* __restrict__ kv_sink,
                                                         const int32_t* __restrict__ kv_ring, int H_kv, int T, int R) {
  constexpr int kPieces = D / 8;
  const int bg = blockIdx.y;
  const int b = bg / H_kv, g = bg % H_kv;
  const int S_g = kv_sink[g], R_g = kv_ring[g];
  const int ks = min(S_g, T), kr = min(R_g, T);
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (ks + kr) * kPieces) return;
  const int k = idx / kPieces, piece = idx % kPieces;
  int t, local;
  if (k < ks) {
    t = k;
    local = k;
  } else {
    t = T - kr + (k - ks);
    local = S_g + t % R_g;
  }
  const size_t src = (static_cast<size_t>(bg) * T + t) * D + 8 * piece;
  const size_t dst = (static_cast<size_t>(b) * R + kv_off[g] + local) * D + 8 * piece;
  *reinterpret_cast<bf16x8*>(Kc + dst) = *reinterpret_cast<const bf16x8*>(K + src);
  *reinterpret_cast<bf16x8*>(Vc + dst) = *reinterpret_cast<const bf16x8*>(V + src);
}

template <int D>
hipError_t decode_d(const void* q, const void* knew, const void* vnew, void* kc, void* vc, const int32_t* pos,
                    const DecodePlanView& pl, int B, int T_max, float scale, void* o, float* lse,
                    int32_t* counters, float* part, hipStream_t stream) {
  const float c = scale * kLog2e;
  if (pl.H_kv != pl.H)
    hipLaunchKernelGGL((decode_kernel<D, true>), dim3(pl.n_chunks, B), dim3(64 * decode_waves<true>()), 0, stream,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(knew), static_cast<const bf16*>(vnew),
                       static_cast<bf16*>(kc), static_cast<bf16*>(vc), pos, pl.chunks, pl.q_cap, pl.q_sink, pl.H,
                       pl.H_kv, pl.rows, T_max, c, counters, part, pl.n_chunks, static_cast<bf16*>(o), lse);
  else
    hipLaunchKernelGGL((decode_kernel<D, false>), dim3(pl.n_chunks, B), dim3(64 * decode_waves<false>()), 0, stream,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(knew), static_cast<const bf16*>(vnew),
                       static_cast<bf16*>(kc), static_cast<bf16*>(vc), pos, pl.chunks, pl.q_cap, pl.q_sink, pl.H,
                       pl.H_kv, pl.rows, T_max, c, counters, part, pl.n_chunks, static_cast<bf16*>(o), lse);
  return hipGetLastError();
}

template <int D>
hipError_t fill_d(const void* k, const void* v, void* kc, void* vc, const DecodePlanView& pl, int B, int T,
                  hipStream_t stream) {
  int max_kept = 0;
  for (int g = 0; g < pl.H_kv; ++g) max_kept = max(max_kept, min(pl.host_kv_sink[g], T) + min(pl.host_kv_ring[g], T));
  const int pieces = max_kept * (D / 8);
  hipLaunchKernelGGL(cache_fill_kernel<D>, dim3((pieces + 255) / 256, B * pl.H_kv), dim3(256), 0, stream,
                     static_cast<const bf16*>(k), static_cast<const bf16*>(v), static_cast<bf16*>(kc),
                     static_cast<bf16*>(vc), pl.kv_off, pl.kv_sink, pl.kv_ring, pl.H_kv, T, pl.rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const void* q, const void* knew, const void* vnew, void* kcache, void* vcache,
                              const int32_t* pos, const DecodePlanView& plan, int B, int T_max, int d, float scale,
                              void* o, float* lse, int32_t* counters, float* partials, hipStream_t stream) {
  switch (d) {
    case 32:
      return decode_d<32>(q, knew, vnew, kcache, vcache, pos, plan, B, T_max, scale, o, lse, counters, partials,
                          stream);
    case 64:
      return decode_d<64>(q, knew, vnew, kcache, vcache, pos, plan, B, T_max, scale, o, lse, counters, partials,
                          stream);
    case 128:
      return decode_d<128>(q, knew, vnew, kcache, vcache, pos, plan, B, T_max, scale, o, lse, counters, partials,
                           stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_cache_fill_bf16(const void* k, const void* v, void* kcache, void* vcache,
                                  const DecodePlanView& plan, int B, int T, int d, hipStream_t stream) {
  switch (d) {
    case 32: return fill_d<32>(k, v, kcache, vcache, plan, B, T, stream);
    case 64: return fill_d<64>(k, v, kcache, vcache, plan, B, T, stream);
    case 128: return fill_d<128>(k, v, kcache, vcache, plan, B, T, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace aah
