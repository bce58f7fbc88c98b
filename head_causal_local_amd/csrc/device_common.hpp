// Device-side helpers shared by the bf16 MFMA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace aah {
namespace dev {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define AAH_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit words, bounds-checked

// v_mfma_f32_32x32x16_bf16 lane layouts (lane l, half h = l / 32):
//   A (32 x 16): lane holds A[l % 32][8 h .. 8 h + 7]
//   B (16 x 32): lane holds B[8 h .. 8 h + 7][l % 32]
//   C (32 x 32): register r holds C[8 (r / 4) + 4 h + r % 4][l % 32]
__device__ inline f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Lanes l and l ^ 32 hold the same MFMA column; combine their values.
__device__ inline float half_swap_max(float x) {
  // permlane32_swap(x, x): lanes < 32 get (own, partner) and lanes >= 32 get (partner, own).
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource covering `bytes` bytes from `p`; loads past the end return zero.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), kBufferFlags);
}

__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_off), 0, 0));
}

// Raw buffer resource words (base, stride 0, range in bytes, flags) for the
// LDS-copy instruction below, which takes them as a scalar quad.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ inline i32x4 rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 r;
  r[0] = static_cast<int>(static_cast<uint32_t>(a));
  r[1] = static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xFFFFu);
  r[2] = static_cast<int>(bytes);
  r[3] = kBufferFlags;
  return r;
}

// The resource words as wave-uniform values.  They always are uniform (built
// from kernel arguments and workgroup-uniform indices), but under register
// pressure the compiler may keep them in vector registers, which the "s"
// operands of the copy instructions below cannot take; reading the first lane
// makes them scalar again (and costs nothing when they already are).
__device__ inline i32x4 uniform(const i32x4& r) {
  i32x4 u;
  u[0] = __builtin_amdgcn_readfirstlane(r[0]);
  u[1] = __builtin_amdgcn_readfirstlane(r[1]);
  u[2] = __builtin_amdgcn_readfirstlane(r[2]);
  u[3] = __builtin_amdgcn_readfirstlane(r[3]);
  return u;
}

// Asynchronous copy of 16 bytes per lane from a buffer straight into LDS
// (buffer_load_dwordx4 ... lds): lane i's bytes land at lds_base + 16 i, where
// lds_base must be uniform across the wave.  Loads past the resource's range
// deliver zeros.  Completion is counted by vmcnt and is the caller's to wait
// for (wait_vm_barrier).  Issued as inline assembly so that the compiler's own
// wait-count bookkeeping does not serialise later LDS reads of other buffers
// behind these copies.  The LDS address goes in M0, which the compiler itself
// sets from the "{m0}" operand (it keeps M0 for its own uses, so the assembly
// names it as an input rather than writing it).
__device__ inline void dma16(const i32x4& rsrc, const void* lds_base, uint32_t byte_off) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(lds_base)));
  __asm__ volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(byte_off), "s"(uniform(rsrc)), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                   : "memory");
}

// As dma16 with 4 bytes per lane (buffer_load_dword ... lds): lane i's word
// lands at lds_base + 4 i.
__device__ inline void dma4(const i32x4& rsrc, const void* lds_base, uint32_t byte_off) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(lds_base)));
  __asm__ volatile("buffer_load_dword %0, %1, 0 offen lds"
                   :
                   : "v"(byte_off), "s"(uniform(rsrc)), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                   : "memory");
}

// Workgroup barrier after waiting until at most n of this wave's vector-memory
// operations (loads, LDS copies) are outstanding; n is a literal 0..15.  The
// memory clobber keeps the compiler from moving memory accesses across it.
#define wait_vm_barrier(n) __asm__ volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(n) : "memory")

// XOR swizzle of the 16-byte chunks of a row-major bf16 tile whose rows hold
// NC chunks (NC = d / 8): logical chunk c of row r is stored at chunk
// c ^ swz<NC>(r).  gfx950's LDS serves 256 bytes per cycle from 64 four-byte
// banks, i.e. sixteen 16-byte bank groups.  The swizzle makes both read
// patterns of the kernels touch every bank group once per cycle:
//   * ds_read_b128 of one logical chunk by 16 consecutive rows (one MFMA
//     operand; 16 lanes per cycle), and
//   * ds_read_b64_tr_b16 of four consecutive rows 4k .. 4k + 3 at four chunks
//     (32 lanes per cycle).
// (A tile probe measured 3.8 conflict cycles per ds_read_b128 without a
// swizzle adapted to 64 banks and none with this one.)
template <int NC>
__device__ constexpr int swz(int r) {
  return NC >= 16 ? (((r & 3) << 2) | ((r >> 2) & 3))
       : NC == 8  ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3))
                  : ((r >> 2) & 3);
}

__device__ inline float load_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(byte_off), 0, 0));
}

// ds_read_b64_tr_b16 works on 16-lane groups: if source lane s of a group
// addresses row R0 + s / 4, columns C0 + 4 (s % 4) .. + 3 of a row-major bf16
// tile, destination lane i of the group receives column C0 + i, rows R0 .. R0 + 3.
// Two reads, the second of rows R0 + 8 .. R0 + 11 (at its own, swizzled,
// address), give eight rows of one column: an MFMA A or B operand whose k index
// runs down the tile.
__device__ inline bf16x8 read_tr(const void* lo, const void* hi) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AAH_LDS s16x4*)(lo));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AAH_LDS s16x4*)(hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Store 4 consecutive fp32 values as bf16 (round to nearest even) with one 8-byte store.
__device__ inline void store_bf16x4(bf16* dst, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = static_cast<bf16>(a);
  v[1] = static_cast<bf16>(b);
  v[2] = static_cast<bf16>(c);
  v[3] = static_cast<bf16>(d);
  *reinterpret_cast<u32x2*>(dst) = __builtin_bit_cast(u32x2, v);
}

// Eight bf16 values times c, each rounded back to bf16 (nearest even).
__device__ inline bf16x8 scale_bf16x8(const bf16x8& x, float c) {
  bf16x8 y;
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = static_cast<bf16>(static_cast<float>(x[i]) * c);
  return y;
}

}  // namespace dev
}  // namespace aah
