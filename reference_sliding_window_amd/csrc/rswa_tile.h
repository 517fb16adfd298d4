// Tile helpers shared by the packed (matrix-core) kernels of librswa. Internal.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rswa {
namespace tile {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// Native vectors for 16- and 8-byte moves (HIP's uint4 is a struct whose copies
// go through private memory).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kD = 128;                   // head dim of the packed kernels
constexpr int kRowBytes = kD * 2;         // 256-byte bf16 rows in LDS, no padding
constexpr float kNegInf = -__builtin_huge_valf();

__device__ constexpr bf16x2_t kOnes = {(__bf16)1.0f, (__bf16)1.0f};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Physical 16-byte chunk of logical chunk c in row r of a 256-byte-row LDS tile:
// c ^ chunk_swz(r). Eight consecutive rows read at one chunk (MFMA row fragments)
// and four consecutive rows read at four neighbouring chunks (transposing reads)
// then hit distinct banks.
__device__ __forceinline__ int chunk_swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// Byte offset of the row fragment lane (l32, hi) reads for k-step ks: row l32,
// logical chunk 2 ks + hi (8 consecutive d starting at 16 ks + 8 hi).
__device__ __forceinline__ uint32_t row_frag_off(int l32, int hi, int ks) {
  return l32 * kRowBytes + 16 * ((2 * ks + hi) ^ chunk_swz(l32));
}

// Byte offset for the transposing read (ds_read_b64_tr_b16) that builds half h2
// of a 32x32x16 MFMA operand holding 8 tile rows x one d per lane: within each
// 16-lane group G = lane / 16, lane s addresses row 8 h2 + 4 (G / 2) + e and
// d = 32 db + 16 (G % 2) + 4 q (e = s / 4 mod 4, q = s mod 4); lane i of the
// group then receives d = 32 db + lane % 32 of the rows base + e, e = 0..3. The
// row-dependent part of the swizzle is the same for every 16-row step st, so
// step st adds 16 st rows.
__device__ __forceinline__ uint32_t tr_off(int lane, int db, int h2) {
  const int G = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
  const int row = 8 * h2 + 4 * (G >> 1) + e;
  const int chunk = (4 * db + 2 * (G & 1) + (q >> 1)) ^ chunk_swz(row);
  return row * kRowBytes + 16 * chunk + 8 * (q & 1);
}

// x combined with the other half-wave's copy (lanes l and l ^ 32 exchange
// through v_permlane32_swap): their max, or their sum.
__device__ __forceinline__ float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The 32x32x16 operand for 16-row step st and d block db from two transposing reads.
__device__ __forceinline__ bf16x8_t tr_operand(const char *tile, uint32_t off0, uint32_t off1, int st) {
  const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(tile + off0 + 16 * st * kRowBytes));
  const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(tile + off1 + 16 * st * kRowBytes));
  const u32x2_t a0 = __builtin_bit_cast(u32x2_t, v0), a1 = __builtin_bit_cast(u32x2_t, v1);
  return as_bf16x8(u32x4_t{a0.x, a0.y, a1.x, a1.y});
}

// LDS DMA (global_load_lds_*) is issued from inline asm so that the compiler
// does not track it: tracked, it makes every transposing LDS read (whose memory
// operand carries no alias information) wait for all DMA in flight, which
// defeats prefetching. The instruction has no register outputs. Callers order
// DMA writes before LDS reads themselves: s_waitcnt vmcnt on the issuing wave,
// then block_barrier(). The LDS base goes in M0 (one wait state before use).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void_t *)p));
}

// 16 bytes per lane from a wave-uniform 64-bit base in scalar registers plus a
// 32-bit per-lane byte offset (the instruction's saddr form). M0 is saved and
// restored around the instruction: the compiler reserves it.
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds_base) {
  // The base is the same in every lane; say so where the compiler cannot tell.
  const uint64_t a = reinterpret_cast<uintptr_t>(sbase);
  // (readfirstlane returns int: each half goes through uint32_t, never sign-extended)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint64_t ua = (uint64_t)lo | ((uint64_t)hi << 32);
  sbase = reinterpret_cast<const void *>(ua);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// 4 bytes per lane from a per-lane 64-bit address.
__device__ __forceinline__ void dma4(const void *src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// Workgroup barrier with no memory fence of its own (a fence would wait for all
// DMA in flight); the compiler may not move memory accesses across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt with only vmcnt = n (n < 16); expcnt and lgkmcnt left at their maximum.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0f70 | n);
}

}  // namespace tile
}  // namespace rswa
