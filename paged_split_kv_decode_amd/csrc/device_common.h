// Device helpers shared by the gfx950 kernels of this library.
//
// Everything here is CDNA4-specific: wave64 lane shuffles, the MFMA operand
// vector types, direct global->LDS loads and the LDS transpose read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pd {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define PD_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
// lse = +inf ends a split-slot list (the slots after it are not read)
__device__ __forceinline__ float end_of_slots() { return __builtin_inff(); }

// 2^x on the hardware transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the hardware unit (v_log_f32).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Lane exchange across the whole wave64 (ds_bpermute based).
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  int src = (lane_id() ^ mask) << 2;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(v)));
}

// Wave64 inclusive prefix sum / prefix max with DPP: four row shifts scan
// each 16-lane row, then two row broadcasts carry the totals of rows 0..2
// forward (row_shr:n = 0x110 + n, row_bcast:15 = 0x142 into rows 1 and 3,
// row_bcast:31 = 0x143 into rows 2 and 3).  Lanes a shift leaves without a
// source take the identity.
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return x;
}
__device__ __forceinline__ int wave_incl_max(int x) {
  constexpr int kMin = -0x7fffffff - 1;
  x = max(x, __builtin_amdgcn_update_dpp(kMin, x, 0x111, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(kMin, x, 0x112, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(kMin, x, 0x114, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(kMin, x, 0x118, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(kMin, x, 0x142, 0xa, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(kMin, x, 0x143, 0xc, 0xf, false));
  return x;
}
// Sum / max over the 64 lanes (every lane gets the result): the last lane
// of the inclusive scan.
__device__ __forceinline__ int wave_sum(int v) { return __builtin_amdgcn_readlane(wave_incl_sum(v), 63); }
__device__ __forceinline__ int wave_max(int v) { return __builtin_amdgcn_readlane(wave_incl_max(v), 63); }

// Exchanges with the lane 16 or 32 apart as VALU permutes (v_permlane16_swap
// / v_permlane32_swap swap row pairs between two registers; with the value
// in both, each lane ends up holding itself and its partner, in some
// order), combined with a commutative operation.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float readlane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// fp32 -> bf16 bits with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
// (converted as a pair: one v_cvt_pk_bf16_f32; two scalar casts became two
// conversions, a shift and an or)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

#define PD_CONST __attribute__((address_space(4)))

// Read-only int32 data the kernel never writes (block tables, lengths),
// viewed through the constant address space: a wave-uniform load from it
// becomes a scalar s_load (counted by lgkmcnt, not vmcnt), which keeps the
// vmcnt bookkeeping of the LDS-DMA page ring exact.
__device__ __forceinline__ const PD_CONST int32_t* as_const(const int32_t* p) {
  return (const PD_CONST int32_t*)p;
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): the wave writes 64 consecutive 16-byte chunks
// starting at LDS byte address `lds_addr` (wave-uniform, goes to M0); lane
// i's chunk comes from `base + voff_i` (base wave-uniform).
//
// Issued as inline asm on purpose: the compiler's own wait insertion treats
// every later LDS read as dependent on every outstanding LDS-DMA and would
// drain the whole ring (vmcnt(0)) before each transpose read.  Callers own
// the ordering instead: `wait_vmcnt<N>()` before reading a slot (vector
// memory ops complete in order) and `wait_lgkmcnt0()` before refilling a
// slot that was just read.  The `s_nop` covers the M0-write -> LDS-DMA hazard.
// A wave-uniform 64-bit address that the asm takes in a scalar register
// pair: read from the first lane, so a value the compiler happened to keep in
// vector registers still fits the "s" operand (free when already scalar).
__device__ __forceinline__ const void* scalar_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void global_to_lds_16(const void* base, uint32_t voff, uint32_t lds_addr) {
  base = scalar_ptr(base);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_addr), "v"(voff), "s"(base)
      : "memory", "m0");
}
// Same, with the LDS address given as a wave-uniform base plus a constant
// byte offset that is added inside the asm, so a run of loads into one LDS
// buffer keeps a single base in a scalar register.  The load carries the
// non-temporal (`nt`) cache policy: data read once should not displace
// anything in the caches, and on MI355X streaming reads marked this way reach
// about 7.1 TB/s against about 6.0 TB/s without it.
template <uint32_t kOff>
__device__ __forceinline__ void global_to_lds_16_stream(const void* base, uint32_t voff, uint32_t lds_base) {
  base = scalar_ptr(base);
  asm volatile(
      "s_add_u32 m0, %0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2 nt"
      :
      : "s"(lds_base), "v"(voff), "s"(base), "i"(kOff)
      : "memory", "m0", "scc");
}
// Same, with a per-lane 64-bit source address (the instruction's vaddr
// form): for rows of one load that come from different pages.
__device__ __forceinline__ void global_to_lds_16_v(const void* src, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(lds_addr), "v"(src)
      : "memory", "m0");
}
// The non-temporal variant of the vaddr form.
template <uint32_t kOff>
__device__ __forceinline__ void global_to_lds_16_stream_v(const void* src, uint32_t lds_base) {
  asm volatile(
      "s_add_u32 m0, %0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt"
      :
      : "s"(lds_base), "v"(src), "i"(kOff)
      : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(PD_LDS const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// s_waitcnt with only the vector-memory counter constrained.  gfx9 encoding:
// vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits 15:14; expcnt (6:4) and
// lgkmcnt (11:8) left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

}  // namespace pd
