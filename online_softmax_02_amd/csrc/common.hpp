// Device helpers shared by the gfx950 kernels: vector types, exp2, wave64
// reductions and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osx {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;  // MFMA bf16 operand: 8 values per lane
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Buffer resource over [base, base + bytes): raw buffer loads past `bytes`
// return zeros, which is how ragged tails are zero-filled without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
}
__device__ __forceinline__ f32x4 buf_ld16f(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maximum): placed where
// all vector-memory loads are known to be complete, so the compiler's waitcnt
// analysis does not carry "maybe pending" loads into the next loop iteration.
// Debug build (OSX_DEBUG_SYNC=1, library libosx_debug_sync.so): an extra full
// wait (vector memory, LDS and scalar memory) and workgroup barrier at every
// LDS stage boundary that all wavefronts of a workgroup pass together, and an
// extra full wait at every wavefront-private LDS stage.  Only the timing
// changes: the results must equal the default build's bit for bit, and a
// difference would mean that some stage was read before it was complete, or
// overwritten while still in use.
#if defined(OSX_DEBUG_SYNC) && OSX_DEBUG_SYNC
#define OSX_DEBUG_SYNC_WG()                 \
  do {                                      \
    __builtin_amdgcn_sched_barrier(0);      \
    __builtin_amdgcn_s_waitcnt(0);          \
    __builtin_amdgcn_s_barrier();           \
    __builtin_amdgcn_sched_barrier(0);      \
  } while (0)
#define OSX_DEBUG_SYNC_WAVE()               \
  do {                                      \
    __builtin_amdgcn_sched_barrier(0);      \
    __builtin_amdgcn_s_waitcnt(0);          \
    __builtin_amdgcn_sched_barrier(0);      \
  } while (0)
#else
#define OSX_DEBUG_SYNC_WG() \
  do {                      \
  } while (0)
#define OSX_DEBUG_SYNC_WAVE() \
  do {                        \
  } while (0)
#endif

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over lane pairs (i, i ^ 32) with v_permlane32_swap, which trades
// the upper 32 lanes of one register for the lower 32 of another in the VALU
// (no LDS round trip).  Swapping two copies of v leaves, in every lane, one
// register with v of lane i mod 32 and one with v of lane i mod 32 + 32, so
// both halves compute the same expression in the same order.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Butterfly reductions over all 64 lanes of a wavefront.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Merge two online-softmax states (m, l) whose m is in the log2 domain:
// l = l_a 2^(m_a - m) + l_b 2^(m_b - m), m = max(m_a, m_b).  Empty states
// carry m = -inf, l = 0.
__device__ __forceinline__ void merge_ml(float& m, float& l, float mb, float lb) {
  float mn = fmaxf(m, mb);
  if (mn == kNegInf) return;  // both empty
  l = l * exp2_fast(m - mn) + lb * exp2_fast(mb - mn);
  m = mn;
}

// Two fp32 -> packed bf16 (round to nearest even) in one 32-bit word.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 h = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                              float a7) {
  u32x4 u = {pack_bf16x2(a0, a1), pack_bf16x2(a2, a3), pack_bf16x2(a4, a5), pack_bf16x2(a6, a7)};
  return __builtin_bit_cast(bf16x8, u);
}

// Eight fp32 values rounded to bf16 (nearest even) and packed as an MFMA
// operand, with their sum (of the rounded values) added to `acc` on the dot2
// unit: each v_dot2_f32_bf16 adds one packed pair times (1, 1).  The pairs are
// summed from the packed 32-bit words themselves, not extracted back out of
// the bf16x8 vector.
__device__ __forceinline__ bf16x8 pack_bf16x8_sum(const float (&p)[8], float& acc) {
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  const uint32_t w0 = pack_bf16x2(p[0], p[1]), w1 = pack_bf16x2(p[2], p[3]);
  const uint32_t w2 = pack_bf16x2(p[4], p[5]), w3 = pack_bf16x2(p[6], p[7]);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), one, acc, false);
  const u32x4 u = {w0, w1, w2, w3};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

}  // namespace osx
