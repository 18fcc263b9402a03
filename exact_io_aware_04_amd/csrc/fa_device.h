// Device helpers shared by the gfx950 attention kernels (fa_fwd.hip,
// fa_bwd.hip): vector types, buffer and wait-count encodings, the matrix-core
// product, conversions to the 16-bit input types and lane-half exchanges.
// Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

typedef __bf16 fa_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 fa_f16x8 __attribute__((ext_vector_type(8)));
typedef float fa_f32x16 __attribute__((ext_vector_type(16)));
typedef float fa_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int fa_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int fa_u32x2 __attribute__((ext_vector_type(2)));
typedef short fa_i16x4 __attribute__((ext_vector_type(4)));

#define FA_AS3 __attribute__((address_space(3)))
#define FA_NEG_INF (-__builtin_inff())
#define FA_LN2 0.69314718055994530942f
// buffer descriptor word 3 for raw (unformatted, unswizzled) buffer access
#define FA_BUF_WORD3 0x00020000
// s_waitcnt immediate for vmcnt <= v and lgkmcnt == 0 (expcnt at its "no
// wait" maximum; vmcnt is split over bits 3:0 and 15:14)
#define FA_WAITCNT_VM_LGKM0(v) ((((v) & 15) | (((v) >> 4) << 14)) | (7 << 4))
// s_waitcnt immediate for lgkmcnt == 0 only (vmcnt and expcnt at their
// "no wait" maxima)
#define FA_WAITCNT_LGKM0 (15 | (3 << 14) | (7 << 4))

// Workgroup barrier without a memory fence: the caller has already waited
// for exactly the memory operations that must be complete.  (A fenced
// barrier would also wait for the K/V blocks still in flight.)  The asm is a
// compiler memory barrier, so no LDS access moves across it.
namespace {

__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// matrix-core products, conversions, lane-half exchange
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ fa_f32x16 mma16(fa_u32x4 a, fa_u32x4 b, fa_f32x16 c) {
  if constexpr (DT == 2)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(fa_bf16x8, a), __builtin_bit_cast(fa_bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(
        __builtin_bit_cast(fa_f16x8, a), __builtin_bit_cast(fa_f16x8, b), c, 0, 0, 0);
}

// Round 8 floats to the 16-bit input type (nearest even), packed in 4 words.
template <int DT>
__device__ __forceinline__ fa_u32x4 pack8(const float* x) {
  if constexpr (DT == 2) {
    fa_bf16x8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (__bf16)x[i];
    return __builtin_bit_cast(fa_u32x4, h);
  } else {
    fa_f16x8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)x[i];
    return __builtin_bit_cast(fa_u32x4, h);
  }
}

template <int DT>
__device__ __forceinline__ fa_u32x2 pack4(float a, float b, float c, float d) {
  if constexpr (DT == 2) {
    __bf16 h[4] = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    return __builtin_bit_cast(fa_u32x2, h);
  } else {
    _Float16 h[4] = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
    return __builtin_bit_cast(fa_u32x2, h);
  }
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// A pointer that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ const unsigned char* uniform_ptr(const unsigned char* ptr) {
  const unsigned long long v = (unsigned long long)ptr;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return (const unsigned char*)(((unsigned long long)hi << 32) | lo);
}

// Lanes l and l^32 hold the same query row: combine their values.  The swap
// leaves each lane with its own value in one result and its partner's in the
// other, so max / sum of the two results is the pair's max / sum.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte chunk swizzles of K and V rows in LDS (chunk position = chunk ^
// swizzle of the row).  K rows are read 16 rows x one chunk per 16 lanes, V
// rows 8 rows x 4 chunks per wavefront by the transposing read; each swizzle
// spreads every such access over distinct chunk slots of the LDS banks.  Rows
// of 128 and 256 elements start on the same bank, so both use the
// 128-element swizzle (it flips chunk bits 0-3 and 2-3, staying inside each
// 16-chunk half row).
template <int D>
__device__ __forceinline__ int kswz(int r) { return D >= 128 ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1)); }
template <int D>
__device__ __forceinline__ int vswz(int r) { return D >= 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

}  // namespace
