// Device helpers for CDNA4 (gfx950) shared by the attention kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

// hipError_t of the last failed launch on this thread, shared by every entry point.
namespace attn_detail {
inline thread_local int last_hip_error = 0;
}  // namespace attn_detail

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kXcds = 8;  // MI355X: 8 XCDs, 32 CUs each; workgroup id w runs on XCD w % 8
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaitVm0 = 0;  // s_waitcnt immediate: every counter zero
// s_waitcnt lgkmcnt(0) only (gfx9 encoding: vmcnt 63, expcnt 7).
constexpr int kWaitLgkm0 = 0xF | (7 << 4) | (3 << 14);
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3 for raw 32-bit access (gfx9)

// v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] B[16x32].  Operand layout:
// lane l holds row (A) or column (B) l%32 and the 8 k-elements 8*(l/32)..+7;
// the accumulator: lane l holds column l%32 and rows 8*(r/4) + 4*(l/32) + r%4
// in register r.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: C[16x16] += A[16x32] B[32x16].  Operand layout:
// lane l holds row (A) or column (B) l%16 and the 8 k-elements 8*(l/16)..+7;
// the accumulator: lane l holds column l%16 and rows 4*(l/16) + r in register r.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max(a, b, c) in one instruction.  fmaxf would make the compiler quiet
// possible signalling NaNs of the MFMA results first (an extra instruction per
// operand); scores here are finite or -inf.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Reductions over the lane pair (l, l^32).  v_permlane32_swap exchanges the
// upper half-wave of one register with the lower half-wave of another; with
// x in both, every lane ends up holding x_l in one result and x_(l^32) in the
// other, so a symmetric combine of the two needs no lane select.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return max3f(__uint_as_float(r[0]), __uint_as_float(r[1]), -INFINITY);
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same over the lane pair (l, l^16) with v_permlane16_swap, which exchanges
// the odd 16-lane rows of one register with the even rows of another.
__device__ __forceinline__ float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return max3f(__uint_as_float(r[0]), __uint_as_float(r[1]), -INFINITY);
}
__device__ __forceinline__ float pair16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// exp2 on the FMA pipe (FlashAttention-4 (papercache summary), section
// 3.1.3, the exponential emulated by a polynomial): Cody-Waite split
// x = n + f, n = floor(x), f in [0, 1); 2^f by a degree-3 polynomial with
// p(0) = 1 whose coefficients are the relative-error minimax fit on [0, 1]
// (Remez exchange; max relative error 8.6e-5 in fp32, far below the 2^-9
// of the bf16 rounding that follows); 2^n inserted by adding n to the
// exponent bits.  x is clamped at -127: there n = -127 and f = 0 give exactly
// +0, so a masked score (-inf) still contributes nothing.  Valid for x < 128.
constexpr float kExp2C1 = 0x1.63e658p-1f;
constexpr float kExp2C2 = 0x1.d2378ap-3f;
constexpr float kExp2C3 = 0x1.3baaa6p-4f;

__device__ __forceinline__ float exp2_poly(float x) {
  x = __builtin_fmaxf(x, -127.f);
  const float n = __builtin_floorf(x);
  const float f = x - n;
  const float p = fmaf(fmaf(fmaf(kExp2C3, f, kExp2C2), f, kExp2C1), f, 1.f);
  return __int_as_float(__float_as_int(p) + (static_cast<int>(n) << 23));
}

// Two transpose reads of LDS, concatenated into one 8-element bf16 operand.
__device__ __forceinline__ bf16x8 read_tr_pair(const __bf16* p0, const __bf16* p1) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

}  // namespace
