// Shared host/device helpers of libnomas (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "nomas.h"

namespace nomas {

// ---- host-side error reporting (thread-local message, see nomas_last_error) ----
int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int32_t ok();
int32_t check_launch(const char* what);   // hipGetLastError after a launch

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Token rows reserved per head in a cache buffer (multiple of the largest key tile).
constexpr int kTokenAlign = 128;

// ---- device-side index checks. In a build with NOMAS_DEVICE_CHECKS defined,
// NOMAS_IN_BOUNDS(c) evaluates c, counts each false one in the source file's
// failure counter and returns it, so the access it guards is skipped instead
// of leaving its buffer; otherwise it is the constant true and c is not even
// evaluated (the kernels compile as if the guard were absent).
#ifdef NOMAS_DEVICE_CHECKS
static __device__ unsigned int g_check_failures;
__device__ __forceinline__ bool in_bounds_counted(bool c) {
  if (!c) atomicAdd(&g_check_failures, 1u);
  return c;
}
#define NOMAS_IN_BOUNDS(c) (::nomas::in_bounds_counted(c))
// this source file's failure count (reset: also clear it); needs the device current
static inline int64_t source_check_failures(int reset) {
  unsigned int v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_check_failures), sizeof v, 0, hipMemcpyDeviceToHost) != hipSuccess)
    return -1;
  if (reset) {
    const unsigned int z = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_check_failures), &z, sizeof z, 0, hipMemcpyHostToDevice) != hipSuccess)
      return -1;
  }
  return v;
}
#else
#define NOMAS_IN_BOUNDS(c) true
static inline int64_t source_check_failures(int) { return -1; }
#endif

// ---- device helpers ----
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16x2, round to nearest even: one v_cvt_pk_bf16_f32 on
// gfx950 (converting the pair as a vector; element-wise casts become one
// conversion per element plus a v_perm to join them)
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}


// ---- INT8 codes (the quantise-append and the fused projection). A vector with
// absmax m has the scale s = fp32(m / 127) (a correctly rounded division) and x
// the code RNE(fp32(x / s)). The fast path forms it from the exact product
// x * r, r = rcp(s) (within 1 ulp of 1/s): with C = 1.5 * 2^23,
// f = fma(x, r, C) is C + RNE(x * r) (one rounding, to an integer, ties to
// even), and d = fma(x, r, C - f) is the distance of x * r from that integer.
// |x*r - x/s| <= 127 * 2^-23 and |fp32(x/s) - x/s| <= 127 * 2^-24, so while
// |d| <= 1/2 - 2^-14 no half-integer lies between x * r and fp32(x/s) and both
// round to the same code. Otherwise (about one code in 8,000), and for scales
// of 0 or below 2^-120 (r is then NaN: rcp would overflow, and the scale's own
// rounding can push |x/s| past 127.5), the code comes from the IEEE quotient,
// clamped. A code c is carried as the float C + c, whose low byte is c in two's
// complement.
constexpr float kMagic = 12582912.0f;            // 1.5 * 2^23
constexpr float kNearHalf = 0.5f - 0x1p-14f;
constexpr float kMinFastScale = 0x1p-120f;

// the reciprocal the fast path multiplies by (NaN sends every code of a scale
// below 2^-120, or of zero, to the exact path)
__device__ __forceinline__ float code_recip(float s) {
  return s >= kMinFastScale ? __builtin_amdgcn_rcpf(s) : __builtin_nanf("");
}
// fast code of x (C + code); clears ok when the exact path must decide
__device__ __forceinline__ float code_fast(float x, float r, bool& ok) {
  const float f = fmaf(x, r, kMagic);
  const float d = fmaf(x, r, kMagic - f);
  ok &= fabsf(d) <= kNearHalf;          // false for NaN
  return f;
}
// exact code of x from the IEEE quotient (C + code)
__device__ __forceinline__ float code_exact(float x, float s) {
  const bool pos = s > 0.f;
  const float q = fminf(fmaxf(rintf(x / (pos ? s : 1.f)), -127.f), 127.f);
  return (pos ? q : 0.f) + kMagic;
}
// low bytes of four code floats -> one dword (bytes in argument order)
__device__ __forceinline__ unsigned pack4(float c0, float c1, float c2, float c3) {
  const unsigned lo = __builtin_amdgcn_perm(__float_as_uint(c1), __float_as_uint(c0), 0x0c0c0400u);
  const unsigned hi = __builtin_amdgcn_perm(__float_as_uint(c3), __float_as_uint(c2), 0x04000c0cu);
  return lo | hi;
}

}  // namespace nomas
