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

}  // namespace nomas
