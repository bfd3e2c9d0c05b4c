// Counter calibration for global -> LDS copies (measurement aid, not part of
// the method).
//
// The attention and projection kernels bring their operand tiles into LDS with
// buffer_load ... lds, 16 bytes per lane. rocprofv3's FETCH_SIZE does not count
// every access pattern at the same scale, so the HBM bytes of those kernels are
// scaled by what the counter reads for this kernel, which moves a known number
// of bytes the same way: each block streams its contiguous 1 MiB slice of the
// source through a 32 KB LDS ring, one 1 KB wave instruction at a time, and
// then writes one word so the copies have an observer. Every source byte is
// fetched exactly once.
#include "nomas_common.hpp"

namespace nomas {

constexpr int64_t kCalSliceBytes = int64_t(1) << 20;

__global__ __launch_bounds__(256) void lds_stream_kernel(const unsigned char* src, int64_t bytes, unsigned* sink) {
  __shared__ __align__(16) unsigned char ring[32 * 1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t base = (int64_t)blockIdx.x * kCalSliceBytes;
  const int n = (int)min(kCalSliceBytes, bytes - base);   // a multiple of 1 KB
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(src) + base, (short)0, n, 0x00020000);
  for (int off = wave * 1024; off < n; off += 4 * 1024) {
    unsigned char* dst = ring + ((off >> 10) & 31) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, lane * 16, off, 0,
                                             0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = *reinterpret_cast<const unsigned*>(ring);
}

}  // namespace nomas

using namespace nomas;

extern "C" int64_t nomas_calibrate_lds_stream_blocks(int64_t bytes) {
  if (bytes <= 0 || bytes % 1024) return -1;
  return (bytes + kCalSliceBytes - 1) / kCalSliceBytes;
}

extern "C" int32_t nomas_calibrate_lds_stream(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  const int64_t blocks = nomas_calibrate_lds_stream_blocks(bytes);
  if (blocks < 1 || blocks > INT32_MAX)
    return fail(NOMAS_E_INVALID, "calibrate_lds_stream: bytes must be a positive multiple of 1024");
  if (!src || !aligned16(src) || !sink || (reinterpret_cast<uintptr_t>(sink) & 3))
    return fail(NOMAS_E_INVALID, "calibrate_lds_stream: src must be 16-byte aligned and sink 4-byte aligned");
  hipLaunchKernelGGL(lds_stream_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const unsigned char*>(src), bytes, sink);
  if (int32_t e = check_launch("calibrate_lds_stream")) return e;
  return ok();
}
