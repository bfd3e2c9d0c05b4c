// QKV projection with the 3D RoPE of the video rows' queries and keys fused into
// the epilogue: y = x W^T, then (q, k of video rows) rotated, one bf16 rounding.
//
// Pages: the DiT block has hidden size 2,048, 16 heads of 128 and 3D RoPE ("Hy-
// Nomas auf einer RTX 4090", inferencekey.com, section "Modell und Dateien";
// blog.authon.dev, section "What Hy-Nomas is"). W holds the query, key and value
// channels in that order (3 * H * D rows of `hidden`); no bias (none is named).
//
// GEMM design (gfx950, v_mfma_f32_16x16x32_bf16, bf16 in, fp32 accumulate):
//  * The product is formed transposed, y^T = W x^T: W rows are the A operand and
//    x rows the B operand (both contiguous along the hidden dimension), so a
//    lane's accumulator holds 4 consecutive channels of one token -- the RoPE
//    pairs (2j, 2j+1) sit in one lane and a store writes 8 contiguous bytes.
//  * Block = 8 waves = 256 channels x 256 tokens; each wave owns 64 channels x
//    128 tokens (4 x 8 accumulator tiles). The hidden dimension is walked in
//    steps of 64: both 256 x 64 operand tiles are copied global -> LDS by the
//    load unit (buffer_load ... lds, double-buffered, one barrier per step),
//    with the 16-byte chunk index XOR-swizzled by (row / 2) % 8, which keeps a
//    16-lane quarter's fragment reads on 16 distinct bank groups.
//  * Fragments of the second half of a step are requested before the first
//    half's MFMAs; two waves per SIMD cover each other's LDS latency.
//  * Blocks are laid out so each XCD works through whole channel tiles: the
//    W tile stays in that XCD's L2 while token tiles stream past it.
#include "nomas_common.hpp"

namespace nomas {

constexpr int kGemmBM = 256;          // channels per block
constexpr int kGemmBN = 256;          // tokens per block
constexpr int kGemmBK = 64;           // hidden elements per step
constexpr int kGemmThreads = 512;
constexpr int kGemmTileBytes = 256 * kGemmBK * 2;   // one operand tile (32 KB)

__device__ __forceinline__ int gemm_swz(int row) { return (row >> 1) & 7; }

struct GemmArgs {
  const uint16_t* x;
  int64_t ld_x;
  int n_rows;
  int hidden;
  const uint16_t* w;
  int64_t ld_w;
  int n_ch;             // 3 * H * D
  int hd;               // H * D
  int head_dim;
  int n_video;
  const float2* table;  // [n_video][head_dim / 2] (cos, sin), or null
  uint16_t* y;
  int64_t ld_y;
  int tiles_m;          // token tiles
  int n_blocks;
  int per_xcd;
};

__global__ __launch_bounds__(kGemmThreads, 1) void qkv_gemm_kernel(const GemmArgs a) {
  __shared__ __align__(16) unsigned char lds[2 * 2 * kGemmTileBytes];
  auto wbuf = [&](int s) { return lds + s * 2 * kGemmTileBytes; };
  auto xbuf = [&](int s) { return lds + s * 2 * kGemmTileBytes + kGemmTileBytes; };

  const int b = blockIdx.x;
  const int logical = (b & 7) * a.per_xcd + (b >> 3);
  if (logical >= a.n_blocks) return;
  const int tn = __builtin_amdgcn_readfirstlane(logical / a.tiles_m);   // channel tile
  const int tm = __builtin_amdgcn_readfirstlane(logical % a.tiles_m);   // token tile
  const int ch0 = tn * kGemmBM, tok0 = tm * kGemmBN;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4, i16 = lane & 15;
  const int wch = (wave & 3) * 64, wtok = (wave >> 2) * 128;   // the wave's sub-tile

  // rows past the ends read as zeros
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.w) + (int64_t)ch0 * a.ld_w, (short)0,
      (int)(max(0, min(kGemmBM, a.n_ch - ch0)) * a.ld_w * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.x) + (int64_t)tok0 * a.ld_x, (short)0,
      (int)(max(0, min(kGemmBN, a.n_rows - tok0)) * a.ld_x * 2), 0x00020000);

  // each wave instruction fills 1 KB of LDS (8 rows of 128 B); the lane fetches
  // the global chunk that the swizzled layout puts at its position
  auto issue = [&](int kt, int s) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int blk = wave * 4 + k, row = blk * 8 + (lane >> 3), c = (lane & 7) ^ gemm_swz(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)(wbuf(s) + blk * 1024), 16,
                                               row * (int)a.ld_w * 2 + c * 16, kt * kGemmBK * 2, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(xbuf(s) + blk * 1024), 16,
                                               row * (int)a.ld_x * 2 + c * 16, kt * kGemmBK * 2, 0, 0);
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // fragments of half kh (32 hidden elements) of stage s
  auto read = [&](int s, int kh, bf16x8 (&fa)[4], bf16x8 (&fb)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wch + 16 * i + i16;
      fa[i] = *reinterpret_cast<const bf16x8*>(wbuf(s) + r * 128 + (((4 * kh + G) ^ gemm_swz(r)) * 16));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = wtok + 16 * j + i16;
      fb[j] = *reinterpret_cast<const bf16x8*>(xbuf(s) + r * 128 + (((4 * kh + G) ^ gemm_swz(r)) * 16));
    }
  };
  auto mma = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  const int nk = a.hidden / kGemmBK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int s = kt & 1;
    if (kt + 1 < nk) issue(kt + 1, s ^ 1);
    bf16x8 fa0[4], fb0[8], fa1[4], fb1[8];
    read(s, 0, fa0, fb0);
    read(s, 1, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    mma(fa0, fb0);
    mma(fa1, fb1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: RoPE on query/key channels of video rows, one bf16 rounding
  const int D = a.head_dim, P = D / 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = ch0 + wch + 16 * i + 4 * G;     // channels ch .. ch+3
    if (ch >= a.n_ch) continue;
    const bool rot = a.table && ch < 2 * a.hd;
    const int p0 = (ch % D) / 2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tok = tok0 + wtok + 16 * j + i16;
      if (tok >= a.n_rows) continue;
      f32x4 v = acc[i][j];
      if (rot && tok < a.n_video) {
        const float2 c0 = a.table[(int64_t)tok * P + p0], c1 = a.table[(int64_t)tok * P + p0 + 1];
        const float u0 = v[0], w0 = v[1], u1 = v[2], w1 = v[3];
        v[0] = fmaf(u0, c0.x, -w0 * c0.y);
        v[1] = fmaf(u0, c0.y, w0 * c0.x);
        v[2] = fmaf(u1, c1.x, -w1 * c1.y);
        v[3] = fmaf(u1, c1.y, w1 * c1.x);
      }
      *reinterpret_cast<uint2*>(a.y + (int64_t)tok * a.ld_y + ch) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  }
}

// table[i][p] = (cos, sin)(pos_axis(i, p) * w[p]) for the video rows of a segment
struct RopeTableFreq {
  float w[64];
};
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ table, int n_rows, int pairs, int t0,
                                                         int grid_h, int grid_w, int pairs_t, int pairs_th,
                                                         RopeTableFreq f) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)n_rows * pairs) return;
  const int row = (int)(i / pairs), p = (int)(i % pairs);
  const int gs = grid_h * grid_w;
  const int pos = p < pairs_t ? t0 + row / gs : (p < pairs_th ? (row / grid_w) % grid_h : row % grid_w);
  float s, c;
  sincosf(static_cast<float>(pos) * f.w[p], &s, &c);
  table[i] = make_float2(c, s);
}

}  // namespace nomas

using namespace nomas;

extern "C" int32_t nomas_rope3d_table(float* table, int32_t head_dim, int32_t t0, int32_t n_frames, int32_t grid_h,
                                      int32_t grid_w, int32_t d_t, int32_t d_h, int32_t d_w, float theta,
                                      int32_t inverse, void* stream) {
  const char* who = "rope3d_table";
  if (!table || (reinterpret_cast<uintptr_t>(table) & 7)) return fail(NOMAS_E_INVALID, "%s: table must be non-NULL and 8-byte aligned", who);
  if (head_dim != 64 && head_dim != 128) return fail(NOMAS_E_UNSUPPORTED, "%s: head_dim must be 64 or 128", who);
  if (d_t < 0 || d_h < 0 || d_w < 0 || (d_t | d_h | d_w) & 1 || d_t + d_h + d_w != head_dim)
    return fail(NOMAS_E_INVALID, "%s: band widths (%d,%d,%d) must be even and sum to head_dim %d", who, d_t, d_h, d_w,
                head_dim);
  if (t0 < 0 || n_frames < 1 || grid_h < 1 || grid_w < 1)
    return fail(NOMAS_E_INVALID, "%s: need t0 >= 0, n_frames >= 1, grid_h >= 1, grid_w >= 1", who);
  if (!(theta > 0.f)) return fail(NOMAS_E_INVALID, "%s: theta must be > 0", who);
  const int64_t n_rows = (int64_t)n_frames * grid_h * grid_w;
  if (n_rows * head_dim > INT32_MAX || (int64_t)t0 + n_frames > (1 << 24))
    return fail(NOMAS_E_INVALID, "%s: too many rows or positions beyond 2^24", who);
  RopeTableFreq f;
  const int widths[3] = {d_t, d_h, d_w};
  const double sign = inverse ? -1.0 : 1.0;
  int p = 0;
  for (int ax = 0; ax < 3; ++ax)
    for (int j = 0; j < widths[ax] / 2; ++j) f.w[p++] = static_cast<float>(sign * pow((double)theta, -2.0 * j / widths[ax]));
  const int pairs = head_dim / 2;
  const int64_t n = n_rows * pairs;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, as_stream(stream),
                     reinterpret_cast<float2*>(table), (int)n_rows, pairs, t0, grid_h, grid_w, d_t / 2,
                     (d_t + d_h) / 2, f);
  return check_launch(who);
}

extern "C" int32_t nomas_qkv_projection(const uint16_t* x, int64_t ld_x, int32_t n_rows, int32_t hidden,
                                        const uint16_t* w, int64_t ld_w, int32_t n_heads, int32_t head_dim,
                                        int32_t n_video, const float* rope_table, uint16_t* qkv, int64_t ld_qkv,
                                        void* stream) {
  const char* who = "qkv_projection";
  if (!x || !w || !qkv) return fail(NOMAS_E_INVALID, "%s: x, w, qkv must be non-NULL", who);
  if (!aligned16(x) || !aligned16(w) || !aligned16(qkv)) return fail(NOMAS_E_INVALID, "%s: x, w, qkv must be 16-byte aligned", who);
  if (rope_table && (reinterpret_cast<uintptr_t>(rope_table) & 7))
    return fail(NOMAS_E_INVALID, "%s: rope_table must be 8-byte aligned", who);
  if (head_dim != 64 && head_dim != 128) return fail(NOMAS_E_UNSUPPORTED, "%s: head_dim must be 64 or 128", who);
  if (n_heads < 1 || n_rows < 1 || hidden < kGemmBK || hidden % kGemmBK)
    return fail(NOMAS_E_INVALID, "%s: need n_heads >= 1, n_rows >= 1, hidden a positive multiple of %d", who, kGemmBK);
  if (n_video < 0 || n_video > n_rows) return fail(NOMAS_E_INVALID, "%s: need 0 <= n_video <= n_rows", who);
  const int64_t n_ch = 3LL * n_heads * head_dim;
  if (ld_x < hidden || ld_x % 8 || ld_w < hidden || ld_w % 8 || ld_qkv < n_ch || ld_qkv % 4)
    return fail(NOMAS_E_INVALID, "%s: ld_x, ld_w >= hidden (multiples of 8), ld_qkv >= 3*n_heads*head_dim (a multiple of 4)", who);
  if ((int64_t)kGemmBM * ld_w * 2 > INT32_MAX || (int64_t)kGemmBN * ld_x * 2 > INT32_MAX || n_ch > (1 << 20))
    return fail(NOMAS_E_INVALID, "%s: sizes out of range", who);
  GemmArgs a;
  a.x = x;
  a.ld_x = ld_x;
  a.n_rows = n_rows;
  a.hidden = hidden;
  a.w = w;
  a.ld_w = ld_w;
  a.n_ch = (int)n_ch;
  a.hd = n_heads * head_dim;
  a.head_dim = head_dim;
  a.n_video = rope_table ? n_video : 0;
  a.table = reinterpret_cast<const float2*>(rope_table);
  a.y = qkv;
  a.ld_y = ld_qkv;
  a.tiles_m = (n_rows + kGemmBN - 1) / kGemmBN;
  const int tiles_n = (int)((n_ch + kGemmBM - 1) / kGemmBM);
  a.n_blocks = tiles_n * a.tiles_m;
  a.per_xcd = (a.n_blocks + 7) / 8;
  hipLaunchKernelGGL(qkv_gemm_kernel, dim3((unsigned)(8 * a.per_xcd)), dim3(kGemmThreads), 0, as_stream(stream), a);
  return check_launch(who);
}
