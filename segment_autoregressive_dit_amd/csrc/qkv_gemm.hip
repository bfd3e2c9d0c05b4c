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
//  * Block = 8 waves = 256 channels x 256 tokens, one block per CU; each wave
//    owns 64 channels x 128 tokens (4 x 8 accumulator tiles). The hidden
//    dimension is walked in steps of 32: both 256 x 32 operand tiles are copied
//    global -> LDS by the load unit (buffer_load ... lds) into a ring of four
//    stages, one barrier per step, with the 16-byte chunk index XOR-swizzled by
//    (row/4) % 4. (Block, wave tile and ring depth are the NOMAS_GEMM_CFG
//    defaults below.)
//  * Software pipeline: a step's MFMAs use fragments read during the previous
//    step, while they read the next step's fragments (from a stage made
//    resident by the previous barrier) and the load unit refills the step's own
//    stage four steps ahead; a step waits only for the copies two steps ahead,
//    so each copy has three steps to land.
//  * Blocks are laid out so each XCD works through whole channel tiles: the
//    W tile stays in that XCD's L2 while token tiles stream past it.
#include <type_traits>

#include "nomas_common.hpp"

namespace nomas {

// Block tile BM channels x BN tokens, wave tile WM x WN, ring of S stages.
#ifndef NOMAS_GEMM_CFG
#define NOMAS_GEMM_CFG 256, 256, 64, 128, 4, 1, 8
#endif
template <int BM_, int BN_, int WM_, int WN_, int S_, int MINB_, int GROUPN_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, S = S_, MINB = MINB_, GROUPN = GROUPN_;
  static constexpr int NW = (BM / WM) * (BN / WN);
  static constexpr int NT = NW * 64;
  static constexpr int BK = 32;                    // hidden elements per step
  static constexpr int TI = WM / 16, TJ = WN / 16; // accumulator tiles per wave
  static constexpr int WBYTES = BM * BK * 2, XBYTES = BN * BK * 2;
  static constexpr int IW = WBYTES / 1024 / NW, IX = XBYTES / 1024 / NW;   // copies per wave and stage
  static constexpr int IPS = IW + IX;
  static_assert(IW * NW * 1024 == WBYTES && IX * NW * 1024 == XBYTES, "tiles must split into 1 KB copies per wave");
  static_assert(S >= 3 && (S - 2) * IPS <= 63, "ring depth");
  static_assert(TJ % 2 == 0 || TI <= TJ, "fragment refill pattern");
};
using GC = GemmCfg<NOMAS_GEMM_CFG>;

// 64-byte rows of 4 chunks; the chunk index is XOR-ed with (row / 4) % 4, so the
// 16 rows a quarter-wave reads at one chunk fall on 16 distinct bank groups
__device__ __forceinline__ int gemm_swz(int row) { return (row >> 2) & 3; }

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
  int tiles_n;          // channel tiles
  int tiles_m;          // token tiles
  int n_blocks;
  int per_xcd;
};

// Workgroup barrier without the memory fence __syncthreads() carries (which
// waits for every outstanding load, the prefetched copies included); the
// compiler may not move memory accesses across it. Callers wait for exactly
// what must have landed first.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt with vmcnt(n), lgkmcnt(0) (expcnt left alone)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

__global__ __launch_bounds__(GC::NT, GC::MINB) void qkv_gemm_kernel(const GemmArgs a) {
  constexpr int BM = GC::BM, BN = GC::BN, WM = GC::WM, WN = GC::WN, S = GC::S, BK = GC::BK;
  constexpr int TI = GC::TI, TJ = GC::TJ, IPS = GC::IPS;
  __shared__ __align__(16) unsigned char lds[S * (GC::WBYTES + GC::XBYTES)];
  auto wbuf = [&](int st) { return lds + st * (GC::WBYTES + GC::XBYTES); };
  auto xbuf = [&](int st) { return lds + st * (GC::WBYTES + GC::XBYTES) + GC::WBYTES; };

  // block -> (channel tile, token tile): an XCD works through a contiguous range,
  // in groups of GROUPN channel tiles cycled fastest, so the blocks running
  // together share both their weight and their token tiles in that XCD's L2
  const int b = blockIdx.x;
  const int logical = (b & 7) * a.per_xcd + (b >> 3);
  if (logical >= a.n_blocks) return;
  const int per_group = GC::GROUPN * a.tiles_m;
  const int first_n = (logical / per_group) * GC::GROUPN;
  const int gsize = min(a.tiles_n - first_n, GC::GROUPN);
  const int tn = __builtin_amdgcn_readfirstlane(first_n + (logical % per_group) % gsize);
  const int tm = __builtin_amdgcn_readfirstlane((logical % per_group) / gsize);
  const int ch0 = tn * BM, tok0 = tm * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4, i16 = lane & 15;
  const int wch = (wave % (BM / WM)) * WM, wtok = (wave / (BM / WM)) * WN;

  // rows past the ends read as zeros; base and size pinned to scalar registers
  // (a descriptor the compiler cannot prove uniform turns every load into a
  // loop over lanes)
  auto scalar_ptr = [](const uint16_t* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v & 0xffffffffu)));
    const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v >> 32)));
    return reinterpret_cast<uint16_t*>(lo | (hi << 32));
  };
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      scalar_ptr(a.w + (int64_t)ch0 * a.ld_w), (short)0,
      __builtin_amdgcn_readfirstlane((int)(max(0, min(BM, a.n_ch - ch0)) * a.ld_w * 2)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      scalar_ptr(a.x + (int64_t)tok0 * a.ld_x), (short)0,
      __builtin_amdgcn_readfirstlane((int)(max(0, min(BN, a.n_rows - tok0)) * a.ld_x * 2)), 0x00020000);

  // each wave instruction fills 1 KB of LDS (16 rows of 64 B); the lane fetches
  // the global chunk that the swizzled layout puts at its position
  auto issue = [&](int kt, int st) {
#pragma unroll
    for (int k = 0; k < GC::IW; ++k) {
      const int blk = wave * GC::IW + k, row = blk * 16 + (lane >> 2), c = (lane & 3) ^ gemm_swz(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)(wbuf(st) + blk * 1024),
                                               16, row * (int)a.ld_w * 2 + c * 16, kt * BK * 2, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < GC::IX; ++k) {
      const int blk = wave * GC::IX + k, row = blk * 16 + (lane >> 2), c = (lane & 3) ^ gemm_swz(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(xbuf(st) + blk * 1024),
                                               16, row * (int)a.ld_x * 2 + c * 16, kt * BK * 2, 0, 0);
    }
  };

  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto read_a = [&](int st, int i) {
    const int r = wch + 16 * i + i16;
    return *reinterpret_cast<const bf16x8*>(wbuf(st) + r * 64 + ((G ^ gemm_swz(r)) * 16));
  };
  auto read_b = [&](int st, int j) {
    const int r = wtok + 16 * j + i16;
    return *reinterpret_cast<const bf16x8*>(xbuf(st) + r * 64 + ((G ^ gemm_swz(r)) * 16));
  };

  // Pipeline over a ring of S stages. Step kt computes from fragments read during
  // step kt-1 (so stage kt%S is free) and meanwhile: the load unit fills stage
  // kt%S with step kt+S, and the wave reads step kt+1's fragments from stage
  // (kt+1)%S. At its end the step waits only for the copies of step kt+2 (the
  // later ones stay in flight: S-1 steps for a copy to land), then a barrier
  // makes them visible and retires every read of the stage refilled next.
  // Token fragment j of the next step goes into the register of token fragment
  // j once its MFMAs are issued; channel fragments alternate two sets.
  const int nk = a.hidden / BK;
  for (int st = 0; st < S && st < nk; ++st) issue(st, st);
  // wait for stages 0 and 1: the copies issued after them may stay in flight
  if (nk >= S) wait_vm_lgkm0<(S - 2) * IPS>();
  else wait_vm_lgkm0<0>();
  barrier_only();
  bf16x8 fa[2][TI], fb[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) fa[0][i] = read_a(0, i);
#pragma unroll
  for (int j = 0; j < TJ; ++j) fb[j] = read_b(0, j);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): stage 0 read out before anyone refills it
  barrier_only();
  // (the last step's reads of the next fragments read a stale stage and go
  // unused: cheaper than a branch per token column)
  auto step = [&](int kt, auto cur_tag) {
    constexpr int C = decltype(cur_tag)::value, N = C ^ 1;
    if (kt + S < nk) issue(kt + S, kt % S);
    const int sn = (kt + 1) % S;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
#pragma unroll
      for (int i = 0; i < TI; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[C][i], fb[j], acc[i][j], 0, 0, 0);
      fb[j] = read_b(sn, j);
      // the next channel fragments, spread over the token columns
#pragma unroll
      for (int i = j * TI / TJ; i < (j + 1) * TI / TJ; ++i) fa[N][i] = read_a(sn, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    // copies issued after step kt+2's (those of steps kt+3 .. kt+S) may stay in
    // flight; near the end, wait for all
    if (kt + S < nk) wait_vm_lgkm0<(S - 2) * IPS>();
    else wait_vm_lgkm0<0>();
    barrier_only();
  };
  using Z = std::integral_constant<int, 0>;
  using O = std::integral_constant<int, 1>;
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, Z{});
    if (kt + 1 < nk) step(kt + 1, O{});
  }

  // ---- epilogue: RoPE on query/key channels of video rows, one bf16 rounding.
  // The block's channels lie in one of query/key/value; the angles of a token's
  // two pairs are one 16-byte load, all of a token column issued at once.
  const int D = a.head_dim, P = D / 2;
  const bool rot_block = a.table && ch0 < 2 * a.hd;
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int tok = tok0 + wtok + 16 * j + i16;
    if (tok >= a.n_rows) continue;
    const bool rot = rot_block && tok < a.n_video;
    f32x4 cs[TI];
    if (rot) {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int p0 = ((ch0 + wch + 16 * i + 4 * G) % D) / 2;   // even: 16-byte aligned
        cs[i] = *reinterpret_cast<const f32x4*>(a.table + (int64_t)tok * P + p0);
      }
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int ch = ch0 + wch + 16 * i + 4 * G;     // channels ch .. ch+3
      if (ch >= a.n_ch) continue;
      f32x4 v = acc[i][j];
      if (rot) {
        const float u0 = v[0], w0 = v[1], u1 = v[2], w1 = v[3];
        v[0] = fmaf(u0, cs[i][0], -w0 * cs[i][1]);
        v[1] = fmaf(u0, cs[i][1], w0 * cs[i][0]);
        v[2] = fmaf(u1, cs[i][2], -w1 * cs[i][3]);
        v[3] = fmaf(u1, cs[i][3], w1 * cs[i][2]);
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
  if (!table || !aligned16(table)) return fail(NOMAS_E_INVALID, "%s: table must be non-NULL and 16-byte aligned", who);
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
  if (rope_table && !aligned16(rope_table)) return fail(NOMAS_E_INVALID, "%s: rope_table must be 16-byte aligned", who);
  if (head_dim != 64 && head_dim != 128) return fail(NOMAS_E_UNSUPPORTED, "%s: head_dim must be 64 or 128", who);
  if (n_heads < 1 || n_rows < 1 || hidden < 64 || hidden % 64)
    return fail(NOMAS_E_INVALID, "%s: need n_heads >= 1, n_rows >= 1, hidden a positive multiple of 64", who);
  if (n_video < 0 || n_video > n_rows) return fail(NOMAS_E_INVALID, "%s: need 0 <= n_video <= n_rows", who);
  const int64_t n_ch = 3LL * n_heads * head_dim;
  if (ld_x < hidden || ld_x % 8 || ld_w < hidden || ld_w % 8 || ld_qkv < n_ch || ld_qkv % 4)
    return fail(NOMAS_E_INVALID, "%s: ld_x, ld_w >= hidden (multiples of 8), ld_qkv >= 3*n_heads*head_dim (a multiple of 4)", who);
  if ((int64_t)GC::BM * ld_w * 2 > INT32_MAX || (int64_t)GC::BN * ld_x * 2 > INT32_MAX || n_ch > (1 << 20))
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
  a.tiles_m = (n_rows + GC::BN - 1) / GC::BN;
  a.tiles_n = (int)((n_ch + GC::BM - 1) / GC::BM);
  a.n_blocks = a.tiles_n * a.tiles_m;
  a.per_xcd = (a.n_blocks + 7) / 8;
  hipLaunchKernelGGL(qkv_gemm_kernel, dim3((unsigned)(8 * a.per_xcd)), dim3(GC::NT), 0, as_stream(stream), a);
  return check_launch(who);
}
