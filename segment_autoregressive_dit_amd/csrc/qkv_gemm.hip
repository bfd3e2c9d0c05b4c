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
//    dimension is walked in steps of 64: both 256 x 64 operand tiles are copied
//    global -> LDS by the load unit (buffer_load ... lds) into two stages, so
//    each copy fetches whole 128-byte lines of its rows; the 16-byte chunk
//    index is XOR-swizzled by (row/2) % 8. (Block, wave tile and ring depth are
//    the NOMAS_GEMM_CFG defaults below.)
//  * Software pipeline, one barrier per step: a step's first 32-deep half runs
//    its MFMAs on fragments already in registers while the second half's
//    fragments are read from the step's stage; after the barrier (every wave's
//    reads of that stage done, the next step's copies landed) the load unit
//    refills the stage with the step after next, and the second half's MFMAs
//    run while the next step's first-half fragments are read. Each copy has a
//    whole step to land.
//  * Blocks are laid out so each XCD works through whole channel tiles: the
//    W tile stays in that XCD's L2 while token tiles stream past it.
#include <type_traits>

#include "nomas_common.hpp"

namespace nomas {

// Block tile BM channels x BN tokens, wave tile WM x WN, ring of S stages.
#ifndef NOMAS_GEMM_CFG
#define NOMAS_GEMM_CFG 256, 256, 64, 128, 2, 1, 8
#endif
template <int BM_, int BN_, int WM_, int WN_, int S_, int MINB_, int GROUPN_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, S = S_, MINB = MINB_, GROUPN = GROUPN_;
  static constexpr int NW = (BM / WM) * (BN / WN);
  static constexpr int NT = NW * 64;
  static constexpr int BK = 64;                    // hidden elements per step
  static constexpr int TI = WM / 16, TJ = WN / 16; // accumulator tiles per wave
  static constexpr int WBYTES = BM * BK * 2, XBYTES = BN * BK * 2;
  static constexpr int IW = WBYTES / 1024 / NW, IX = XBYTES / 1024 / NW;   // copies per wave and stage
  static constexpr int IPS = IW + IX;
  static_assert(IW * NW * 1024 == WBYTES && IX * NW * 1024 == XBYTES, "tiles must split into 1 KB copies per wave");
  static_assert(S == 2, "two stages of 64-deep steps");
  static_assert(TJ % 2 == 0 || TI <= TJ, "fragment refill pattern");
};
using GC = GemmCfg<NOMAS_GEMM_CFG>;

// 128-byte rows of 8 chunks; the chunk index is XOR-ed with (row / 2) % 8, so
// the 16 rows a quarter-wave reads at one chunk fall on 16 distinct bank groups
// (rows 2m and 2m+1 in the two halves of a 256-byte bank row, m picking the
// chunk)
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
  int tiles_n;          // channel tiles
  int tiles_m;          // token tiles
  int n_blocks;
  int per_xcd;
  // the ring cache written by the final-step variant (video rows
  // [app_row0, n_video) go to the slots of frames frames_written + skip, ...)
  void* kc;
  void* vc;
  float* ks;
  float* vs;
  int pitch;
  int tpf;
  int cap;
  int base_slot;        // slot of the first written frame
  int app_row0;         // first video row written (rows of frames beyond the capacity are skipped)
  uint16_t* vt;         // V^T [H*D][ld_vt] of all rows, or null
  int64_t ld_vt;
};

// cache token row of video row r (app_row0 <= r < n_video)
__device__ __forceinline__ int gemm_slot_token(const GemmArgs& a, int r) {
  const int fi = (r - a.app_row0) / a.tpf;
  int slot = a.base_slot + fi;
  if (slot >= a.cap) slot -= a.cap;
  return slot * a.tpf + r % a.tpf;
}

enum { kAppNone = 0, kAppBf16 = 1, kAppInt8 = 2 };

// Workgroup barrier without the memory fence __syncthreads() carries (which
// waits for every outstanding load, the prefetched copies included); the
// compiler may not move memory accesses across it. Callers wait for exactly
// what must have landed first.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- value and cache epilogue. The wave's accumulators hold channels
// c0 + 16i + 4G .. +3 of tokens t0 + 16j + i16 (G = lane/16, i16 = lane%16),
// already the bf16 values the projection stored; its 64 channels lie in one
// head of the query, key or value part.
//  * VT: the value channels also go out transposed, V^T[h*D + d][token], for
//    attention's value operand (which then needs no transpose pass).
//  * APP (final step): the segment's keys and values into the ring cache as
//    the quantise-append would write them. INT8: a token's absmax over the head
//    (the lane's 16 channels, the wave's 4 channel lanes by two row swaps, for
//    head dim 128 the partner wave's through LDS), scale m/127, codes by the
//    shared code arithmetic. Keys go out as 4-channel pieces of their cache
//    rows.
// Transposed values are staged in LDS as [channel][token] and leave in runs of
// 16 tokens (cache: tokens per frame a multiple of 16, else element by
// element).
template <int APP, bool VT, int TI, int TJ, int WN>
__device__ __forceinline__ void kv_epilogue(const GemmArgs& a, f32x4 (&acc)[TI][TJ], unsigned char* lds, int c0,
                                            int t0, int wave, int lane) {
  constexpr bool I8 = APP == kAppInt8;
  constexpr int ES = I8 ? 1 : 2;                       // bytes per cached element
  constexpr int WM = 16 * TI;                          // the wave's channels (64)
  constexpr int CH = WN / 16;                          // 16-token runs per channel row
  static_assert(WM == 64, "a wave's channels are one head (D 64) or half of one (D 128, partner wave ^ 1)");
  static_assert(GC::NW * WM * WN * 2 <= GC::S * (GC::WBYTES + GC::XBYTES), "bf16 staging fits the operand ring");
  static_assert((GC::BM / WM) % 2 == 0, "partner waves (wave ^ 1) hold the two channel halves of a 128-wide head");
  const int G = lane >> 4, i16 = lane & 15;
  const int D = a.head_dim;
  const int part = c0 < a.n_ch ? c0 / a.hd : 3;        // 1: keys, 2: values
  const int hc = c0 - part * a.hd;                     // channel within the part
  const int h = hc / D, cin0 = hc % D;                 // head, first channel within the head
  __syncthreads();                                      // every wave is done with the ring

  // INT8 scales: per token j of the lane, s = absmax/127 and its reciprocal
  float sc[TJ], rc[TJ];
  if constexpr (I8) {
    float* red = reinterpret_cast<float*>(lds + GC::S * (GC::WBYTES + GC::XBYTES));   // [NW][WN]
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < TI; ++i) m = fmaxf(m, fmaxf(fmaxf(fabsf(acc[i][j][0]), fabsf(acc[i][j][1])),
                                                     fmaxf(fabsf(acc[i][j][2]), fabsf(acc[i][j][3]))));
      const unsigned u = __float_as_uint(m);
      const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      const float m2 = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
      const unsigned u2 = __float_as_uint(m2);
      const auto q = __builtin_amdgcn_permlane32_swap(u2, u2, false, false);
      sc[j] = fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
      if (G == 0) red[wave * WN + 16 * j + i16] = sc[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      // head dim 128: the head's other 64 channels are the partner wave's (wave ^ 1)
      if (D > WM) sc[j] = fmaxf(sc[j], red[(wave ^ 1) * WN + 16 * j + i16]);
      sc[j] = sc[j] / 127.0f;
      rc[j] = code_recip(sc[j]);
    }
  }
  unsigned char* st = lds + wave * WM * WN * 2;         // the wave's staging area

  // ---- V^T of every row of the call
  if (VT && part == 2) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          reinterpret_cast<uint16_t*>(st)[(16 * i + 4 * G + e) * WN + 16 * j + i16] =
              static_cast<uint16_t>(__float_as_uint(acc[i][j][e]) >> 16);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's staging stores have landed
    uint16_t* vt = a.vt + (int64_t)hc * a.ld_vt;
#pragma unroll
    for (int k = 0; k < WM * CH / 64; ++k) {
      const int cl = (k * 64 + lane) / CH, chunk = (k * 64 + lane) % CH;
      const int r = t0 + 16 * chunk;
      uint16_t* dst = vt + (int64_t)cl * a.ld_vt + r;
      const uint16_t* src = reinterpret_cast<const uint16_t*>(st) + cl * WN + 16 * chunk;
      if (!NOMAS_IN_BOUNDS(hc + cl < a.hd && r >= 0 && a.n_rows <= a.ld_vt)) continue;
      if (r + 16 <= a.n_rows) {
        reinterpret_cast<u32x4*>(dst)[0] = reinterpret_cast<const u32x4*>(src)[0];
        reinterpret_cast<u32x4*>(dst)[1] = reinterpret_cast<const u32x4*>(src)[1];
      } else {
        for (int e = 0; e < 16 && r + e < a.n_rows; ++e) dst[e] = src[e];
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // its reads are done before the area is staged again
  }
  if constexpr (APP == kAppNone) return;
  if (part != 1 && part != 2) return;
  void* cache = part == 1 ? a.kc : a.vc;

  // scales: by the head's first wave, lanes of channel group 0
  if constexpr (I8) {
    if (cin0 == 0 && G == 0) {
      float* sdst = (part == 1 ? a.ks : a.vs) + (int64_t)h * a.pitch;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int r = t0 + 16 * j + i16;
        if (r >= a.app_row0 && r < a.n_video) {
          const int st = gemm_slot_token(a, r);
          if (NOMAS_IN_BOUNDS(st >= 0 && st < a.cap * a.tpf)) sdst[st] = sc[j];
        }
      }
    }
  }

  // the cached form of element e of acc[i][j]: C + code (INT8) or the bf16 value
  auto cached = [&](int i, int j, float (&f)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = acc[i][j][e];
    if constexpr (I8) {
      bool ok = true;
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = code_fast(acc[i][j][e], rc[j], ok);
      if (!ok) {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = code_exact(acc[i][j][e], sc[j]);
      }
    }
  };

  if (part == 1) {
    // keys: 4 channels of one token per store
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int r = t0 + 16 * j + i16;
      if (r < a.app_row0 || r >= a.n_video) continue;
      const int stk = gemm_slot_token(a, r);
      if (!NOMAS_IN_BOUNDS(stk >= 0 && stk < a.cap * a.tpf && cin0 + WM <= D)) continue;
      unsigned char* row = static_cast<unsigned char*>(cache) + ((int64_t)h * a.pitch + stk) * D * ES;
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        float f[4];
        cached(i, j, f);
        const int cin = cin0 + 16 * i + 4 * G;
        if constexpr (I8) *reinterpret_cast<unsigned*>(row + cin) = pack4(f[0], f[1], f[2], f[3]);
        else *reinterpret_cast<uint2*>(row + 2 * cin) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
      }
    }
    return;
  }

  // values: staged [64 channels][WN tokens] in the wave's area
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      float f[4];
      cached(i, j, f);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int off = (16 * i + 4 * G + e) * WN + 16 * j + i16;
        if constexpr (I8) st[off] = static_cast<unsigned char>(__float_as_uint(f[e]) & 0xffu);
        else reinterpret_cast<uint16_t*>(st)[off] = static_cast<uint16_t>(__float_as_uint(f[e]) >> 16);
      }
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's staging stores have landed
  unsigned char* vt = static_cast<unsigned char*>(cache) + ((int64_t)h * D + cin0) * a.pitch * ES;
  if (a.tpf % 16 == 0) {
    // 8 lanes per channel row, 16 tokens (one run of slots) each
#pragma unroll
    for (int k = 0; k < WM * CH / 64; ++k) {
      const int cl = (k * 64 + lane) / CH, chunk = (k * 64 + lane) % CH;
      const int r = t0 + 16 * chunk;
      if (r < a.app_row0 || r >= a.n_video) continue;
      const int sv = gemm_slot_token(a, r);
      if (!NOMAS_IN_BOUNDS(sv >= 0 && sv + 16 <= a.cap * a.tpf)) continue;
      unsigned char* dst = vt + ((int64_t)cl * a.pitch + sv) * ES;
      const unsigned char* src = st + (cl * WN + 16 * chunk) * ES;
#pragma unroll
      for (int b = 0; b < ES; ++b)
        reinterpret_cast<u32x4*>(dst)[b] = reinterpret_cast<const u32x4*>(src)[b];
    }
  } else {
    for (int k = lane; k < WM * WN; k += 64) {
      const int cl = k / WN, tl = k % WN, r = t0 + tl;
      if (r < a.app_row0 || r >= a.n_video) continue;
      const int sv = gemm_slot_token(a, r);
      if (!NOMAS_IN_BOUNDS(sv >= 0 && sv < a.cap * a.tpf)) continue;
      unsigned char* dst = vt + ((int64_t)cl * a.pitch + sv) * ES;
      const unsigned char* src = st + (cl * WN + tl) * ES;
#pragma unroll
      for (int b = 0; b < ES; ++b) dst[b] = src[b];
    }
  }
}

// s_waitcnt with vmcnt(n), lgkmcnt(0) (expcnt left alone)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// APP: kAppNone (the projection alone), kAppBf16 / kAppInt8 (the final-step
// variant that also writes the segment's keys and values into the ring cache);
// VT: the values also go out transposed
template <int APP, bool VT>
__global__ __launch_bounds__(GC::NT, GC::MINB) void qkv_gemm_kernel(const GemmArgs a) {
  constexpr int BM = GC::BM, BN = GC::BN, WM = GC::WM, WN = GC::WN, S = GC::S, BK = GC::BK;
  constexpr int TI = GC::TI, TJ = GC::TJ, IPS = GC::IPS;
  // (the final-step variant reuses the ring for its value staging, then 4 KB of
  // per-wave maxima)
  __shared__ __align__(16) unsigned char lds[S * (GC::WBYTES + GC::XBYTES) + (APP == kAppInt8 ? GC::NW * WN * 4 : 0)];
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

  // each wave instruction fills 1 KB of LDS (8 rows of 128 B); the lane fetches
  // the global chunk that the swizzled layout puts at its position
  auto issue = [&](int kt, int st) {
#pragma unroll
    for (int k = 0; k < GC::IW; ++k) {
      const int blk = wave * GC::IW + k, row = blk * 8 + (lane >> 3), c = (lane & 7) ^ gemm_swz(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)(wbuf(st) + blk * 1024),
                                               16, row * (int)a.ld_w * 2 + c * 16, kt * BK * 2, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < GC::IX; ++k) {
      const int blk = wave * GC::IX + k, row = blk * 8 + (lane >> 3), c = (lane & 7) ^ gemm_swz(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(xbuf(st) + blk * 1024),
                                               16, row * (int)a.ld_x * 2 + c * 16, kt * BK * 2, 0, 0);
    }
  };

  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto read_a = [&](int st, int kk, int i) {
    const int r = wch + 16 * i + i16;
    return *reinterpret_cast<const bf16x8*>(wbuf(st) + r * 128 + (((4 * kk + G) ^ gemm_swz(r)) * 16));
  };
  auto read_b = [&](int st, int kk, int j) {
    const int r = wtok + 16 * j + i16;
    return *reinterpret_cast<const bf16x8*>(xbuf(st) + r * 128 + (((4 * kk + G) ^ gemm_swz(r)) * 16));
  };

  // Two stages of 64-deep steps. Step kt: the first half's MFMAs (fragments in
  // registers) while the second half's fragments are read from stage kt%2;
  // then every wave waits for the copies of step kt+1 and for its own reads,
  // a barrier, the copies of step kt+2 into stage kt%2 (now read out), and the
  // second half's MFMAs while step kt+1's first-half fragments are read from
  // stage (kt+1)%2. One barrier per step; each copy has a whole step to land.
  const int nk = a.hidden / BK;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  if (nk > 1) wait_vm_lgkm0<IPS>();
  else wait_vm_lgkm0<0>();
  barrier_only();
  bf16x8 fa[2][TI], fb[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) fa[0][i] = read_a(0, 0, i);
#pragma unroll
  for (int j = 0; j < TJ; ++j) fb[j] = read_b(0, 0, j);
  // (the last step's reads of the next fragments read a stale stage and go
  // unused: cheaper than a branch per token column)
  auto half = [&](int st_next, int kk_next, auto cur_tag) {
    constexpr int C = decltype(cur_tag)::value, N = C ^ 1;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
#pragma unroll
      for (int i = 0; i < TI; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[C][i], fb[j], acc[i][j], 0, 0, 0);
      fb[j] = read_b(st_next, kk_next, j);
#pragma unroll
      for (int i = j * TI / TJ; i < (j + 1) * TI / TJ; ++i) fa[N][i] = read_a(st_next, kk_next, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using Z = std::integral_constant<int, 0>;
  using O = std::integral_constant<int, 1>;
  for (int kt = 0; kt < nk; ++kt) {
    const int sc = kt & 1;
    half(sc, 1, Z{});
    wait_vm_lgkm0<0>();
    barrier_only();
    if (kt + 2 < nk) issue(kt + 2, sc);
    half(sc ^ 1, 0, O{});
  }

  // ---- epilogue: RoPE on query/key channels of video rows, one bf16 rounding.
  // A block may straddle the key/value boundary 2*H*D (head dim 64 with an odd
  // head count), so the rotation is decided per 4-channel group; a group never
  // straddles it (4-aligned groups, boundary a multiple of 128). The angles of a
  // token's two pairs are one 16-byte load, all of a token column issued at
  // once (also for value channels of such a block: the table index stays in
  // range, the values go unused).
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
      if (rot && ch < 2 * a.hd) {
        const float u0 = v[0], w0 = v[1], u1 = v[2], w1 = v[3];
        v[0] = fmaf(u0, cs[i][0], -w0 * cs[i][1]);
        v[1] = fmaf(u0, cs[i][1], w0 * cs[i][0]);
        v[2] = fmaf(u1, cs[i][2], -w1 * cs[i][3]);
        v[3] = fmaf(u1, cs[i][3], w1 * cs[i][2]);
      }
      const unsigned p01 = pack_bf16x2(v[0], v[1]), p23 = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(a.y + (int64_t)tok * a.ld_y + ch) = make_uint2(p01, p23);
      // the value and cache outputs take what the projection stored: the bf16 values
      if constexpr (APP != kAppNone || VT) acc[i][j] = (f32x4){bf16_lo(p01), bf16_hi(p01), bf16_lo(p23), bf16_hi(p23)};
    }
  }
  if constexpr (APP != kAppNone || VT) kv_epilogue<APP, VT, TI, TJ, WN>(a, acc, lds, ch0 + wch, tok0 + wtok, wave, lane);
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

namespace nomas {
int32_t validate_cache(const nomas_kvcache* c, const char* who);
int64_t check_failures_qkv(int reset) { return source_check_failures(reset); }

static int32_t qkv_projection_impl(const char* who, const uint16_t* x, int64_t ld_x, int32_t n_rows, int32_t hidden,
                                   const uint16_t* w, int64_t ld_w, int32_t n_heads, int32_t head_dim,
                                   int32_t n_video, const float* rope_table, uint16_t* qkv, int64_t ld_qkv,
                                   uint16_t* v_t, int64_t ld_vt, nomas_kvcache* c, void* stream) {
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
  if (v_t && (!aligned16(v_t) || ld_vt < n_rows || ld_vt % 8))
    return fail(NOMAS_E_INVALID, "%s: v_t must be 16-byte aligned with ld_vt >= n_rows and a multiple of 8", who);
  GemmArgs a{};
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
  a.vt = v_t;
  a.ld_vt = ld_vt;
  a.tiles_m = (n_rows + GC::BN - 1) / GC::BN;
  a.tiles_n = (int)((n_ch + GC::BM - 1) / GC::BM);
  a.n_blocks = a.tiles_n * a.tiles_m;
  a.per_xcd = (a.n_blocks + 7) / 8;
  int app = kAppNone;
  int n_frames = 0;
  if (c) {
    if (int32_t e = validate_cache(c, who)) return e;
    if (c->n_heads != n_heads || c->head_dim != head_dim)
      return fail(NOMAS_E_INVALID, "%s: the cache holds %d heads of %d, the projection %d of %d", who, c->n_heads,
                  c->head_dim, n_heads, head_dim);
    const int tpf = c->tokens_per_frame, cap = c->capacity_frames;
    if (n_video < tpf || n_video % tpf)
      return fail(NOMAS_E_INVALID, "%s: n_video %d must be a positive multiple of tokens_per_frame %d", who, n_video, tpf);
    n_frames = n_video / tpf;
    const int skip = n_frames > cap ? n_frames - cap : 0;   // frames overwritten within this append
    // the cached keys are the stored (rotated) ones; without a table nothing is rotated
    a.n_video = n_video;
    a.kc = c->k;
    a.vc = c->v;
    a.ks = c->k_scale;
    a.vs = c->v_scale;
    a.pitch = c->token_pitch;
    a.tpf = tpf;
    a.cap = cap;
    a.base_slot = (int)((c->frames_written + skip) % cap);
    a.app_row0 = skip * tpf;
    app = c->kv_dtype == NOMAS_KV_INT8 ? kAppInt8 : kAppBf16;
  }
  const dim3 grid((unsigned)(8 * a.per_xcd)), block(GC::NT);
  const hipStream_t st = as_stream(stream);
  const bool vt = v_t != nullptr;
  if (app == kAppInt8) {
    if (vt) hipLaunchKernelGGL((qkv_gemm_kernel<kAppInt8, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((qkv_gemm_kernel<kAppInt8, false>), grid, block, 0, st, a);
  } else if (app == kAppBf16) {
    if (vt) hipLaunchKernelGGL((qkv_gemm_kernel<kAppBf16, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((qkv_gemm_kernel<kAppBf16, false>), grid, block, 0, st, a);
  } else {
    if (vt) hipLaunchKernelGGL((qkv_gemm_kernel<kAppNone, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((qkv_gemm_kernel<kAppNone, false>), grid, block, 0, st, a);
  }
  if (int32_t e = check_launch(who)) return e;
  if (c) c->frames_written += n_frames;
  return ok();
}
}  // namespace nomas

extern "C" int32_t nomas_qkv_projection(const uint16_t* x, int64_t ld_x, int32_t n_rows, int32_t hidden,
                                        const uint16_t* w, int64_t ld_w, int32_t n_heads, int32_t head_dim,
                                        int32_t n_video, const float* rope_table, uint16_t* qkv, int64_t ld_qkv,
                                        void* stream) {
  return qkv_projection_impl("qkv_projection", x, ld_x, n_rows, hidden, w, ld_w, n_heads, head_dim, n_video,
                             rope_table, qkv, ld_qkv, nullptr, 0, nullptr, stream);
}

extern "C" int32_t nomas_qkv_projection_vt(const uint16_t* x, int64_t ld_x, int32_t n_rows, int32_t hidden,
                                           const uint16_t* w, int64_t ld_w, int32_t n_heads, int32_t head_dim,
                                           int32_t n_video, const float* rope_table, uint16_t* qkv, int64_t ld_qkv,
                                           uint16_t* v_t, int64_t ld_vt, void* stream) {
  if (!v_t) return fail(NOMAS_E_INVALID, "qkv_projection_vt: v_t is NULL");
  return qkv_projection_impl("qkv_projection_vt", x, ld_x, n_rows, hidden, w, ld_w, n_heads, head_dim, n_video,
                             rope_table, qkv, ld_qkv, v_t, ld_vt, nullptr, stream);
}

extern "C" int32_t nomas_qkv_projection_append(const uint16_t* x, int64_t ld_x, int32_t n_rows, int32_t hidden,
                                               const uint16_t* w, int64_t ld_w, int32_t n_heads, int32_t head_dim,
                                               int32_t n_video, const float* rope_table, uint16_t* qkv,
                                               int64_t ld_qkv, uint16_t* v_t, int64_t ld_vt, nomas_kvcache* c,
                                               void* stream) {
  if (!c) return fail(NOMAS_E_INVALID, "qkv_projection_append: cache descriptor is NULL");
  return qkv_projection_impl("qkv_projection_append", x, ld_x, n_rows, hidden, w, ld_w, n_heads, head_dim, n_video,
                             rope_table, qkv, ld_qkv, v_t, ld_vt, c, stream);
}
