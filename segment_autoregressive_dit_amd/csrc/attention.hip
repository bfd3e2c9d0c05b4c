// Block-causal segment attention: the current segment's queries against the
// retained cache frames plus the whole current segment.
//
// Pages: "segment-wise causal joint attention" (madebyagents.com model page
// "Hy-Nomas", component "Segment-Autoregressive DiT"); the history enters as a
// KV cache that is the attention context (orcarouter.ai, section "Die Schleife");
// INT8 cache entries are computed in BF16 ("Hy-Nomas auf einer RTX 4090",
// inferencekey.com, section "Das Single-GPU-Preset").
//
// Kernel design (gfx950, wave64, v_mfma_f32_16x16x32_bf16):
//  * One block = NW waves = NW*QB*16 queries of one head and one key split.
//    Each wave owns QB blocks of 16 queries; their Q fragments stay in VGPRs.
//  * Logits are formed transposed, S^T = K Q^T, so a lane holds one query
//    (lane % 16) and 4 keys per MFMA: a row max needs only two cross-lane steps
//    (lanes 16 and 32 apart), and the row sums come from an MFMA against an
//    all-ones operand.
//  * The 32 keys of a group are fed to the two S^T MFMAs in a permuted row
//    order so that lane group G ends up holding keys 8G..8G+7 in register
//    order; that is exactly the B operand (P^T) layout of the value MFMA
//    O^T += V^T P^T, so P never goes through LDS.
//  * V^T operand rows are contiguous key runs: the cache stores V transposed and
//    the current segment's V is transposed once into the workspace.
//  * K and V^T tiles of BC keys are staged in LDS, with the 16-byte chunk index
//    XOR-swizzled by the row so that the strided 128-bit operand reads are
//    bank-conflict free: three K and two V^T stages (all 160 KB) for bf16
//    tiles, two K and three V^T stages for INT8. bf16 tiles are copied global -> LDS by the load unit
//    (buffer_load ... lds).
//  * Head dim 128 runs a ping-pong schedule: the block's 8 waves form two
//    groups, one wave of each on every SIMD, one barrier apart, so that on every
//    SIMD one wave issues MFMAs (values of tile t-1, logits of tile t, at issue
//    priority 1) while the other runs the softmax of its tile. With three K
//    stages the copies are all issued from the softmax phases (group A: K two
//    tiles ahead, group B: V^T one tile ahead). Head dim 64 runs two 4-wave
//    blocks per CU, tile by tile.
//  * Online softmax in the log2 domain with a fixed reference max per query that
//    is only raised when a tile's max exceeds it by more than kTau (probabilities
//    stay <= 2^kTau, exact in fp32 and bf16 range), so the O rescale is rare.
//  * INT8 cache tiles stage their codes through registers: key codes are
//    converted to bf16 exactly and the key scale multiplies the fp32 logit of
//    its key (folded into the softmax's exponent coefficient); values are
//    dequantised (code * scale, rounded once to bf16) on the way into LDS. The
//    scales themselves go global -> LDS by the load unit.
//  * Split-KV: the key tiles are cut into contiguous chunks; each block writes a
//    normalised fp32 partial and its log-sum-exp, merged in fixed order.
//  * Block ids are remapped so the blocks that the hardware places on one XCD
//    share (head, split): they stream the same K/V through that XCD's L2.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "nomas_common.hpp"

namespace nomas {

int32_t validate_cache(const nomas_kvcache* c, const char* who);

constexpr float kTau = 8.0f;

// wave -> ping-pong group; waves of a block are dealt to the 4 SIMDs round-robin,
// so with 8 waves, waves w and w+4 share a SIMD and go to different groups
#ifndef PP_GROUP
#define PP_GROUP(w) ((w) >> 2)
#endif
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kcur;
  int64_t ld_qkv;
  const uint16_t* vtcur;   // [H][D][pitch_cur] bf16, zero beyond n_cur
  int pitch_cur;
  const void* kc;
  const void* vc;
  const float* ks;
  const float* vs;
  int pitch_c;
  int n_cached;            // cache keys attended: c_na + c_nb
  int c_a0;                // in physical cache tokens: [c_a0, c_a0 + c_na), then [0, c_nb)
  int c_na;                // (a frame range that wraps round the ring is two runs)
  int c_nb;
  int n_cur;
  int n_q;
  int H;
  float c2;                // softmax_scale * log2(e)
  uint16_t* out;
  int64_t ld_out;
  float* lse;
  float* part_o;           // [S][H][n_q][D] or null
  float* part_lse;         // [S][H][n_q]
  int n_splits;
  int tiles_c;
  int tiles_total;
  int n_qtiles;
  int n_blocks;
  int per_xcd;
  const int32_t* blist;    // sparse: [H][nqb_sp][n_sel] candidate blocks of 128 cache rows
  int n_sel;
  int nqb_sp;
};

constexpr int kSpKeyBlock = NOMAS_SPARSE_KEY_BLOCK;
constexpr int kSpQueryBlock = NOMAS_SPARSE_QUERY_BLOCK;
enum { kModeCached = 0, kModeSegments = 1, kModeSparse = 2 };

// Segments of a multi-segment call (the joint sequence [video_0; text_0;
// video_1; ...]): segment s owns rows [row0[s], row0[s+1]), its first nv[s] rows
// being video of frames t0[s], t0[s]+1, ... (tpf rows each); its query tiles are
// the global tiles [qtile0[s], qtile0[s+1]). window < 0: no window.
constexpr int kMaxSegments = 64;
struct SegTable {
  int n_seg;
  int tpf;
  int window;
  int row0[kMaxSegments + 1];
  int nv[kMaxSegments];
  int t0[kMaxSegments];
  int qtile0[kMaxSegments + 1];
};

template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? ((row & 3) | (((row >> 3) & 3) << 2)) : ((row & 3) | (((row >> 3) & 1) << 2));
}
template <int BC>
__device__ __forceinline__ int swz_v(int d) {
  return BC == 128 ? (d & 15) : ((d >> 1) & 7);
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
// with the gfx950 row-swap permutes; every lane ends with the same value.
__device__ __forceinline__ float xmax16(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xadd16(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xadd32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 int8 codes -> 16 bf16 (exact: |code| <= 127 < 2^8)
__device__ __forceinline__ void i8x16_to_bf16(const u32x4 w, u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int x = static_cast<int>(w[e]);
    const float f0 = static_cast<float>((x << 24) >> 24);
    const float f1 = static_cast<float>((x << 16) >> 24);
    const float f2 = static_cast<float>((x << 8) >> 24);
    const float f3 = static_cast<float>(x >> 24);
    if (e < 2) {
      lo[2 * e] = pack_bf16x2(f0, f1);
      lo[2 * e + 1] = pack_bf16x2(f2, f3);
    } else {
      hi[2 * (e - 2)] = pack_bf16x2(f0, f1);
      hi[2 * (e - 2) + 1] = pack_bf16x2(f2, f3);
    }
  }
}

// 16 int8 codes of 16 consecutive keys -> bf16(code_k * scale_k), one rounding
__device__ __forceinline__ void i8x16_dequant_bf16(const u32x4 w, const f32x4 (&sc)[4], u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int x = static_cast<int>(w[e]);
    const float f0 = static_cast<float>((x << 24) >> 24) * sc[e][0];
    const float f1 = static_cast<float>((x << 16) >> 24) * sc[e][1];
    const float f2 = static_cast<float>((x << 8) >> 24) * sc[e][2];
    const float f3 = static_cast<float>(x >> 24) * sc[e][3];
    if (e < 2) {
      lo[2 * e] = pack_bf16x2(f0, f1);
      lo[2 * e + 1] = pack_bf16x2(f2, f3);
    } else {
      hi[2 * (e - 2)] = pack_bf16x2(f0, f1);
      hi[2 * (e - 2) + 1] = pack_bf16x2(f2, f3);
    }
  }
}

template <int D, int QB, int NW, int BC, bool I8, bool PIPE, bool VPF>
struct AttnCfg {
  static constexpr int NT = NW * 64;
  static constexpr int KC = D / 8;                 // 16-byte chunks per K row (bf16)
  static constexpr int VC = BC / 8;                // 16-byte chunks per V^T row (bf16)
  static constexpr int KT_BYTES = BC * D * 2;
  static constexpr int VT_BYTES = D * BC * 2;
  static constexpr int KSTAGE = KT_BYTES + (I8 ? BC * 4 : 0); // K tile (+ INT8: its per-key K scales)
  static constexpr int VSTAGE = VT_BYTES;          // V^T tile
  static constexpr int NVS = PIPE && VPF ? 3 : 2;  // V^T stages
  static constexpr int NKS = PIPE && !VPF ? 3 : 2; // K stages
  // INT8: each wave's own copy of a tile's value scales
  static constexpr int VSC_OFF = NKS * KSTAGE + NVS * VSTAGE;
  static constexpr int VSC_BYTES = I8 ? NW * BC * 4 : 0;
  static constexpr int LDS_BYTES = VSC_OFF + VSC_BYTES;
  static constexpr int NK8 = BC * D / 16 / NT;     // int8 K chunks (16 codes) per thread
  static constexpr int NV8 = D * BC / 16 / NT;     // int8 V chunks per thread
  static constexpr int BR = NW * QB * 16;          // queries per block
  static constexpr int NKB = BC / 16;              // 16-key blocks of a tile
  static constexpr int KK = D / 32;                // d-steps of the logit MFMA
  static constexpr int KI = KT_BYTES / 1024 / NW;  // 1 KB LDS-copy instructions per wave (K)
  static constexpr int VI = VT_BYTES / 1024 / NW;  // (V^T)
  static_assert(KT_BYTES % (1024 * NW) == 0 && VT_BYTES % (1024 * NW) == 0, "tile must split into 1 KB copies");
  static_assert((BC * D / 16) % NT == 0 && NK8 >= 1 && NV8 >= 1, "int8 tile must split evenly over threads");
  static_assert(BC % 64 == 0, "scales are copied 64 keys per instruction");
  static_assert(NT % (BC / 16) == 0, "a lane's int8 value chunks share their keys");
};

// MODE: kModeCached (a segment against the cache), kModeSegments (multi-segment
// call: no cache, keys are rows of the joint sequence, see SegTable) or
// kModeSparse (against the cache blocks of a per-query-block list).
template <int D, int QB, int NW, int BC, bool I8, bool PIPE, bool VPF, int MODE>
__global__ __launch_bounds__(NW * 64, PIPE ? 1 : 2) void attn_kernel(const AttnArgs a, const SegTable st) {
  using C = AttnCfg<D, QB, NW, BC, I8, PIPE, VPF>;
  constexpr bool MS = MODE == kModeSegments, SP = MODE == kModeSparse;
  static_assert(kSpKeyBlock % BC == 0 && kSpQueryBlock % C::BR == 0, "sparse blocks must be whole tiles");
  constexpr int NKB = C::NKB, KK = C::KK;
  constexpr int ES = I8 ? 1 : 2;   // bytes per cached element
  // C::NKS K buffers, then C::NVS V^T buffers
  static_assert(C::LDS_BYTES <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) unsigned char lds[C::LDS_BYTES];
  auto kbuf = [&](int i) { return lds + i * C::KSTAGE; };
  auto vbuf = [&](int i) { return lds + C::NKS * C::KSTAGE + i * C::VSTAGE; };

  const int b = blockIdx.x;
  const int logical = (b & 7) * a.per_xcd + (b >> 3);
  if (logical >= a.n_blocks) return;
  // block -> (query tile, split, head); results pinned to scalar registers
  const int qt = __builtin_amdgcn_readfirstlane(logical % a.n_qtiles);
  const int hs = __builtin_amdgcn_readfirstlane(logical / a.n_qtiles);
  const int split = __builtin_amdgcn_readfirstlane(hs % a.n_splits);
  const int h = __builtin_amdgcn_readfirstlane(hs / a.n_splits);

  // cache tiles of this block: the full tiles of the run [c_a0, c_a0 + c_na),
  // those of [0, c_nb), then the partial tail of each run; or (sparse) the tiles
  // of its list, whose last block may be shorter than 128 rows
  const int full_a = a.c_na / BC;
  int full_c_b = full_a + a.c_nb / BC;
  int tiles_c_b = full_c_b + (a.c_na % BC != 0) + (a.c_nb % BC != 0);
  int tiles_total_b = tiles_c_b + (a.n_cur + BC - 1) / BC;
  const int32_t* blist = nullptr;
  constexpr int TPB = kSpKeyBlock / BC;     // tiles per candidate block
  if constexpr (SP) {
    blist = a.blist + ((int64_t)h * a.nqb_sp + qt * C::BR / kSpQueryBlock) * a.n_sel;
    tiles_c_b = full_c_b = 0;
    if (a.n_sel > 0) {
      const int last = __builtin_amdgcn_readfirstlane(blist[a.n_sel - 1]);
      const int rem = max(0, min(kSpKeyBlock, a.n_cached - last * kSpKeyBlock));
      tiles_c_b = (a.n_sel - 1) * TPB + (rem + BC - 1) / BC;
      full_c_b = (a.n_sel - 1) * TPB + rem / BC;
    }
    tiles_total_b = tiles_c_b + (a.n_cur + BC - 1) / BC;
  }
  const int t_begin = __builtin_amdgcn_readfirstlane((int)((int64_t)split * tiles_total_b / a.n_splits));
  const int t_end = __builtin_amdgcn_readfirstlane((int)((int64_t)(split + 1) * tiles_total_b / a.n_splits));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4, i16 = lane & 15;

  // the block's query rows [q_row0, q_row0 + BR) clipped to q_end; MS: the
  // segment the query tile belongs to
  int seg = 0, q_row0 = qt * C::BR, q_end = a.n_q;
  if constexpr (MS) {
    while (seg + 1 < st.n_seg && st.qtile0[seg + 1] <= qt) ++seg;
    q_row0 = st.row0[seg] + (qt - st.qtile0[seg]) * C::BR;
    q_end = st.row0[seg + 1];
  }

  // ---- Q fragments (B operand of S^T = K Q^T): lane -> query i16, dims 32kk+8G..+8
  bf16x8 qf[QB][KK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = q_row0 + (wave * QB + qb) * 16 + i16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 v = {0, 0, 0, 0};
      if (row < q_end) v = *reinterpret_cast<const u32x4*>(a.q + (int64_t)row * a.ld_qkv + (int64_t)h * D + 32 * kk + 8 * G);
      qf[qb][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // O accumulators; row sums of the bf16 probabilities, accumulated by an MFMA
  // with an all-ones operand, so every lane holds its query's full sum
  f32x4 o[QB][D / 16];
  f32x4 lacc[QB];
  float m_ref[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = 0.f;
    lacc[qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[qb][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // ---- buffer descriptors. The range check covers a load's per-lane offset,
  // not its scalar (tile) offset, so what keeps every read in bounds is the
  // tile walk: cache tiles read rows inside the head's token_pitch rows, full
  // current tiles lie inside the segment, and its partial tail gets a
  // descriptor of its own (start_k_tail). Rows of a partial tile outside its
  // valid rows may hold anything and are masked (logits) and zeroed (values).
  const int c_end = a.c_a0 + a.c_na;   // one past the last physical cache row attended
  const __amdgpu_buffer_rsrc_t rk_c = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<char*>(const_cast<void*>(a.kc)) + (int64_t)h * a.pitch_c * D * ES, (short)0, c_end * D * ES, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv_c = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<char*>(const_cast<void*>(a.vc)) + (int64_t)h * D * a.pitch_c * ES, (short)0, D * a.pitch_c * ES, 0x00020000);
  const __amdgpu_buffer_rsrc_t rk_n = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.kcur) + (int64_t)h * D, (short)0, (int)(a.n_cur * a.ld_qkv * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv_n = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.vtcur) + (int64_t)h * D * a.pitch_cur, (short)0, D * a.pitch_cur * 2, 0x00020000);

  // per-key scales of the attended cache tokens
  const __amdgpu_buffer_rsrc_t rks_c = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.ks) + (int64_t)h * a.pitch_c, (short)0, I8 ? c_end * 4 : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t rvs_c = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.vs) + (int64_t)h * a.pitch_c, (short)0, I8 ? c_end * 4 : 0, 0x00020000);

  // bf16 tiles are copied global -> LDS by the load unit straight into their
  // swizzled places. INT8 cache tiles: the codes are staged through registers
  // (16 per lane per piece) and expanded into place by the lane that loaded
  // them; the key scales are copied by the load unit straight to the stage,
  // and each wave copies the value scales it needs to its own LDS slot.
  u32x4 stk[I8 ? C::NK8 : 1], stv[I8 ? C::NV8 : 1];
  // (LDS copy targets are formed from scalar values where they are used, so
  // that the copy's base address is known to be uniform)
  auto vsc = [&]() { return lds + C::VSC_OFF + wave * BC * 4; };

  // MS: the key range [kbase, kend) of the joint sequence being visited
  int kbase = 0, kend = 0;
  // Every run of tiles is of one kind, known at compile time: cache tiles
  // (cache_tag true) or tiles of the current segment / joint sequence.
  // tile t -> (first key inside its part, valid keys); the valid keys are the
  // tile's rows [klo, klo + nvalid) (klo > 0 only for a partial cache tile
  // moved back to keep its rows inside the head's token_pitch rows)
  auto tile_rows = [&](int t, auto cache_tag, int& key0, int& nvalid, int& klo) {
    constexpr bool CACHE = decltype(cache_tag)::value;
    klo = 0;
    // (the list entry is the same for the whole block: keep it scalar)
    if constexpr (MS) {
      key0 = kbase + t * BC;
      nvalid = min(BC, kend - key0);
    } else if constexpr (SP && CACHE) {
      key0 = __builtin_amdgcn_readfirstlane(blist[t / TPB]) * kSpKeyBlock + (t % TPB) * BC;
      nvalid = min(BC, a.n_cached - key0);
    } else if constexpr (CACHE) {
      // full tiles of the first run, of the second, then the partial tails
      int k0, n;
      if (t < full_a) k0 = a.c_a0 + t * BC, n = BC;
      else if (t < full_c_b) k0 = (t - full_a) * BC, n = BC;
      else if (t == full_c_b && a.c_na % BC) k0 = a.c_a0 + full_a * BC, n = a.c_na % BC;
      else k0 = a.c_nb / BC * BC, n = a.c_nb % BC;
      // a tile reads rows [k0, k0 + BC); the first run's tail can end near the
      // head's last row, so the read is moved back to end at token_pitch (a
      // multiple of 128, >= BC) and its leading rows are masked too
      if (k0 + BC > a.pitch_c) klo = k0 - (a.pitch_c - BC), k0 = a.pitch_c - BC;
      key0 = __builtin_amdgcn_readfirstlane(k0);
      nvalid = __builtin_amdgcn_readfirstlane(n);
      klo = __builtin_amdgcn_readfirstlane(klo);
    } else {
      key0 = __builtin_amdgcn_readfirstlane((t - tiles_c_b) * BC);
      nvalid = min(BC, a.n_cur - key0);
    }
#ifdef NOMAS_DEVICE_CHECKS
    // checking build: a tile that would read outside its buffer reads rows
    // [0, BC) instead, all masked
    const bool fits = CACHE ? key0 >= 0 && key0 + BC <= a.pitch_c && klo >= 0 && klo + nvalid <= BC
                            : key0 >= 0 && key0 + nvalid <= a.n_cur && key0 + BC <= a.pitch_cur;
    if (!NOMAS_IN_BOUNDS(fits)) key0 = 0, nvalid = 0, klo = 0;
#endif
  };
  auto tile_info = [&](int t, auto cache_tag, int& key0, int& nvalid) {
    int klo;
    tile_rows(t, cache_tag, key0, nvalid, klo);
  };

  // ---- issue the loads of tile t's keys / values into K / V buffer i
  auto start_k = [&](int t, int i, auto ct) {
    constexpr bool cache = decltype(ct)::value;
    int key0, nvalid;
    tile_info(t, ct, key0, nvalid);
    if constexpr (I8 && cache) {
      unsigned char* Ks = kbuf(i);
#pragma unroll
      for (int j = 0; j < C::NK8; ++j) {
        const int c = (j * NW + wave) * 64 + lane, row = c / (D / 16), cc = c % (D / 16);
        stk[j] = __builtin_amdgcn_raw_buffer_load_b128(rk_c, row * D + cc * 16, key0 * D, 0);
      }
      if (wave == 0)
#pragma unroll
        for (int j = 0; j < BC / 64; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rks_c, (__attribute__((address_space(3))) void*)(Ks + C::KT_BYTES + j * 256),
                                                   4, (j * 64 + lane) * 4, key0 * 4, 0, 0);
    } else {
      // each wave instruction fills 1 KB of LDS, lane l at byte 16*l; the lane
      // fetches the global chunk that the swizzled layout puts there
      const __amdgpu_buffer_rsrc_t rk = cache ? rk_c : rk_n;
      const int kstride = cache ? D * 2 : (int)a.ld_qkv * 2;
      unsigned char* Ks = kbuf(i);
#pragma unroll
      for (int k = 0; k < C::KI; ++k) {
        const int blk = wave * C::KI + k, p = blk * 64 + lane;
        const int row = p / C::KC, c = (p % C::KC) ^ swz_k<D>(row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(Ks + blk * 1024), 16,
                                                 row * kstride + c * 16, key0 * kstride, 0, 0);
      }
    }
  };
  // the last, partial key tile of the current segment (or of a range of the
  // joint sequence): its rows past the end must not be fetched at all, and the
  // scalar offset of a buffer load lies outside the range check, so the tile
  // gets a descriptor based at its first row and bounded by its valid rows
  auto start_k_tail = [&](int t) {
    int key0, nvalid;
    tile_info(t, std::false_type{}, key0, nvalid);
    key0 = __builtin_amdgcn_readfirstlane(key0);
    nvalid = __builtin_amdgcn_readfirstlane(nvalid);
    const uint64_t base = reinterpret_cast<uint64_t>(a.kcur + (int64_t)key0 * a.ld_qkv + (int64_t)h * D);
    const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(base & 0xffffffffu)));
    const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(base >> 32)));
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(lo | (hi << 32)), (short)0, (int)(nvalid * a.ld_qkv * 2), 0x00020000);
    const int kstride = (int)a.ld_qkv * 2;
    unsigned char* Ks = kbuf(0);
#pragma unroll
    for (int k = 0; k < C::KI; ++k) {
      const int blk = wave * C::KI + k, p = blk * 64 + lane;
      const int row = p / C::KC, c = (p % C::KC) ^ swz_k<D>(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(Ks + blk * 1024), 16,
                                               row * kstride + c * 16, 0, 0, 0);
    }
  };
  auto start_v = [&](int t, int i, auto ct) {
    constexpr bool cache = decltype(ct)::value;
    int key0, nvalid;
    tile_info(t, ct, key0, nvalid);
    if constexpr (I8 && cache) {
#pragma unroll
      for (int j = 0; j < C::NV8; ++j) {
        const int c = (j * NW + wave) * 64 + lane, d = c / (BC / 16), cc = c % (BC / 16);
        stv[j] = __builtin_amdgcn_raw_buffer_load_b128(rv_c, d * a.pitch_c + cc * 16, key0, 0);
      }
#pragma unroll
      for (int j = 0; j < BC / 64; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rvs_c, (__attribute__((address_space(3))) void*)(vsc() + j * 256), 4,
                                                 (j * 64 + lane) * 4, key0 * 4, 0, 0);
    } else {
      const __amdgpu_buffer_rsrc_t rv = cache ? rv_c : rv_n;
      const int vstride = (cache ? a.pitch_c : a.pitch_cur) * 2;
      unsigned char* Vs = vbuf(i);
#pragma unroll
      for (int k = 0; k < C::VI; ++k) {
        const int blk = wave * C::VI + k, p = blk * 64 + lane;
        const int d = p / C::VC, c = (p % C::VC) ^ swz_v<BC>(d);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(Vs + blk * 1024), 16,
                                                 d * vstride + c * 16, key0 * 2, 0, 0);
      }
    }
  };

  // bf16 tiles copied by the four waves of one group (1 KB blocks gw*KG .. +KG)
  auto copy_k4 = [&](int t, int i, auto ct) {
    constexpr bool cache = decltype(ct)::value;
    constexpr int KG = C::KT_BYTES / 1024 / 4;
    int key0, nvalid;
    tile_info(t, ct, key0, nvalid);
    const __amdgpu_buffer_rsrc_t rk = cache ? rk_c : rk_n;
    const int kstride = cache ? D * 2 : (int)a.ld_qkv * 2;
    unsigned char* Ks = kbuf(i);
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const int blk = (wave & 3) * KG + k, p = blk * 64 + lane;
      const int row = p / C::KC, c = (p % C::KC) ^ swz_k<D>(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(Ks + blk * 1024), 16,
                                               row * kstride + c * 16, key0 * kstride, 0, 0);
    }
  };
  auto copy_v4 = [&](int t, int i, auto ct) {
    constexpr bool cache = decltype(ct)::value;
    constexpr int VG = C::VT_BYTES / 1024 / 4;
    int key0, nvalid;
    tile_info(t, ct, key0, nvalid);
    const __amdgpu_buffer_rsrc_t rv = cache ? rv_c : rv_n;
    const int vstride = (cache ? a.pitch_c : a.pitch_cur) * 2;
    unsigned char* Vs = vbuf(i);
#pragma unroll
    for (int k = 0; k < VG; ++k) {
      const int blk = (wave & 3) * VG + k, p = blk * 64 + lane;
      const int d = p / C::VC, c = (p % C::VC) ^ swz_v<BC>(d);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(Vs + blk * 1024), 16,
                                               d * vstride + c * 16, key0 * 2, 0, 0);
    }
  };

  // ---- complete the staging of tile t's keys / values (INT8: convert + store),
  // after wait_copies(): this wave's own loads and copies have landed
  auto finish_k = [&](int t, int i, auto ct) {
    constexpr bool cache = decltype(ct)::value;
    int key0, nvalid;
    tile_info(t, ct, key0, nvalid);
    if constexpr (I8 && cache) {
      unsigned char* Ks = kbuf(i);
#pragma unroll
      for (int j = 0; j < C::NK8; ++j) {
        const int c = (j * NW + wave) * 64 + lane, row = c / (D / 16), cc = c % (D / 16);
        u32x4 lo, hi;
        i8x16_to_bf16(stk[j], lo, hi);
        const int s = swz_k<D>(row);
        *reinterpret_cast<u32x4*>(Ks + row * D * 2 + (((2 * cc) ^ s) * 16)) = lo;
        *reinterpret_cast<u32x4*>(Ks + row * D * 2 + (((2 * cc + 1) ^ s) * 16)) = hi;
        __builtin_amdgcn_sched_barrier(0);   // one piece at a time: few live registers
      }
      // the key scales wave 0 copied (its copies have landed) become the
      // exponent coefficients scale * c2, once per tile for the whole block
      if (wave == 0) {
        float* ksc = reinterpret_cast<float*>(Ks + C::KT_BYTES);
#pragma unroll
        for (int j = 0; j < BC / 64; ++j) ksc[j * 64 + lane] *= a.c2;
      }
    }
  };
  // INT8: the value scales of the lane's 16 keys (keys 16*cc .. 16*cc+15)
  auto read_vsc = [&](f32x4 (&sc)[4]) {
    const int cc = lane % (BC / 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[e] = *reinterpret_cast<const f32x4*>(vsc() + (cc * 16 + 4 * e) * 4);
  };
  auto finish_v_sc = [&](int t, int i, auto ct, const f32x4 (&sc)[4]) {
    constexpr bool cache = decltype(ct)::value;
    if constexpr (I8 && cache) {
      unsigned char* Vs = vbuf(i);
      // a lane's chunks all cover keys 16*cc .. 16*cc+15
      const int cc = lane % (BC / 16);
#pragma unroll
      for (int j = 0; j < C::NV8; ++j) {
        const int d = ((j * NW + wave) * 64 + lane) / (BC / 16);
        u32x4 lo, hi;
        i8x16_dequant_bf16(stv[j], sc, lo, hi);
        const int s = swz_v<BC>(d);
        *reinterpret_cast<u32x4*>(Vs + d * BC * 2 + (((2 * cc) ^ s) * 16)) = lo;
        *reinterpret_cast<u32x4*>(Vs + d * BC * 2 + (((2 * cc + 1) ^ s) * 16)) = hi;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto finish_v = [&](int t, int i, auto ct) {
    f32x4 sc[4];
    if constexpr (I8 && decltype(ct)::value) read_vsc(sc);
    finish_v_sc(t, i, ct, sc);
  };
  auto wait_copies = [&]() { __builtin_amdgcn_s_waitcnt(0); };

  // zero the values of the keys of a partial tile outside its rows [klo, khi)
  // (all waves' data landed)
  auto zero_tail = [&](int i, int klo, int khi) {
    unsigned char* Vs = vbuf(i);
    for (int idx = tid; idx < D * BC; idx += C::NT) {
      const int d = idx / BC, k = idx % BC;
      if (k < klo || k >= khi)
        *reinterpret_cast<uint16_t*>(Vs + d * BC * 2 + (((k >> 3) ^ swz_v<BC>(d)) * 16) + (k & 7) * 2) = 0;
    }
  };

  const int krow0 = 8 * (i16 >> 2) + (i16 & 3);   // K row of key block 0 for this lane
  const int ksw = swz_k<D>(krow0);                 // the same for every key block

  // S^T = K Q^T from K buffer i into s, in steps of KH key blocks x one 32-wide
  // d-slice (QB*KH independent accumulators per step); each step's K fragments
  // are requested before the previous step's MFMAs, so the LDS latency hides
  // behind them (the scheduling barriers keep that order). INT8 keys: the key
  // scales are folded into the softmax's exponent coefficient, kcs = k_scale *
  // c2 per key, so the exponent is s * kcs - m_ref (one fma per logit, as for
  // bf16 keys).
  constexpr int KH = NKB > 4 ? 4 : NKB;
  constexpr int NSTEP = NKB / KH * KK;
  auto read_kstep = [&](int i, int st, bf16x8 (&dst)[KH]) {
    const unsigned char* Ks = kbuf(i);
    const int h = st / KK, kk = st % KK;
#pragma unroll
    for (int j = 0; j < KH; ++j) {
      const int kb = h * KH + j;
      const int row = krow0 + 32 * (kb >> 1) + 4 * (kb & 1);
      dst[j] = *reinterpret_cast<const bf16x8*>(Ks + row * D * 2 + (((4 * kk + G) ^ ksw) * 16));
    }
  };
  auto read_k0 = [&](int i, bf16x8 (&dst)[KH]) { read_kstep(i, 0, dst); };
  // k0: the first step's fragments, already requested by the caller
  f32x4 kcs[NKB];   // INT8 cache tiles: per-key exponent coefficients k_scale * c2
  auto logits_from = [&](int i, const bf16x8 (&k0)[KH], f32x4 (&s)[QB][NKB], auto scaled_tag) {
    constexpr bool SCALED = decltype(scaled_tag)::value;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    bf16x8 kf[2][KH];
#pragma unroll
    for (int j = 0; j < KH; ++j) kf[0][j] = k0[j];
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      if (st + 1 < NSTEP) read_kstep(i, st + 1, kf[(st + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const int h = st / KK, kk = st % KK;
#pragma unroll
      for (int j = 0; j < KH; ++j)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][h * KH + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[st & 1][j], qf[qb][kk], s[qb][h * KH + j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SCALED) {
      const float* sc = reinterpret_cast<const float*>(kbuf(i) + C::KT_BYTES);   // scale * c2 per key
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) kcs[kb] = *reinterpret_cast<const f32x4*>(sc + 32 * (kb >> 1) + 8 * G + 4 * (kb & 1));
    }
  };

  auto logits = [&](int i, f32x4 (&s)[QB][NKB], auto scaled_tag) {
    bf16x8 k0[KH];
    read_k0(i, k0);
    logits_from(i, k0, s, scaled_tag);
  };

  // keys of a partial tile outside its rows [klo, khi) never win
  auto mask_tail = [&](f32x4 (&s)[QB][NKB], int klo, int khi) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (const int key = 32 * (kb >> 1) + 8 * G + 4 * (kb & 1) + r; key < klo || key >= khi) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb][r] = -INFINITY;
          kcs[kb][r] = a.c2;   // a zero scale would turn -inf into NaN
        }
  };

  // raise the reference max of query block qb by up (log2 units); the first
  // tile of a block sets it outright (O and the sums are still zero)
  bool fresh = true;
  auto raise_ref = [&](int qb, float up) {
    if (!fresh) {
      const float alpha = __builtin_amdgcn_exp2f(-up);
      lacc[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[qb][db] *= alpha;
    }
    m_ref[qb] += up;
  };

  // P = exp2(c2*s - m_ref) as bf16 MFMA operands, against a running reference
  // max per query. The exponents t = c2*s - m_ref are formed in place first and
  // each lane tests the maximum of its own (fma results, so the max needs no NaN
  // quieting): the reference is raised -- O and the sums rescaled -- only when a
  // t exceeds kTau, so every probability is at most 2^kTau and raises are rare
  // after the first tile. A raise takes the exact tile max over the query's four
  // lanes and never lowers the reference; the block's first tile (reference 0,
  // t = c2*s) always takes it and sets the reference to that max.
  auto probs = [&](f32x4 (&s)[QB][NKB], bf16x8 (&pf)[QB][BC / 32], auto scaled_tag) {
    constexpr bool SCALED = decltype(scaled_tag)::value;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float nm = -m_ref[qb];
      float tm = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s[qb][kb][r] = fmaf(s[qb][kb][r], SCALED ? kcs[kb][r] : a.c2, nm);
        tm = fmaxf(tm, fmaxf(fmaxf(s[qb][kb][0], s[qb][kb][1]), fmaxf(s[qb][kb][2], s[qb][kb][3])));
      }
      if (fresh || __any(tm > kTau)) {
        float up = xmax32(xmax16(tm));
        if (!fresh) up = fmaxf(up, 0.f);
        raise_ref(qb, up);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[qb][kb] -= up;
      }
#pragma unroll
      for (int g = 0; g < BC / 32; ++g) {
        float p[8];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) p[4 * bb + r] = __builtin_amdgcn_exp2f(s[qb][2 * g + bb][r]);
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
        pf[qb][g] = __builtin_bit_cast(bf16x8, w);
      }
    }
    fresh = false;
  };

  // O^T += V^T P^T from V buffer i, plus the row sums by an all-ones A operand. The V fragments of key group g+1 are requested into
  // the registers of group g as each is consumed, so their LDS latency hides
  // behind the remaining MFMAs (the scheduling barriers keep that order).
  const bf16x8 ones = __builtin_bit_cast(bf16x8, (u32x4){0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  auto vread = [&](int i, int g, int db) {
    const int d = 16 * db + i16;
    return *reinterpret_cast<const bf16x8*>(vbuf(i) + d * BC * 2 + (((4 * g + G) ^ swz_v<BC>(d)) * 16));
  };
  auto read_v0 = [&](int i, bf16x8 (&vf)[D / 16]) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db) vf[db] = vread(i, 0, db);
  };
  // vf: key group 0's fragments, already requested
  auto values_from = [&](int i, const bf16x8 (&pf)[QB][BC / 32], bf16x8 (&vf)[D / 16]) {
#pragma unroll
    for (int g = 0; g < BC / 32; ++g) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[qb][g], lacc[qb], 0, 0, 0);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pf[qb][g], o[qb][db], 0, 0, 0);
        if (g + 1 < BC / 32) vf[db] = vread(i, g + 1, db);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // then() runs right after the first group's requests (the caller's next reads)
  auto values = [&](int i, const bf16x8 (&pf)[QB][BC / 32], auto&& then) {
    bf16x8 vf[D / 16];
    read_v0(i, vf);
    then();
    __builtin_amdgcn_sched_barrier(0);
    values_from(i, pf, vf);
  };
  auto no_reads = []() {};

  // ---- a run of n full tiles [t0, t0+n) of one kind.
  // PIPE: two wave groups in ping-pong, one issuing MFMAs while the other runs
  // the softmax. bf16 tiles take the three-K-stage schedule (no copies in the
  // MFMA phases), INT8 cache tiles the two-stage one. Otherwise: tile by tile,
  // the next tile's copies in flight during its MFMAs.
  auto run_full = [&](int t0, int n, auto ct) {
    if (n <= 0) return;
    const std::bool_constant<I8 && decltype(ct)::value> scaled_tag;
    if constexpr (PIPE && !VPF && !I8) {
      // bf16 ping-pong, three K stages. Slot X(t) = [A: H1(t) | B: H2(t-1)],
      // slot Y(t) = [A: H2(t) | B: H1(t)]; H1 = values of t-1 + logits of t (MFMA),
      // H2 = softmax of t. The MFMA phases issue no copies: A copies K(t+2)
      // whole at the top of its H2(t) (slot Y(t); K buffer (t+2)%3 was last read
      // in slot Y(t-1)) and waits for K(t+1) at its end; B copies V(t+1) whole at
      // the top of its H2(t) (slot X(t+1); V buffer (t+1)%2 was last read in slot
      // Y(t)) and waits for it at the end of its H1(t+1).
      constexpr int KG = C::KT_BYTES / 1024 / 4;
      const int grp = PP_GROUP(wave);
      start_k(t0, 0, ct);
      if (n > 1) start_k(t0 + 1, 1, ct);
      start_v(t0, 0, ct);
      wait_copies();
      __syncthreads();
      f32x4 sacc[QB][NKB];
      bf16x8 pf[QB][BC / 32];
      if (grp == 1) __syncthreads();   // group B runs one slot behind
      int kb = 0;                      // K buffer of tile t: t % 3
      for (int t = 0; t < n; ++t) {
        __builtin_amdgcn_s_setprio(1);
        bf16x8 k0[KH];
        if (t >= 1) values((t - 1) & 1, pf, [&]() { read_k0(kb, k0); });
        else read_k0(kb, k0);
        logits_from(kb, k0, sacc, scaled_tag);
        __builtin_amdgcn_s_setprio(0);
        if (grp == 1) wait_copies();
        __syncthreads();
        const int kb2 = kb == 0 ? 2 : kb - 1;   // (t + 2) % 3
        if (grp == 0 && t + 2 < n) copy_k4(t0 + t + 2, kb2, ct);
        if (grp == 1 && t + 1 < n) copy_v4(t0 + t + 1, (t + 1) & 1, ct);
        probs(sacc, pf, scaled_tag);
        if (grp == 0) {
          if (t + 2 < n) __builtin_amdgcn_s_waitcnt((KG & 15) | (7 << 4) | ((KG >> 4) << 14));
          else wait_copies();
        }
        __syncthreads();
        kb = kb == 2 ? 0 : kb + 1;
      }
      values((n - 1) & 1, pf, no_reads);
      __syncthreads();
      if (grp == 0) __syncthreads();   // group A's idle last slot
    } else if constexpr (PIPE) {
      // INT8 ping-pong, two K stages and three V^T stages: each tile is an MFMA
      // phase H1(t) = [values of t-1, logits of t] and a VALU phase H2(t) =
      // [softmax of t], the two groups one barrier apart. K(s) and V(s) travel
      // together: group A loads its half at the top of its H1(s-1), group B at
      // the top of its H2(s-2), and each converts its half into K buffer s%2 and
      // V buffer s%3 before the barrier that opens A's H1(s). With the third V
      // stage each wave's H2(s) already requests V(s)'s first fragments for its
      // next H1, across the barrier.
      static_assert(VPF, "the two-stage schedule serves INT8 tiles, whose K and V travel together");
      const int grp = PP_GROUP(wave);
      auto issue = [&](int s) {
        if (s < n) {
          start_k(t0 + s, s & 1, ct);
          start_v(t0 + s, s % 3, ct);
        }
      };
      // (the value scales are requested first: their LDS latency hides behind
      // the key conversion)
      auto complete = [&](int s) {
        wait_copies();
        if (s < n) {
          f32x4 sc[4];
          if constexpr (decltype(ct)::value) read_vsc(sc);
          finish_k(t0 + s, s & 1, ct);
          finish_v_sc(t0 + s, s % 3, ct, sc);
        }
      };
      start_k(t0, 0, ct);
      start_v(t0, 0, ct);
      wait_copies();
      finish_k(t0, 0, ct);
      finish_v(t0, 0, ct);
      __syncthreads();
      f32x4 sacc[QB][NKB];
      bf16x8 pf[QB][BC / 32];
      bf16x8 vf[D / 16];
      // Cache tiles (codes staged through registers): group B converts its half
      // of tile s in its H2(s-2), the slot of A's H1(s-1), and then requests
      // tile s+1; so each slot carries one group's conversion (A's in Y, B's in
      // X). K buffer s%2 then holds tile s-2 and V buffer s%3 tile s-3, both
      // read by both groups in earlier slots, and the key scales stay with wave
      // 0 (group A). Current-segment tiles, copied straight into LDS, cannot be
      // requested three tiles ahead (the copy would land in a buffer still
      // read): B converts them in its H1(s-1) as requested in its H2(s-2).
      constexpr bool AHEAD = decltype(ct)::value;
      if (grp == 1) {     // group B's first slot
        issue(1);
        if constexpr (AHEAD) {
          complete(1);
          issue(2);
        }
        __syncthreads();
      }
      for (int t = 0; t < n; ++t) {
        // H1(t), at issue priority 1 so that each MFMA goes out as soon as the
        // matrix core frees
        __builtin_amdgcn_s_setprio(1);
        if (grp == 0) issue(t + 1);
        bf16x8 k0[KH];   // first K fragments of tile t, landing during the value MFMAs
        read_k0(t & 1, k0);
        if (t >= 1) values_from((t - 1) % 3, pf, vf);
        logits_from(t & 1, k0, sacc, scaled_tag);
        __builtin_amdgcn_s_setprio(0);
        if (!AHEAD && grp == 1) complete(t + 1);
        __syncthreads();
        // H2(t)
        if (!AHEAD && grp == 1) issue(t + 2);
        probs(sacc, pf, scaled_tag);
        read_v0(t % 3, vf);
        if (grp == 0) complete(t + 1);
        if (AHEAD && grp == 1) {
          complete(t + 2);
          issue(t + 3);
        }
        __syncthreads();
      }
      values_from((n - 1) % 3, pf, vf);
      __syncthreads();
      if (grp == 0) __syncthreads();   // group A's idle last slot
    } else {
      start_k(t0, 0, ct);
      start_v(t0, 0, ct);
      wait_copies();
      finish_k(t0, 0, ct);
      finish_v(t0, 0, ct);
      __syncthreads();
      for (int j = 0; j < n; ++j) {
        const int i = j & 1;
        const bool more = j + 1 < n;
        if (more) {
          start_k(t0 + j + 1, i ^ 1, ct);
          start_v(t0 + j + 1, i ^ 1, ct);
        }
        f32x4 s[QB][NKB];
        logits(i, s, scaled_tag);
        bf16x8 pf[QB][BC / 32];
        probs(s, pf, scaled_tag);
        values(i, pf, no_reads);
        if (more) {
          wait_copies();
          finish_k(t0 + j + 1, i ^ 1, ct);
          finish_v(t0 + j + 1, i ^ 1, ct);
        }
        __syncthreads();
      }
    }
  };

  // ---- one partial tile (keys past nvalid masked), unpipelined
  auto run_partial = [&](int t, auto ct) {
    const std::bool_constant<I8 && decltype(ct)::value> scaled_tag;
    int key0, nvalid, klo;
    tile_rows(t, ct, key0, nvalid, klo);
    if constexpr (decltype(ct)::value) start_k(t, 0, ct);   // cache tiles read inside the head's rows
    else start_k_tail(t);
    start_v(t, 0, ct);
    wait_copies();
    finish_k(t, 0, ct);
    finish_v(t, 0, ct);
    __syncthreads();
    zero_tail(0, klo, klo + nvalid);
    __syncthreads();
    f32x4 s[QB][NKB];
    logits(0, s, scaled_tag);
    mask_tail(s, klo, klo + nvalid);
    bf16x8 pf[QB][BC / 32];
    probs(s, pf, scaled_tag);
    values(0, pf, no_reads);
    __syncthreads();
  };

  using T_ = std::true_type;
  using F_ = std::false_type;
  if constexpr (MS) {
    // block-causal visibility of a query in segment seg: every row of seg, and
    // the video rows of each earlier segment whose frame is >= t0[seg] - window
    for (int r = 0; r <= seg; ++r) {
      kbase = st.row0[r];
      kend = st.row0[r + 1];
      if (r < seg) {
        const int nf = st.nv[r] / st.tpf;
        const int fmin = st.window < 0 ? st.t0[r] : max(st.t0[r], st.t0[seg] - st.window);
        if (fmin >= st.t0[r] + nf) continue;
        kbase += (fmin - st.t0[r]) * st.tpf;
        kend = st.row0[r] + st.nv[r];
      }
      const int nfull = (kend - kbase) / BC;
      run_full(0, nfull, F_{});
      if (nfull * BC < kend - kbase) run_partial(nfull, F_{});
    }
  } else {
    // this split's tiles: full cache tiles, full current tiles, then the partial
    // tails (one per cache run, one of the segment; key order does not matter
    // to attention)
    const int full_c = full_c_b, full_n = a.n_cur / BC;
    const int c_lo = min(t_begin, full_c), c_hi = min(t_end, full_c);
    const int n_lo = max(t_begin, tiles_c_b), n_hi = min(t_end, tiles_c_b + full_n);
    run_full(c_lo, c_hi - c_lo, T_{});
    run_full(n_lo, max(0, n_hi - n_lo), F_{});
    if (full_c < tiles_c_b && t_begin <= full_c && full_c < t_end) run_partial(full_c, T_{});
    if (full_c + 1 < tiles_c_b && t_begin <= full_c + 1 && full_c + 1 < t_end) run_partial(full_c + 1, T_{});
    const int pn = tiles_c_b + full_n;
    if (pn < tiles_total_b && t_begin <= pn && pn < t_end) run_partial(pn, F_{});
  }

  // ---- epilogue. A sparse block whose list leaves its split no key tile (its
  // last candidate block is short, so it has fewer tiles than the split count
  // was planned for) has l = 0: it writes O = 0 and lse = -inf, which the merge
  // weighs by exp(-inf) = 0. Any block that ran a tile has l >= 1 (the tile's
  // largest key enters with probability 1).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = lacc[qb][0];
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const int row = q_row0 + (wave * QB + qb) * 16 + i16;
    if (row >= q_end) continue;
    const float lse = l > 0.f ? (m_ref[qb] + log2f(l)) * kLn2 : -INFINITY;
    if (!a.part_o) {
      uint16_t* dst = a.out + (int64_t)row * a.ld_out + (int64_t)h * D + 4 * G;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const f32x4 v = o[qb][db] * inv;
        *reinterpret_cast<uint2*>(dst + 16 * db) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
      if (a.lse && G == 0) a.lse[(int64_t)h * a.n_q + row] = lse;
    } else {
      const int64_t prow = ((int64_t)split * a.H + h) * a.n_q + row;
      float* dst = a.part_o + prow * D + 4 * G;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db) = o[qb][db] * inv;
      if (G == 0) a.part_lse[prow] = lse;
    }
  }
}

// ---- merge of split partials: O = sum_s exp(lse_s - lse) O_s, fixed order
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                                         int S, int H, int n_q, uint16_t* __restrict__ out,
                                                         int64_t ld_out, float* __restrict__ lse) {
  constexpr int TPR = D / 4;                  // threads per (head, query) row
  const int r = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (r >= H * n_q) return;
  const int h = r / n_q, row = r % n_q;
  const int d0 = (threadIdx.x % TPR) * 4;
  float m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmaxf(m, part_lse[((int64_t)s * H + h) * n_q + row]);
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    // an empty split (lse = -inf, O = 0) gets weight 0; m is finite because
    // some split of every row has keys
    const int64_t pr = ((int64_t)s * H + h) * n_q + row;
    const float w = expf(part_lse[pr] - m);
    wsum += w;
    acc += w * *reinterpret_cast<const f32x4*>(part_o + pr * D + d0);
  }
  acc *= 1.0f / wsum;
  *reinterpret_cast<uint2*>(out + (int64_t)row * ld_out + (int64_t)h * D + d0) =
      make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
  if (lse && d0 == 0) lse[(int64_t)h * n_q + row] = m + logf(wsum);
}

// ---- current segment's V -> V^T [H][D][pitch] (zero beyond n). A lane moves an
// 8 x 8 block (8 tokens x 8 channels): eight 16-byte row loads, a transpose in
// registers (each output word joins two 16-bit halves), eight 16-byte stores;
// no LDS. A block is 128 tokens x D channels of one head, one wave per 64 x 64
// quarter; lane = 8 * channel chunk + token group, so a load instruction reads
// 8 rows x 128 contiguous bytes and a store writes 8 channel rows x 128
// contiguous bytes.
template <int D>
__global__ __launch_bounds__(2 * D) void v_transpose_kernel(const uint16_t* __restrict__ v, int64_t ld, int n,
                                                           uint16_t* __restrict__ vt, int pitch) {
  const int h = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * 128 + (wave & 1) * 64 + 8 * (lane & 7);   // the lane's first token
  const int d0 = (wave >> 1) * 64 + 8 * (lane >> 3);                     // and first channel
  u32x4 in[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {   // rows past n (n >= 1) read row n-1 and keep zeros
    in[i] = *reinterpret_cast<const u32x4*>(v + (int64_t)min(t0 + i, n - 1) * ld + (int64_t)h * D + d0);
    if (t0 + i >= n) in[i] = (u32x4){0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a = in[2 * k][j >> 1], b = in[2 * k + 1][j >> 1];
      o[k] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    *reinterpret_cast<u32x4*>(vt + ((int64_t)h * D + d0 + j) * pitch + t0) = o;
  }
}
static_assert(kTokenAlign % 128 == 0, "V^T pitches are whole 128-token blocks");

// ---------------------------------------------------------------- host side
struct Plan {
  int bc;
  int br;
  int n_cached, n_q, pitch_cur, tiles_c, tiles_total, n_qtiles, splits;
  size_t off_part_o, off_part_lse, bytes;
};

// Tile shape per head dim and cache type: keys per tile, waves per block,
// 16-query blocks per wave, ping-pong schedule, V prefetch across the barrier
// (three V stages). INT8 tiles stage their codes through registers, which
// leaves no room for 128-key tiles in the ping-pong register budget (two waves
// per SIMD, 256 registers each).
template <int D, bool I8> struct Shape;
#ifndef NOMAS_ATTN_BC
#define NOMAS_ATTN_BC 128
#endif
template <bool I8> struct Shape<128, I8> {
  static constexpr int BC = I8 ? 64 : NOMAS_ATTN_BC, NW = 8, QB = 2;
  static constexpr bool PIPE = true, VPF = I8;
};
template <bool I8> struct Shape<64, I8> {
  static constexpr int BC = 64, NW = 4, QB = 2;
  static constexpr bool PIPE = false, VPF = false;
};
static_assert(Shape<128, true>::NW * Shape<128, true>::QB == Shape<128, false>::NW * Shape<128, false>::QB,
              "both cache types tile the queries alike");
constexpr int kCUs = 256;
static int block_queries(int D) { return D == 128 ? Shape<128, false>::NW * Shape<128, false>::QB * 16 : Shape<64, false>::NW * Shape<64, false>::QB * 16; }
static int key_tile(int D, bool i8) {
  if (D == 128) return i8 ? Shape<128, true>::BC : Shape<128, false>::BC;
  return i8 ? Shape<64, true>::BC : Shape<64, false>::BC;
}
// resident blocks per CU: the ping-pong schedule runs one 8-wave block per CU
static int blocks_per_cu(int D) { return (D == 128 ? Shape<128, false>::PIPE : Shape<64, false>::PIPE) ? 1 : 2; }

// Split count for a call whose query-tile blocks do not fill the chip. With s
// splits the call runs ceil(blocks * s / slots) rounds of resident blocks, each
// block taking 1/s of a whole block's keys; the plan takes the smallest s whose
// makespan is within 10 % of the shortest (each split adds an fp32 partial that
// the blocks write and the merge reads).
// Splits keep at least 16 key tiles each; more than one per CU never pays.
static int auto_splits(int n_qtiles, int H, int tiles_total, int per_cu) {
  const int64_t blocks = (int64_t)n_qtiles * H, slots = (int64_t)per_cu * kCUs;
  if (blocks >= slots) return 1;
  const int max_s = std::min(kCUs, tiles_total / 16);
  if (max_s <= 1) return 1;
  auto makespan = [&](int s) { return (double)((blocks * s + slots - 1) / slots) / s; };
  double best = makespan(1);
  for (int s = 2; s <= max_s; ++s) best = std::min(best, makespan(s));
  for (int s = 1; s < max_s; ++s)
    if (makespan(s) <= best * 1.10) return s;
  return max_s;
}

static bool make_plan(int n_video, int n_text, int64_t n_cached, int H, int D, int kv_dtype, int n_splits,
                      Plan& p) {
  if (n_video < 0 || n_text < 0 || (int64_t)n_video + n_text < 1 || H < 1 || (D != 64 && D != 128) ||
      n_cached < 0 || n_splits < 0 || (kv_dtype != NOMAS_KV_BF16 && kv_dtype != NOMAS_KV_INT8))
    return false;
  if ((int64_t)n_video + n_text > (1 << 26) || n_cached > ((int64_t)1 << 30)) return false;
  p.bc = key_tile(D, kv_dtype == NOMAS_KV_INT8);
  p.br = block_queries(D);
  p.n_cached = (int)n_cached;
  p.n_q = n_video + n_text;
  p.pitch_cur = (int)round_up(p.n_q, kTokenAlign);
  p.tiles_c = (int)((n_cached + p.bc - 1) / p.bc);
  p.tiles_total = p.tiles_c + (p.n_q + p.bc - 1) / p.bc;
  p.n_qtiles = (p.n_q + p.br - 1) / p.br;
  int s = n_splits ? n_splits : auto_splits(p.n_qtiles, H, p.tiles_total, blocks_per_cu(D));
  if (s > p.tiles_total) s = p.tiles_total;
  p.splits = s;
  size_t off = round_up((int64_t)H * D * p.pitch_cur * 2, 256);
  p.off_part_o = off;
  if (s > 1) {
    off += round_up((int64_t)s * H * p.n_q * D * 4, 256);
    p.off_part_lse = off;
    off += round_up((int64_t)s * H * p.n_q * 4, 256);
  } else {
    p.off_part_lse = off;
  }
  p.bytes = off;
  return true;
}

template <int D, bool I8, int MODE = kModeCached>
static void launch_attn(const AttnArgs& a, hipStream_t st, const SegTable& seg) {
  const dim3 grid((unsigned)(8 * a.per_xcd));
  using S = Shape<D, I8>;
  hipLaunchKernelGGL((attn_kernel<D, S::QB, S::NW, S::BC, I8, S::PIPE, S::VPF, MODE>), grid, dim3(S::NW * 64), 0, st,
                     a, seg);
}

}  // namespace nomas

using namespace nomas;

extern "C" size_t nomas_segment_attention_workspace_bytes(int32_t n_video, int32_t n_text, int64_t n_cached,
                                                          int32_t n_heads, int32_t head_dim, int32_t kv_dtype,
                                                          int32_t n_splits) {
  Plan p;
  if (!make_plan(n_video, n_text, n_cached, n_heads, head_dim, kv_dtype, n_splits, p)) return 0;
  return p.bytes;
}

extern "C" int32_t nomas_segment_attention_splits(int32_t n_video, int32_t n_text, int64_t n_cached,
                                                  int32_t n_heads, int32_t head_dim, int32_t kv_dtype,
                                                  int32_t n_splits) {
  Plan p;
  if (!make_plan(n_video, n_text, n_cached, n_heads, head_dim, kv_dtype, n_splits, p)) return -1;
  return p.splits;
}

// The cached tokens a call attends to, as runs of physical cache tokens:
// [a0, a0 + na) then [0, nb). All retained frames are read in slot order (one
// run); a frame range that wraps round the ring is two.
struct CacheRuns {
  int64_t a0, na, nb;
};
static CacheRuns all_retained(const nomas_kvcache* c) {
  return CacheRuns{0, nomas_kvcache_valid_frames(c) * c->tokens_per_frame, 0};
}

// the cached call, dense (sparse = false) or restricted to the block lists; the
// current values from v_cur (transposed into the workspace) or, when v_t is
// given, from the caller's V^T [H*D][ld_vt]
static int32_t segment_attention_impl(const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur, int64_t ld_qkv,
                                      const uint16_t* v_t, int64_t ld_vt, int32_t n_video, int32_t n_text,
                                      const nomas_kvcache* c, const CacheRuns& runs, bool sparse,
                                      const int32_t* block_list, int32_t n_select, uint16_t* out, int64_t ld_out,
                                      float* lse, float softmax_scale, int32_t n_splits, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (int32_t e = validate_cache(c, "segment_attention")) return e;
  const int H = c->n_heads, D = c->head_dim;
  if (!q || !k_cur || !(v_cur || v_t) || !out)
    return fail(NOMAS_E_INVALID, "segment_attention: q, k_cur, out and v_cur (or v_t) must be non-NULL");
  if (!aligned16(q) || !aligned16(k_cur) || (v_cur && !aligned16(v_cur)) || !aligned16(out))
    return fail(NOMAS_E_INVALID, "segment_attention: q, k_cur, v_cur, out must be 16-byte aligned");
  // (key tiles read whole 128-row blocks of V^T columns: ld_vt covers them)
  if (v_t && (!aligned16(v_t) || ld_vt < round_up((int64_t)n_video + n_text, 128) || ld_vt % 8 ||
              (int64_t)D * ld_vt * 2 > INT32_MAX))
    return fail(NOMAS_E_INVALID,
                "segment_attention: v_t must be 16-byte aligned with ld_vt >= n_video + n_text rounded up to a "
                "multiple of 128, a multiple of 8, and head_dim * ld_vt * 2 bytes below 2 GiB");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return fail(NOMAS_E_INVALID, "segment_attention: lse must be 4-byte aligned");
  if (ld_qkv < (int64_t)H * D || ld_qkv % 8 || ld_out < (int64_t)H * D || ld_out % 8)
    return fail(NOMAS_E_INVALID, "segment_attention: ld_qkv and ld_out must be >= n_heads*head_dim and multiples of 8");
  if (n_video < 0 || n_text < 0 || (int64_t)n_video + n_text < 1)
    return fail(NOMAS_E_INVALID, "segment_attention: need n_video >= 0, n_text >= 0, n_video + n_text >= 1");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(NOMAS_E_INVALID, "segment_attention: softmax_scale must be finite and > 0");
  if (n_splits < 0) return fail(NOMAS_E_INVALID, "segment_attention: n_splits must be >= 0");
  // 32-bit byte ranges of the kernels' loads of the current rows and of V^T
  if (((int64_t)n_video + n_text) * ld_qkv * 2 > INT32_MAX ||
      (int64_t)D * round_up((int64_t)n_video + n_text, kTokenAlign) * 2 > INT32_MAX)
    return fail(NOMAS_E_INVALID, "segment_attention: (n_video + n_text) * ld_qkv * 2 bytes must stay below 2 GiB");
  const int64_t n_cached = runs.na + runs.nb;
  const int64_t n_cand = (n_cached + kSpKeyBlock - 1) / kSpKeyBlock;
  if (sparse) {
    if (n_select < 0 || n_select > n_cand)
      return fail(NOMAS_E_INVALID, "segment_attention_sparse: n_select %d outside [0, %lld] (candidate blocks)", n_select,
                  (long long)n_cand);
    if (n_select > 0 && (!block_list || (reinterpret_cast<uintptr_t>(block_list) & 3)))
      return fail(NOMAS_E_INVALID, "segment_attention_sparse: block_list must be non-NULL and 4-byte aligned");
  }
  // splits and workspace are planned for the listed rows (an upper bound)
  Plan p;
  if (!make_plan(n_video, n_text, sparse ? (int64_t)n_select * kSpKeyBlock : n_cached, H, D, c->kv_dtype, n_splits, p))
    return fail(NOMAS_E_INVALID, "segment_attention: sizes out of range");
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(NOMAS_E_WORKSPACE, "segment_attention: workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < p.bytes)
    return fail(NOMAS_E_WORKSPACE, "segment_attention: workspace of %zu bytes, need %zu", workspace_bytes, p.bytes);

  const hipStream_t st = as_stream(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const uint16_t* vt = v_t;
  int pitch_cur = (int)ld_vt;
  if (!v_t) {
    uint16_t* vw = reinterpret_cast<uint16_t*>(ws);
    const dim3 grid((unsigned)(p.pitch_cur / 128), (unsigned)H);
    if (D == 128) hipLaunchKernelGGL(v_transpose_kernel<128>, grid, dim3(256), 0, st, v_cur, ld_qkv, p.n_q, vw, p.pitch_cur);
    else hipLaunchKernelGGL(v_transpose_kernel<64>, grid, dim3(128), 0, st, v_cur, ld_qkv, p.n_q, vw, p.pitch_cur);
    if (int32_t e = check_launch("segment_attention (v transpose)")) return e;
    vt = vw;
    pitch_cur = p.pitch_cur;
  }

  AttnArgs a{};
  a.q = q;
  a.kcur = k_cur;
  a.ld_qkv = ld_qkv;
  a.vtcur = vt;
  a.pitch_cur = pitch_cur;
  a.kc = c->k;
  a.vc = c->v;
  a.ks = c->k_scale;
  a.vs = c->v_scale;
  a.pitch_c = c->token_pitch;
  a.n_cached = (int)n_cached;
  a.c_a0 = (int)runs.a0;
  a.c_na = (int)runs.na;
  a.c_nb = (int)runs.nb;
  a.n_cur = p.n_q;
  a.n_q = p.n_q;
  a.H = H;
  a.c2 = softmax_scale * kLog2e;
  a.out = out;
  a.ld_out = ld_out;
  a.lse = lse;
  a.part_o = p.splits > 1 ? reinterpret_cast<float*>(ws + p.off_part_o) : nullptr;
  a.part_lse = p.splits > 1 ? reinterpret_cast<float*>(ws + p.off_part_lse) : nullptr;
  a.n_splits = p.splits;
  a.tiles_c = p.tiles_c;
  a.tiles_total = p.tiles_total;
  a.n_qtiles = p.n_qtiles;
  a.n_blocks = p.n_qtiles * H * p.splits;
  a.per_xcd = (a.n_blocks + 7) / 8;
  a.blist = block_list;
  a.n_sel = sparse ? n_select : 0;
  a.nqb_sp = (p.n_q + kSpQueryBlock - 1) / kSpQueryBlock;
  const bool i8 = c->kv_dtype == NOMAS_KV_INT8;
  const SegTable none{};
  if (sparse) {
    if (D == 128) {
      if (i8) launch_attn<128, true, kModeSparse>(a, st, none);
      else launch_attn<128, false, kModeSparse>(a, st, none);
    } else {
      if (i8) launch_attn<64, true, kModeSparse>(a, st, none);
      else launch_attn<64, false, kModeSparse>(a, st, none);
    }
  } else if (D == 128) {
    if (i8) launch_attn<128, true>(a, st, none);
    else launch_attn<128, false>(a, st, none);
  } else {
    if (i8) launch_attn<64, true>(a, st, none);
    else launch_attn<64, false>(a, st, none);
  }
  if (int32_t e = check_launch("segment_attention")) return e;
  if (p.splits > 1) {
    const int rows = H * p.n_q;
    const int rows_per_block = 256 / (D / 4);
    const dim3 grid((unsigned)((rows + rows_per_block - 1) / rows_per_block));
    if (D == 128)
      hipLaunchKernelGGL(attn_merge_kernel<128>, grid, dim3(256), 0, st, a.part_o, a.part_lse, p.splits, H, p.n_q, out, ld_out, lse);
    else
      hipLaunchKernelGGL(attn_merge_kernel<64>, grid, dim3(256), 0, st, a.part_o, a.part_lse, p.splits, H, p.n_q, out, ld_out, lse);
    if (int32_t e = check_launch("segment_attention (merge)")) return e;
  }
  return ok();
}

extern "C" int32_t nomas_segment_attention(const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                                           int64_t ld_qkv, int32_t n_video, int32_t n_text, const nomas_kvcache* c,
                                           uint16_t* out, int64_t ld_out, float* lse, float softmax_scale,
                                           int32_t n_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (int32_t e = validate_cache(c, "segment_attention")) return e;
  return segment_attention_impl(q, k_cur, v_cur, ld_qkv, nullptr, 0, n_video, n_text, c, all_retained(c), false,
                                nullptr, 0, out, ld_out, lse, softmax_scale, n_splits, workspace, workspace_bytes,
                                stream);
}

extern "C" int32_t nomas_segment_attention_frames(const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                                                  int64_t ld_qkv, const uint16_t* v_t, int64_t ld_vt,
                                                  int32_t n_video, int32_t n_text, const nomas_kvcache* c,
                                                  int64_t first_frame, int32_t n_frames, uint16_t* out,
                                                  int64_t ld_out, float* lse, float softmax_scale, int32_t n_splits,
                                                  void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "segment_attention_frames";
  if (int32_t e = validate_cache(c, who)) return e;
  const int64_t fw = c->frames_written, valid = nomas_kvcache_valid_frames(c);
  if (n_frames < 0 || first_frame < fw - valid || first_frame + n_frames > fw)
    return fail(NOMAS_E_INVALID, "%s: frames [%lld, %lld) are not all retained (retained: [%lld, %lld))", who,
                (long long)first_frame, (long long)first_frame + n_frames, (long long)(fw - valid), (long long)fw);
  const int64_t tpf = c->tokens_per_frame, cap = c->capacity_frames;
  CacheRuns runs = all_retained(c);
  if (n_frames < valid) {
    const int64_t s = first_frame % cap;
    const int64_t na = std::min<int64_t>(n_frames, cap - s);
    runs = CacheRuns{s * tpf, na * tpf, (n_frames - na) * tpf};
  }
  return segment_attention_impl(q, k_cur, v_cur, ld_qkv, v_t, ld_vt, n_video, n_text, c, runs, false, nullptr, 0, out,
                                ld_out, lse, softmax_scale, n_splits, workspace, workspace_bytes, stream);
}

extern "C" int32_t nomas_segment_attention_sparse(const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                                                  int64_t ld_qkv, int32_t n_video, int32_t n_text,
                                                  const nomas_kvcache* c, const int32_t* block_list,
                                                  int32_t n_select, uint16_t* out, int64_t ld_out, float* lse,
                                                  float softmax_scale, int32_t n_splits, void* workspace,
                                                  size_t workspace_bytes, void* stream) {
  if (int32_t e = validate_cache(c, "segment_attention_sparse")) return e;
  return segment_attention_impl(q, k_cur, v_cur, ld_qkv, nullptr, 0, n_video, n_text, c, all_retained(c), true,
                                block_list, n_select, out, ld_out, lse, softmax_scale, n_splits, workspace,
                                workspace_bytes, stream);
}

// ---------------------------------------------------------------- no-allocation variant
// The workspace of nomas_segment_attention_noalloc: a device array of the
// library, one copy on every GPU it runs on, held until the process ends. Host
// code never passes the array's name to a kernel or a copy (in host code it is
// a stand-in, not a device address): it uses the address hipGetSymbolAddress
// returns for the current device, looked up on the entry point's first call
// there and kept per device.
namespace nomas {
int64_t check_failures_attention(int reset) { return source_check_failures(reset); }
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static int32_t scratch_address(void** out, const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(NOMAS_E_HIP, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(NOMAS_E_UNSUPPORTED, "%s: device %d beyond %d", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(NOMAS_E_HIP, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", who, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NOMAS_OK;
}
}  // namespace nomas

extern "C" size_t nomas_segment_attention_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int32_t nomas_segment_attention_noalloc(const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                                                   int64_t ld_qkv, int32_t n_video, int32_t n_text,
                                                   const nomas_kvcache* c, uint16_t* out, int64_t ld_out,
                                                   float* lse, float softmax_scale, int32_t n_splits, void* stream) {
  const char* who = "segment_attention_noalloc";
  if (int32_t e = validate_cache(c, who)) return e;
  // the workspace these sizes need must fit the scratch array (checked before
  // anything touches the device)
  const size_t need = nomas_segment_attention_workspace_bytes(
      n_video, n_text, nomas_kvcache_valid_frames(c) * c->tokens_per_frame, c->n_heads, c->head_dim, c->kv_dtype,
      n_splits);
  if (need == 0) return fail(NOMAS_E_INVALID, "%s: sizes out of range", who);
  if (need > kNoAllocScratchBytes)
    return fail(NOMAS_E_WORKSPACE, "%s: these sizes need %zu bytes of workspace, beyond the %zu-byte scratch array",
                who, need, kNoAllocScratchBytes);
  if (stream) {
    int sdev = -1, cur = -1;
    if (hipStreamGetDevice(as_stream(stream), &sdev) != hipSuccess || hipGetDevice(&cur) != hipSuccess || sdev != cur)
      return fail(NOMAS_E_INVALID, "%s: the stream must belong to the calling thread's current device", who);
  }
  void* ws = nullptr;
  if (int32_t e = scratch_address(&ws, who)) return e;
  return segment_attention_impl(q, k_cur, v_cur, ld_qkv, nullptr, 0, n_video, n_text, c, all_retained(c), false,
                                nullptr, 0, out, ld_out, lse, softmax_scale, n_splits, ws, kNoAllocScratchBytes,
                                stream);
}

// ---------------------------------------------------------------- multi-segment calls
namespace nomas {

struct SegPlan {
  SegTable t;
  int n_rows, pitch, n_qtiles;
  size_t bytes;
};

static int32_t make_seg_plan(const nomas_segment* segs, int32_t n_segments, int32_t tpf, int32_t window, int H, int D,
                             SegPlan& p, const char* who) {
  if (!segs || n_segments < 1 || n_segments > kMaxSegments)
    return fail(NOMAS_E_INVALID, "%s: need 1 <= n_segments <= %d and a segment array", who, kMaxSegments);
  if (tpf < 1) return fail(NOMAS_E_INVALID, "%s: tokens_per_frame must be >= 1", who);
  if (H < 1 || (D != 64 && D != 128)) return fail(NOMAS_E_UNSUPPORTED, "%s: head_dim must be 64 or 128, n_heads >= 1", who);
  p.t = SegTable{};
  p.t.n_seg = n_segments;
  p.t.tpf = tpf;
  p.t.window = window < 0 ? -1 : window;
  const int br = block_queries(D);
  int64_t rows = 0, tiles = 0;
  for (int s = 0; s < n_segments; ++s) {
    const nomas_segment& g = segs[s];
    if (g.n_video < 0 || g.n_text < 0 || (int64_t)g.n_video + g.n_text < 1 || g.n_video % tpf || g.t0 < 0)
      return fail(NOMAS_E_INVALID,
                  "%s: segment %d needs n_video >= 0 (a multiple of tokens_per_frame), n_text >= 0, "
                  "n_video + n_text >= 1, t0 >= 0", who, s);
    p.t.row0[s] = (int)rows;
    p.t.nv[s] = g.n_video;
    p.t.t0[s] = g.t0;
    p.t.qtile0[s] = (int)tiles;
    rows += (int64_t)g.n_video + g.n_text;
    tiles += ((int64_t)g.n_video + g.n_text + br - 1) / br;
    if (rows > (1 << 26)) return fail(NOMAS_E_INVALID, "%s: more than 2^26 rows", who);
  }
  p.t.row0[n_segments] = (int)rows;
  p.t.qtile0[n_segments] = (int)tiles;
  p.n_rows = (int)rows;
  p.n_qtiles = (int)tiles;
  // V^T pitch: a range's partial tail tile starts anywhere (segments are not
  // tile-aligned) and reads a whole tile of columns, so one more 128-column
  // block of (zero) padding keeps every tile's columns inside the buffer
  p.pitch = (int)round_up(rows, kTokenAlign) + kTokenAlign;
  p.bytes = round_up((int64_t)H * D * p.pitch * 2, 256);
  return NOMAS_OK;
}

}  // namespace nomas

extern "C" size_t nomas_block_causal_attention_workspace_bytes(const nomas_segment* segs, int32_t n_segments,
                                                               int32_t tokens_per_frame, int32_t n_heads,
                                                               int32_t head_dim) {
  SegPlan p;
  if (make_seg_plan(segs, n_segments, tokens_per_frame, -1, n_heads, head_dim, p, "block_causal_attention")) return 0;
  return p.bytes;
}

extern "C" int32_t nomas_block_causal_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_qkv,
                                                const nomas_segment* segs, int32_t n_segments,
                                                int32_t tokens_per_frame, int32_t window_frames, int32_t n_heads,
                                                int32_t head_dim, uint16_t* out, int64_t ld_out, float* lse,
                                                float softmax_scale, void* workspace, size_t workspace_bytes,
                                                void* stream) {
  const char* who = "block_causal_attention";
  const int H = n_heads, D = head_dim;
  SegPlan p;
  if (int32_t e = make_seg_plan(segs, n_segments, tokens_per_frame, window_frames, H, D, p, who)) return e;
  if (!q || !k || !v || !out) return fail(NOMAS_E_INVALID, "%s: q, k, v, out must be non-NULL", who);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(NOMAS_E_INVALID, "%s: q, k, v, out must be 16-byte aligned", who);
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return fail(NOMAS_E_INVALID, "%s: lse must be 4-byte aligned", who);
  if (ld_qkv < (int64_t)H * D || ld_qkv % 8 || ld_out < (int64_t)H * D || ld_out % 8)
    return fail(NOMAS_E_INVALID, "%s: ld_qkv and ld_out must be >= n_heads*head_dim and multiples of 8", who);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(NOMAS_E_INVALID, "%s: softmax_scale must be finite and > 0", who);
  if ((int64_t)p.n_rows * ld_qkv * 2 > INT32_MAX || (int64_t)D * p.pitch * 2 > INT32_MAX)
    return fail(NOMAS_E_INVALID, "%s: rows * ld_qkv * 2 bytes must stay below 2 GiB", who);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(NOMAS_E_WORKSPACE, "%s: workspace must be non-NULL and 256-byte aligned", who);
  if (workspace_bytes < p.bytes)
    return fail(NOMAS_E_WORKSPACE, "%s: workspace of %zu bytes, need %zu", who, workspace_bytes, p.bytes);

  const hipStream_t st = as_stream(stream);
  uint16_t* vt = static_cast<uint16_t*>(workspace);
  {
    const dim3 grid((unsigned)(p.pitch / 128), (unsigned)H);
    if (D == 128) hipLaunchKernelGGL(v_transpose_kernel<128>, grid, dim3(256), 0, st, v, ld_qkv, p.n_rows, vt, p.pitch);
    else hipLaunchKernelGGL(v_transpose_kernel<64>, grid, dim3(128), 0, st, v, ld_qkv, p.n_rows, vt, p.pitch);
    if (int32_t e = check_launch("block_causal_attention (v transpose)")) return e;
  }
  AttnArgs a{};
  a.q = q;
  a.kcur = k;
  a.ld_qkv = ld_qkv;
  a.vtcur = vt;
  a.pitch_cur = p.pitch;
  a.kc = k;          // no cache: the descriptors over it are never read
  a.vc = v;
  a.ks = nullptr;
  a.vs = nullptr;
  a.pitch_c = 0;
  a.n_cached = 0;
  a.n_cur = p.n_rows;
  a.n_q = p.n_rows;
  a.H = H;
  a.c2 = softmax_scale * kLog2e;
  a.out = out;
  a.ld_out = ld_out;
  a.lse = lse;
  a.part_o = nullptr;
  a.part_lse = nullptr;
  a.n_splits = 1;
  a.tiles_c = 0;
  a.tiles_total = 0;
  a.n_qtiles = p.n_qtiles;
  a.n_blocks = p.n_qtiles * H;
  a.per_xcd = (a.n_blocks + 7) / 8;
  if (D == 128) launch_attn<128, false, kModeSegments>(a, st, p.t);
  else launch_attn<64, false, kModeSegments>(a, st, p.t);
  return check_launch(who);
}
