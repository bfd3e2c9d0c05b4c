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
//    (lane % 16) and 4 keys per MFMA: row max / row sum need only two
//    cross-lane steps (lanes 16 and 32 apart) per key tile.
//  * The 32 keys of a group are fed to the two S^T MFMAs in a permuted row
//    order so that lane group G ends up holding keys 8G..8G+7 in register
//    order; that is exactly the B operand (P^T) layout of the value MFMA
//    O^T += V^T P^T, so P never goes through LDS.
//  * V^T operand rows are contiguous key runs: the cache stores V transposed and
//    the current segment's V is transposed once into the workspace.
//  * K and V^T tiles of BC keys are double-buffered in LDS (one barrier per
//    tile), with the 16-byte chunk index XOR-swizzled by the row so that the
//    strided 128-bit operand reads are bank-conflict free. The next tile's
//    global loads are issued before the current tile's MFMAs.
//  * Online softmax in the log2 domain with a fixed reference max per query that
//    is only raised when a tile's max exceeds it by more than kTau (probabilities
//    stay <= 2^kTau, exact in fp32 and bf16 range), so the O rescale is rare.
//  * INT8 cache tiles: codes are converted to bf16 exactly while staging into
//    LDS; the key scale multiplies the logit of its key and the value scale
//    multiplies the probability of its key, both in fp32.
//  * Split-KV: the key tiles are cut into contiguous chunks; each block writes a
//    normalised fp32 partial and its log-sum-exp, merged in fixed order.
//  * Block ids are remapped so the blocks that the hardware places on one XCD
//    share (head, split): they stream the same K/V through that XCD's L2.
#include <cmath>
#include <cstdlib>

#include "nomas_common.hpp"

namespace nomas {

int32_t validate_cache(const nomas_kvcache* c, const char* who);

constexpr float kTau = 8.0f;
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
  int n_cached;
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
};

template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? ((row & 3) | (((row >> 3) & 3) << 2)) : ((row & 3) | (((row >> 3) & 1) << 2));
}
template <int BC>
__device__ __forceinline__ int swz_v(int d) {
  return BC == 128 ? (d & 15) : ((d >> 1) & 7);
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

template <int D, int QB, int NW, int BC, bool I8>
struct AttnCfg {
  static constexpr int NT = NW * 64;
  static constexpr int KC = D / 8;                 // bf16 chunks per K row
  static constexpr int VC = BC / 8;                // bf16 chunks per V^T row
  static constexpr int KT_BYTES = BC * D * 2;
  static constexpr int VT_BYTES = D * BC * 2;
  static constexpr int STAGE = KT_BYTES + VT_BYTES + 2 * BC * 4;
  static constexpr int NKB = BC * KC / NT;         // bf16 K chunks per thread
  static constexpr int NVB = D * VC / NT;          // bf16 V chunks per thread
  static constexpr int NSTG = NKB + NVB;
  static constexpr int BR = NW * QB * 16;          // queries per block
  static_assert(BC * KC % NT == 0 && D * VC % NT == 0, "tile must split evenly over threads");
  static_assert(NKB % 2 == 0 && NVB % 2 == 0, "int8 staging uses half the chunks");
};

template <int D, int QB, int NW, int BC, bool I8>
__global__ __launch_bounds__(NW * 64) void attn_kernel(const AttnArgs a) {
  using C = AttnCfg<D, QB, NW, BC, I8>;
  __shared__ __align__(16) unsigned char lds[2 * C::STAGE];

  const int b = blockIdx.x;
  const int logical = (b & 7) * a.per_xcd + (b >> 3);
  if (logical >= a.n_blocks) return;
  const int qt = logical % a.n_qtiles;
  const int hs = logical / a.n_qtiles;
  const int split = hs % a.n_splits;
  const int h = hs / a.n_splits;
  const int t_begin = (int)((int64_t)split * a.tiles_total / a.n_splits);
  const int t_end = (int)((int64_t)(split + 1) * a.tiles_total / a.n_splits);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int G = lane >> 4, i16 = lane & 15;

  // ---- Q fragments (B operand of S^T = K Q^T): lane -> query i16, dims 32kk+8G..+8
  bf16x8 qf[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qt * C::BR + (wave * QB + qb) * 16 + i16;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      u32x4 v = {0, 0, 0, 0};
      if (row < a.n_q) v = *reinterpret_cast<const u32x4*>(a.q + (int64_t)row * a.ld_qkv + (int64_t)h * D + 32 * kk + 8 * G);
      qf[qb][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 o[QB][D / 16];
  float m_ref[QB], l_sum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = -INFINITY;
    l_sum[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[qb][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  u32x4 stg[C::NSTG];

  // tile t -> (is cache tile, first key inside its part, valid keys)
  auto tile_info = [&](int t, bool& cache, int& key0, int& nvalid) {
    cache = t < a.tiles_c;
    if (cache) {
      key0 = t * BC;
      nvalid = min(BC, a.n_cached - key0);
    } else {
      key0 = (t - a.tiles_c) * BC;
      nvalid = min(BC, a.n_cur - key0);
    }
  };

  // ---- global -> registers
  auto load_tile = [&](int t) {
    bool cache;
    int key0, nvalid;
    tile_info(t, cache, key0, nvalid);
    if (I8 && cache) {
      const int8_t* kc = static_cast<const int8_t*>(a.kc);
      const int8_t* vc = static_cast<const int8_t*>(a.vc);
#pragma unroll
      for (int j = 0; j < C::NKB / 2; ++j) {
        const int c = tid + C::NT * j;
        const int row = c / (D / 16), cc = c % (D / 16);
        u32x4 v = {0, 0, 0, 0};
        if (row < nvalid) v = *reinterpret_cast<const u32x4*>(kc + ((int64_t)h * a.pitch_c + key0 + row) * D + cc * 16);
        stg[j] = v;
      }
#pragma unroll
      for (int j = 0; j < C::NVB / 2; ++j) {
        const int c = tid + C::NT * j;
        const int d = c / (BC / 16), cc = c % (BC / 16);
        stg[C::NKB / 2 + j] = *reinterpret_cast<const u32x4*>(vc + ((int64_t)h * D + d) * a.pitch_c + key0 + cc * 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < C::NKB; ++j) {
        const int c = tid + C::NT * j;
        const int row = c / C::KC, cc = c % C::KC;
        u32x4 v = {0, 0, 0, 0};
        if (row < nvalid) {
          const uint16_t* src = cache ? static_cast<const uint16_t*>(a.kc) + ((int64_t)h * a.pitch_c + key0 + row) * D + cc * 8
                                      : a.kcur + (int64_t)(key0 + row) * a.ld_qkv + (int64_t)h * D + cc * 8;
          v = *reinterpret_cast<const u32x4*>(src);
        }
        stg[j] = v;
      }
#pragma unroll
      for (int j = 0; j < C::NVB; ++j) {
        const int c = tid + C::NT * j;
        const int d = c / C::VC, cc = c % C::VC;
        const uint16_t* src = cache ? static_cast<const uint16_t*>(a.vc) + ((int64_t)h * D + d) * a.pitch_c + key0 + cc * 8
                                    : a.vtcur + ((int64_t)h * D + d) * a.pitch_cur + key0 + cc * 8;
        stg[C::NKB + j] = *reinterpret_cast<const u32x4*>(src);
      }
    }
  };

  // ---- registers -> LDS stage (with int8 -> bf16 conversion and key masking)
  auto store_tile = [&](int t, int stage) {
    bool cache;
    int key0, nvalid;
    tile_info(t, cache, key0, nvalid);
    unsigned char* Ks = lds + stage * C::STAGE;
    unsigned char* Vs = Ks + C::KT_BYTES;
    float* sc = reinterpret_cast<float*>(Vs + C::VT_BYTES);
    if (I8 && cache) {
#pragma unroll
      for (int j = 0; j < C::NKB / 2; ++j) {
        const int c = tid + C::NT * j;
        const int row = c / (D / 16), cc = c % (D / 16);
        u32x4 lo, hi;
        i8x16_to_bf16(stg[j], lo, hi);
        const int s = swz_k<D>(row);
        *reinterpret_cast<u32x4*>(Ks + row * D * 2 + (((2 * cc) ^ s) * 16)) = lo;
        *reinterpret_cast<u32x4*>(Ks + row * D * 2 + (((2 * cc + 1) ^ s) * 16)) = hi;
      }
#pragma unroll
      for (int j = 0; j < C::NVB / 2; ++j) {
        const int c = tid + C::NT * j;
        const int d = c / (BC / 16), cc = c % (BC / 16);
        u32x4 lo, hi;
        i8x16_to_bf16(stg[C::NKB / 2 + j], lo, hi);
        if (nvalid < BC) {   // zero the codes of keys past the valid range
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k0 = cc * 16 + 2 * e;
            if (k0 >= nvalid) lo[e] = 0; else if (k0 + 1 >= nvalid) lo[e] &= 0xffffu;
            const int k1 = cc * 16 + 8 + 2 * e;
            if (k1 >= nvalid) hi[e] = 0; else if (k1 + 1 >= nvalid) hi[e] &= 0xffffu;
          }
        }
        const int s = swz_v<BC>(d);
        *reinterpret_cast<u32x4*>(Vs + d * BC * 2 + (((2 * cc) ^ s) * 16)) = lo;
        *reinterpret_cast<u32x4*>(Vs + d * BC * 2 + (((2 * cc + 1) ^ s) * 16)) = hi;
      }
      // scales (0 for keys past the valid range)
      for (int j = tid; j < 2 * BC; j += C::NT) {
        const int kidx = j % BC;
        const float* src = j < BC ? a.ks : a.vs;
        sc[j] = kidx < nvalid ? src[(int64_t)h * a.pitch_c + key0 + kidx] : 0.f;
      }
    } else {
#pragma unroll
      for (int j = 0; j < C::NKB; ++j) {
        const int c = tid + C::NT * j;
        const int row = c / C::KC, cc = c % C::KC;
        *reinterpret_cast<u32x4*>(Ks + row * D * 2 + ((cc ^ swz_k<D>(row)) * 16)) = stg[j];
      }
#pragma unroll
      for (int j = 0; j < C::NVB; ++j) {
        const int c = tid + C::NT * j;
        const int d = c / C::VC, cc = c % C::VC;
        u32x4 v = stg[C::NKB + j];
        if (nvalid < BC) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k0 = cc * 8 + 2 * e;
            if (k0 >= nvalid) v[e] = 0; else if (k0 + 1 >= nvalid) v[e] &= 0xffffu;
          }
        }
        *reinterpret_cast<u32x4*>(Vs + d * BC * 2 + ((cc ^ swz_v<BC>(d)) * 16)) = v;
      }
    }
  };

  // ---- one tile of MFMA work from an LDS stage
  auto compute_tile = [&](int t, int stage) {
    bool cache;
    int key0, nvalid;
    tile_info(t, cache, key0, nvalid);
    const bool scaled = I8 && cache;
    const unsigned char* Ks = lds + stage * C::STAGE;
    const unsigned char* Vs = Ks + C::KT_BYTES;
    const float* sc = reinterpret_cast<const float*>(Vs + C::VT_BYTES);

    f32x4 s[QB][BC / 32][2];
#pragma unroll
    for (int g = 0; g < BC / 32; ++g) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int row = 32 * g + 8 * (i16 >> 2) + 4 * bb + (i16 & 3);
        const int sw = swz_k<D>(row);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][g][bb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + row * D * 2 + (((4 * kk + G) ^ sw) * 16));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][g][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][kk], s[qb][g][bb], 0, 0, 0);
        }
      }
    }

    if (scaled) {
#pragma unroll
      for (int g = 0; g < BC / 32; ++g)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const f32x4 ksv = *reinterpret_cast<const f32x4*>(sc + 32 * g + 8 * G + 4 * bb);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][g][bb] *= ksv;
        }
    }
    if (nvalid < BC) {
#pragma unroll
      for (int g = 0; g < BC / 32; ++g)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (32 * g + 8 * G + 4 * bb + r >= nvalid)
#pragma unroll
              for (int qb = 0; qb < QB; ++qb) s[qb][g][bb][r] = -INFINITY;
    }

    bf16x8 pf[QB][BC / 32];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int g = 0; g < BC / 32; ++g)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[qb][g][bb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mt = mx * a.c2;
      if (__any(mt > m_ref[qb] + kTau)) {
        const float mn = fmaxf(m_ref[qb], mt);
        const float alpha = __builtin_amdgcn_exp2f(m_ref[qb] - mn);
        l_sum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) o[qb][db] *= alpha;
        m_ref[qb] = mn;
      }
      const float nm = -m_ref[qb];
#pragma unroll
      for (int g = 0; g < BC / 32; ++g) {
        float p[8];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(s[qb][g][bb][r], a.c2, nm));
            l_sum[qb] += e;
            p[4 * bb + r] = e;
          }
        if (scaled) {
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(sc + BC + 32 * g + 8 * G);
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(sc + BC + 32 * g + 8 * G + 4);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[r] *= v0[r];
            p[4 + r] *= v1[r];
          }
        }
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
        pf[qb][g] = __builtin_bit_cast(bf16x8, pk);
      }
    }

#pragma unroll
    for (int g = 0; g < BC / 32; ++g) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const int d = 16 * db + i16;
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vs + d * BC * 2 + (((4 * g + G) ^ swz_v<BC>(d)) * 16));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb][g], o[qb][db], 0, 0, 0);
      }
    }
  };

  // ---- main loop: double-buffered LDS, next tile's global loads in flight
  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(t_begin, 0);
    __syncthreads();
    for (int t = t_begin; t < t_end; ++t) {
      const int stage = (t - t_begin) & 1;
      const bool more = t + 1 < t_end;
      if (more) load_tile(t + 1);
      compute_tile(t, stage);
      if (more) store_tile(t + 1, stage ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l = l_sum[qb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = 1.0f / l;
    const int row = qt * C::BR + (wave * QB + qb) * 16 + i16;
    if (row >= a.n_q) continue;
    const float lse = (m_ref[qb] + log2f(l)) * kLn2;
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

// ---- current segment's V -> V^T [H][D][pitch] (zero beyond n)
template <int D>
__global__ __launch_bounds__(256) void v_transpose_kernel(const uint16_t* __restrict__ v, int64_t ld, int n,
                                                          uint16_t* __restrict__ vt, int pitch) {
  constexpr int TT = 64;                      // tokens per block
  constexpr int RP = TT + 8;                  // padded LDS row (elements)
  __shared__ __align__(16) uint16_t tile[D * RP];
  const int h = blockIdx.y, t0 = blockIdx.x * TT;
  for (int c = threadIdx.x; c < TT * D / 8; c += 256) {
    const int t = c / (D / 8), cc = c % (D / 8);
    u32x4 x = {0, 0, 0, 0};
    if (t0 + t < n) x = *reinterpret_cast<const u32x4*>(v + (int64_t)(t0 + t) * ld + (int64_t)h * D + cc * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[(cc * 8 + 2 * e) * RP + t] = static_cast<uint16_t>(x[e] & 0xffffu);
      tile[(cc * 8 + 2 * e + 1) * RP + t] = static_cast<uint16_t>(x[e] >> 16);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < D * (TT / 8); i += 256) {
    const int d = i / (TT / 8), g = i % (TT / 8);
    *reinterpret_cast<u32x4*>(vt + ((int64_t)h * D + d) * pitch + t0 + 8 * g) =
        *reinterpret_cast<const u32x4*>(&tile[d * RP + 8 * g]);
  }
}

// ---------------------------------------------------------------- host side
struct Plan {
  int bc;
  int br;
  int n_cached, n_q, pitch_cur, tiles_c, tiles_total, n_qtiles, splits;
  size_t off_part_o, off_part_lse, bytes;
};

// Tile shape per head dim: keys per tile, waves per block, 16-query blocks per wave.
template <int D> struct Shape;
template <> struct Shape<128> { static constexpr int BC = 64, NW = 8, QB = 2; };
template <> struct Shape<64> { static constexpr int BC = 64, NW = 4, QB = 2; };
constexpr int kCUs = 256;
static int block_queries(int D) { return D == 128 ? Shape<128>::NW * Shape<128>::QB * 16 : Shape<64>::NW * Shape<64>::QB * 16; }
static int key_tile(int D) { return D == 128 ? Shape<128>::BC : Shape<64>::BC; }

static int auto_splits(int n_qtiles, int H, int tiles_total) {
  const int blocks = n_qtiles * H;
  if (blocks >= 2 * kCUs) return 1;
  int s = (2 * kCUs + blocks - 1) / blocks;
  const int max_s = tiles_total / 16;   // at least 16 key tiles per split
  if (s > max_s) s = max_s;
  return s < 1 ? 1 : s;
}

static bool make_plan(int n_video, int n_text, int64_t n_cached, int H, int D, int n_splits, Plan& p) {
  if (n_video < 0 || n_text < 0 || (int64_t)n_video + n_text < 1 || H < 1 || (D != 64 && D != 128) ||
      n_cached < 0 || n_splits < 0)
    return false;
  if ((int64_t)n_video + n_text > (1 << 26) || n_cached > ((int64_t)1 << 30)) return false;
  p.bc = key_tile(D);
  p.br = block_queries(D);
  p.n_cached = (int)n_cached;
  p.n_q = n_video + n_text;
  p.pitch_cur = (int)round_up(p.n_q, kTokenAlign);
  p.tiles_c = (int)((n_cached + p.bc - 1) / p.bc);
  p.tiles_total = p.tiles_c + (p.n_q + p.bc - 1) / p.bc;
  p.n_qtiles = (p.n_q + p.br - 1) / p.br;
  int s = n_splits ? n_splits : auto_splits(p.n_qtiles, H, p.tiles_total);
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

template <int D, bool I8>
static void launch_attn(const AttnArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(8 * a.per_xcd));
  using S = Shape<D>;
  hipLaunchKernelGGL((attn_kernel<D, S::QB, S::NW, S::BC, I8>), grid, dim3(S::NW * 64), 0, st, a);
}

}  // namespace nomas

using namespace nomas;

extern "C" size_t nomas_segment_attention_workspace_bytes(int32_t n_video, int32_t n_text, int64_t n_cached,
                                                          int32_t n_heads, int32_t head_dim, int32_t n_splits) {
  Plan p;
  if (!make_plan(n_video, n_text, n_cached, n_heads, head_dim, n_splits, p)) return 0;
  return p.bytes;
}

extern "C" int32_t nomas_segment_attention_splits(int32_t n_video, int32_t n_text, int64_t n_cached,
                                                  int32_t n_heads, int32_t head_dim, int32_t n_splits) {
  Plan p;
  if (!make_plan(n_video, n_text, n_cached, n_heads, head_dim, n_splits, p)) return -1;
  return p.splits;
}

extern "C" int32_t nomas_segment_attention(const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                                           int64_t ld_qkv, int32_t n_video, int32_t n_text, const nomas_kvcache* c,
                                           uint16_t* out, int64_t ld_out, float* lse, float softmax_scale,
                                           int32_t n_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (int32_t e = validate_cache(c, "segment_attention")) return e;
  const int H = c->n_heads, D = c->head_dim;
  if (!q || !k_cur || !v_cur || !out) return fail(NOMAS_E_INVALID, "segment_attention: q, k_cur, v_cur, out must be non-NULL");
  if (!aligned16(q) || !aligned16(k_cur) || !aligned16(v_cur) || !aligned16(out))
    return fail(NOMAS_E_INVALID, "segment_attention: q, k_cur, v_cur, out must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return fail(NOMAS_E_INVALID, "segment_attention: lse must be 4-byte aligned");
  if (ld_qkv < (int64_t)H * D || ld_qkv % 8 || ld_out < (int64_t)H * D || ld_out % 8)
    return fail(NOMAS_E_INVALID, "segment_attention: ld_qkv and ld_out must be >= n_heads*head_dim and multiples of 8");
  if (n_video < 0 || n_text < 0 || (int64_t)n_video + n_text < 1)
    return fail(NOMAS_E_INVALID, "segment_attention: need n_video >= 0, n_text >= 0, n_video + n_text >= 1");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(NOMAS_E_INVALID, "segment_attention: softmax_scale must be finite and > 0");
  if (n_splits < 0) return fail(NOMAS_E_INVALID, "segment_attention: n_splits must be >= 0");
  const int64_t n_cached = nomas_kvcache_valid_frames(c) * c->tokens_per_frame;
  Plan p;
  if (!make_plan(n_video, n_text, n_cached, H, D, n_splits, p))
    return fail(NOMAS_E_INVALID, "segment_attention: sizes out of range");
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(NOMAS_E_WORKSPACE, "segment_attention: workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < p.bytes)
    return fail(NOMAS_E_WORKSPACE, "segment_attention: workspace of %zu bytes, need %zu", workspace_bytes, p.bytes);

  const hipStream_t st = as_stream(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  uint16_t* vt = reinterpret_cast<uint16_t*>(ws);
  {
    const dim3 grid((unsigned)(p.pitch_cur / 64), (unsigned)H);
    if (D == 128) hipLaunchKernelGGL(v_transpose_kernel<128>, grid, dim3(256), 0, st, v_cur, ld_qkv, p.n_q, vt, p.pitch_cur);
    else hipLaunchKernelGGL(v_transpose_kernel<64>, grid, dim3(256), 0, st, v_cur, ld_qkv, p.n_q, vt, p.pitch_cur);
    if (int32_t e = check_launch("segment_attention (v transpose)")) return e;
  }

  AttnArgs a;
  a.q = q;
  a.kcur = k_cur;
  a.ld_qkv = ld_qkv;
  a.vtcur = vt;
  a.pitch_cur = p.pitch_cur;
  a.kc = c->k;
  a.vc = c->v;
  a.ks = c->k_scale;
  a.vs = c->v_scale;
  a.pitch_c = c->token_pitch;
  a.n_cached = p.n_cached;
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
  const bool i8 = c->kv_dtype == NOMAS_KV_INT8;
  if (D == 128) {
    if (i8) launch_attn<128, true>(a, st);
    else launch_attn<128, false>(a, st);
  } else {
    if (i8) launch_attn<64, true>(a, st);
    else launch_attn<64, false>(a, st);
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
