// Append a segment's K/V frames to the ring-buffer window, quantising to INT8
// when the cache is INT8.
//
// Pages: the DiT carries earlier latents' keys and values in a cache
// ("Hy-Nomas: Was Tencent mit seinem frei formbaren interaktiven Weltmodell
// tatsaechlich macht", orcarouter.ai, section "Die Schleife"); the single-GPU
// preset keeps only the last 18 latent frames on the GPU and stores KV in INT8,
// computing in BF16 ("Hy-Nomas auf einer RTX 4090", inferencekey.com, section
// "Das Single-GPU-Preset"; blog.authon.dev config excerpt). Scale granularity and
// rounding (per token and head, absmax/127, nearest-even) are this library's
// reading.
//
// Ring arithmetic (host): frame f of the session lives in slot f mod capacity.
// An append of n frames writes only its last min(n, capacity) frames, so no two
// tokens of one launch target the same slot and the launch is race-free.
//
// INT8 kernel (kv_append_i8_kernel): one wave = a run of tokens of one head; codes
// from a reciprocal product with an exact test that sends the rare codes near a
// rounding boundary to the IEEE quotient; V transposed in registers. The BF16
// cache has a copy kernel of its own (kv_append_bf16_kernel). Both are described
// where they are defined.
#include "nomas_common.hpp"

namespace nomas {

struct AppendArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t ld;
  int rows;            // token rows written by this launch
  int tpf;
  int cap;
  int base_slot;       // slot of the first written frame
  int pitch;
  int n_heads;
  void* kc;
  void* vc;
  float* ks;
  float* vs;
};

// head h exists and slot tokens [s, s + n) lie inside the ring's capacity * tpf
// rows (NOMAS_IN_BOUNDS)
__device__ __forceinline__ bool slots_in_ring(const AppendArgs& a, int h, int s, int n) {
  return h >= 0 && h < a.n_heads && s >= 0 && s + n <= a.cap * a.tpf;
}

__device__ __forceinline__ int slot_token(const AppendArgs& a, int r) {
  const int fi = r / a.tpf;
  int slot = a.base_slot + fi;
  if (slot >= a.cap) slot -= a.cap;
  return slot * a.tpf + (r - fi * a.tpf);
}

// max |x| over the 8 bf16 of a 16-byte chunk (on the bit patterns: for values
// >= 0 the order of the patterns is the order of the values), as a float
__device__ __forceinline__ float absmax8(const u32x4 w) {
  typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;
  // (each element copied to a scalar before its bit cast: a bit cast of a
  // vector element reads element 0 with this compiler)
  const unsigned w0 = w[0] & 0x7fff7fffu;
  u16x2 m = __builtin_bit_cast(u16x2, w0);
#pragma unroll
  for (int e = 1; e < 4; ++e) {
    const unsigned we = w[e] & 0x7fff7fffu;
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, we));
  }
  const unsigned mx = m[0] > m[1] ? m[0] : m[1];
  return __uint_as_float(mx << 16);
}

// orders a wave's LDS writes before its later LDS reads of other lanes' data:
// the compiler may not move memory operations across the fences, and the LDS
// executes one wave's operations in issue order
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// the 8 codes (as C + code floats, see code_fast / code_exact in
// nomas_common.hpp) of one token's 16-byte chunk
__device__ __forceinline__ bool codes8(const u32x4 w, float s, float r, float (&f)[8]) {
  bool ok = true;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = code_fast((e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]), r, ok);
  if (!ok) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = code_exact((e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]), s);
  }
  return ok;
}

// independent waves per block: the waves share nothing, and one per block
// measured fastest (21.6-21.7 us at the layer shape against 21.8 for two or
// four, 23.2 for eight and 23.4 for sixteen)
constexpr int kAppendWaves = 1;

// One wave = TW tokens x D channels of one head (D = 128: 32 tokens, D = 64:
// 64), a block of kAppendWaves independent waves. Lane = cc + CL*tg: channels
// 8cc..8cc+7 of the run's tokens 8tg..8tg+7, so a lane loads 8 rows x 16 bytes
// of K and of V and each load instruction covers TG whole rows. A token's
// absmax forms inside the wave: the lanes put their chunk maxima into the
// wave's own LDS region, one lane per (K or V, token) reduces the CL chunk
// maxima of its token and forms the scale and its reciprocal, and every lane
// reads back those of its 8 tokens. A wave only reads what it wrote itself, so
// no block barrier holds one wave for another. K codes go out as 8-byte row
// pieces (the CL lanes of a token store its D bytes); V codes are transposed
// in registers (8 tokens x 8 channels), so the TG lanes of a channel store a
// TW-byte run of its slots.
// VEC8 (tokens per frame a multiple of 8): a lane's 8 tokens sit in 8
// consecutive slots; otherwise V^T goes out byte by byte.
template <int D, bool VEC8>
__global__ __launch_bounds__(64 * kAppendWaves) void kv_append_i8_kernel(AppendArgs a) {
  constexpr int CL = D / 8, TG = 64 / CL, TW = 8 * TG, NV = 2 * TW;   // NV: (K or V, token) pairs
  constexpr int RP = NV + 4;                          // padded row: chunk rows start 16 B apart in the banks
  __shared__ __align__(16) float red[kAppendWaves][CL * RP];   // per wave: chunk maxima [chunk][kv * TW + token]
  __shared__ __align__(16) float2 sr[kAppendWaves][NV];        // per wave: (scale, reciprocal) [kv * TW + token]
  const int h = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cc = lane % CL, tg = lane / CL;
  const int tok0 = (blockIdx.x * kAppendWaves + wave) * TW;
  if (tok0 >= a.rows) return;                        // the whole wave
  const int r0 = tok0 + 8 * tg;                      // the lane's first row
  const int c0 = 8 * cc;                             // and first channel

  u32x4 kx[8], vx[8];
  if constexpr (VEC8) {
    // a lane's 8 rows are all live or all past the end (rows is a multiple of
    // 8); a lane past the end re-reads the last 8 rows and stores nothing. One
    // base per tensor, rows a scalar stride apart.
    const int64_t src = (int64_t)min(r0, a.rows - 8) * a.ld + (int64_t)h * D + c0;
    const uint16_t* kp = a.k_new + src;
    const uint16_t* vp = a.v_new + src;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kx[i] = *reinterpret_cast<const u32x4*>(kp + i * a.ld);
      vx[i] = *reinterpret_cast<const u32x4*>(vp + i * a.ld);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {   // rows past the end re-read the last row and are not stored
      const int64_t src = (int64_t)min(r0 + i, a.rows - 1) * a.ld + (int64_t)h * D + c0;
      kx[i] = *reinterpret_cast<const u32x4*>(a.k_new + src);
      vx[i] = *reinterpret_cast<const u32x4*>(a.v_new + src);
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // all 16 loads in flight before the first wait

  // ---- absmax of each token: chunk maxima -> LDS -> one lane per (K or V, token)
  float* rw = &red[wave][cc * RP + 8 * tg];
  *reinterpret_cast<f32x4*>(rw) = (f32x4){absmax8(kx[0]), absmax8(kx[1]), absmax8(kx[2]), absmax8(kx[3])};
  *reinterpret_cast<f32x4*>(rw + 4) = (f32x4){absmax8(kx[4]), absmax8(kx[5]), absmax8(kx[6]), absmax8(kx[7])};
  *reinterpret_cast<f32x4*>(rw + TW) = (f32x4){absmax8(vx[0]), absmax8(vx[1]), absmax8(vx[2]), absmax8(vx[3])};
  *reinterpret_cast<f32x4*>(rw + TW + 4) = (f32x4){absmax8(vx[4]), absmax8(vx[5]), absmax8(vx[6]), absmax8(vx[7])};
  wave_lds_sync();
#pragma unroll
  for (int p = lane; p < NV; p += 64) {
    float m = red[wave][p];
#pragma unroll
    for (int j = 1; j < CL; ++j) m = fmaxf(m, red[wave][j * RP + p]);
    const float sc = m / 127.0f;
    sr[wave][p] = make_float2(sc, code_recip(sc));
    const int t = tok0 + p % TW;
    if (t < a.rows) {
      const int st = slot_token(a, t);
      if (NOMAS_IN_BOUNDS(slots_in_ring(a, h, st, 1))) (p >= TW ? a.vs : a.ks)[(int64_t)h * a.pitch + st] = sc;
    }
  }
  wave_lds_sync();
  if (r0 >= a.rows) return;

  int slot[8];
  if constexpr (VEC8) {   // rows is a multiple of tpf, so all 8 rows are live
    const int s0 = slot_token(a, r0);
#pragma unroll
    for (int i = 0; i < 8; ++i) slot[i] = s0 + i;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) slot[i] = r0 + i < a.rows ? slot_token(a, r0 + i) : -1;
  }

  // ---- K: codes token by token, 8-byte row pieces
  f32x4 q4[4];   // (scale, reciprocal) of the lane's 8 tokens, K then V
#pragma unroll
  for (int j = 0; j < 4; ++j) q4[j] = *reinterpret_cast<const f32x4*>(&sr[wave][8 * tg + 2 * j]);
  int8_t* kc = static_cast<int8_t*>(a.kc) + (int64_t)h * a.pitch * D + c0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float f[8];
    codes8(kx[i], q4[i >> 1][2 * (i & 1)], q4[i >> 1][2 * (i & 1) + 1], f);
    if ((VEC8 || slot[i] >= 0) && NOMAS_IN_BOUNDS(slots_in_ring(a, h, slot[i], 1)))
      *reinterpret_cast<uint2*>(kc + (int64_t)slot[i] * D) = make_uint2(pack4(f[0], f[1], f[2], f[3]),
                                                                       pack4(f[4], f[5], f[6], f[7]));
  }

  // ---- V: codes of 8 tokens x 8 channels, transposed to channel rows
  float fv[8][8];
#pragma unroll
  for (int j = 0; j < 4; ++j) q4[j] = *reinterpret_cast<const f32x4*>(&sr[wave][TW + 8 * tg + 2 * j]);
#pragma unroll
  for (int i = 0; i < 8; ++i) codes8(vx[i], q4[i >> 1][2 * (i & 1)], q4[i >> 1][2 * (i & 1) + 1], fv[i]);
  int8_t* vc = static_cast<int8_t*>(a.vc) + ((int64_t)h * D + c0) * a.pitch;
  if constexpr (VEC8) {
    if (!NOMAS_IN_BOUNDS(slots_in_ring(a, h, slot[0], 8))) return;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint2*>(vc + (int64_t)e * a.pitch + slot[0]) =
          make_uint2(pack4(fv[0][e], fv[1][e], fv[2][e], fv[3][e]), pack4(fv[4][e], fv[5][e], fv[6][e], fv[7][e]));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (slot[i] < 0) break;
      if (!NOMAS_IN_BOUNDS(slots_in_ring(a, h, slot[i], 1))) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vc[(int64_t)e * a.pitch + slot[i]] = static_cast<int8_t>(__float_as_uint(fv[i][e]) & 0xffu);
    }
  }
}

// BF16 cache: a plain copy, K rows in place and V transposed in registers. A
// block is 128 rows x D channels of one head, one wave per 64 x 64 quarter; a
// lane moves 8 rows x 8 channels: eight 16-byte loads from each of K and V,
// eight 16-byte K row stores and, after an 8 x 8 transpose, eight 16-byte V^T
// stores (lane = 8 * channel chunk + row group, so every load and store
// instruction covers 8 rows of 128 contiguous bytes). VEC8 (tokens per frame a
// multiple of 8): a lane's 8 rows share a frame and land in 8 consecutive,
// 16-byte aligned slots; otherwise each row finds its own slot.
template <int D, bool VEC8>
__global__ __launch_bounds__(2 * D) void kv_append_bf16_kernel(AppendArgs a) {
  const int h = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = blockIdx.x * 128 + (wave & 1) * 64 + 8 * (lane & 7);   // the lane's first row
  const int d0 = (wave >> 1) * 64 + 8 * (lane >> 3);                     // and first channel
  if (r0 >= a.rows) return;
  u32x4 kx[8], vx[8];
  if constexpr (VEC8) {   // rows is a multiple of 8: all 8 rows are live; one base, a scalar stride
    const int64_t src = (int64_t)r0 * a.ld + (int64_t)h * D + d0;
    const uint16_t* kp = a.k_new + src;
    const uint16_t* vp = a.v_new + src;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kx[i] = *reinterpret_cast<const u32x4*>(kp + i * a.ld);
      vx[i] = *reinterpret_cast<const u32x4*>(vp + i * a.ld);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {   // rows past the end re-read the last row and are not stored
      const int64_t src = (int64_t)min(r0 + i, a.rows - 1) * a.ld + (int64_t)h * D + d0;
      kx[i] = *reinterpret_cast<const u32x4*>(a.k_new + src);
      vx[i] = *reinterpret_cast<const u32x4*>(a.v_new + src);
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // all 16 loads in flight before the first store
  uint16_t* kc = static_cast<uint16_t*>(a.kc);
  uint16_t* vc = static_cast<uint16_t*>(a.vc);
  if constexpr (VEC8) {   // rows is a multiple of tpf, so all 8 rows are live
    const int s0 = slot_token(a, r0);
    if (!NOMAS_IN_BOUNDS(slots_in_ring(a, h, s0, 8))) return;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(kc + ((int64_t)h * a.pitch + s0 + i) * D + d0) = kx[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t x = vx[2 * k][j >> 1], y = vx[2 * k + 1][j >> 1];
        o[k] = (j & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
      }
      *reinterpret_cast<u32x4*>(vc + ((int64_t)h * D + d0 + j) * a.pitch + s0) = o;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (r0 + i >= a.rows) break;
      const int st = slot_token(a, r0 + i);
      if (!NOMAS_IN_BOUNDS(slots_in_ring(a, h, st, 1))) continue;
      *reinterpret_cast<u32x4*>(kc + ((int64_t)h * a.pitch + st) * D + d0) = kx[i];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        vc[((int64_t)h * D + d0 + j) * a.pitch + st] = static_cast<uint16_t>((j & 1) ? vx[i][j >> 1] >> 16 : vx[i][j >> 1] & 0xffffu);
    }
  }
}

template <int D>
static void launch_append_bf16(const AppendArgs& a, bool vec8, hipStream_t s) {
  const dim3 grid((unsigned)((a.rows + 127) / 128), (unsigned)a.n_heads);
  if (vec8)
    hipLaunchKernelGGL((kv_append_bf16_kernel<D, true>), grid, dim3(2 * D), 0, s, a);
  else
    hipLaunchKernelGGL((kv_append_bf16_kernel<D, false>), grid, dim3(2 * D), 0, s, a);
}

template <int D>
static void launch_append_int8(const AppendArgs& a, bool vec8, hipStream_t s) {
  constexpr int TB = kAppendWaves * 8 * (64 / (D / 8));   // tokens per block: waves of 8 * (64 / (D/8))
  const dim3 grid((unsigned)((a.rows + TB - 1) / TB), (unsigned)a.n_heads);
  if (vec8)
    hipLaunchKernelGGL((kv_append_i8_kernel<D, true>), grid, dim3(64 * kAppendWaves), 0, s, a);
  else
    hipLaunchKernelGGL((kv_append_i8_kernel<D, false>), grid, dim3(64 * kAppendWaves), 0, s, a);
}

int32_t validate_cache(const nomas_kvcache* c, const char* who) {
  if (!c) return fail(NOMAS_E_INVALID, "%s: cache descriptor is NULL", who);
  if (c->n_heads < 1 || (c->head_dim != 64 && c->head_dim != 128) || c->tokens_per_frame < 1 ||
      c->capacity_frames < 1 || (c->kv_dtype != NOMAS_KV_BF16 && c->kv_dtype != NOMAS_KV_INT8))
    return fail(NOMAS_E_INVALID, "%s: cache descriptor is not initialised (use nomas_kvcache_init)", who);
  if (c->token_pitch != nomas_kvcache_token_pitch(c->tokens_per_frame, c->capacity_frames))
    return fail(NOMAS_E_INVALID, "%s: cache token_pitch does not match its sizes", who);
  if ((int64_t)c->token_pitch * c->head_dim * (c->kv_dtype == NOMAS_KV_INT8 ? 1 : 2) > INT32_MAX)
    return fail(NOMAS_E_INVALID, "%s: one head's cache slice must stay below 2 GiB", who);
  if (!c->k || !c->v || !aligned16(c->k) || !aligned16(c->v))
    return fail(NOMAS_E_INVALID, "%s: cache buffers must be non-NULL and 16-byte aligned", who);
  if (c->kv_dtype == NOMAS_KV_INT8 && (!c->k_scale || !c->v_scale))
    return fail(NOMAS_E_INVALID, "%s: INT8 cache without scale buffers", who);
  if (c->frames_written < 0) return fail(NOMAS_E_INVALID, "%s: negative frames_written", who);
  return NOMAS_OK;
}

}  // namespace nomas

namespace nomas {
int64_t check_failures_append(int reset) { return source_check_failures(reset); }
}  // namespace nomas

using namespace nomas;

extern "C" int32_t nomas_kvcache_append(nomas_kvcache* c, const uint16_t* k_new, const uint16_t* v_new, int64_t ld,
                                        int32_t n_frames, void* stream) {
  if (int32_t e = validate_cache(c, "kvcache_append")) return e;
  if (!k_new || !v_new) return fail(NOMAS_E_INVALID, "kvcache_append: k_new and v_new must be non-NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(NOMAS_E_INVALID, "kvcache_append: k_new and v_new must be 16-byte aligned");
  if (n_frames < 1) return fail(NOMAS_E_INVALID, "kvcache_append: n_frames must be >= 1 (got %d)", n_frames);
  const int H = c->n_heads, D = c->head_dim, tpf = c->tokens_per_frame, cap = c->capacity_frames;
  if (ld < (int64_t)H * D || ld % 8)
    return fail(NOMAS_E_INVALID, "kvcache_append: ld must be >= n_heads*head_dim and a multiple of 8");
  if ((int64_t)n_frames * tpf > INT32_MAX / 2) return fail(NOMAS_E_INVALID, "kvcache_append: too many rows");

  const int skip = n_frames > cap ? n_frames - cap : 0;    // frames overwritten within this append
  AppendArgs a;
  a.k_new = k_new + (int64_t)skip * tpf * ld;
  a.v_new = v_new + (int64_t)skip * tpf * ld;
  a.ld = ld;
  a.rows = (n_frames - skip) * tpf;
  a.tpf = tpf;
  a.cap = cap;
  a.base_slot = (int)((c->frames_written + skip) % cap);
  a.pitch = c->token_pitch;
  a.n_heads = H;
  a.kc = c->k;
  a.vc = c->v;
  a.ks = c->k_scale;
  a.vs = c->v_scale;
  const bool vec8 = tpf % 8 == 0;
  const hipStream_t s = as_stream(stream);
  const bool int8 = c->kv_dtype == NOMAS_KV_INT8;
  if (D == 128) {
    if (int8) launch_append_int8<128>(a, vec8, s);
    else launch_append_bf16<128>(a, vec8, s);
  } else {
    if (int8) launch_append_int8<64>(a, vec8, s);
    else launch_append_bf16<64>(a, vec8, s);
  }
  if (int32_t e = check_launch("kvcache_append")) return e;
  c->frames_written += n_frames;
  return ok();
}
