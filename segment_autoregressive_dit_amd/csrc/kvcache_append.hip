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
// INT8 kernel: one block = 64 tokens of one head. Each token's head_dim values
// are spread over head_dim/8 consecutive lanes (16-byte chunks), which reduce
// the absmax with lane shuffles. K rows are written token-major; V is written
// transposed ([head][dim][token]) through an LDS tile so that each wave stores
// whole 64-token runs of one dim. The BF16 cache has a copy kernel of its own
// (kv_append_bf16_kernel, below).
#include "nomas_common.hpp"

namespace nomas {

constexpr int kAppTok = 64;
constexpr int kAppThreads = 256;

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

__device__ __forceinline__ int slot_token(const AppendArgs& a, int r) {
  const int fi = r / a.tpf;
  int slot = a.base_slot + fi;
  if (slot >= a.cap) slot -= a.cap;
  return slot * a.tpf + (r - fi * a.tpf);
}

// Correctly rounded float32 quotient; the build keeps IEEE division (no fast-math).
__device__ __forceinline__ float div_rn(float x, float y) { return x / y; }

template <int D, bool VEC4>
__global__ __launch_bounds__(kAppThreads) void kv_append_kernel(AppendArgs a) {
  constexpr int CPR = D / 8;                       // chunks per token row
  constexpr int CHUNKS = kAppTok * CPR;
  constexpr int PER_THREAD = CHUNKS / kAppThreads;
  constexpr int ROWB = kAppTok + 16;               // padded LDS row of the V^T code tile (bytes)
  __shared__ __align__(16) unsigned char vt[D * ROWB];
  __shared__ int slots[kAppTok];

  const int h = blockIdx.y;
  const int tok0 = blockIdx.x * kAppTok;
  const int tid = threadIdx.x;
  if (tid < kAppTok) slots[tid] = tok0 + tid < a.rows ? slot_token(a, tok0 + tid) : 0;
  __syncthreads();

#pragma unroll
  for (int it = 0; it < PER_THREAD; ++it) {
    const int c = tid + it * kAppThreads;
    const int t = c / CPR, cc = c - t * CPR;       // lanes of one token are consecutive
    const int r = tok0 + t;
    const bool live = r < a.rows;
    const int64_t src = (int64_t)r * a.ld + (int64_t)h * D + cc * 8;
    u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
    if (live) {
      kx = *reinterpret_cast<const u32x4*>(a.k_new + src);
      vx = *reinterpret_cast<const u32x4*>(a.v_new + src);
    }
    const int st = slots[t];
    const int64_t krow = ((int64_t)h * a.pitch + st) * D + cc * 8;
    {
      float kf[8], vf[8];
      float km = 0.f, vm = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = bf16_lo(kx[e]);
        kf[2 * e + 1] = bf16_hi(kx[e]);
        vf[2 * e] = bf16_lo(vx[e]);
        vf[2 * e + 1] = bf16_hi(vx[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        km = fmaxf(km, fabsf(kf[e]));
        vm = fmaxf(vm, fabsf(vf[e]));
      }
#pragma unroll
      for (int m = CPR / 2; m >= 1; m >>= 1) {
        km = fmaxf(km, __shfl_xor(km, m, CPR));
        vm = fmaxf(vm, __shfl_xor(vm, m, CPR));
      }
      const float ksc = div_rn(km, 127.f), vsc = div_rn(vm, 127.f);
      unsigned kq[2] = {0, 0}, vq[2] = {0, 0};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kr = km > 0.f ? fminf(fmaxf(rintf(div_rn(kf[e], ksc)), -127.f), 127.f) : 0.f;
        const float vr = vm > 0.f ? fminf(fmaxf(rintf(div_rn(vf[e], vsc)), -127.f), 127.f) : 0.f;
        kq[e / 4] |= (static_cast<unsigned>(static_cast<int>(kr)) & 0xffu) << (8 * (e % 4));
        vq[e / 4] |= (static_cast<unsigned>(static_cast<int>(vr)) & 0xffu) << (8 * (e % 4));
        vt[(cc * 8 + e) * ROWB + t] = static_cast<unsigned char>(static_cast<int>(vr) & 0xff);
      }
      if (live) {
        *reinterpret_cast<uint2*>(static_cast<int8_t*>(a.kc) + krow) = make_uint2(kq[0], kq[1]);
        if (cc == 0) {
          a.ks[(int64_t)h * a.pitch + st] = ksc;
          a.vs[(int64_t)h * a.pitch + st] = vsc;
        }
      }
    }
  }
  __syncthreads();

  // transposed V store: lanes run along tokens (4 per lane), waves along dims
  const int n_live = min(kAppTok, a.rows - tok0);
  constexpr int GROUPS = kAppTok / 4;
  for (int i = tid; i < D * GROUPS; i += kAppThreads) {
    const int d = i / GROUPS, g = i - d * GROUPS;
    const int t = 4 * g;
    if (t >= n_live) continue;
    const int64_t vrow = ((int64_t)h * D + d) * a.pitch;
    if (VEC4) {   // 4 tokens of one frame, contiguous and aligned slots
      *reinterpret_cast<unsigned*>(static_cast<int8_t*>(a.vc) + vrow + slots[t]) =
          *reinterpret_cast<const unsigned*>(&vt[d * ROWB + t]);
    } else {
      for (int e = 0; e < 4 && t + e < n_live; ++e)
        static_cast<int8_t*>(a.vc)[vrow + slots[t + e]] = static_cast<int8_t>(vt[d * ROWB + t + e]);
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
#pragma unroll
  for (int i = 0; i < 8; ++i) {   // rows past the end re-read the last row and are not stored
    const int64_t src = (int64_t)min(r0 + i, a.rows - 1) * a.ld + (int64_t)h * D + d0;
    kx[i] = *reinterpret_cast<const u32x4*>(a.k_new + src);
    vx[i] = *reinterpret_cast<const u32x4*>(a.v_new + src);
  }
  uint16_t* kc = static_cast<uint16_t*>(a.kc);
  uint16_t* vc = static_cast<uint16_t*>(a.vc);
  if constexpr (VEC8) {   // rows is a multiple of tpf, so all 8 rows are live
    const int s0 = slot_token(a, r0);
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
static void launch_append_int8(const AppendArgs& a, bool vec4, hipStream_t s) {
  const dim3 grid((unsigned)((a.rows + kAppTok - 1) / kAppTok), (unsigned)a.n_heads);
  if (vec4)
    hipLaunchKernelGGL((kv_append_kernel<D, true>), grid, dim3(kAppThreads), 0, s, a);
  else
    hipLaunchKernelGGL((kv_append_kernel<D, false>), grid, dim3(kAppThreads), 0, s, a);
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
  const bool vec4 = tpf % 4 == 0;
  const hipStream_t s = as_stream(stream);
  const bool int8 = c->kv_dtype == NOMAS_KV_INT8;
  if (D == 128) {
    if (int8) launch_append_int8<128>(a, vec4, s);
    else launch_append_bf16<128>(a, tpf % 8 == 0, s);
  } else {
    if (int8) launch_append_int8<64>(a, vec4, s);
    else launch_append_bf16<64>(a, tpf % 8 == 0, s);
  }
  if (int32_t e = check_launch("kvcache_append")) return e;
  c->frames_written += n_frames;
  return ok();
}
