// Host side of libnomas: error state, version, and the cache descriptor helpers.
// The ring-buffer arithmetic of the window (which frames are retained and where)
// lives in kvcache_append.hip next to the kernel that writes it.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "nomas_common.hpp"

namespace nomas {

static thread_local char g_err[512];

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int32_t ok() {
  g_err[0] = '\0';
  return NOMAS_OK;
}

int32_t check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(NOMAS_E_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// failure counters of the checking build, one per source file with checks
int64_t check_failures_append(int reset);
int64_t check_failures_qkv(int reset);
int64_t check_failures_attention(int reset);
int64_t check_failures_sparse(int reset);
int64_t check_failures_rope(int reset);

}  // namespace nomas

using namespace nomas;

extern "C" {

int32_t nomas_version(void) { return (0 << 16) | 1; }

int64_t nomas_device_check_failures(int32_t reset) {
  const int64_t parts[5] = {check_failures_append(reset), check_failures_qkv(reset), check_failures_attention(reset),
                            check_failures_sparse(reset), check_failures_rope(reset)};
  int64_t total = 0;
  for (int64_t p : parts) {
    if (p < 0) return -1;
    total += p;
  }
  return total;
}

const char* nomas_last_error(void) { return g_err; }

int64_t nomas_kvcache_token_pitch(int32_t tokens_per_frame, int32_t capacity_frames) {
  if (tokens_per_frame < 1 || capacity_frames < 1) return -1;
  int64_t n = (int64_t)tokens_per_frame * capacity_frames;
  int64_t p = round_up(n, kTokenAlign);
  if (p > INT32_MAX) return -1;
  return p;
}

size_t nomas_kvcache_bytes(int32_t n_heads, int32_t head_dim, int32_t tokens_per_frame,
                           int32_t capacity_frames, int32_t kv_dtype, int32_t which) {
  if (n_heads < 1 || (head_dim != 64 && head_dim != 128)) return 0;
  if (kv_dtype != NOMAS_KV_BF16 && kv_dtype != NOMAS_KV_INT8) return 0;
  int64_t pitch = nomas_kvcache_token_pitch(tokens_per_frame, capacity_frames);
  if (pitch < 0) return 0;
  size_t elem = kv_dtype == NOMAS_KV_INT8 ? 1 : 2;
  switch (which) {
    case 0:
    case 1: return (size_t)n_heads * (size_t)pitch * (size_t)head_dim * elem;
    case 2: return kv_dtype == NOMAS_KV_INT8 ? (size_t)n_heads * (size_t)pitch * sizeof(float) : 0;
    default: return 0;
  }
}

int32_t nomas_kvcache_init(nomas_kvcache* c, int32_t n_heads, int32_t head_dim, int32_t tokens_per_frame,
                           int32_t capacity_frames, int32_t kv_dtype, void* k, void* v, float* k_scale,
                           float* v_scale) {
  if (!c) return fail(NOMAS_E_INVALID, "kvcache_init: descriptor is NULL");
  if (n_heads < 1) return fail(NOMAS_E_INVALID, "kvcache_init: n_heads must be >= 1 (got %d)", n_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(NOMAS_E_UNSUPPORTED, "kvcache_init: head_dim must be 64 or 128 (got %d)", head_dim);
  if (tokens_per_frame < 1 || capacity_frames < 1)
    return fail(NOMAS_E_INVALID, "kvcache_init: tokens_per_frame and capacity_frames must be >= 1");
  if (kv_dtype != NOMAS_KV_BF16 && kv_dtype != NOMAS_KV_INT8)
    return fail(NOMAS_E_INVALID, "kvcache_init: unknown kv_dtype %d", kv_dtype);
  int64_t pitch = nomas_kvcache_token_pitch(tokens_per_frame, capacity_frames);
  if (pitch < 0) return fail(NOMAS_E_INVALID, "kvcache_init: capacity too large");
  if ((int64_t)n_heads * head_dim * pitch > ((int64_t)1 << 40))
    return fail(NOMAS_E_INVALID, "kvcache_init: cache larger than 1 TiB");
  // the kernels address one head's K or V slice with 32-bit byte offsets
  if (pitch * head_dim * (kv_dtype == NOMAS_KV_INT8 ? 1 : 2) > INT32_MAX)
    return fail(NOMAS_E_INVALID, "kvcache_init: one head's cache slice (token_pitch*head_dim*element size) must stay below 2 GiB");
  if (!k || !v) return fail(NOMAS_E_INVALID, "kvcache_init: k and v buffers must be non-NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(NOMAS_E_INVALID, "kvcache_init: k and v must be 16-byte aligned");
  if (kv_dtype == NOMAS_KV_INT8) {
    if (!k_scale || !v_scale) return fail(NOMAS_E_INVALID, "kvcache_init: INT8 cache needs k_scale and v_scale");
    if (!aligned16(k_scale) || !aligned16(v_scale))
      return fail(NOMAS_E_INVALID, "kvcache_init: scales must be 16-byte aligned");
  } else if (k_scale || v_scale) {
    return fail(NOMAS_E_INVALID, "kvcache_init: BF16 cache takes no scales (pass NULL)");
  }
  c->n_heads = n_heads;
  c->head_dim = head_dim;
  c->tokens_per_frame = tokens_per_frame;
  c->capacity_frames = capacity_frames;
  c->kv_dtype = kv_dtype;
  c->token_pitch = (int32_t)pitch;
  c->k = k;
  c->v = v;
  c->k_scale = k_scale;
  c->v_scale = v_scale;
  c->frames_written = 0;
  return ok();
}

int64_t nomas_kvcache_valid_frames(const nomas_kvcache* c) {
  if (!c) return -1;
  return c->frames_written < c->capacity_frames ? c->frames_written : c->capacity_frames;
}

}  // extern "C"
