// Archive of frames leaving the ring cache: device -> pinned host records by the
// copy engines (hipMemcpy2DAsync, no compute units), and the way back.
//
// Pages: the model keeps a persistent, lifelong KV cache, with frames that leave
// the GPU window held in CPU memory ("Hy-Nomas", madebyagents.com, component
// "Persistent Lifelong KV Cache"; orcarouter.ai, section "Die Schleife").
//
// A frame's record is its slot contents in cache order: K [H][tpf][D], V^T
// [H][D][tpf] (int8 codes or bf16), then (INT8) the key scales [H][tpf] and the
// value scales [H][tpf], float32. Every copy is a 2-D strided copy: one row per
// head (K, scales) or per (head, channel) (V^T), the row pitch being the cache's
// token pitch.
#include "nomas_common.hpp"

namespace nomas {

int32_t validate_cache(const nomas_kvcache* c, const char* who);

struct RecordLayout {
  size_t k, v, sc, total;   // byte sizes of the parts
};

static RecordLayout record_layout(const nomas_kvcache* c) {
  const size_t es = c->kv_dtype == NOMAS_KV_INT8 ? 1 : 2;
  const size_t H = c->n_heads, D = c->head_dim, tpf = c->tokens_per_frame;
  RecordLayout r;
  r.k = H * tpf * D * es;
  r.v = H * D * tpf * es;
  r.sc = c->kv_dtype == NOMAS_KV_INT8 ? H * tpf * 4 : 0;
  r.total = r.k + r.v + 2 * r.sc;
  return r;
}

// slot `slot` of the cache <-> one record at `rec` (to_host: cache -> record)
static int32_t copy_slot(const nomas_kvcache* c, int slot, unsigned char* rec, bool to_host, hipStream_t st,
                         const char* who) {
  const RecordLayout L = record_layout(c);
  const size_t es = c->kv_dtype == NOMAS_KV_INT8 ? 1 : 2;
  const size_t H = c->n_heads, D = c->head_dim, tpf = c->tokens_per_frame, pitch = c->token_pitch;
  const size_t t0 = (size_t)slot * tpf;
  unsigned char* kc = static_cast<unsigned char*>(c->k) + t0 * D * es;
  unsigned char* vc = static_cast<unsigned char*>(c->v) + t0 * es;
  struct Part {
    unsigned char* dev;
    size_t dev_pitch, width, height;
    unsigned char* host;
  } parts[4] = {
      {kc, pitch * D * es, tpf * D * es, H, rec},
      {vc, pitch * es, tpf * es, H * D, rec + L.k},
      {reinterpret_cast<unsigned char*>(c->k_scale + t0), pitch * 4, tpf * 4, H, rec + L.k + L.v},
      {reinterpret_cast<unsigned char*>(c->v_scale + t0), pitch * 4, tpf * 4, H, rec + L.k + L.v + L.sc},
  };
  const int n_parts = c->kv_dtype == NOMAS_KV_INT8 ? 4 : 2;
  for (int i = 0; i < n_parts; ++i) {
    const Part& p = parts[i];
    const hipError_t e =
        to_host ? hipMemcpy2DAsync(p.host, p.width, p.dev, p.dev_pitch, p.width, p.height, hipMemcpyDeviceToHost, st)
                : hipMemcpy2DAsync(p.dev, p.dev_pitch, p.host, p.width, p.width, p.height, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return fail(NOMAS_E_HIP, "%s: hipMemcpy2DAsync: %s", who, hipGetErrorString(e));
  }
  return NOMAS_OK;
}

static int32_t export_frames(const nomas_kvcache* c, int64_t first_frame, int32_t n_frames, void* host_dst,
                             hipStream_t st, const char* who) {
  const int64_t valid = nomas_kvcache_valid_frames(c);
  const int64_t lo = c->frames_written - valid;
  if (n_frames < 0 || first_frame < lo || first_frame + n_frames > c->frames_written)
    return fail(NOMAS_E_INVALID, "%s: frames [%lld, %lld) are not all retained (retained: [%lld, %lld))", who,
                (long long)first_frame, (long long)(first_frame + n_frames), (long long)lo,
                (long long)c->frames_written);
  if (n_frames > 0 && !host_dst) return fail(NOMAS_E_INVALID, "%s: host_dst is NULL", who);
  const size_t rec = record_layout(c).total;
  for (int32_t i = 0; i < n_frames; ++i) {
    const int slot = (int)((first_frame + i) % c->capacity_frames);
    if (int32_t e = copy_slot(c, slot, static_cast<unsigned char*>(host_dst) + i * rec, true, st, who)) return e;
  }
  return NOMAS_OK;
}

}  // namespace nomas

using namespace nomas;

extern "C" size_t nomas_kvcache_record_bytes(const nomas_kvcache* c) {
  if (validate_cache(c, "kvcache_record_bytes")) return 0;
  return record_layout(c).total;
}

extern "C" int32_t nomas_kvcache_export_frames(const nomas_kvcache* c, int64_t first_frame, int32_t n_frames,
                                               void* host_dst, void* stream) {
  const char* who = "kvcache_export_frames";
  if (int32_t e = validate_cache(c, who)) return e;
  if (int32_t e = export_frames(c, first_frame, n_frames, host_dst, as_stream(stream), who)) return e;
  return ok();
}

extern "C" int32_t nomas_kvcache_append_archive(nomas_kvcache* c, const uint16_t* k_new, const uint16_t* v_new,
                                                int64_t ld, int32_t n_frames, void* host_evicted,
                                                int32_t* n_evicted, void* stream) {
  const char* who = "kvcache_append_archive";
  if (int32_t e = validate_cache(c, who)) return e;
  if (!n_evicted) return fail(NOMAS_E_INVALID, "%s: n_evicted is NULL", who);
  // the append's own checks, before anything is enqueued
  const int64_t HD = (int64_t)c->n_heads * c->head_dim;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))
    return fail(NOMAS_E_INVALID, "%s: k_new and v_new must be non-NULL and 16-byte aligned", who);
  if (ld < HD || ld % 8) return fail(NOMAS_E_INVALID, "%s: ld must be >= n_heads*head_dim and a multiple of 8", who);
  if (n_frames < 1 || n_frames > c->capacity_frames)
    return fail(NOMAS_E_INVALID, "%s: n_frames must be in [1, capacity_frames] (got %d)", who, n_frames);
  const int64_t valid = nomas_kvcache_valid_frames(c);
  const int32_t ev = (int32_t)(valid + n_frames > c->capacity_frames ? valid + n_frames - c->capacity_frames : 0);
  const hipStream_t st = as_stream(stream);
  // the records are taken on the stream before the append kernel overwrites them
  if (int32_t e = export_frames(c, c->frames_written - valid, ev, host_evicted, st, who)) return e;
  if (int32_t e = nomas_kvcache_append(c, k_new, v_new, ld, n_frames, stream)) return e;
  *n_evicted = ev;
  return ok();
}

extern "C" int32_t nomas_kvcache_restore_frames(nomas_kvcache* c, const void* host_src, int32_t n_frames,
                                                void* stream) {
  const char* who = "kvcache_restore_frames";
  if (int32_t e = validate_cache(c, who)) return e;
  if (n_frames < 1 || n_frames > c->capacity_frames)
    return fail(NOMAS_E_INVALID, "%s: n_frames must be in [1, capacity_frames] (got %d)", who, n_frames);
  if (!host_src) return fail(NOMAS_E_INVALID, "%s: host_src is NULL", who);
  const size_t rec = record_layout(c).total;
  const hipStream_t st = as_stream(stream);
  for (int32_t i = 0; i < n_frames; ++i) {
    const int slot = (int)((c->frames_written + i) % c->capacity_frames);
    if (int32_t e = copy_slot(c, slot, const_cast<unsigned char*>(static_cast<const unsigned char*>(host_src)) + i * rec,
                              false, st, who))
      return e;
  }
  c->frames_written += n_frames;
  return ok();
}
