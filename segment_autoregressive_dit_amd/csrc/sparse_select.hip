// Candidate-block selection for block-sparse segment attention.
//
// Pages: after two dense denoising steps, attention keeps 25 % of the candidate
// video blocks ("Hy-Nomas auf einer RTX 4090", inferencekey.com, section "Das
// Single-GPU-Preset", citing the tech report's section 6.2). The rule below is a
// reading (the pages give none): per head and block of 256 query rows,
// candidate block c of 128 cached keys scores mean_q . mean_k(c), and the
// n_select highest scores are kept, equal scores going to the lower index; the
// list is written in ascending order.
//
// Kernels: block means of Q and of the cached keys (INT8 keys as code*scale, the
// key the attention sees) into the workspace, then one workgroup per (query
// block, head) scores every candidate into LDS and ranks them.
#include "nomas_common.hpp"

namespace nomas {

int32_t validate_cache(const nomas_kvcache* c, const char* who);

constexpr int kSpKeyBlock = NOMAS_SPARSE_KEY_BLOCK;
constexpr int kSpQueryBlock = NOMAS_SPARSE_QUERY_BLOCK;
constexpr int kSpMaxCandidates = 8192;   // scores of one (query block, head) held in LDS

// Row means: a thread takes 8 consecutive channels of one row per step (one
// 16-byte load for bf16, 8 bytes for int8); D/8 threads cover a row and the
// 256/(D/8) row groups are summed through LDS at the end.
template <int D>
__device__ __forceinline__ void add_bf16x8(float (&acc)[8], const u32x4 w) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] += bf16_lo(w[e]);
    acc[2 * e + 1] += bf16_hi(w[e]);
  }
}

template <int D>
__device__ __forceinline__ void finish_mean(float (&acc)[8], float* __restrict__ dst, int count) {
  constexpr int TPR = D / 8, RG = 256 / TPR;
  __shared__ float part[RG][D];
  const int g = threadIdx.x / TPR, c0 = (threadIdx.x % TPR) * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) part[g][c0 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < RG; ++i) s += part[i][threadIdx.x];
    dst[threadIdx.x] = s / (float)count;
  }
}

// mean over the rows of query block b of head h: mq[h][b][d]
template <int D>
__global__ __launch_bounds__(256) void sp_mean_q_kernel(const uint16_t* __restrict__ q, int64_t ld, int n_q,
                                                        float* __restrict__ mq, int nqb) {
  constexpr int TPR = D / 8, RG = 256 / TPR;
  const int b = blockIdx.x, h = blockIdx.y;
  const int g = threadIdx.x / TPR, c0 = (threadIdx.x % TPR) * 8;
  const int r0 = b * kSpQueryBlock, r1 = min(n_q, r0 + kSpQueryBlock);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int r = r0 + g; r < r1; r += RG)
    add_bf16x8<D>(acc, *reinterpret_cast<const u32x4*>(q + (int64_t)r * ld + (int64_t)h * D + c0));
  finish_mean<D>(acc, mq + ((int64_t)h * nqb + b) * D, r1 - r0);
}

// mean over the keys of candidate block c of head h: mk[h][c][d] (INT8 keys as
// code * scale)
template <int D, bool I8>
__global__ __launch_bounds__(256) void sp_mean_k_kernel(const void* __restrict__ kc, const float* __restrict__ ks,
                                                        int pitch, int n_cached, float* __restrict__ mk, int nc) {
  constexpr int TPR = D / 8, RG = 256 / TPR;
  const int c = blockIdx.x, h = blockIdx.y;
  const int g = threadIdx.x / TPR, c0 = (threadIdx.x % TPR) * 8;
  const int r0 = c * kSpKeyBlock, r1 = min(n_cached, r0 + kSpKeyBlock);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int r = r0 + g; r < r1; r += RG) {
    const int64_t row = (int64_t)h * pitch + r;
    if (!NOMAS_IN_BOUNDS(r < pitch)) break;
    if constexpr (I8) {
      const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(kc) + row * D + c0);
      const float sc = ks[row];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += static_cast<float>(static_cast<int>(w.x << (24 - 8 * e)) >> 24) * sc;
        acc[4 + e] += static_cast<float>(static_cast<int>(w.y << (24 - 8 * e)) >> 24) * sc;
      }
    } else {
      add_bf16x8<D>(acc, *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(kc) + row * D + c0));
    }
  }
  finish_mean<D>(acc, mk + ((int64_t)h * nc + c) * D, r1 - r0);
}

// scores of all candidates for (query block b, head h), then the n_select best
// (rank = candidates with a higher score, or an equal one at a lower index),
// written ascending
template <int D>
__global__ __launch_bounds__(256) void sp_select_kernel(const float* __restrict__ mq, const float* __restrict__ mk,
                                                        int nqb, int nc, int n_select, int32_t* __restrict__ list) {
  __shared__ float score[kSpMaxCandidates];
  __shared__ unsigned char keep[kSpMaxCandidates];
  __shared__ float qv[D];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  if (tid < D) qv[tid] = mq[((int64_t)h * nqb + b) * D + tid];
  __syncthreads();
  if (!NOMAS_IN_BOUNDS(nc <= kSpMaxCandidates)) return;
  for (int c = tid; c < nc; c += 256) {
    const float* kr = mk + ((int64_t)h * nc + c) * D;
    float s = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], kr[d], s);
    score[c] = s;
  }
  __syncthreads();
  for (int c = tid; c < nc; c += 256) {
    const float sc = score[c];
    int rank = 0;
    for (int o = 0; o < nc; ++o) rank += (score[o] > sc) || (score[o] == sc && o < c);
    keep[c] = rank < n_select;
  }
  __syncthreads();
  int32_t* out = list + ((int64_t)h * nqb + b) * n_select;
  for (int c = tid; c < nc; c += 256) {
    if (!keep[c]) continue;
    int pos = 0;
    for (int o = 0; o < c; ++o) pos += keep[o];
    if (pos < n_select) out[pos] = c;   // ranks are distinct for finite scores

  }
}

int64_t check_failures_sparse(int reset) { return source_check_failures(reset); }

}  // namespace nomas

using namespace nomas;

static int sp_qblocks(int n_q) { return (n_q + kSpQueryBlock - 1) / kSpQueryBlock; }

extern "C" int32_t nomas_sparse_candidates(int64_t n_cached) {
  if (n_cached < 0) return -1;
  return (int32_t)((n_cached + kSpKeyBlock - 1) / kSpKeyBlock);
}

extern "C" size_t nomas_sparse_select_workspace_bytes(int32_t n_q, int64_t n_cached, int32_t n_heads,
                                                      int32_t head_dim) {
  if (n_q < 1 || n_cached < 0 || n_heads < 1 || (head_dim != 64 && head_dim != 128)) return 0;
  const int64_t nc = (n_cached + kSpKeyBlock - 1) / kSpKeyBlock;
  return (size_t)(round_up((int64_t)n_heads * sp_qblocks(n_q) * head_dim * 4, 256) +
                  round_up((int64_t)n_heads * nc * head_dim * 4, 256));
}

extern "C" int32_t nomas_sparse_select(const uint16_t* q, int64_t ld_q, int32_t n_q, const nomas_kvcache* c,
                                       int32_t n_select, int32_t* block_list, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const char* who = "sparse_select";
  if (int32_t e = validate_cache(c, who)) return e;
  const int H = c->n_heads, D = c->head_dim;
  const int64_t n_cached = nomas_kvcache_valid_frames(c) * c->tokens_per_frame;
  const int nc = (int)((n_cached + kSpKeyBlock - 1) / kSpKeyBlock);
  if (!q || !aligned16(q)) return fail(NOMAS_E_INVALID, "%s: q must be non-NULL and 16-byte aligned", who);
  if (ld_q < (int64_t)H * D || ld_q % 8) return fail(NOMAS_E_INVALID, "%s: ld_q must be >= n_heads*head_dim, a multiple of 8", who);
  if (n_q < 1) return fail(NOMAS_E_INVALID, "%s: n_q must be >= 1", who);
  if (n_select < 0 || n_select > nc)
    return fail(NOMAS_E_INVALID, "%s: n_select %d outside [0, %d] (candidate blocks of the cache)", who, n_select, nc);
  if (nc > kSpMaxCandidates) return fail(NOMAS_E_UNSUPPORTED, "%s: more than %d candidate blocks", who, kSpMaxCandidates);
  if (n_select == 0) return ok();
  if (!block_list || (reinterpret_cast<uintptr_t>(block_list) & 3))
    return fail(NOMAS_E_INVALID, "%s: block_list must be non-NULL and 4-byte aligned", who);
  const size_t need = nomas_sparse_select_workspace_bytes(n_q, n_cached, H, D);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(NOMAS_E_WORKSPACE, "%s: workspace must be non-NULL and 256-byte aligned", who);
  if (workspace_bytes < need) return fail(NOMAS_E_WORKSPACE, "%s: workspace of %zu bytes, need %zu", who, workspace_bytes, need);
  const int nqb = sp_qblocks(n_q);
  float* mq = static_cast<float*>(workspace);
  float* mk = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + round_up((int64_t)H * nqb * D * 4, 256));
  const hipStream_t st = as_stream(stream);
  const bool i8 = c->kv_dtype == NOMAS_KV_INT8;
  if (D == 128) {
    hipLaunchKernelGGL(sp_mean_q_kernel<128>, dim3(nqb, H), dim3(256), 0, st, q, ld_q, n_q, mq, nqb);
    if (i8) hipLaunchKernelGGL((sp_mean_k_kernel<128, true>), dim3(nc, H), dim3(256), 0, st, c->k, c->k_scale, c->token_pitch, (int)n_cached, mk, nc);
    else hipLaunchKernelGGL((sp_mean_k_kernel<128, false>), dim3(nc, H), dim3(256), 0, st, c->k, c->k_scale, c->token_pitch, (int)n_cached, mk, nc);
    hipLaunchKernelGGL(sp_select_kernel<128>, dim3(nqb, H), dim3(256), 0, st, mq, mk, nqb, nc, n_select, block_list);
  } else {
    hipLaunchKernelGGL(sp_mean_q_kernel<64>, dim3(nqb, H), dim3(256), 0, st, q, ld_q, n_q, mq, nqb);
    if (i8) hipLaunchKernelGGL((sp_mean_k_kernel<64, true>), dim3(nc, H), dim3(256), 0, st, c->k, c->k_scale, c->token_pitch, (int)n_cached, mk, nc);
    else hipLaunchKernelGGL((sp_mean_k_kernel<64, false>), dim3(nc, H), dim3(256), 0, st, c->k, c->k_scale, c->token_pitch, (int)n_cached, mk, nc);
    hipLaunchKernelGGL(sp_select_kernel<64>, dim3(nqb, H), dim3(256), 0, st, mq, mk, nqb, nc, n_select, block_list);
  }
  return check_launch(who);
}
