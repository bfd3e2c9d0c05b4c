// 3D rotary position embedding of Q and K video rows, in place.
//
// Pages: the model card lists "3D RoPE" among the DiT's features ("Hy-Nomas auf
// einer RTX 4090", inferencekey.com, section "Modell und Dateien"; blog.authon.dev,
// section "What Hy-Nomas is"). Band split (d_t, d_h, d_w), adjacent-pair order and
// theta are arguments; the per-pair law is pos * theta^(-2j/d) inside each band.
//
// HBM-bound: every element is read once and written once. One block handles
// kTok consecutive tokens: it first evaluates the token's head_dim/2 angles once
// (sincosf, shared by all heads and by Q and K through LDS), then streams the
// rows in 16-byte chunks (8 bf16 = 4 pairs) with consecutive threads on
// consecutive chunks, so each wave reads/writes 1 KB contiguous per instruction.
#include "nomas_common.hpp"

namespace nomas {

constexpr int kRopeTok = 4;
constexpr int kRopeThreads = 256;
// chunks a thread loads before it rotates any (at the layer shape 19.95-20.1 us
// against 20.2-20.4 for 4, 20.6-20.8 for 2, 21.0-21.2 one at a time)
constexpr int kRopeBatch = 8;

struct RopeFreq {
  float w[64];   // angle per unit position of pair p (sign of `inverse` folded in)
};

template <int D>
__global__ __launch_bounds__(kRopeThreads) void rope3d_kernel(uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                                             int64_t ld, int n_heads, int n_rows, int t0,
                                                             int grid_h, int grid_w, int pairs_t, int pairs_th,
                                                             RopeFreq f) {
  constexpr int P = D / 2;          // pairs per head row
  constexpr int CPR = D / 8;        // 16-byte chunks per head row
  __shared__ float2 cs[kRopeTok][P];
  const int row0 = blockIdx.x * kRopeTok;
  const int gs = grid_h * grid_w;

  for (int i = threadIdx.x; i < kRopeTok * P; i += kRopeThreads) {
    const int tk = i / P, p = i % P, row = row0 + tk;
    float c = 1.f, s = 0.f;
    if (row < n_rows) {
      const int pos = p < pairs_t ? t0 + row / gs : (p < pairs_th ? (row / grid_w) % grid_h : row % grid_w);
      sincosf(static_cast<float>(pos) * f.w[p], &s, &c);
    }
    cs[tk][p] = make_float2(c, s);
  }
  __syncthreads();

  // chunks in batches of kRopeBatch per thread: the batch's loads are all in
  // flight before the first rotation. Every load is issued (a chunk that is not
  // rotated reads the block's first chunk, which exists), so no branch sits
  // between them; only the stores are conditional.
  const int chunks_per_tensor = n_heads * CPR;
  const int n_tensors = k ? 2 : 1;
  const int total = kRopeTok * n_tensors * chunks_per_tensor;
  for (int i0 = threadIdx.x; i0 < total; i0 += kRopeBatch * kRopeThreads) {
    u32x4* ptr[kRopeBatch];
    bool live[kRopeBatch];
    u32x4 v[kRopeBatch];
    int tkb[kRopeBatch], d0b[kRopeBatch];
#pragma unroll
    for (int b = 0; b < kRopeBatch; ++b) {
      const int i = i0 + b * kRopeThreads;
      const int tk = i / (n_tensors * chunks_per_tensor);
      const int rem = i - tk * n_tensors * chunks_per_tensor;
      const int tensor = rem / chunks_per_tensor;
      const int c = rem - tensor * chunks_per_tensor;
      const int row = row0 + tk;
      const int h = c / CPR, d0 = (c - h * CPR) * 8;
      tkb[b] = tk;
      d0b[b] = d0;
      live[b] = i < total && row < n_rows &&
                NOMAS_IN_BOUNDS(h < n_heads && d0 + 8 <= D && (int64_t)n_heads * D <= ld);
      uint16_t* base = tensor ? k : q;
      ptr[b] = live[b] ? reinterpret_cast<u32x4*>(base + (int64_t)row * ld + (int64_t)h * D + d0)
                       : reinterpret_cast<u32x4*>(q + (int64_t)row0 * ld);
      v[b] = *ptr[b];
    }
#pragma unroll
    for (int b = 0; b < kRopeBatch; ++b) {
      if (!live[b]) continue;
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 r = cs[tkb[b]][d0b[b] / 2 + e];
        const float u = bf16_lo(v[b][e]), w = bf16_hi(v[b][e]);
        o[e] = pack_bf16x2(fmaf(u, r.x, -w * r.y), fmaf(u, r.y, w * r.x));
      }
      *ptr[b] = o;
    }
  }
}

int64_t check_failures_rope(int reset) { return source_check_failures(reset); }

}  // namespace nomas

using namespace nomas;

extern "C" int32_t nomas_rope3d(uint16_t* q, uint16_t* k, int64_t ld, int32_t n_heads, int32_t head_dim,
                                int32_t t0, int32_t n_frames, int32_t grid_h, int32_t grid_w, int32_t d_t,
                                int32_t d_h, int32_t d_w, float theta, int32_t inverse, void* stream) {
  if (!q) return fail(NOMAS_E_INVALID, "rope3d: q is NULL");
  if (n_heads < 1) return fail(NOMAS_E_INVALID, "rope3d: n_heads must be >= 1");
  if (head_dim != 64 && head_dim != 128)
    return fail(NOMAS_E_UNSUPPORTED, "rope3d: head_dim must be 64 or 128 (got %d)", head_dim);
  if (d_t < 0 || d_h < 0 || d_w < 0 || (d_t | d_h | d_w) & 1 || d_t + d_h + d_w != head_dim)
    return fail(NOMAS_E_INVALID, "rope3d: band widths (%d,%d,%d) must be even and sum to head_dim %d", d_t, d_h,
                d_w, head_dim);
  if (t0 < 0 || n_frames < 1 || grid_h < 1 || grid_w < 1)
    return fail(NOMAS_E_INVALID, "rope3d: need t0 >= 0, n_frames >= 1, grid_h >= 1, grid_w >= 1");
  if (!(theta > 0.f)) return fail(NOMAS_E_INVALID, "rope3d: theta must be > 0");
  if (ld < (int64_t)n_heads * head_dim || ld % 8)
    return fail(NOMAS_E_INVALID, "rope3d: ld must be >= n_heads*head_dim and a multiple of 8");
  if (!aligned16(q) || (k && !aligned16(k))) return fail(NOMAS_E_INVALID, "rope3d: q and k must be 16-byte aligned");
  const int64_t n_rows = (int64_t)n_frames * grid_h * grid_w;
  if (n_rows > INT32_MAX / 2 || (int64_t)t0 + n_frames > (1 << 24))
    return fail(NOMAS_E_INVALID, "rope3d: too many rows or positions beyond 2^24");
  if (n_rows * ld > ((int64_t)1 << 40)) return fail(NOMAS_E_INVALID, "rope3d: tensor larger than 1 TiB");

  RopeFreq f;
  const int widths[3] = {d_t, d_h, d_w};
  const double sign = inverse ? -1.0 : 1.0;
  int p = 0;
  for (int a = 0; a < 3; ++a)
    for (int j = 0; j < widths[a] / 2; ++j)
      f.w[p++] = static_cast<float>(sign * pow((double)theta, -2.0 * j / widths[a]));
  const int pairs_t = d_t / 2, pairs_th = (d_t + d_h) / 2;
  const dim3 grid((unsigned)((n_rows + kRopeTok - 1) / kRopeTok));
  if (head_dim == 128)
    hipLaunchKernelGGL(rope3d_kernel<128>, grid, dim3(kRopeThreads), 0, as_stream(stream), q, k, ld, n_heads,
                       (int)n_rows, t0, grid_h, grid_w, pairs_t, pairs_th, f);
  else
    hipLaunchKernelGGL(rope3d_kernel<64>, grid, dim3(kRopeThreads), 0, as_stream(stream), q, k, ld, n_heads,
                       (int)n_rows, t0, grid_h, grid_w, pairs_t, pairs_th, f);
  return check_launch("rope3d");
}
