// Chunked prefill, the in-chunk part of the linear-attention state: for the
// virtual query of token t of a chunk (its own decode at its own position,
// SPLA Technical Summary 2.2), o_bar_t = phi(q_t)^T S_t with S_t the state up
// to and including token t.  The decode kernels of the chunk see the state
// before the chunk, S_0; this kernel adds the chunk's own tokens up to t:
//   o_bar_t += sum_{i <= t} (phi(q_t) . phi(k_i)) v_i,   phi(q_t).z += sum_{i <= t} phi(q_t) . phi(k_i),
// into the first row chunk of the o_bar / phi(q).z partials the combine sums.
#include "decode_common.h"

namespace spla {

namespace {

// grid (m, G): virtual query t (token t of the chunk), KV head g; its R query
// heads.  k_new / v_new / q address the chunk's first token.  Thread = token i
// for the linear weights w[i][h] (a D-long dot product each); then thread =
// (value channel, token split) for sum_i w[i][h] v_i, the splits meeting in
// LDS.  fp32 throughout.
template <bool BF16, int R, int D>
__global__ __launch_bounds__(kThreads) void k_chunk_la(const void* k_new, const void* v_new, const void* q,
                                                        float* obar_part, float* dz_part, int32_t G, int32_t H) {
  constexpr int CHUNKS = D / (1024 / D);  // o_bar partials per (query, KV head)
  constexpr int NS = kThreads / D;        // token splits of the weighted sum
  __shared__ float fq[R][D];
  __shared__ float wl[kThreads][R];
  __shared__ float red[NS][R][D];
  __shared__ float zred[NS][R];
  const int t = blockIdx.x, g = blockIdx.y;
  const int n = t + 1;  // tokens 0 .. t of the chunk
  for (int i = threadIdx.x; i < R * D; i += kThreads) {
    const int h = i / D, c = i % D;
    fq[h][c] = phi_f(load_elem<BF16>(q, ((size_t)t * H + g * R + h) * D + c));
  }
  __syncthreads();
  if ((int)threadIdx.x < n) {
    const size_t row = ((size_t)threadIdx.x * G + g) * D;
    float w[R];
#pragma unroll
    for (int h = 0; h < R; ++h) w[h] = 0.f;
    for (int c = 0; c < D; ++c) {
      const float f = phi_f(load_elem<BF16>(k_new, row + c));
#pragma unroll
      for (int h = 0; h < R; ++h) w[h] = fmaf(fq[h][c], f, w[h]);
    }
#pragma unroll
    for (int h = 0; h < R; ++h) wl[threadIdx.x][h] = w[h];
  }
  __syncthreads();
  const int c = threadIdx.x % D, sp = threadIdx.x / D;
  float acc[R], zs[R];
#pragma unroll
  for (int h = 0; h < R; ++h) acc[h] = zs[h] = 0.f;
  for (int i = sp; i < n; i += NS) {
    const float v = load_elem<BF16>(v_new, ((size_t)i * G + g) * D + c);
#pragma unroll
    for (int h = 0; h < R; ++h) {
      acc[h] = fmaf(wl[i][h], v, acc[h]);
      zs[h] += wl[i][h];
    }
  }
#pragma unroll
  for (int h = 0; h < R; ++h) {
    red[sp][h][c] = acc[h];
    if (c == 0) zred[sp][h] = zs[h];
  }
  __syncthreads();
  const size_t bg = (size_t)t * G + g;
  for (int i = threadIdx.x; i < R * D; i += kThreads) {
    const int h = i / D, cc = i % D;
    float s = red[0][h][cc];
#pragma unroll
    for (int k = 1; k < NS; ++k) s += red[k][h][cc];
    obar_part[((bg * CHUNKS + 0) * R + h) * D + cc] += s;
  }
  if ((int)threadIdx.x < R) {
    const int h = threadIdx.x;
    float s = zred[0][h];
#pragma unroll
    for (int k = 1; k < NS; ++k) s += zred[k][h];
    dz_part[(bg * CHUNKS + 0) * R + h] += s;
  }
}

}  // namespace

hipError_t launch_chunk_la(const DecodeArgs& a, bool bf16, const void* k_new, const void* v_new, const Launch& l) {
  const dim3 grid(a.B, a.G);
  if (bf16)
    SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_chunk_la<true, RR, DD>, grid, l, k_new, v_new, a.q, a.obar_part,
                                             a.dz_part, a.G, a.H))
  SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_chunk_la<false, RR, DD>, grid, l, k_new, v_new, a.q, a.obar_part,
                                           a.dz_part, a.G, a.H))
}

}  // namespace spla
