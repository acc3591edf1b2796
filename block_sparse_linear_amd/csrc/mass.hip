// Exact attention mass of every candidate block: for (b, g) and block j in
// 1 .. nb-2, LGx(j) = log sum_h (1/Bk) sum_{i in j} exp(q_hat_h . k_i), the
// quantity the second-order Taylor score estimates (SPLA Technical Summary
// 2.1: a block's integrated probability mass, here in the per-token mean form
// of the score formula, summed over the query heads of the KV group).  It
// reads every key of every candidate block: an evaluation pass for measuring
// how well a block score ranks blocks, not part of a decode.
#include "attend_mfma.h"

namespace spla {

namespace {

// logsumexp over the R per-head values held (uniform) in v
template <int R>
__device__ __forceinline__ float group_lse(const float (&v)[8]) {
  float m = v[0];
#pragma unroll
  for (int h = 1; h < R; ++h) m = fmaxf(m, v[h]);
  float e = 0.f;
#pragma unroll
  for (int h = 0; h < R; ++h) e += __expf(v[h] - m);
  return m + __logf(e);
}

// bf16 keys on the matrix cores.  grid (ceil(max candidates / 4), G, B);
// wavefront w of workgroup x takes block j = 1 + 4 x + w.  Product: the
// 16-row A operand holds the R queries (other rows zero), B the block's K
// tile read straight from its page, 16 tokens per tile.  Lane (l16, lg4)
// holds rows 4 lg4 .. 4 lg4 + 3 (heads) of token l16 of each tile.  No
// barriers: each wavefront is on its own, and leaves at once past the
// sequence's last candidate.
template <int R, int D, int BK>
__global__ __launch_bounds__(kThreads) void k_block_mass(const void* q, const int32_t* block_table, float* lgx,
                                                          int32_t G, int32_t H, int32_t max_blocks,
                                                          const DecodeArgs a) {
  constexpr int NKS = D / 32;  // k-steps
  constexpr int NT = BK / 16;  // 16-token tiles
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64, l16 = lane % 16, lg4 = lane / 16;
  const int g = blockIdx.y, b = blockIdx.z;
  const int j = 1 + 4 * blockIdx.x + w;
  // queries: row l16 of A is head l16 (rows >= R are masked to zero)
  uint4 aq[NKS];
  const int hq = l16 < R ? l16 : 0;
  const uint32_t mq = l16 < R ? 0xffffffffu : 0u;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) +
                                                    ((size_t)b * H + g * R + hq) * D + 32 * ks + 8 * lg4);
    aq[ks] = make_uint4(v.x & mq, v.y & mq, v.z & mq, v.w & mq);
  }
  SPLA_SCALARS_READY("s"(a.lens[b]), "s"(a.bk), "s"(a.k_pages), "s"(a.num_pages), "s"(a.inv_sqrt_d), "s"(a.err));
  const int nb = n_blocks(a, b);
  if (j > nb - 2) return;
  const int page = block_table[(size_t)b * max_blocks + j];
  if (page < 0 || page >= a.num_pages) {
    if (lane == 0) atomicOr(a.err, kErrPage);
    return;
  }
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.k_pages) + ((size_t)page * G + g) * BK * D;
  uint4 kraw[NT][NKS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kraw[nt][ks] = *reinterpret_cast<const uint4*>(kp + (size_t)(nt * 16 + l16) * D + 32 * ks + 8 * lg4);
  f32x4_t c[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    c[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) c[nt] = mfma_bf16(aq[ks], kraw[nt][ks], c[nt]);
  }
  // per head: log of the mean of exp(s) over the block's tokens
  const float sc = a.inv_sqrt_d;
  float lm[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) m = fmaxf(m, c[nt][i] * sc);
    m = row16_max(m);
    float e = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) e += __expf(c[nt][i] * sc - m);
    e = row16_sum(e);
    lm[i] = m + __logf(e) - __logf((float)BK);
  }
  float v[8];
#pragma unroll
  for (int h = 0; h < 8; ++h)
    v[h] = h < R ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lm[h % 4]), 16 * (h / 4))) : 0.f;
  if (lane == 0) lgx[((size_t)b * G + g) * max_blocks + j] = group_lse<R>(v);
}

// fp32 keys on the VALU: wavefront = block, lane = token (two tokens per lane
// at Bk = 128); the queries are uniform loads
template <int R, int D, int BK>
__global__ __launch_bounds__(kThreads) void k_block_mass_f32(const void* q, const int32_t* block_table, float* lgx,
                                                              int32_t G, int32_t H, int32_t max_blocks,
                                                              const DecodeArgs a) {
  constexpr int TPL = BK / 64;  // tokens per lane
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  const int g = blockIdx.y, b = blockIdx.z;
  const int j = 1 + 4 * blockIdx.x + w;
  const int nb = n_blocks(a, b);
  if (j > nb - 2) return;
  const int page = block_table[(size_t)b * max_blocks + j];
  if (page < 0 || page >= a.num_pages) {
    if (lane == 0) atomicOr(a.err, kErrPage);
    return;
  }
  const float* kp = reinterpret_cast<const float*>(a.k_pages) + ((size_t)page * G + g) * BK * D;
  const float* qg = reinterpret_cast<const float*>(q) + ((size_t)b * H + g * R) * D;
  float s[TPL][R];
#pragma unroll
  for (int u = 0; u < TPL; ++u)
#pragma unroll
    for (int h = 0; h < R; ++h) s[u][h] = 0.f;
  for (int c4 = 0; c4 < D / 4; ++c4) {
    float4 kv[TPL];
#pragma unroll
    for (int u = 0; u < TPL; ++u) kv[u] = reinterpret_cast<const float4*>(kp + (size_t)(lane + 64 * u) * D)[c4];
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const float4 qv = reinterpret_cast<const float4*>(qg + (size_t)h * D)[c4];
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        s[u][h] = fmaf(qv.x, kv[u].x, s[u][h]);
        s[u][h] = fmaf(qv.y, kv[u].y, s[u][h]);
        s[u][h] = fmaf(qv.z, kv[u].z, s[u][h]);
        s[u][h] = fmaf(qv.w, kv[u].w, s[u][h]);
      }
    }
  }
  float v[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) v[h] = 0.f;
#pragma unroll
  for (int h = 0; h < R; ++h) {
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < TPL; ++u) m = fmaxf(m, s[u][h] * a.inv_sqrt_d);
    m = wave_max(m);
    float e = 0.f;
#pragma unroll
    for (int u = 0; u < TPL; ++u) e += __expf(s[u][h] * a.inv_sqrt_d - m);
    e = wave_sum(e);
    v[h] = m + __logf(e) - __logf((float)BK);
  }
  if (lane == 0) lgx[((size_t)b * G + g) * max_blocks + j] = group_lse<R>(v);
}

template <int R, int D>
hipError_t launch_mass_rd(const DecodeArgs& a, bool bf16, float* lgx, const dim3& grid, const Launch& l) {
  if (bf16) {
    if (a.bk == 64) return launch_kernel(k_block_mass<R, D, 64>, grid, l, a.q, a.block_table, lgx, a.G, a.H, a.max_blocks, a);
    return launch_kernel(k_block_mass<R, D, 128>, grid, l, a.q, a.block_table, lgx, a.G, a.H, a.max_blocks, a);
  }
  if (a.bk == 64) return launch_kernel(k_block_mass_f32<R, D, 64>, grid, l, a.q, a.block_table, lgx, a.G, a.H, a.max_blocks, a);
  return launch_kernel(k_block_mass_f32<R, D, 128>, grid, l, a.q, a.block_table, lgx, a.G, a.H, a.max_blocks, a);
}

}  // namespace

hipError_t launch_block_mass(const DecodeArgs& a, bool bf16, float* lgx, int max_cand, const Launch& l) {
  const dim3 grid((max_cand + 3) / 4, a.G, a.B);
  SPLA_DISPATCH_RD(a.r, a.d, (launch_mass_rd<RR, DD>(a, bf16, lgx, grid, l)))
}

}  // namespace spla
