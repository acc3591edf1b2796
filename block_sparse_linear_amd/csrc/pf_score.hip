// Block scorer of a chunked-prefill group on the matrix cores.  Every virtual
// query (token) of the group is scored against every candidate block with the
// decode scorer's log-domain second-order Taylor score (SPLA Technical Summary
// 2.1, diagonal covariance):
//   ls_h(j) = q_h . mu_j / sqrt(d) + log(1 + sum_c q_hc^2 var_jc / (2 d)),
//   LG(j)   = logsumexp over the R query heads of the group,
// or the first-order (mean-pooling) form.  Over a group both sums are matrix
// products, [tokens x d] by [d x blocks] per query head, so one workgroup
// reads a 64-block statistics tile once for 32 tokens instead of once per
// token.  fp32 queries use the fp32 matrix cores (16x16x4, fp32 in and out,
// k_pf_score); bf16 queries use the bf16 matrix cores on exact bf16 splits of
// the fp32 operands (k_pf_score_bf), which gives the same products in a
// quarter of the matrix-core time.
#include "decode_common.h"

namespace spla {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float f4_at(const float4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// grid (score_tiles, G, ceil(m / 32)).  Wavefront w takes tokens 32 z +
// 16 (w / 2) .. + 15, the 16 rows of the A operand, against blocks 32 (w % 2)
// .. + 31 of tile t as two 16-column tiles (B operand = statistics, columns =
// blocks).  Channel c = kk * KS + ks is contracted at k-step ks in k slot kk
// = lane / 16, so a lane's query channels are contiguous and its statistics
// arrive as float4s of one channel quartet of the tile layout (64 blocks side
// by side per quartet).  Accumulators: column tile x query head x (mean,
// variance).  bf16 queries are held packed for the whole kernel; the
// statistics stream one channel quartet ahead of the products, behind a
// scheduling barrier (left alone, the scheduler sinks the loads to their first
// use).  Up to four query heads, three wavefronts share a SIMD (168 registers
// per lane at 4 x 128, a few spilled).
template <bool BF16, int R, int D, bool TAYLOR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(R <= 4 ? 3 : 1))) void k_pf_score(const float* mean, const float* var, const void* q,
                                                        int32_t n_tiles, int32_t G, int32_t H, int32_t m,
                                                        const DecodeArgs a) {
  constexpr int KS = D / 4;            // k-steps, and channels per k slot
  constexpr int KQ = KS / 4;           // channel quartets per k slot
  constexpr int NC = 2;                // column tiles per wavefront
  const int t = blockIdx.x, g = blockIdx.y;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64, l16 = lane % 16, kk = lane / 16;
  const int tok0 = 32 * blockIdx.z + 16 * (w >> 1);  // first token of this wavefront
  const int n0 = NC * (w & 1);                       // its first column tile
  const int tok = min(tok0 + l16, m - 1);     // A row (rows past the group repeat the last token, never stored)

  // ---- statistics loads of one channel quartet (all four column tiles)
  const float4* mean4 = reinterpret_cast<const float4*>(mean);
  const float4* var4 = reinterpret_cast<const float4*>(var);
  const size_t base = ((size_t)g * n_tiles + t) * (size_t)(D / 4) * kTile + (size_t)(kk * KQ) * kTile + l16;
  constexpr int NBUF = 2;              // quartets in registers: the current one and one in flight
  float4 bm[NBUF][NC], bv[NBUF][NC];
  auto load_b = [&](int j, int buf) {
#pragma unroll
    for (int n = 0; n < NC; ++n) {
      const size_t at = base + (size_t)j * kTile + 16 * (n0 + n);
      bm[buf][n] = mean4[at];
      bv[buf][n] = TAYLOR ? var4[at] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  // ---- A: this lane's KS query channels of every head.  bf16 queries are
  // held packed for the whole kernel (KS / 2 registers per head); fp32 ones
  // stream a channel quartet at a time, two quartets ahead like the
  // statistics.
  constexpr int QW = BF16 ? KS / 8 : 1;  // 16-byte pieces of packed bf16 per head
  uint4 qp[R][QW];
  if constexpr (BF16) {
#pragma unroll
    for (int h = 0; h < R; ++h)
#pragma unroll
      for (int i = 0; i < QW; ++i)
        qp[h][i] = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) +
                                                  ((size_t)tok * H + g * R + h) * D + kk * KS)[i];
  }
  float4 qa[NBUF][R];
  auto load_a = [&](int j, int buf) {
    if constexpr (!BF16) {
#pragma unroll
      for (int h = 0; h < R; ++h)
        qa[buf][h] = *reinterpret_cast<const float4*>(static_cast<const float*>(q) +
                                                      ((size_t)tok * H + g * R + h) * D + kk * KS + 4 * j);
    }
  };
  load_b(0, 0);
  load_a(0, 0);
  SPLA_SCALARS_READY("s"(a.bk), "s"(a.lg), "s"(a.lg_out), "s"(a.max_blocks), "s"(a.inv_sqrt_d));

  const float half_inv_d = 0.5f / (float)D;
  const size_t row = (size_t)n_tiles * kTile;
  {
    // ---- products: quartet j of this wavefront's column tiles, the next quartet in flight
    f32x4_t cm[NC][R], cv[NC][R];
#pragma unroll
    for (int n = 0; n < NC; ++n)
#pragma unroll
      for (int h = 0; h < R; ++h) cm[n][h] = cv[n][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KQ; ++j) {
      if (j + 1 < KQ) {
        load_b(j + 1, (j + 1) % NBUF);
        load_a(j + 1, (j + 1) % NBUF);
      }
      // the prefetch stays ahead of this step's products (left alone, the
      // scheduler sinks the loads to their first use)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int h = 0; h < R; ++h) {
          float qk;
          if constexpr (BF16) {
            const int c = 4 * j + e;  // channel of the lane's run
            const uint4& u = qp[h][c / 8];
            const uint32_t wd = (c % 8) / 2 == 0 ? u.x : (c % 8) / 2 == 1 ? u.y : (c % 8) / 2 == 2 ? u.z : u.w;
            qk = c % 2 == 0 ? bf16_lo_f(wd) : bf16_hi_f(wd);
          } else {
            qk = f4_at(qa[j % NBUF][h], e);
          }
          const float q2 = qk * qk;
#pragma unroll
          for (int n = 0; n < NC; ++n) {
            cm[n][h] = __builtin_amdgcn_mfma_f32_16x16x4f32(qk, f4_at(bm[j % NBUF][n], e), cm[n][h], 0, 0, 0);
            if (TAYLOR)
              cv[n][h] = __builtin_amdgcn_mfma_f32_16x16x4f32(q2, f4_at(bv[j % NBUF][n], e), cv[n][h], 0, 0, 0);
          }
        }
      }
    }

    // ---- log scores, group logsumexp: lane holds tokens 4 kk + i, block 16 n + l16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = tok0 + 4 * kk + i;
      if (tk >= m) continue;
      const int nb = (a.lens[tk] + a.bk - 1) / a.bk;
#pragma unroll
      for (int n = 0; n < NC; ++n) {
        float ls[R];
#pragma unroll
        for (int h = 0; h < R; ++h)
          ls[h] = TAYLOR ? cm[n][h][i] * a.inv_sqrt_d + __logf(1.f + fmaxf(cv[n][h][i], 0.f) * half_inv_d)
                         : cm[n][h][i] * a.inv_sqrt_d;
        float lg = ls[0];
        if constexpr (R > 1) {
          float mx = ls[0];
#pragma unroll
          for (int h = 1; h < R; ++h) mx = fmaxf(mx, ls[h]);
          float e[R];
#pragma unroll
          for (int h = 0; h < R; ++h) e[h] = __expf(ls[h] - mx);
          // pairwise, in the decode scorer's order
#pragma unroll
          for (int st = 1; st < R; st *= 2)
#pragma unroll
            for (int h = 0; h < R; h += 2 * st) e[h] += e[h + st];
          lg = mx + __logf(e[0]);
        }
        const int jb = t * kTile + 16 * (n0 + n) + l16;
        const bool cand = jb >= 1 && jb <= nb - 2;
        a.lg[((size_t)tk * G + g) * row + jb] = cand ? lg : -INFINITY;
        if (a.lg_out && cand) a.lg_out[((size_t)tk * G + g) * a.max_blocks + jb] = lg;
      }
    }
  }
}

// The same scorer for bf16 queries on the bf16 matrix cores (16x16x32,
// fp32 sums).  The products stay exact to fp32 level: q is bf16 already;
// every statistic is split exactly into three bf16 parts (hi, mid, lo: 8 bits
// each of its 24) and q^2 into two; q . mean takes the three parts and
// q^2 . var the five products of the parts above 2^-32 of their sum.  At
// eight 16x16x32 products per 32 channels and (column tile, head) against
// sixteen 16x16x4 fp32 ones, the matrix cores take a quarter of the time.
// Mapping as in k_pf_score; lane (l16, lg4) takes channels 32 ks + 8 lg4 ..
// + 7 of k-step ks: its A row is token l16's query, its B column block l16's
// statistics (two float4 channel quartets of the tile layout).  The splits
// are made once per workgroup and k-step and shared in LDS.
typedef __bf16 bf16x8s_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma_bf16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8s_t, a), __builtin_bit_cast(bf16x8s_t, b),
                                                  c, 0, 0, 0);
}

// 8 floats -> bf16 hi, mid, lo parts (hi + mid + lo == x exactly), pairs packed
__device__ __forceinline__ void split3(const float4& u, const float4& v, uint4& hi, uint4& mid, uint4& lo) {
  const float x[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    h[p] = pack_bf16(x[2 * p], x[2 * p + 1]);
    const float r0 = x[2 * p] - bf16_lo_f(h[p]), r1 = x[2 * p + 1] - bf16_hi_f(h[p]);
    m[p] = pack_bf16(r0, r1);
    l[p] = pack_bf16(r0 - bf16_lo_f(m[p]), r1 - bf16_hi_f(m[p]));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  mid = make_uint4(m[0], m[1], m[2], m[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

template <int R, int D, bool TAYLOR>
__global__ __launch_bounds__(kThreads) void k_pf_score_bf(const float* mean, const float* var, const void* q,
                                                           int32_t n_tiles, int32_t G, int32_t H, int32_t m,
                                                           const DecodeArgs a) {
  constexpr int KS = D / 32;  // k-steps of 32 channels
  constexpr int NC = 2;       // column tiles per wavefront
  constexpr int NQ = (2 * R * 64 + kThreads - 1) / kThreads;  // query units per thread
  const int t = blockIdx.x, g = blockIdx.y;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64, l16 = lane % 16, lg4 = lane / 16;
  const int tok0 = 32 * blockIdx.z + 16 * (w >> 1);
  const int n0 = NC * (w & 1);
  // Each k-step's bf16 operands are formed once per workgroup and shared in
  // LDS (two wavefronts read every statistics column and every query row):
  // thread (block b = tid % 64, channel group cg = tid / 64) splits the
  // statistics the B operand of lane (b % 16, cg) of column tile b / 16
  // holds; query unit u (lane u % 64, head u / 64 % R, token tile u / 64R)
  // loads the A operand of that lane and splits its square.
  __shared__ uint4 sM[3][4][64], sV[TAYLOR ? 3 : 1][4][64];
  __shared__ uint4 sQ[TAYLOR ? 3 : 1][2][R][64];
  const int sb = threadIdx.x % 64, scg = threadIdx.x / 64;
  const float4* mean4 = reinterpret_cast<const float4*>(mean);
  const float4* var4 = reinterpret_cast<const float4*>(var);
  const size_t sbase = ((size_t)g * n_tiles + t) * (size_t)(D / 4) * kTile + sb;
  const uint16_t* qg = static_cast<const uint16_t*>(q);
  struct Raw {
    float4 bm[2], bv[2];
    uint4 qa[NQ];
  };
  auto load = [&](int ks, Raw& r) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const size_t at = sbase + (size_t)(8 * ks + 2 * scg + e) * kTile;
      r.bm[e] = mean4[at];
      r.bv[e] = TAYLOR ? var4[at] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      const int u = min((int)threadIdx.x + kThreads * k, 2 * R * 64 - 1);
      const int ul = u % 64, uh = (u / 64) % R, ut = u / (64 * R);
      const int tk = min(32 * (int)blockIdx.z + 16 * ut + ul % 16, m - 1);
      r.qa[k] = *reinterpret_cast<const uint4*>(qg + ((size_t)tk * H + g * R + uh) * D + 32 * ks + 8 * (ul / 16));
    }
  };
  Raw cur, nxt;
  load(0, cur);
  SPLA_SCALARS_READY("s"(a.bk), "s"(a.lg), "s"(a.lg_out), "s"(a.max_blocks), "s"(a.inv_sqrt_d));
  f32x4_t cm[NC][R], cv[NC][R];
#pragma unroll
  for (int n = 0; n < NC; ++n)
#pragma unroll
    for (int h = 0; h < R; ++h) cm[n][h] = cv[n][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    // ---- form this k-step's operands in LDS
    {
      uint4 hi, mid, lo;
      split3(cur.bm[0], cur.bm[1], hi, mid, lo);
      sM[0][scg][sb] = hi;
      sM[1][scg][sb] = mid;
      sM[2][scg][sb] = lo;
      if (TAYLOR) {
        split3(cur.bv[0], cur.bv[1], hi, mid, lo);
        sV[0][scg][sb] = hi;
        sV[TAYLOR ? 1 : 0][scg][sb] = mid;
        sV[TAYLOR ? 2 : 0][scg][sb] = lo;
      }
#pragma unroll
      for (int k = 0; k < NQ; ++k) {
        const int u = (int)threadIdx.x + kThreads * k;
        if (u < 2 * R * 64) {
          const int ul = u % 64, uh = (u / 64) % R, ut = u / (64 * R);
          const uint4 qv = cur.qa[k];
          sQ[0][ut][uh][ul] = qv;
          if (TAYLOR) {
            const uint32_t in[4] = {qv.x, qv.y, qv.z, qv.w};
            uint32_t oh[4], ol[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const float a0 = bf16_lo_f(in[p]), a1 = bf16_hi_f(in[p]);
              const float s0 = a0 * a0, s1 = a1 * a1;  // exact: 16 significant bits
              oh[p] = pack_bf16(s0, s1);
              ol[p] = pack_bf16(s0 - bf16_lo_f(oh[p]), s1 - bf16_hi_f(oh[p]));
            }
            sQ[TAYLOR ? 1 : 0][ut][uh][ul] = make_uint4(oh[0], oh[1], oh[2], oh[3]);
            sQ[TAYLOR ? 2 : 0][ut][uh][ul] = make_uint4(ol[0], ol[1], ol[2], ol[3]);
          }
        }
      }
    }
    __syncthreads();
    // the next k-step's loads go out while this one's products run
    if (ks + 1 < KS) load(ks + 1, nxt);
    // ---- products of this wavefront's token tile and column tiles
    uint4 mh[NC], mm[NC], ml[NC], vh[NC], vm[NC], vl[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
      const int ct = n0 + n;
      mh[n] = sM[0][lg4][16 * ct + l16];
      mm[n] = sM[1][lg4][16 * ct + l16];
      ml[n] = sM[2][lg4][16 * ct + l16];
      if (TAYLOR) {
        vh[n] = sV[0][lg4][16 * ct + l16];
        vm[n] = sV[TAYLOR ? 1 : 0][lg4][16 * ct + l16];
        vl[n] = sV[TAYLOR ? 2 : 0][lg4][16 * ct + l16];
      }
    }
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const uint4 qv = sQ[0][w >> 1][h][lane];
      uint4 sh, sl;
      if (TAYLOR) {
        sh = sQ[TAYLOR ? 1 : 0][w >> 1][h][lane];
        sl = sQ[TAYLOR ? 2 : 0][w >> 1][h][lane];
      }
#pragma unroll
      for (int n = 0; n < NC; ++n) {
        cm[n][h] = mfma_bf16x32(qv, ml[n], cm[n][h]);
        cm[n][h] = mfma_bf16x32(qv, mm[n], cm[n][h]);
        cm[n][h] = mfma_bf16x32(qv, mh[n], cm[n][h]);
        if (TAYLOR) {
          cv[n][h] = mfma_bf16x32(sl, vm[n], cv[n][h]);
          cv[n][h] = mfma_bf16x32(sh, vl[n], cv[n][h]);
          cv[n][h] = mfma_bf16x32(sl, vh[n], cv[n][h]);
          cv[n][h] = mfma_bf16x32(sh, vm[n], cv[n][h]);
          cv[n][h] = mfma_bf16x32(sh, vh[n], cv[n][h]);
        }
      }
    }
    if (ks + 1 < KS) {
      __syncthreads();  // every wavefront has read this k-step's operands
      cur = nxt;
    }
  }

  // ---- log scores, group logsumexp: lane holds tokens 4 lg4 + i, block 16 n + l16
  const float half_inv_d = 0.5f / (float)D;
  const size_t row = (size_t)n_tiles * kTile;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tk = tok0 + 4 * lg4 + i;
    if (tk >= m) continue;
    const int nb = (a.lens[tk] + a.bk - 1) / a.bk;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
      float ls[R];
#pragma unroll
      for (int h = 0; h < R; ++h)
        ls[h] = TAYLOR ? cm[n][h][i] * a.inv_sqrt_d + __logf(1.f + fmaxf(cv[n][h][i], 0.f) * half_inv_d)
                       : cm[n][h][i] * a.inv_sqrt_d;
      float lg = ls[0];
      if constexpr (R > 1) {
        float mx = ls[0];
#pragma unroll
        for (int h = 1; h < R; ++h) mx = fmaxf(mx, ls[h]);
        float e[R];
#pragma unroll
        for (int h = 0; h < R; ++h) e[h] = __expf(ls[h] - mx);
        // pairwise, in the decode scorer's order
#pragma unroll
        for (int st = 1; st < R; st *= 2)
#pragma unroll
          for (int h = 0; h < R; h += 2 * st) e[h] += e[h + st];
        lg = mx + __logf(e[0]);
      }
      const int jb = t * kTile + 16 * (n0 + n) + l16;
      const bool cand = jb >= 1 && jb <= nb - 2;
      a.lg[((size_t)tk * G + g) * row + jb] = cand ? lg : -INFINITY;
      if (a.lg_out && cand) a.lg_out[((size_t)tk * G + g) * a.max_blocks + jb] = lg;
    }
  }
}

template <bool BF16, bool TAYLOR>
hipError_t launch_pf_score_form(const DecodeArgs& a, const Launch& l) {
  const dim3 grid(a.score_tiles, a.G, (a.B + 31) / 32);
  if constexpr (BF16) {
    SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_pf_score_bf<RR, DD, TAYLOR>, grid, l, a.blk_mean, a.blk_var, a.q,
                                             a.n_tiles, a.G, a.H, a.B, a))
  } else {
    SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_pf_score<BF16, RR, DD, TAYLOR>, grid, l, a.blk_mean, a.blk_var,
                                             a.q, a.n_tiles, a.G, a.H, a.B, a))
  }
}

}  // namespace

// virtual queries only: a.B tokens of one sequence, whose statistics rows the
// pointers address
hipError_t launch_pf_score(const DecodeArgs& a, bool bf16, const Launch& l) {
  if (!a.virtual_queries || a.score_tiles <= 0) return hipErrorInvalidValue;
  const bool mean = a.score_form == kScoreMean;
  if (bf16) return mean ? launch_pf_score_form<true, false>(a, l) : launch_pf_score_form<true, true>(a, l);
  return mean ? launch_pf_score_form<false, false>(a, l) : launch_pf_score_form<false, true>(a, l);
}

}  // namespace spla
