// Block scorer: log-domain second-order Taylor score of every candidate block,
// summed over the query heads of a KV group (SPLA Technical Summary 2.1, score
// formula with the diagonal covariance of its implementation paragraph), and
// the fused decode-step kernel that also carries the one-token append.
#include "decode_common.h"

namespace spla {

namespace {

// ============================================================== score
// Arguments the first loads of a score tile need.  The kernels take them
// ahead of their argument struct, so with kernel-argument preloading they are
// in SGPRs when the wave starts.
struct ScorePre {
  const float* mean;
  const float* var;
  const void* q;
  int32_t n_tiles, G, H;
  int32_t tiles_all;  // tiles every sequence of the batch has: their loads need no length
};

// grid (score_tiles, G, B); lane = block within a 64-block tile, the four
// wavefronts split the channels and meet in LDS.  Every wavefront issues its
// query loads and then all of its statistics loads before the first wait.
// TAYLOR = false is the first-order (mean-pooling) score q_hat . mean, which
// reads no variances: the baseline the second-order selection is measured
// against.
template <bool BF16, int R, int D, bool TAYLOR>
__device__ void score_tile(const DecodeArgs& a, const int t, const int g, const int b, const ScorePre& p) {
  constexpr int NC4 = D / 16;  // channel quartets per wavefront
  constexpr int CW = D / 4;    // channels per wavefront
  constexpr int QPL = (R * CW + 63) / 64;  // query elements per lane
  __shared__ float4 qs[4][R][CW / 4];
  __shared__ float4 q2s[4][R][CW / 4];
  __shared__ float red[4][2 * R][kTile];
  if (t >= p.tiles_all) {
    // a tile that only some sequences have: this one's length decides first
    const int nbs = n_blocks(a, b);
    if (nbs <= a.top_k || t * kTile > nbs - 2) return;
  }
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  // queries of this wavefront's channel quarter
  // (loads are unconditional, from clamped in-range addresses, and masked
  // afterwards: a load under a branch makes the compiler wait for it there)
  float qv[QPL];
#pragma unroll
  for (int i = 0; i < QPL; ++i) {
    const int e = min(lane + 64 * i, R * CW - 1);
    const int h = e / CW, c = e - h * CW;
    qv[i] = load_elem<BF16>(p.q, ((size_t)b * p.H + g * R + h) * D + w * CW + c);
  }
  // statistics of the tile: 64 blocks x this wavefront's channels
  const float4* mean4 = reinterpret_cast<const float4*>(p.mean);
  const float4* var4 = reinterpret_cast<const float4*>(p.var);
  const size_t base = (((size_t)b * p.G + g) * p.n_tiles + t) * (size_t)(D / 4) * kTile +
                      (size_t)(w * NC4) * kTile + lane;
  float4 m[NC4], v[NC4];
#pragma unroll
  for (int i = 0; i < NC4; ++i) m[i] = mean4[base + (size_t)i * kTile];
#pragma unroll
  for (int i = 0; i < NC4; ++i) v[i] = TAYLOR ? var4[base + (size_t)i * kTile] : make_float4(0.f, 0.f, 0.f, 0.f);
  // keep every load above this point: the whole tile is in flight before the
  // first use
  __builtin_amdgcn_sched_barrier(0);
  // the rest of the arguments, while the tile is in flight
  const int T = a.lens[b];
  SPLA_SCALARS_READY("s"(T), "s"(a.bk), "s"(a.lg), "s"(a.lg_out), "s"(a.max_blocks), "s"(a.inv_sqrt_d));
  const int nb = (T + a.bk - 1) / a.bk;
  const int j0 = t * kTile;
  // wavefront-private staging of q and q^2 (LDS operations of one wavefront
  // complete in order, so no barrier is needed)
  float* qf = reinterpret_cast<float*>(&qs[w][0][0]);
  float* q2f = reinterpret_cast<float*>(&q2s[w][0][0]);
#pragma unroll
  for (int i = 0; i < QPL; ++i) {
    const int e = lane + 64 * i;
    if (e < R * CW) {
      qf[e] = qv[i];
      q2f[e] = qv[i] * qv[i];
    }
  }
  float dot[R], qq[R];
#pragma unroll
  for (int h = 0; h < R; ++h) dot[h] = qq[h] = 0.f;
#pragma unroll
  for (int i = 0; i < NC4; ++i) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const float4 q = qs[w][h][i];
      const float4 q2 = q2s[w][h][i];
      dot[h] = fmaf(q.x, m[i].x, dot[h]);
      dot[h] = fmaf(q.y, m[i].y, dot[h]);
      dot[h] = fmaf(q.z, m[i].z, dot[h]);
      dot[h] = fmaf(q.w, m[i].w, dot[h]);
      if (!TAYLOR) continue;
      qq[h] = fmaf(q2.x, v[i].x, qq[h]);
      qq[h] = fmaf(q2.y, v[i].y, qq[h]);
      qq[h] = fmaf(q2.z, v[i].z, qq[h]);
      qq[h] = fmaf(q2.w, v[i].w, qq[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < R; ++h) {
    red[w][h][lane] = dot[h];
    red[w][R + h][lane] = qq[h];
  }
  __syncthreads();
  // finalisation spread over the four wavefronts: lane = (block, head), the
  // R lanes of a block combine their log scores with DPP (max, exp-sum)
  constexpr int BPW = 64 / R;  // blocks per wavefront pass
  const float half_inv_d = 0.5f / (float)D;
  const int h = lane % R;
  for (int blk0 = w * BPW; blk0 < kTile; blk0 += 4 * BPW) {
    const int blk = blk0 + lane / R;
    const float dd = (red[0][h][blk] + red[1][h][blk]) + (red[2][h][blk] + red[3][h][blk]);
    const float vv = (red[0][R + h][blk] + red[1][R + h][blk]) + (red[2][R + h][blk] + red[3][R + h][blk]);
    const float ls = TAYLOR ? dd * a.inv_sqrt_d + __logf(1.f + fmaxf(vv, 0.f) * half_inv_d) : dd * a.inv_sqrt_d;
    float lg = ls;
    if constexpr (R > 1) {
      float mx = ls;
      mx = fmaxf(mx, dpp_f<kDppXor1>(mx, mx));
      if constexpr (R > 2) mx = fmaxf(mx, dpp_f<kDppXor2>(mx, mx));
      if constexpr (R > 4) mx = fmaxf(mx, dpp_f<kDppRowHalfMirror>(mx, mx));
      float e = __expf(ls - mx);
      e += dpp_f<kDppXor1>(0.f, e);
      if constexpr (R > 2) e += dpp_f<kDppXor2>(0.f, e);
      if constexpr (R > 4) e += dpp_f<kDppRowHalfMirror>(0.f, e);
      lg = mx + __logf(e);
    }
    const int j = j0 + blk;
    if (h == 0) {
      const bool cand = j >= 1 && j <= nb - 2;
      a.lg[((size_t)b * p.G + g) * (size_t)(p.n_tiles * kTile) + j] = cand ? lg : -INFINITY;
      if (a.lg_out && cand) a.lg_out[((size_t)b * p.G + g) * a.max_blocks + j] = lg;
    }
  }
}

// ============================================================== S_all rows
// One chunk of 1024 / D rows x of S_all for (b, g) (thread = row x, value
// channel quartet c4), in the first kernel of a decode:
//   update   (fused step) S[x][:] += phi(k[x]) v and z[x] += phi(k[x]) for
//            the step's token, with the same rounding as the append kernel
//            (phi(k) v formed alone, then added);
//   o_bar    partial phi(q_h)^T S and phi(q_h).z over the chunk's rows for
//            every query head h of the group, from the rows just read or
//            updated (so the token attends to itself): the combine sums the
//            D * D / 1024 chunks and never reads S_all.
template <bool BF16, int R, int D, bool UPDATE>
__device__ void state_rows(const DecodeArgs& dc, const StateRefs& st, int b, int g, int rc) {
  constexpr int ROWS = 1024 / D, C4N = D / 4, CHUNKS = D / ROWS;
  __shared__ float4 red[R][ROWS][C4N];
  __shared__ float zred[R][ROWS];
  const int xr = threadIdx.x / C4N, c4 = threadIdx.x % C4N;
  const int x = rc * ROWS + xr;
  const size_t bg = (size_t)b * dc.G + g;
  float4* S = reinterpret_cast<float4*>(st.s_all) + (bg * D + x) * C4N + c4;
  float* z = st.z_all + bg * D + x;
  float4 s = *S;
  float zx = *z;
  float qx[R];
#pragma unroll
  for (int h = 0; h < R; ++h) qx[h] = load_elem<BF16>(dc.q, ((size_t)b * dc.H + g * R + h) * D + x);
  if constexpr (UPDATE) {
    const float f = phi_f(load_elem<BF16>(st.k_new, bg * D + x));
    const float4 v = load4<BF16>(st.v_new, bg * D + c4 * 4);
    s = make_float4(s.x + fmaf(f, v.x, 0.f), s.y + fmaf(f, v.y, 0.f), s.z + fmaf(f, v.z, 0.f),
                    s.w + fmaf(f, v.w, 0.f));
    zx = zx + (0.f + f);
    *S = s;
    if (c4 == 0) *z = zx;
  }
#pragma unroll
  for (int h = 0; h < R; ++h) {
    const float fq = phi_f(qx[h]);
    red[h][xr][c4] = make_float4(fq * s.x, fq * s.y, fq * s.z, fq * s.w);
    if (c4 == 0) {
      zred[h][xr] = fq * zx;
      // phi(q) of row x as bf16 hi + lo for the attend kernel's matrix-core
      // operands (hi + lo carries phi to ~2^-16 relative)
      const uint32_t hi = pack_bf16(fq, 0.f) & 0xffffu;
      const uint32_t lo = pack_bf16(fq - bf16_lo_f(hi), 0.f) & 0xffffu;
      uint16_t* dst = dc.phq + ((size_t)b * dc.H + g * R + h) * 2 * D + x;
      dst[0] = (uint16_t)hi;
      dst[D] = (uint16_t)lo;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < R * C4N; i += kThreads) {
    const int h = i / C4N, c = i % C4N;
    float4 acc = red[h][0][c];
#pragma unroll
    for (int r = 1; r < ROWS; ++r) {
      const float4 t = red[h][r][c];
      acc = make_float4(acc.x + t.x, acc.y + t.y, acc.z + t.z, acc.w + t.w);
    }
    reinterpret_cast<float4*>(dc.obar_part)[((bg * CHUNKS + rc) * R + h) * C4N + c] = acc;
  }
  if ((int)threadIdx.x < R) {
    const int h = threadIdx.x;
    float acc = zred[h][0];
#pragma unroll
    for (int r = 1; r < ROWS; ++r) acc += zred[h][r];
    dc.dz_part[(bg * CHUNKS + rc) * R + h] = acc;
  }
}

// spla_decode, first launch, grid (score_tiles + D * D / 1024, G, B): for
// each (b, g) the scorer's tiles, then the o_bar partials of the S_all row
// chunks.
template <bool BF16, int R, int D, bool TAYLOR>
__global__ __launch_bounds__(kThreads) void k_score(const float* mean, const float* var, const void* q,
                                                     int32_t n_tiles, int32_t G, int32_t H, int32_t tiles_all,
                                                     int32_t score_tiles, const StepArgs a) {
  const int x = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (x < score_tiles) {
    const ScorePre p{mean, var, q, n_tiles, G, H, tiles_all};
    score_tile<BF16, R, D, TAYLOR>(a.dec, x, g, b, p);
    return;
  }
  SPLA_SCALARS_READY("s"(a.st.s_all), "s"(a.st.z_all), "s"(a.dec.obar_part), "s"(a.dec.dz_part));
  state_rows<BF16, R, D, false>(a.dec, a.st, b, g, x - score_tiles);
}

// Fused decode step, first launch, grid (score_tiles + D * D / 1024 + 1, G,
// B): for each (b, g), the scorer's tiles, then the S_all / z_all update of
// this step's token in row chunks (with their o_bar partials), then the
// token's page row and the statistics of the block it completes.  The two
// parts are independent: the scorer reads statistics of candidate blocks
// 1..nb-2 only, all completed by earlier appends, and neither pages nor
// S_all.
template <bool BF16, int R, int D, bool TAYLOR>
__global__ __launch_bounds__(kThreads) void k_step_score(const float* mean, const float* var, const void* q,
                                                          int32_t n_tiles, int32_t G, int32_t H, int32_t tiles_all,
                                                          int32_t score_tiles, const StepArgs a) {
  constexpr int kChunks = D / (1024 / D);  // S_all row chunks per (b, g)
  const DecodeArgs& dc = a.dec;
  const int x = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (x < score_tiles) {
    const ScorePre p{mean, var, q, n_tiles, G, H, tiles_all};
    score_tile<BF16, R, D, TAYLOR>(dc, x, g, b, p);
    return;
  }
  SPLA_SCALARS_READY("s"(dc.bk), "s"(a.st.k_new), "s"(a.st.v_new), "s"(a.st.s_all), "s"(a.st.z_all),
                     "s"(dc.obar_part), "s"(dc.dz_part), "s"(a.st.block_table), "s"(a.st.k_pages),
                     "s"(a.st.v_pages));
  if (x < score_tiles + kChunks) {
    state_rows<BF16, R, D, true>(dc, a.st, b, g, x - score_tiles);
    return;
  }
  const int T = dc.lens[b];  // after the append
  const AppendEntry E{b, 1, T - 1, b};
  append_page_row_head<BF16>(a.st, E, g);
  if (T % dc.bk == 0) append_block_stats<BF16>(a.st, E, T / dc.bk - 1, g);
}

template <bool TAYLOR>
hipError_t launch_score_form(const StepArgs& a, bool bf16, const Launch& l) {
  const DecodeArgs& d = a.dec;
  const int chunks = d.d / (1024 / d.d);
  const dim3 grid(d.score_tiles + chunks, d.G, d.B);
  if (bf16)
    SPLA_DISPATCH_RD(d.r, d.d, launch_kernel(k_score<true, RR, DD, TAYLOR>, grid, l, d.blk_mean, d.blk_var,
                                             d.q, d.n_tiles, d.G, d.H, d.tiles_all, d.score_tiles, a))
  SPLA_DISPATCH_RD(d.r, d.d, launch_kernel(k_score<false, RR, DD, TAYLOR>, grid, l, d.blk_mean, d.blk_var,
                                           d.q, d.n_tiles, d.G, d.H, d.tiles_all, d.score_tiles, a))
}

template <bool TAYLOR>
hipError_t launch_step_score_form(const StepArgs& a, bool bf16, const Launch& l) {
  const int chunks = a.dec.d / (1024 / a.dec.d);
  const dim3 grid(a.dec.score_tiles + chunks + 1, a.dec.G, a.dec.B);
  const DecodeArgs& d = a.dec;
  if (bf16)
    SPLA_DISPATCH_RD(d.r, d.d, launch_kernel(k_step_score<true, RR, DD, TAYLOR>, grid, l, d.blk_mean, d.blk_var,
                                             d.q, d.n_tiles, d.G, d.H, d.tiles_all, d.score_tiles, a))
  SPLA_DISPATCH_RD(d.r, d.d, launch_kernel(k_step_score<false, RR, DD, TAYLOR>, grid, l, d.blk_mean, d.blk_var,
                                           d.q, d.n_tiles, d.G, d.H, d.tiles_all, d.score_tiles, a))
}

}  // namespace

hipError_t launch_score(const StepArgs& a, bool bf16, const Launch& l) {
  if (a.dec.virtual_queries) return hipErrorInvalidValue;  // a prefill group is scored by k_pf_score
  return a.dec.score_form == kScoreMean ? launch_score_form<false>(a, bf16, l) : launch_score_form<true>(a, bf16, l);
}

hipError_t launch_step_score(const StepArgs& a, bool bf16, const Launch& l) {
  return a.dec.score_form == kScoreMean ? launch_step_score_form<false>(a, bf16, l)
                                        : launch_step_score_form<true>(a, bf16, l);
}

}  // namespace spla
