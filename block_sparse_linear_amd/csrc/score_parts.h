// Work items of the first kernel of a decode (block scores of one 64-block
// tile; the S_all row chunks with their o_bar partials), shared by the
// scorer kernels and the one-kernel decode step.  Each function is executed
// by a whole 256-thread workgroup; its LDS comes in as a struct, so a kernel
// that runs several kinds of item can overlay them.
#pragma once

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
template <int R, int D>
struct ScoreTileLds {
  float4 qs[4][R][D / 16];   // q of each wavefront's channel quarter
  float4 q2s[4][R][D / 16];  // and its square
  float red[4][2 * R][kTile];
};

// a float4 that is read (or written) once per call, streamed past the caches
__device__ __forceinline__ float4 load_stream4(const float4* p) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const v4f x = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
  return make_float4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ void store_stream4(float4* p, const float4& v) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  v4f x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<v4f*>(p));
}

template <bool BF16, int R, int D, bool TAYLOR>
__device__ void score_tile(const DecodeArgs& a, const int t, const int g, const int b, const ScorePre& p,
                           ScoreTileLds<R, D>& L) {
  constexpr int NC4 = D / 16;  // channel quartets per wavefront
  constexpr int CW = D / 4;    // channels per wavefront
  constexpr int QPL = (R * CW + 63) / 64;  // query elements per lane
  auto& qs = L.qs;
  auto& q2s = L.q2s;
  auto& red = L.red;
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
  for (int i = 0; i < NC4; ++i) m[i] = load_stream4(&mean4[base + (size_t)i * kTile]);
#pragma unroll
  for (int i = 0; i < NC4; ++i)
    v[i] = TAYLOR ? load_stream4(&var4[base + (size_t)i * kTile]) : make_float4(0.f, 0.f, 0.f, 0.f);
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
// CPW > 1: one workgroup takes CPW consecutive chunks (for batches with so
// many (b, g) pairs that a workgroup per chunk costs more in workgroup
// overhead than it gains in spread).
template <int R, int D>
struct StateRowsLds {
  float4 red[R][1024 / D][D / 4];
  float zred[R][1024 / D];
};

template <bool BF16, int R, int D, bool UPDATE, int CPW = 1, bool STREAM = false>
__device__ void state_rows(const DecodeArgs& dc, const StateRefs& st, int b, int g, int rc0, StateRowsLds<R, D>& L) {
  constexpr int ROWS = 1024 / D, C4N = D / 4, CHUNKS = D / ROWS;
  auto& red = L.red;
  auto& zred = L.zred;
  const int xr = threadIdx.x / C4N, c4 = threadIdx.x % C4N;
  const size_t bg = (size_t)b * dc.G + g;
  // CPW consecutive chunks rc0 .. rc0 + CPW - 1: every load first, then one
  // chunk after the other through the same LDS (each chunk's arithmetic and
  // partials as when it has a workgroup of its own)
  float4 s[CPW];
  float zx[CPW], qx[CPW][R], kx[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int x = (rc0 + c) * ROWS + xr;
    const float4* sp = reinterpret_cast<const float4*>(st.s_all) + (bg * D + x) * C4N + c4;
    s[c] = STREAM ? load_stream4(sp) : *sp;
    zx[c] = st.z_all[bg * D + x];
#pragma unroll
    for (int h = 0; h < R; ++h) qx[c][h] = load_elem<BF16>(dc.q, ((size_t)b * dc.H + g * R + h) * D + x);
    if constexpr (UPDATE) kx[c] = load_elem<BF16>(st.k_new, bg * D + x);
  }
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (UPDATE) v = load4<BF16>(st.v_new, bg * D + c4 * 4);
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int rc = rc0 + c, x = rc * ROWS + xr;
    if (c > 0) __syncthreads();  // the previous chunk's partials are read out of LDS
    if constexpr (UPDATE) {
      const float f = phi_f(kx[c]);
      s[c] = make_float4(s[c].x + fmaf(f, v.x, 0.f), s[c].y + fmaf(f, v.y, 0.f), s[c].z + fmaf(f, v.z, 0.f),
                         s[c].w + fmaf(f, v.w, 0.f));
      zx[c] = zx[c] + (0.f + f);
      float4* sp = reinterpret_cast<float4*>(st.s_all) + (bg * D + x) * C4N + c4;
      if constexpr (STREAM) {
        store_stream4(sp, s[c]);
      } else {
        *sp = s[c];
      }
      if (c4 == 0) st.z_all[bg * D + x] = zx[c];
    }
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const float fq = phi_f(qx[c][h]);
      red[h][xr][c4] = make_float4(fq * s[c].x, fq * s[c].y, fq * s[c].z, fq * s[c].w);
      if (c4 == 0) {
        zred[h][xr] = fq * zx[c];
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
      const int h = i / C4N, cc = i % C4N;
      float4 acc = red[h][0][cc];
#pragma unroll
      for (int r = 1; r < ROWS; ++r) {
        const float4 t = red[h][r][cc];
        acc = make_float4(acc.x + t.x, acc.y + t.y, acc.z + t.z, acc.w + t.w);
      }
      reinterpret_cast<float4*>(dc.obar_part)[((bg * CHUNKS + rc) * R + h) * C4N + cc] = acc;
    }
    if ((int)threadIdx.x < R) {
      const int h = threadIdx.x;
      float acc = zred[h][0];
#pragma unroll
      for (int r = 1; r < ROWS; ++r) acc += zred[h][r];
      dc.dz_part[(bg * CHUNKS + rc) * R + h] = acc;
    }
  }
}

// the LDS of the three kinds of item a decode step's first kernel runs (a
// workgroup runs one kind, so they overlay)
template <bool BF16, int R, int D>
union ProducerLds {
  ScoreTileLds<R, D> score;
  StateRowsLds<R, D> state;
  BlockStatsLds<BF16> stats;
};

}  // namespace
}  // namespace spla
