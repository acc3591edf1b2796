// Attend + correct on the matrix cores (bf16 K/V): for one selected block,
// the exact-softmax partials (max, sum, sum p v) and the linear-attention
// partials (sum w v, sum w, w = phi(q).phi(k)) from the same K/V tile (SPLA
// Technical Summary 2.2: o_tilde from the blocks already loaded for the
// sparse pass).  Shared by the attend kernel and the fused select + attend
// kernel.
#pragma once

#include "decode_common.h"

namespace spla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));


__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  c, 0, 0, 0);
}

__device__ __forceinline__ float phi_fast(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// phi of 8 packed bf16 values as bf16 hi + lo pairs (hi = phi rounded to
// bf16, lo = the rounding of what is left), so hi + lo holds phi to ~2^-16
__device__ __forceinline__ void phi_bf16_split(const uint4& raw, uint4& hi, uint4& lo) {
  const uint32_t in[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t oh[4], ol[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x0 = phi_fast(bf16_lo_f(in[k])), x1 = phi_fast(bf16_hi_f(in[k]));
    oh[k] = pack_bf16(x0, x1);
    ol[k] = pack_bf16(x0 - bf16_lo_f(oh[k]), x1 - bf16_hi_f(oh[k]));
  }
  hi = make_uint4(oh[0], oh[1], oh[2], oh[3]);
  lo = make_uint4(ol[0], ol[1], ol[2], ol[3]);
}

// A operands of product (1) for this lane: row m = lane % 16 holds query m
// (m < R), or bf16 hi / lo of phi(query m - WB) (from the phi(q) array the
// first kernel of the decode wrote); other rows read row 0 and are masked
// when the operands are formed
template <int R, int D>
__device__ __forceinline__ void load_q_mfma(const void* q, const uint16_t* phq, int H, int g, int b,
                                            uint4 (&qraw)[D / 32], uint4 (&fh)[D / 32], uint4 (&fl)[D / 32]) {
  constexpr int WB = R <= 4 ? 4 : 8;
  const int lane = threadIdx.x % 64, m = lane % 16, lg4 = lane / 16;
  const int hq = m < R ? m : 0;
  const int hw = (m >= WB && m < WB + R) ? m - WB : 0;
  const uint16_t* fq = phq + ((size_t)b * H + g * R + hw) * 2 * D;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    qraw[ks] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) +
                                               ((size_t)b * H + g * R + hq) * D + 32 * ks + 8 * lg4);
    fh[ks] = *reinterpret_cast<const uint4*>(fq + 32 * ks + 8 * lg4);
    fl[ks] = *reinterpret_cast<const uint4*>(fq + D + 32 * ks + 8 * lg4);
  }
}

// Block j (page `page`) of (b, g), all R query heads, bf16 K/V; writes the
// partial record of `slot`.  Matrix cores do both contractions:
//   (1) logits s = q.k and linear weights w = phi(q).phi(k) of the block's
//       tokens: rows of the 16-row A operand are the R queries and the R
//       phi(q) (bf16 hi/lo split), B is the K tile read straight from the
//       page plus phi(K) hi/lo computed in registers; wavefront w takes 16
//       (Bk = 64) or 32 (Bk = 128) tokens;
//   (2) sum_t p_t v_t and sum_t w_t v_t: rows of A are p and w (hi/lo split,
//       from LDS), B is the V tile staged transposed in LDS; wavefront w
//       takes a quarter of the value channels.
// Softmax max / sums cross the wavefronts through LDS (two barriers).
// j < 0 (an unused slot) returns at once; j and page must be uniform over
// the workgroup.
template <int R, int D, int BK>
__device__ __forceinline__ void attend_block_mfma(const DecodeArgs& a, int slot, int g, int b, int j, int page,
                                                  const uint4 (&qraw)[D / 32], const uint4 (&fh)[D / 32],
                                                  const uint4 (&fl)[D / 32]) {
  constexpr int NKS = D / 32;              // k-steps per channel block
  constexpr int NT1W = BK / 64;            // 16-token tiles per wavefront
  constexpr int WB = R <= 4 ? 4 : 8;       // first linear-weight row of product (1)
  constexpr int NT2W = D / 64;             // 16-channel tiles per wavefront
  constexpr int MT2 = (4 * R + 15) / 16;   // row tiles of product (2): hi/lo rows of p and w
  constexpr int KS2 = BK / 32;             // token k-steps of product (2)
  constexpr int VS = BK + 8;               // row stride (elements) of the transposed V tile
  constexpr int PS = BK + 8;               // row stride of the p / w rows
  constexpr int NV = BK * D / (16 * kThreads);  // token-pair x 8-channel pieces per thread
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VS];
  __shared__ __attribute__((aligned(16))) uint16_t pw[MT2 * 16 * PS];
  __shared__ float s_max[4][R], s_l[4][R], s_sw[4][R];

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64, l16 = lane % 16, lg4 = lane / 16;
  const int m = l16;  // A-operand row of this lane in product (1)
  if (j < 0) return;
  const int T = a.lens[b];
  const int nb = n_blocks(a, b);
  if (j >= nb) {
    if (threadIdx.x == 0) atomicOr(a.err, kErrSel);
    return;
  }
  if (page < 0 || page >= a.num_pages) {
    if (threadIdx.x == 0) atomicOr(a.err, kErrPage);
    return;
  }
  const int ntok = min(BK, T - j * BK);
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.k_pages) + ((size_t)page * a.G + g) * BK * D;
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(a.v_pages) + ((size_t)page * a.G + g) * BK * D;

  // ---- issue every global load first: K operands, V pieces, queries
  uint4 kraw[NT1W][NKS];
#pragma unroll
  for (int nt = 0; nt < NT1W; ++nt) {
    const int tok = (w * NT1W + nt) * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kraw[nt][ks] = *reinterpret_cast<const uint4*>(kp + (size_t)tok * D + 32 * ks + 8 * lg4);
  }
  uint4 vr[NV][2];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = threadIdx.x + kThreads * i;
    const int tp = idx % (BK / 2), cg = idx / (BK / 2);
    vr[i][0] = *reinterpret_cast<const uint4*>(vp + (size_t)(2 * tp) * D + 8 * cg);
    vr[i][1] = *reinterpret_cast<const uint4*>(vp + (size_t)(2 * tp + 1) * D + 8 * cg);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (R < 4) {
    for (int i = threadIdx.x; i < MT2 * 16 * PS / 2; i += kThreads) reinterpret_cast<uint32_t*>(pw)[i] = 0u;
  }

  // ---- A operands of product (1)
  const bool is_q = m < R, is_w = m >= WB && m < WB + R;
  // rows that are not queries / phi(q) rows are zero (bit masks keep this
  // plain VALU work)
  const uint32_t mq = is_q ? 0xffffffffu : 0u, mw = is_w ? 0xffffffffu : 0u;
  uint4 aq[NKS], afh[NKS], afl[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    aq[ks] = make_uint4(qraw[ks].x & mq, qraw[ks].y & mq, qraw[ks].z & mq, qraw[ks].w & mq);
    afh[ks] = make_uint4(fh[ks].x & mw, fh[ks].y & mw, fh[ks].z & mw, fh[ks].w & mw);
    afl[ks] = make_uint4(fl[ks].x & mw, fl[ks].y & mw, fl[ks].z & mw, fl[ks].w & mw);
  }

  // ---- product (1): logits and linear weights of this wavefront's tokens
  f32x4_t c1[NT1W];
#pragma unroll
  for (int nt = 0; nt < NT1W; ++nt) {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      // w = phi(q).phi(k) from hi / lo pairs of both (the lo x lo product,
      // ~2^-18 relative, is left out).  A single bf16 phi(k) would leave
      // ~1e-4 relative error in sum w, which the subtraction
      // D = phi(q).z_all - sum w magnifies when few tokens are unselected.
      uint4 fkh, fkl;
      phi_bf16_split(kraw[nt][ks], fkh, fkl);
      c = mfma_bf16(aq[ks], kraw[nt][ks], c);
      c = mfma_bf16(afh[ks], fkh, c);
      c = mfma_bf16(afl[ks], fkh, c);
      c = mfma_bf16(afh[ks], fkl, c);
    }
    c1[nt] = c;
  }
  // lane (lg4, reg i) holds row 4*lg4 + i of the 16 x 16 result, token l16
  const float inv_sqrt_d = a.inv_sqrt_d;
  float mloc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int nt = 0; nt < NT1W; ++nt) {
    const int tok = (w * NT1W + nt) * 16 + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * lg4 + i;
      if (row < R && tok < ntok) mloc[i] = fmaxf(mloc[i], c1[nt][i] * inv_sqrt_d);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) mloc[i] = row16_max(mloc[i]);
  if (l16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * lg4 + i;
      if (row < R) s_max[w][row] = mloc[i];
    }
  }
  __syncthreads();
  // ---- p = exp(s - m) and w, split hi/lo, into the rows of product (2)
  float lsum[4] = {0.f, 0.f, 0.f, 0.f}, wsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < NT1W; ++nt) {
    const int tok = (w * NT1W + nt) * 16 + l16;
    const bool valid = tok < ntok;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * lg4 + i;
      int kind = -1, h = 0;
      float x = 0.f;
      if (row < R) {
        h = row;
        const float mh = fmaxf(fmaxf(s_max[0][h], s_max[1][h]), fmaxf(s_max[2][h], s_max[3][h]));
        x = valid ? __expf(c1[nt][i] * inv_sqrt_d - mh) : 0.f;
        lsum[i] += x;
        kind = 0;
      } else if (row >= WB && row < WB + R) {
        h = row - WB;
        x = valid ? c1[nt][i] : 0.f;
        wsum[i] += x;
        kind = 1;
      }
      if (kind >= 0) {
        // product (2) rows: pair pi = kind * R + h owns rows 2 pi (hi) and
        // 2 pi + 1 (lo), so one lane of the result holds both halves
        const uint32_t hb = pack_bf16(x, 0.f) & 0xffffu;
        const uint32_t lb = pack_bf16(x - bf16_lo_f(hb), 0.f) & 0xffffu;
        const int rh = 2 * (kind * R + h);
        pw[rh * PS + tok] = (uint16_t)hb;
        pw[(rh + 1) * PS + tok] = (uint16_t)lb;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lsum[i] = row16_sum(lsum[i]);
    wsum[i] = row16_sum(wsum[i]);
  }
  if (l16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * lg4 + i;
      if (row < R) s_l[w][row] = lsum[i];
      if (row >= WB && row < WB + R) s_sw[w][row - WB] = wsum[i];
    }
  }
  // ---- V tile, transposed into LDS (rows past the block's end are zero)
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = threadIdx.x + kThreads * i;
    const int tp = idx % (BK / 2), cg = idx / (BK / 2);
    const bool v0 = 2 * tp < ntok, v1 = 2 * tp + 1 < ntok;
    const uint32_t r0[4] = {vr[i][0].x, vr[i][0].y, vr[i][0].z, vr[i][0].w};
    const uint32_t r1[4] = {vr[i][1].x, vr[i][1].y, vr[i][1].z, vr[i][1].w};
    uint32_t* dst = reinterpret_cast<uint32_t*>(vt) + (size_t)(8 * cg) * (VS / 2) + tp;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a0 = v0 ? r0[k] : 0u, a1 = v1 ? r1[k] : 0u;
      dst[(2 * k) * (VS / 2)] = (a0 & 0xffffu) | (a1 << 16);
      dst[(2 * k + 1) * (VS / 2)] = (a0 >> 16) | (a1 & 0xffff0000u);
    }
  }
  __syncthreads();
  // ---- product (2)
  const int rec = 2 * D + kPartHdr;
  float* part0 = a.part + (((size_t)b * a.H + g * R) * a.top_k + slot) * rec;
#pragma unroll
  for (int nt2 = 0; nt2 < NT2W; ++nt2) {
    const int ch = (w * NT2W + nt2) * 16 + l16;
#pragma unroll
    for (int mt = 0; mt < MT2; ++mt) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS2; ++ks) {
        const uint4 av = *reinterpret_cast<const uint4*>(&pw[(mt * 16 + l16) * PS + 32 * ks + 8 * lg4]);
        const uint4 bv = *reinterpret_cast<const uint4*>(&vt[ch * VS + 32 * ks + 8 * lg4]);
        c = mfma_bf16(av, bv, c);
      }
      // lane group lg4 holds rows 4 lg4 .. 4 lg4 + 3 of tile mt: pairs
      // pi0 = 8 mt + 2 lg4 (hi + lo in c[0], c[1]) and pi0 + 1 (c[2], c[3])
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int pi = 8 * mt + 2 * lg4 + e;
        if (pi < 2 * R) {
          const int kind = pi / R, h = pi % R;
          part0[(size_t)h * a.top_k * rec + kPartHdr + (kind ? D : 0) + ch] = c[2 * e] + c[2 * e + 1];
        }
      }
    }
  }
  if (threadIdx.x < R) {
    const int h = threadIdx.x;
    float* dst = part0 + (size_t)h * a.top_k * rec;
    dst[0] = fmaxf(fmaxf(s_max[0][h], s_max[1][h]), fmaxf(s_max[2][h], s_max[3][h])) ;
    dst[1] = (s_l[0][h] + s_l[1][h]) + (s_l[2][h] + s_l[3][h]);
    dst[2] = (s_sw[0][h] + s_sw[1][h]) + (s_sw[2][h] + s_sw[3][h]);
    dst[3] = 0.f;
  }
}


}  // namespace
}  // namespace spla
