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

// 16 bytes of a K/V tile: read once per call, streamed past the caches
__device__ __forceinline__ uint4 load_stream_u4(const uint16_t* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
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

// V tiles in LDS are row-major (token rows of D bf16), each row's 16-byte
// chunks permuted by the row: chunk c of token row t sits at chunk position
// c ^ vswz(t).  The transposing reads of product (2) take 8 bytes from each of
// 16 rows (4 rows 8 apart per 16-lane group); the permutation spreads those
// rows over the LDS banks so that every bank serves two of the 64 reads, the
// fewest 512 bytes allow.
template <int D>
__device__ __forceinline__ int vswz(int t) {
  return (2 * (((t >> 3) & 3) | ((t & 1) << 2))) & (D / 8 - 1);
}

typedef __bf16 bf16x4v_t __attribute__((__vector_size__(4 * sizeof(__bf16))));

// 16-lane groups of a transposing LDS read (gfx950): source lane 4 e + q of
// the group gives the address of 4 consecutive bf16 (positions 0..3); lane i
// of the group receives position i % 4 of source lanes i / 4, 4 + i / 4,
// 8 + i / 4, 12 + i / 4, in that order
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const auto lp = (__attribute__((address_space(3))) bf16x4v_t*)(p);
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}

// 16 bytes from global memory into LDS, lane i of the wavefront to
// lds_block + 16 i (lds_block uniform over the wavefront), no registers
__device__ __forceinline__ void load_to_lds16(const void* src, uint16_t* lds_block) {
  __builtin_amdgcn_global_load_lds(const_cast<void*>(src), (__attribute__((address_space(3))) void*)(lds_block), 16, 0,
                                   0);
}

// A operands of product (1), loaded before the block is known.  A row of a
// matrix product depends on that row of A alone, so rows that hold nothing
// useful read any valid data and their results are never used.
//  - Packed (R <= 4): one row set per k-step.  Row m < R holds query m, row
//    4 + h the bf16 hi part of phi(query h), row 8 + h its lo part (from the
//    phi(q) array the first kernel of the decode wrote).  Three products per
//    k-step, against K, phi(K) hi and phi(K) lo, give q.k in rows < R of one
//    accumulator and the hi and lo halves of phi(q).phi(k) in rows 4 + h and
//    8 + h of another.
//  - Otherwise (R = 8): q in rows m < R, phi(q) hi and lo in rows 8 + h of two
//    more row sets, masked to zero elsewhere, all in one accumulator.
template <int R, int D>
struct QOps {
  static constexpr bool kPacked = R <= 4;
  static constexpr int kRows = kPacked ? 1 : 3;
  uint4 a[kRows][D / 32];
};

// this lane's A-row pointer of the packed form: q rows, phi(q) hi / lo rows,
// or query 0 for the unused rows
template <int R, int D>
__device__ __forceinline__ const uint16_t* packed_row(const void* q, const uint16_t* phq, int H, int g, int b,
                                                      bool with_phi) {
  const int m = (threadIdx.x % 64) % 16;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(q) + ((size_t)b * H + g * R) * D;
  const uint16_t* fp = phq + ((size_t)b * H + g * R) * 2 * D;
  if (m < R) return qp + (size_t)m * D;
  if (with_phi && m >= 4 && m < 4 + R) return fp + (size_t)(m - 4) * 2 * D;
  if (with_phi && m >= 8 && m < 8 + R) return fp + (size_t)(m - 8) * 2 * D + D;
  return qp;
}

// the rows that come from q (the packed form's phi rows get query 0 for now)
template <int R, int D>
__device__ __forceinline__ void load_qops_q(const void* q, int H, int g, int b, QOps<R, D>& o) {
  const int lane = threadIdx.x % 64, m = lane % 16, lg4 = lane / 16;
  if constexpr (QOps<R, D>::kPacked) {
    const uint16_t* p = packed_row<R, D>(q, reinterpret_cast<const uint16_t*>(q), H, g, b, false);  // no phi rows
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) o.a[0][ks] = *reinterpret_cast<const uint4*>(p + 32 * ks + 8 * lg4);
  } else {
    const int hq = m < R ? m : 0;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      o.a[0][ks] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) +
                                                   ((size_t)b * H + g * R + hq) * D + 32 * ks + 8 * lg4);
  }
}

// the rows that come from phi(q) (after load_qops_q)
template <int R, int D>
__device__ __forceinline__ void load_qops_phi(const uint16_t* phq, int H, int g, int b, QOps<R, D>& o) {
  const int lane = threadIdx.x % 64, m = lane % 16, lg4 = lane / 16;
  if constexpr (QOps<R, D>::kPacked) {
    const bool hi = m >= 4 && m < 4 + R, lo = m >= 8 && m < 8 + R;
    const uint16_t* fq = phq + ((size_t)b * H + g * R + (hi ? m - 4 : (lo ? m - 8 : 0))) * 2 * D + (lo ? D : 0);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const uint4 v = *reinterpret_cast<const uint4*>(fq + 32 * ks + 8 * lg4);
      if (hi || lo) o.a[0][ks] = v;
    }
  } else {
    constexpr int WB = 8;
    const int hw = (m >= WB && m < WB + R) ? m - WB : 0;
    const uint16_t* fq = phq + ((size_t)b * H + g * R + hw) * 2 * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      o.a[1][ks] = *reinterpret_cast<const uint4*>(fq + 32 * ks + 8 * lg4);
      o.a[2][ks] = *reinterpret_cast<const uint4*>(fq + D + 32 * ks + 8 * lg4);
    }
  }
}

// both: one load per k-step in the packed form
template <int R, int D>
__device__ __forceinline__ void load_qops(const void* q, const uint16_t* phq, int H, int g, int b, QOps<R, D>& o) {
  if constexpr (QOps<R, D>::kPacked) {
    const int lg4 = (threadIdx.x % 64) / 16;
    const uint16_t* p = packed_row<R, D>(q, phq, H, g, b, true);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) o.a[0][ks] = *reinterpret_cast<const uint4*>(p + 32 * ks + 8 * lg4);
  } else {
    load_qops_q<R, D>(q, H, g, b, o);
    load_qops_phi<R, D>(phq, H, g, b, o);
  }
}

// Block j (page `page`) of (b, g), all R query heads, bf16 K/V; writes the
// partial record of `slot`.  Matrix cores do both contractions:
//   (1) logits s = q.k and linear weights w = phi(q).phi(k) of the block's
//       tokens: rows of the 16-row A operand are the R queries and the R
//       phi(q) (bf16 hi/lo split; layouts at QOps), B is the K tile read
//       straight from the page plus phi(K) hi/lo computed in registers;
//       wavefront w takes 16 (Bk = 64) or 32 (Bk = 128) tokens;
//   (2) sum_t p_t v_t and sum_t w_t v_t: rows of A are p and w (hi/lo split,
//       from LDS), B is the V tile in LDS; wavefront w takes a quarter of the
//       value channels.  VLDS: the V tile goes from the page straight into
//       LDS (row-major, chunks permuted by vswz), with no registers and whole
//       1 KB runs per load instruction, and B is read with transposing LDS
//       reads; the compiler then waits for V as well as K before product
//       (1).  Otherwise V is loaded into registers with K and written
//       transposed into LDS after product (1), so product (1) waits for K
//       only: the form for a kernel bound by one workgroup's latency.
// Softmax max / sums cross the wavefronts through LDS (two barriers).
// j < 0 (an unused slot) returns at once; j and page must be uniform over
// the workgroup.
template <int R, int D, int BK, bool VLDS = false>
__device__ __forceinline__ void attend_block_mfma(const DecodeArgs& a, int slot, int g, int b, int j, int page,
                                                  const QOps<R, D>& qo) {
  constexpr int NKS = D / 32;              // k-steps per channel block
  constexpr int NT1W = BK / 64;            // 16-token tiles per wavefront
  constexpr int WB = R <= 4 ? 4 : 8;       // first linear-weight row of product (1)
  constexpr int NT2W = D / 64;             // 16-channel tiles per wavefront
  constexpr int MT2 = (4 * R + 15) / 16;   // row tiles of product (2): hi/lo rows of p and w
  constexpr int KS2 = BK / 32;             // token k-steps of product (2)
  constexpr int PS = BK + 8;               // row stride of the p / w rows
  // VLDS: row-major V tile
  constexpr int NC = D / 8;                // 16-byte chunks of a V row
  constexpr int RPI = 64 * 16 / (2 * D);   // V rows per 1 KB load instruction of a wavefront
  constexpr int NVI = BK * D * 2 / (kThreads * 16);  // V load instructions per wavefront
  // otherwise: V tile transposed (channel rows)
  constexpr int VS = BK + 8;               // row stride (elements) of the transposed V tile
  constexpr int NV = BK * D / (16 * kThreads);  // token-pair x 8-channel pieces per thread
  __shared__ __attribute__((aligned(16))) uint16_t vs[VLDS ? BK * D : D * VS];
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

  // ---- issue every global load first: K operands, V, queries
  uint4 kraw[NT1W][NKS];
#pragma unroll
  for (int nt = 0; nt < NT1W; ++nt) {
    const int tok = (w * NT1W + nt) * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kraw[nt][ks] = load_stream_u4(kp + (size_t)tok * D + 32 * ks + 8 * lg4);
  }
  uint4 vr[VLDS ? 1 : NV][2];
  if constexpr (VLDS) {
    // 1 KB block bl = NVI w + i of the tile per instruction, lane -> token
    // row bl RPI + lane / NC, chunk position lane % NC (holding chunk
    // (lane % NC) ^ vswz(row) of the row).  Rows past the block's end take
    // token 0's data instead: their p and w are exactly zero in product (2),
    // so finite values there add exactly zero, and no page row past the last
    // written token is read.
#pragma unroll
    for (int i = 0; i < NVI; ++i) {
      const int bl = NVI * w + i;
      const int t = bl * RPI + lane / NC, cp = lane % NC;
      load_to_lds16(vp + (size_t)(t < ntok ? t : 0) * D + 8 * (cp ^ vswz<D>(t)), vs + bl * 512);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = threadIdx.x + kThreads * i;
      const int tp = idx % (BK / 2), cg = idx / (BK / 2);
      vr[i][0] = load_stream_u4(vp + (size_t)(2 * tp) * D + 8 * cg);
      vr[i][1] = load_stream_u4(vp + (size_t)(2 * tp + 1) * D + 8 * cg);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (R < 4) {
    for (int i = threadIdx.x; i < MT2 * 16 * PS / 2; i += kThreads) reinterpret_cast<uint32_t*>(pw)[i] = 0u;
  }

  // ---- product (1): logits and linear weights of this wavefront's tokens.
  // w = phi(q).phi(k) from bf16 hi / lo pairs of both: a single bf16 phi(k)
  // would leave ~1e-4 relative error in sum w, which the subtraction
  // D = phi(q).z_all - sum w magnifies when few tokens are unselected.
  // c1: lane (lg4, reg i) holds row 4 lg4 + i of the 16 x 16 result for
  // token l16, with rows < R the logits and rows WB + h the linear weights
  f32x4_t c1[NT1W];
  if constexpr (QOps<R, D>::kPacked) {
#pragma unroll
    for (int nt = 0; nt < NT1W; ++nt) {
      f32x4_t cs = {0.f, 0.f, 0.f, 0.f}, cw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint4 fkh, fkl;
        phi_bf16_split(kraw[nt][ks], fkh, fkl);
        cs = mfma_bf16(qo.a[0][ks], kraw[nt][ks], cs);
        cw = mfma_bf16(qo.a[0][ks], fkh, cw);
        cw = mfma_bf16(qo.a[0][ks], fkl, cw);
      }
      // rows 4 + h (lane group 1) hold phi_hi(q_h).phi(k), rows 8 + h (lane
      // group 2, 16 lanes up) phi_lo(q_h).phi(k): their sum is w
      const int src = ((lane + 16) & 63) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float up = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(cw[i])));
        c1[nt][i] = lg4 == 1 ? cw[i] + up : cs[i];
      }
    }
  } else {
    // q rows and phi(q) rows in one accumulator: rows that are not queries /
    // phi(q) rows of each operand are zero (bit masks keep this plain VALU
    // work); the lo x lo product (~2^-18 relative) is left out
    const bool is_q = m < R, is_w = m >= WB && m < WB + R;
    const uint32_t mq = is_q ? 0xffffffffu : 0u, mw = is_w ? 0xffffffffu : 0u;
    uint4 aq[NKS], afh[NKS], afl[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint4 q0 = qo.a[0][ks], f0 = qo.a[1 % QOps<R, D>::kRows][ks], f1 = qo.a[2 % QOps<R, D>::kRows][ks];
      aq[ks] = make_uint4(q0.x & mq, q0.y & mq, q0.z & mq, q0.w & mq);
      afh[ks] = make_uint4(f0.x & mw, f0.y & mw, f0.z & mw, f0.w & mw);
      afl[ks] = make_uint4(f1.x & mw, f1.y & mw, f1.z & mw, f1.w & mw);
    }
#pragma unroll
    for (int nt = 0; nt < NT1W; ++nt) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint4 fkh, fkl;
        phi_bf16_split(kraw[nt][ks], fkh, fkl);
        c = mfma_bf16(aq[ks], kraw[nt][ks], c);
        c = mfma_bf16(afh[ks], fkh, c);
        c = mfma_bf16(afl[ks], fkh, c);
        c = mfma_bf16(afh[ks], fkl, c);
      }
      c1[nt] = c;
    }
  }
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
  if constexpr (VLDS) {
    // this wavefront's V rows are in LDS once its loads are done (the barrier
    // then shows every wavefront's rows to all)
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    // ---- V tile, transposed into LDS (rows past the block's end are zero)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = threadIdx.x + kThreads * i;
      const int tp = idx % (BK / 2), cg = idx / (BK / 2);
      const bool v0 = 2 * tp < ntok, v1 = 2 * tp + 1 < ntok;
      const uint32_t r0[4] = {vr[i][0].x, vr[i][0].y, vr[i][0].z, vr[i][0].w};
      const uint32_t r1[4] = {vr[i][1].x, vr[i][1].y, vr[i][1].z, vr[i][1].w};
      uint32_t* dst = reinterpret_cast<uint32_t*>(vs) + (size_t)(8 * cg) * (VS / 2) + tp;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t a0 = v0 ? r0[k] : 0u, a1 = v1 ? r1[k] : 0u;
        dst[(2 * k) * (VS / 2)] = (a0 & 0xffffu) | (a1 << 16);
        dst[(2 * k + 1) * (VS / 2)] = (a0 >> 16) | (a1 & 0xffff0000u);
      }
    }
  }
  __syncthreads();
  // ---- product (2)
  const int rec = 2 * D;
  float* part0 = a.part + (((size_t)b * a.H + g * R) * a.top_k + slot) * rec;
#pragma unroll
  for (int nt2 = 0; nt2 < NT2W; ++nt2) {
    const int ch = (w * NT2W + nt2) * 16 + l16;
    // B operands: lane (lg4, n = l16) holds tokens 32 ks + 8 lg4 + 0..7 of
    // channel ch
    uint4 bvs[KS2];
#pragma unroll
    for (int ks = 0; ks < KS2; ++ks) {
      if constexpr (VLDS) {
        // two transposing reads; as a source this lane addresses token
        // 32 ks + 8 lg4 + 4 h + l16 / 4, channels ch0 + 4 (l16 % 4) .. + 3
        const int chs = (w * NT2W + nt2) * 16 + 4 * (l16 % 4);
        uint2 hv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t = 32 * ks + 8 * lg4 + 4 * h + l16 / 4;
          hv[h] = lds_read_tr16(&vs[t * D + 8 * ((chs / 8) ^ vswz<D>(t)) + chs % 8]);
        }
        bvs[ks] = make_uint4(hv[0].x, hv[0].y, hv[1].x, hv[1].y);
      } else {
        bvs[ks] = *reinterpret_cast<const uint4*>(&vs[ch * VS + 32 * ks + 8 * lg4]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT2; ++mt) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS2; ++ks) {
        const uint4 av = *reinterpret_cast<const uint4*>(&pw[(mt * 16 + l16) * PS + 32 * ks + 8 * lg4]);
        c = mfma_bf16(av, bvs[ks], c);
      }
      // lane group lg4 holds rows 4 lg4 .. 4 lg4 + 3 of tile mt: pairs
      // pi0 = 8 mt + 2 lg4 (hi + lo in c[0], c[1]) and pi0 + 1 (c[2], c[3])
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int pi = 8 * mt + 2 * lg4 + e;
        if (pi < 2 * R) {
          const int kind = pi / R, h = pi % R;
          part0[(size_t)h * a.top_k * rec + (kind ? D : 0) + ch] = c[2 * e] + c[2 * e + 1];
        }
      }
    }
  }
  if (threadIdx.x < R) {
    const int h = threadIdx.x;
    *reinterpret_cast<float4*>(a.part_hdr + ((((size_t)b * a.H + g * R + h) * a.top_k + slot) * kPartHdr)) =
        make_float4(fmaxf(fmaxf(s_max[0][h], s_max[1][h]), fmaxf(s_max[2][h], s_max[3][h])),
                    (s_l[0][h] + s_l[1][h]) + (s_l[2][h] + s_l[3][h]),
                    (s_sw[0][h] + s_sw[1][h]) + (s_sw[2][h] + s_sw[3][h]), 0.f);
  }
}


}  // namespace
}  // namespace spla
