// Attend + correct kernels, grid (top_k, G, B): one selected block of one
// (sequence, KV head) per workgroup, reading the selection the selector wrote
// (or the caller's override).  fp32 K/V on the vector ALUs, bf16 K/V on the
// matrix cores.
#include "attend_mfma.h"

namespace spla {

namespace {

// ============================================================== attend
// grid (top_k, G, B): one selected block of one (b, g) per workgroup, all R
// query heads of the group.  Tokens in chunks of 64: K chunk staged in LDS as
// fp32, lane = token for the two dot products, then thread = value channel for
// the weighted sums (V read straight from the page, coalesced along d).
template <bool BF16, int R, int D>
__global__ __launch_bounds__(kThreads) void k_attend(const DecodeArgs a) {
  constexpr int KS = D + 1;  // padded row stride of the K chunk (floats)
  __shared__ float ks[64 * KS];
  __shared__ float qs[R][D];
  __shared__ float fq[R][D];
  __shared__ float red[4][2 * R][64];
  __shared__ float pw[2 * R][64];  // p (softmax numerators) then w (linear weights)
  __shared__ float sf[R];          // rescale of the running sums for this chunk
  __shared__ float s_m[R], s_l[R], s_sw[R];
  const int slot = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  constexpr int d = D;
  const int bk = a.bk;
  const int32_t* selp = a.sel_in ? a.sel_in : a.sel;
  const int j = selp[((size_t)b * a.G + g) * a.top_k + slot];
  if (j < 0) return;
  const int T = a.lens[b];
  const int nb = n_blocks(a, b);
  if (j >= nb) {
    if (threadIdx.x == 0) atomicOr(a.err, kErrSel);
    return;
  }
  // the selector's page ids (the block table only for the test hook)
  const int page = a.sel_in ? a.block_table[(size_t)b * a.max_blocks + j]
                            : a.sel_page[((size_t)b * a.G + g) * a.top_k + slot];
  if (page < 0 || page >= a.num_pages) {
    if (threadIdx.x == 0) atomicOr(a.err, kErrPage);
    return;
  }
  const int ntok = min(bk, T - j * bk);
  for (int i = threadIdx.x; i < R * d; i += kThreads) {
    const int h = i / d, c = i - h * d;
    const float v = load_elem<BF16>(a.q, ((size_t)b * a.H + g * R + h) * d + c);
    qs[h][c] = v;
    fq[h][c] = phi_f(v);
  }
  if (threadIdx.x < R) {
    s_m[threadIdx.x] = -INFINITY;
    s_l[threadIdx.x] = 0.f;
    s_sw[threadIdx.x] = 0.f;
  }
  const size_t page_base = (((size_t)page * a.G + g) * bk) * d;
  // per-thread accumulators: value channel c, pairs (kind, head) strided by the group count
  constexpr int ngrp = kThreads / d;
  constexpr int npair = (2 * R + ngrp - 1) / ngrp;
  const int c = threadIdx.x % d;
  const int grp = threadIdx.x / d;
  float acc[npair];
#pragma unroll
  for (int k = 0; k < npair; ++k) acc[k] = 0.f;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  constexpr int cq = d / 4;  // channels per wavefront in the dot phase
  for (int c0 = 0; c0 < ntok; c0 += 64) {
    const int n = min(64, ntok - c0);
    __syncthreads();
    // stage K chunk (n x d) as fp32
    for (int i = threadIdx.x; i < n * (d / 4); i += kThreads) {
      const int tok = i / (d / 4), q4 = i - tok * (d / 4);
      const float4 k4 = load4<BF16>(a.k_pages, page_base + (size_t)(c0 + tok) * d + q4 * 4);
      float* dst = &ks[tok * KS + q4 * 4];
      dst[0] = k4.x;
      dst[1] = k4.y;
      dst[2] = k4.z;
      dst[3] = k4.w;
    }
    __syncthreads();
    float sp[R], wp[R];
#pragma unroll
    for (int h = 0; h < R; ++h) sp[h] = wp[h] = 0.f;
    if (lane < n) {
      for (int cc = w * cq; cc < (w + 1) * cq; ++cc) {
        const float kv = ks[lane * KS + cc];
        const float fk = phi_f(kv);
#pragma unroll
        for (int h = 0; h < R; ++h) {
          sp[h] = fmaf(qs[h][cc], kv, sp[h]);
          wp[h] = fmaf(fq[h][cc], fk, wp[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < R; ++h) {
      red[w][h][lane] = sp[h];
      red[w][R + h][lane] = wp[h];
    }
    __syncthreads();
    // softmax bookkeeping: wavefront w handles heads w, w+4
    for (int h = w; h < R; h += 4) {
      float s = -INFINITY, wv = 0.f;
      if (lane < n) {
        s = (red[0][h][lane] + red[1][h][lane] + red[2][h][lane] + red[3][h][lane]) * a.inv_sqrt_d;
        wv = red[0][R + h][lane] + red[1][R + h][lane] + red[2][R + h][lane] + red[3][R + h][lane];
      }
      const float mc = wave_max(s);
      const float m_old = s_m[h];
      const float m_new = fmaxf(m_old, mc);
      const float p = lane < n ? expf(s - m_new) : 0.f;
      const float ps = wave_sum(p);
      const float ws = wave_sum(wv);
      pw[h][lane] = p;
      pw[R + h][lane] = wv;
      if (lane == 0) {
        const float scale = expf(m_old - m_new);  // 0 on the first chunk
        sf[h] = scale;
        s_l[h] = s_l[h] * scale + ps;
        s_m[h] = m_new;
        s_sw[h] += ws;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < npair; ++k) {
      const int p = grp + k * ngrp;
      if (p < 2 * R) {
        const bool is_sm = p < R;
        float x = is_sm ? acc[k] * sf[p] : acc[k];
        const float* wt = pw[p];
        for (int i = 0; i < n; ++i) {
          const float v = load_elem<BF16>(a.v_pages, page_base + (size_t)(c0 + i) * d + c);
          x = fmaf(wt[i], v, x);
        }
        acc[k] = x;
      }
    }
  }
  __syncthreads();
  const int rec = 2 * d;
#pragma unroll
  for (int k = 0; k < npair; ++k) {
    const int p = grp + k * ngrp;
    if (p < 2 * R) {
      const int h = p < R ? p : p - R;
      float* dst = a.part + (((size_t)b * a.H + g * R + h) * a.top_k + slot) * rec + (p < R ? 0 : d);
      dst[c] = acc[k];
    }
  }
  if (threadIdx.x < R) {
    const int h = threadIdx.x;
    *reinterpret_cast<float4*>(a.part_hdr + (((size_t)b * a.H + g * R + h) * a.top_k + slot) * kPartHdr) =
        make_float4(s_m[h], s_l[h], s_sw[h], 0.f);
  }
}


// bf16 K/V: the selected block of this slot and its page, then the MFMA body
template <int R, int D, int BK>
__global__ __launch_bounds__(kThreads) void k_attend_mfma(const DecodeArgs a) {
  const int slot = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  SPLA_SCALARS_READY("s"(a.lens[b]), "s"(a.bk), "s"(a.top_k), "s"(a.sel_in), "s"(a.sel), "s"(a.sel_page),
                     "s"(a.G), "s"(a.q), "s"(a.H), "s"(a.k_pages), "s"(a.v_pages));
  QOps<R, D> qo;
  load_qops<R, D>(a.q, a.phq, a.H, g, b, qo);  // independent of the selection: issued first
  const size_t srow = ((size_t)b * a.G + g) * a.top_k + slot;
  int j, page;
  if (a.sel_in) {
    j = a.sel_in[srow];
    page = (j >= 0 && j < a.max_blocks) ? a.block_table[(size_t)b * a.max_blocks + j] : -1;
  } else {
    j = a.sel[srow];
    page = a.sel_page[srow];
  }
  // many workgroups per CU here: V straight into LDS (fewer registers, more
  // workgroups resident)
  attend_block_mfma<R, D, BK, true>(a, slot, g, b, j, page, qo);
}

}  // namespace

hipError_t launch_attend(const DecodeArgs& a, bool bf16, const Launch& l) {
  const dim3 grid(a.top_k, a.G, a.B);
  if (!bf16) SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_attend<false, RR, DD>, grid, l, a))
  if (a.bk == 64) SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_attend_mfma<RR, DD, 64>, grid, l, a))
  SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_attend_mfma<RR, DD, 128>, grid, l, a))
}


}  // namespace spla
