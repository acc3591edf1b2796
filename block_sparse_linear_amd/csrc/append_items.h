// Work items of the append (SPLA Technical Summary 2.1: pages and block
// statistics), shared by the append kernel and the fused decode-step kernel.
// Each function is executed by a whole 256-thread workgroup.
#pragma once

#include "spla_common.h"

namespace spla {

// copy appended tokens [i0, i0 + ntok_max) of entry E (all KV heads) into the
// pages
template <bool BF16>
__device__ void append_page_rows(const StateRefs& a, const AppendEntry& E, int i0, int ntok_max) {
  const int ntok = min(ntok_max, E.n - i0);
  const int es = BF16 ? 2 : 4;
  const int vec_per_row = a.d * es / 16;
  const int per_tok = a.G * vec_per_row;
  const int total = ntok * per_tok;
  const uint4* kn = reinterpret_cast<const uint4*>(a.k_new);
  const uint4* vn = reinterpret_cast<const uint4*>(a.v_new);
  uint4* kp = reinterpret_cast<uint4*>(a.k_pages);
  uint4* vp = reinterpret_cast<uint4*>(a.v_pages);
  for (int idx = threadIdx.x; idx < total; idx += kThreads) {
    const int i = idx / per_tok;
    const int rem = idx - i * per_tok;
    const int g = rem / vec_per_row;
    const int v = rem - g * vec_per_row;
    const int p = E.t0 + i0 + i;
    const int j = p / a.bk;
    const int page = a.block_table[(size_t)E.seq * a.max_blocks + j];
    if (page < 0 || page >= a.num_pages) {
      atomicOr(a.err, kErrPage);
      continue;
    }
    const size_t src = (((size_t)(E.row + i0 + i)) * a.G + g) * vec_per_row + v;
    const size_t dst = (((size_t)page * a.G + g) * a.bk + (p % a.bk)) * vec_per_row + v;
    kp[dst] = kn[src];
    vp[dst] = vn[src];
  }
}

// the page row of entry E's first appended token, KV head g only (threads
// 0 .. d * element size / 16 - 1 copy one 16-byte piece each of k and v)
template <bool BF16>
__device__ void append_page_row_head(const StateRefs& a, const AppendEntry& E, int g) {
  const int vec_per_row = a.d * (BF16 ? 2 : 4) / 16;
  const int v = threadIdx.x;
  if (v >= vec_per_row) return;
  const int p = E.t0;
  const int page = a.block_table[(size_t)E.seq * a.max_blocks + p / a.bk];
  if (page < 0 || page >= a.num_pages) {
    if (v == 0) atomicOr(a.err, kErrPage);
    return;
  }
  const size_t src = ((size_t)E.row * a.G + g) * vec_per_row + v;
  const size_t dst = (((size_t)page * a.G + g) * a.bk + (p % a.bk)) * vec_per_row + v;
  reinterpret_cast<uint4*>(a.k_pages)[dst] = reinterpret_cast<const uint4*>(a.k_new)[src];
  reinterpret_cast<uint4*>(a.v_pages)[dst] = reinterpret_cast<const uint4*>(a.v_new)[src];
}

// mean and population variance (two passes) of block j of entry E's
// sequence, KV head g, completed by this append: tokens older than the
// append come from the pages, the new ones from k_new.  Every key of the
// block is loaded at once, 16 bytes per load (thread = (token group, 16-byte
// column of the row)), and held in registers for both passes; the per-column
// sums meet in LDS.
template <bool BF16>
struct BlockStatsLds {
  float red[kThreads * (BF16 ? 8 : 4)];  // per-column partial sums of every thread
};

template <bool BF16, int D>
__device__ void append_block_stats(const StateRefs& a, const AppendEntry& E, int j, int g, BlockStatsLds<BF16>& L) {
  constexpr int VE = BF16 ? 8 : 4;  // elements per 16-byte vector
  constexpr int d = D;
  constexpr int vr = d / VE;        // vectors per token row
  constexpr int tg = kThreads / vr;  // token groups
  constexpr int MAXV = 128 / tg;    // vectors (tokens) per thread at Bk = 128
  float* red = L.red;
  const int bk = a.bk;
  const int nv = bk / tg;           // vectors (tokens) per thread
  const int col = threadIdx.x % vr, t0 = threadIdx.x / vr;
  const int page = a.block_table[(size_t)E.seq * a.max_blocks + j];
  const bool page_ok = page >= 0 && page < a.num_pages;
  if (!page_ok && j * bk < E.t0) {
    if (threadIdx.x == 0) atomicOr(a.err, kErrPage);
    return;
  }
  const uint4* kp = reinterpret_cast<const uint4*>(a.k_pages);
  const uint4* kn = reinterpret_cast<const uint4*>(a.k_new);
  uint4 raw[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    if (i < nv) {
      const int p = j * bk + t0 + tg * i;  // token of this vector
      raw[i] = p < E.t0 ? kp[(((size_t)page * a.G + g) * bk + (p % bk)) * vr + col]
                        : kn[((size_t)(E.row + p - E.t0) * a.G + g) * vr + col];
    }
  }
  auto elem = [](uint4 v, int e) -> float {
    const uint32_t w = e < 2 * (VE / 4) ? (e < VE / 4 ? v.x : v.y) : (e < 3 * (VE / 4) ? v.z : v.w);
    if constexpr (BF16) return (e & 1) ? bf16_hi_f(w) : bf16_lo_f(w);
    return __uint_as_float(w);
  };
  // pass 1: per-column sums
  float s[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) s[e] = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    if (i < nv)
#pragma unroll
      for (int e = 0; e < VE; ++e) s[e] += elem(raw[i], e);
#pragma unroll
  for (int e = 0; e < VE; ++e) red[(t0 * vr + col) * VE + e] = s[e];
  __syncthreads();
  float mean[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    float tot = 0.f;
    for (int q = 0; q < tg; ++q) tot += red[(q * vr + col) * VE + e];
    mean[e] = tot / (float)bk;
  }
  __syncthreads();
  // pass 2: per-column sums of squared deviations, from the same registers
#pragma unroll
  for (int e = 0; e < VE; ++e) s[e] = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    if (i < nv)
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const float dv = elem(raw[i], e) - mean[e];
        s[e] = fmaf(dv, dv, s[e]);
      }
#pragma unroll
  for (int e = 0; e < VE; ++e) red[(t0 * vr + col) * VE + e] = s[e];
  __syncthreads();
  if (t0 == 0) {
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      float t2 = 0.f;
      for (int q = 0; q < tg; ++q) t2 += red[(q * vr + col) * VE + e];
      const int c = col * VE + e;
      const size_t idx = ((((size_t)E.seq * a.G + g) * a.n_tiles + j / kTile) * (d / 4) + c / 4) * (kTile * 4) +
                         (j % kTile) * 4 + (c % 4);
      a.blk_mean[idx] = mean[e];
      a.blk_var[idx] = t2 / (float)bk;
    }
  }
}

}  // namespace spla
