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
// append come from the pages, the new ones from k_new
template <bool BF16>
__device__ void append_block_stats(const StateRefs& a, const AppendEntry& E, int j, int g) {
  __shared__ float red[kThreads];
  const int d = a.d, bk = a.bk;
  const int groups = kThreads / d;
  const int c = threadIdx.x % d;
  const int grp = threadIdx.x / d;
  const int tpg = bk / groups;
  const int page = a.block_table[(size_t)E.seq * a.max_blocks + j];
  const bool page_ok = page >= 0 && page < a.num_pages;
  if (!page_ok && j * bk < E.t0) {
    if (threadIdx.x == 0) atomicOr(a.err, kErrPage);
    return;
  }
  auto key = [&](int p) -> float {
    if (p < E.t0) {
      return load_elem<BF16>(a.k_pages, (((size_t)page * a.G + g) * bk + (p % bk)) * d + c);
    }
    return load_elem<BF16>(a.k_new, ((size_t)(E.row + p - E.t0) * a.G + g) * d + c);
  };
  const int p0 = j * bk + grp * tpg;
  float s = 0.f;
  for (int i = 0; i < tpg; ++i) s += key(p0 + i);
  red[threadIdx.x] = s;
  __syncthreads();
  float tot = 0.f;
  for (int q = 0; q < groups; ++q) tot += red[q * d + c];
  const float mean = tot / (float)bk;
  __syncthreads();
  float s2 = 0.f;
  for (int i = 0; i < tpg; ++i) {
    const float dv = key(p0 + i) - mean;
    s2 = fmaf(dv, dv, s2);
  }
  red[threadIdx.x] = s2;
  __syncthreads();
  if (grp == 0) {
    float t2 = 0.f;
    for (int q = 0; q < groups; ++q) t2 += red[q * d + c];
    const size_t idx = ((((size_t)E.seq * a.G + g) * a.n_tiles + j / kTile) * (d / 4) + c / 4) * (kTile * 4) +
                       (j % kTile) * 4 + (c % 4);
    a.blk_mean[idx] = mean;
    a.blk_var[idx] = t2 / (float)bk;
  }
}

}  // namespace spla
