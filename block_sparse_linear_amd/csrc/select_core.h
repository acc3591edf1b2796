// Top-k block selection of one (sequence, KV head) by one 256-thread
// workgroup: the sink (block 0), the current block (nb - 1) and the top_k - 2
// candidates 1 .. nb - 2 with the largest group log score, ties to the
// smaller block id (SPLA Technical Summary 1 and 2.1: only the most relevant
// blocks are loaded; the Baidu Cloud sparse-attention article, section 5:
// score, sort, keep the top K).  Shared by the stand-alone selector and the
// fused select + attend kernel.
#pragma once

#include <type_traits>

#include "decode_common.h"

namespace spla {
namespace {

constexpr int kSelMax = kMaxBlocksPerSeq - 2;  // candidates per (b, g) the selector handles
constexpr int kSelLevels = 12;                 // bucket refinement levels
constexpr int kSelRank = 256;                  // threshold-bucket size ranked exactly

// bucket of x at one refinement level: monotone non-decreasing in x
__device__ __forceinline__ int sel_bucket(float x, float lo, float scale) {
  const float f = (x - lo) * scale;
  return f >= 255.f ? 255 : (f <= 0.f ? 0 : (int)f);
}

// LDS of the selector (the ranking and chosen lists are padded with sentinels
// so the rank and position counts read them four at a time)
struct __attribute__((aligned(16))) SelectLds {
  int hist[4][256];  // one histogram per wavefront
  float mkey[kSelRank + 4];  // ranking list: keys of the threshold bucket
  int midx[kSelRank + 4];    // their candidate indices
  int mpage[kSelRank];       // page of midx[i]
  int cid[kThreads + 4];     // chosen list: candidate indices (top_k - 2 <= 254 entries)
  int cpg[kThreads];         // page of cid[i]
  float s_mn[4], s_mx[4];
  int s_cnt[4];
  int s_bt, s_above, s_cbt, s_nm;
};

// one thread's candidates: scores and page ids (candidate i = thread + 256 u,
// block id i + 1), plus the pages of the sink and the current block
template <int KPT>
struct SelectKeys {
  float x[KPT];
  int pg[KPT];
  int pg_sink, pg_cur;
};

// Issue the candidate loads of a selection: scores and page ids of
// candidates 0 .. KPT * 256 - 1, clamped into the score row of b and the
// block table row brow (b, or 0 for the virtual queries of one sequence's
// prefill chunk).  They need no sequence length, so a kernel can issue them
// first (lg, block_table and the sizes are kernel arguments ahead of the
// argument struct).  The pages of the sink and the current block come with
// select_pages once the length is known.
template <int KPT>
__device__ __forceinline__ void select_load(const float* lg, const int32_t* block_table, int n_tiles, int max_blocks,
                                            int G, int g, int b, int brow, SelectKeys<KPT>& k) {
  const int cap = max(min(n_tiles * kTile, max_blocks) - 2, 0);  // last candidate index inside both rows
  const int32_t* btab = block_table + (size_t)brow * max_blocks;
  const float* row = lg + ((size_t)b * G + g) * (size_t)(n_tiles * kTile) + 1;  // row[i] = LG(i + 1)
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int i = min((int)threadIdx.x + u * kThreads, cap);
    k.x[u] = row[i];
    k.pg[u] = btab[min(i + 1, max_blocks - 1)];
  }
}

// Pages of the sink and the current block.  They are read with vector
// loads (the offset is a zero the compiler cannot see as uniform): a scalar
// load would be waited for at every LDS barrier of the selection, which waits
// on the scalar-load counter too.
template <int KPT>
__device__ __forceinline__ void select_pages(const int32_t* block_table, int max_blocks, int brow, int nb,
                                             SelectKeys<KPT>& k) {
  int zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  const int32_t* btab = block_table + (size_t)brow * max_blocks;
  k.pg_sink = btab[zero];
  k.pg_cur = btab[min(max(nb - 1, 0), max_blocks - 1) + zero];
}

// Bucket select over the scores held in registers (KPT per thread,
// KPT * 256 >= nb - 2): the scores are binned into 256 buckets spread over
// [min, max] of the remaining candidates; every candidate in a bucket above
// the one holding the k'-th largest is taken, and that bucket is refined the
// same way until it holds at most kSelRank candidates (then ranked exactly by
// (score desc, id asc)) or only equal scores (then taken by ascending id).
// The bucket index is a monotone function of the score, so the result is the
// exact top k'.  The k' chosen candidates are gathered in a list (those above
// the threshold bucket by reserved places, the threshold bucket's picks at
// their rank), and each one's ascending output position is the count of
// chosen candidates with a smaller index.
//
// Requires nb > top_k and the keys of select_load; every thread of the
// workgroup must call it.  For each output position pos in [0, top_k),
// exactly one thread calls emit(pos, block id, page id).
template <int KPT, typename Emit>
__device__ __forceinline__ void select_core(const DecodeArgs& a, int nb, const SelectKeys<KPT>& k, SelectLds& L,
                                            Emit&& emit) {
  using Mask = typename std::conditional<(KPT <= 32), uint32_t, uint64_t>::type;
  const int nc = nb - 2;
  const int kp = a.top_k - 2;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  Mask memb = 0, above = 0;  // bit u: key u still in the threshold bucket / already taken
#pragma unroll
  for (int u = 0; u < KPT; ++u) memb |= (Mask)((int)threadIdx.x + u * kThreads < nc) << u;
  if (threadIdx.x == 0) L.s_nm = 0;
  L.mkey[threadIdx.x] = -INFINITY;
  L.midx[threadIdx.x] = 0x7fffffff;
  L.cid[threadIdx.x] = 0x7fffffff;
  if (threadIdx.x < 4) {
    L.mkey[kSelRank + threadIdx.x] = -INFINITY;
    L.midx[kSelRank + threadIdx.x] = 0x7fffffff;
    L.cid[kThreads + threadIdx.x] = 0x7fffffff;
  }
  // the counters and sentinels above are used by every wavefront after the
  // bucket loop; its first barrier orders them when it runs (more than
  // kSelRank candidates), otherwise this one does (nc is uniform)
  if (nc <= kSelRank) __syncthreads();
  int need = kp;
  bool equal_mode = false;
  // members of the threshold bucket: all candidates at first, then the count
  // the histogram gives for the bucket picked (no extra pass to count them)
  int cnt = nc;
  for (int lev = 0; cnt > kSelRank; ++lev) {
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const bool in = (memb >> u) & 1;
      mn = fminf(mn, in ? k.x[u] : INFINITY);
      mx = fmaxf(mx, in ? k.x[u] : -INFINITY);
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
#pragma unroll
    for (int q = 0; q < 4; ++q) L.hist[q][threadIdx.x] = 0;
    if (lane == 0) {
      L.s_mn[wv] = mn;
      L.s_mx[wv] = mx;
    }
    __syncthreads();
    mn = fminf(fminf(L.s_mn[0], L.s_mn[1]), fminf(L.s_mn[2], L.s_mn[3]));
    mx = fmaxf(fmaxf(L.s_mx[0], L.s_mx[1]), fmaxf(L.s_mx[2], L.s_mx[3]));
    const float range = mx - mn;
    if (!(range > 0.f) || !(range < INFINITY) || lev == kSelLevels) {
      equal_mode = true;  // equal scores (or a degenerate range): take by id
      if (range > 0.f && threadIdx.x == 0) atomicOr(a.err, kErrSel);
      break;
    }
    const float scale = 256.f / range;
    int bkt[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      bkt[u] = sel_bucket(k.x[u], mn, scale);
      atomicAdd(&L.hist[wv][bkt[u]], (int)((memb >> u) & 1));  // non-members add 0: no branch
    }
    __syncthreads();
    if (wv == 0) {
      int c[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int bin = 255 - 4 * lane - q;
        c[q] = (L.hist[0][bin] + L.hist[1][bin]) + (L.hist[2][bin] + L.hist[3][bin]);
        sum += c[q];
      }
      int run = wave_incl_scan_i(sum) - sum;  // keys in buckets above this lane's
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (run < need && run + c[q] >= need) {
          L.s_bt = 255 - 4 * lane - q;
          L.s_above = run;
          L.s_cbt = c[q];
        }
        run += c[q];
      }
    }
    __syncthreads();
    const int bt = L.s_bt;
    need -= L.s_above;
    cnt = L.s_cbt;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const Mask bit = (Mask)1 << u;
      const bool in = (memb & bit) != 0;
      above |= (in && bkt[u] > bt) ? bit : (Mask)0;
      memb &= (in && bkt[u] == bt) ? ~(Mask)0 : ~bit;
    }
  }
  if (equal_mode) {
    // equal scores: the `need` smallest ids among the members; find the id
    // bound by bisection on counts
    int lo = 0, hi = nc;  // smallest X with #members(id < X) >= need
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      int c = 0;
#pragma unroll
      for (int u = 0; u < KPT; ++u) c += ((memb >> u) & 1) && ((int)threadIdx.x + u * kThreads < mid);
      c = wave_sum_i(c);
      __syncthreads();
      if (lane == 0) L.s_cnt[wv] = c;
      __syncthreads();
      c = (L.s_cnt[0] + L.s_cnt[1]) + (L.s_cnt[2] + L.s_cnt[3]);
      if (c >= need) hi = mid; else lo = mid + 1;
    }
    Mask low = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      low |= (((memb >> u) & 1) && (int)threadIdx.x + u * kThreads < lo) ? ((Mask)1 << u) : (Mask)0;
    above |= low;
    memb = 0;
  }
  // every key above a threshold bucket (or taken by id) goes to the chosen
  // list, the threshold bucket's keys to the ranking list: lanes count theirs
  // (both counts packed in one int, members in the low 16 bits), one LDS
  // atomic per wavefront reserves the places in both, then every lane stores
  // its own
  {
    const int packed = (__popcll((uint64_t)above) << 16) | __popcll((uint64_t)memb);
    const int incl = wave_incl_scan_i(packed);
    int base = 0;
    if (lane == 63 && incl > 0) base = atomicAdd(&L.s_nm, incl);  // lane 63: the wavefront's totals
    const int b0 = __builtin_amdgcn_readlane(base, 63) + incl - packed;
    int pa = b0 >> 16, pm = b0 & 0xffff;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int i = threadIdx.x + u * kThreads;
      if ((above >> u) & 1) {
        L.cid[pa] = i;
        L.cpg[pa] = k.pg[u];
        ++pa;
      }
      if ((memb >> u) & 1) {
        L.mkey[pm] = k.x[u];
        L.midx[pm] = i;
        L.mpage[pm] = k.pg[u];
        ++pm;
      }
    }
  }
  __syncthreads();
  // the final bucket (<= kSelRank candidates): exact rank by (score desc, id
  // asc); the first `need` go to the chosen list after the na keys above it
  const int nm = L.s_nm & 0xffff, na = L.s_nm >> 16;  // na + need == kp
  if (nm > 0) {
    if ((int)threadIdx.x < nm) {
      const float xv = L.mkey[threadIdx.x];
      const int my = L.midx[threadIdx.x];
      int rank = 0;
#pragma unroll 4
      for (int v = 0; v < nm; v += 4) {
        const float4 y = *reinterpret_cast<const float4*>(&L.mkey[v]);
        const int4 iy = *reinterpret_cast<const int4*>(&L.midx[v]);
        rank += (y.x > xv) || (y.x == xv && iy.x < my);
        rank += (y.y > xv) || (y.y == xv && iy.y < my);
        rank += (y.z > xv) || (y.z == xv && iy.z < my);
        rank += (y.w > xv) || (y.w == xv && iy.w < my);
      }
      if (rank < need) {
        L.cid[na + rank] = my;
        L.cpg[na + rank] = L.mpage[threadIdx.x];
      }
    }
    __syncthreads();
  }
  // output position of chosen entry t: 1 + the chosen candidates with a
  // smaller index (the list is padded with sentinels past kp)
  if ((int)threadIdx.x < kp) {
    const int my = L.cid[threadIdx.x];
    int pos = 1;
    for (int v = 0; v < kp; v += 4) {
      const int4 c = *reinterpret_cast<const int4*>(&L.cid[v]);
      pos += (c.x < my) + (c.y < my) + (c.z < my) + (c.w < my);
    }
    emit(pos, my + 1, L.cpg[threadIdx.x]);
  }
  if (threadIdx.x == 0) emit(0, 0, k.pg_sink);
  if (threadIdx.x == kThreads - 1) emit(kp + 1, nb - 1, k.pg_cur);
}

// keys-per-thread sizes compiled for a selector: the smallest one that holds
// the longest sequence's candidates is launched
template <int... Ks>
struct SelectSizes {};

// candidates of the longest sequence that has more blocks than top_k (0 if none)
inline int max_candidates(const DecodeArgs& a) {
  int nc = 0;
  for (int b = 0; b < a.B; ++b) {
    const int nb = (a.lens[b] + a.bk - 1) / a.bk;
    if (nb > a.top_k) nc = nc > nb - 2 ? nc : nb - 2;
  }
  return nc;
}

}  // namespace
}  // namespace spla
