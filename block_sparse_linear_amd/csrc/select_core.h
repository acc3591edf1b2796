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

constexpr int kFastCap = 256;  // candidates per wavefront list of the threshold path

// LDS of the selector (the ranking and chosen lists are padded with sentinels
// so the rank and position counts read them several at a time)
struct __attribute__((aligned(16))) SelectLds {
  // threshold path: per-wavefront lists of the candidates at or above the
  // bound as packed keys (score key << 32 | ~candidate index: one integer
  // order for (score desc, id asc)) and pages, the group maxima of the bound
  // and the partial ranks of every listed candidate against each list
  uint64_t fkey[4][kFastCap + 2];
  int fpg[4][kFastCap];
  int4 prank[kThreads];
  float pool[kThreads];
  int s_fcnt[4];
  // bucket path
  int hist[4][256];  // one histogram per wavefront
  float mkey[kSelRank + 4];  // ranking list: keys of the threshold bucket
  int midx[kSelRank + 4];    // their candidate indices
  int mpage[kSelRank];       // page of midx[i]
  int cid[kThreads + 4];     // chosen list: candidate indices (top_k - 2 <= 254 entries)
  int cpg[kThreads];         // page of cid[i]
  float s_mn[4], s_mx[4];
  int s_cnt[4];
  int s_bt, s_above, s_cbt, s_nm;
  int s_j, s_page;  // one slot's block and page (select_slot's bucket path)
};

// One thread's candidates: scores and page ids of candidates i = w * 64 KPT
// + 64 u + lane of wavefront w (each wavefront a contiguous range, its lanes
// strided through it: loads are whole-wavefront runs, and a list written in
// (u, lane) order is in candidate order), block id i + 1; plus the pages of
// the sink and the current block.
template <int KPT>
struct SelectKeys {
  float x[KPT];
  int pg[KPT];
  int pg_sink, pg_cur;
  __device__ __forceinline__ static int cand(int u) {
    return (int)(threadIdx.x >> 6) * (64 * KPT) + 64 * u + (int)(threadIdx.x & 63);
  }
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
    const int i = min(SelectKeys<KPT>::cand(u), cap);
    k.x[u] = row[i];
    k.pg[u] = btab[min(i + 1, max_blocks - 1)];
  }
}

// The two halves of select_load, for a kernel that has the page ids before
// the scores exist: the candidates' page ids, then (later) their scores.
template <int KPT>
__device__ __forceinline__ void select_load_pages(const int32_t* block_table, int n_tiles, int max_blocks, int brow,
                                                  SelectKeys<KPT>& k) {
  const int cap = max(min(n_tiles * kTile, max_blocks) - 2, 0);
  const int32_t* btab = block_table + (size_t)brow * max_blocks;
#pragma unroll
  for (int u = 0; u < KPT; ++u) k.pg[u] = btab[min(min(SelectKeys<KPT>::cand(u), cap) + 1, max_blocks - 1)];
}
template <int KPT>
__device__ __forceinline__ void select_load_scores(const float* lg, int n_tiles, int max_blocks, int G, int g, int b,
                                                   SelectKeys<KPT>& k) {
  const int cap = max(min(n_tiles * kTile, max_blocks) - 2, 0);
  const float* row = lg + ((size_t)b * G + g) * (size_t)(n_tiles * kTile) + 1;
#pragma unroll
  for (int u = 0; u < KPT; ++u) k.x[u] = row[min(SelectKeys<KPT>::cand(u), cap)];
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

// packed key: larger score first, then the smaller candidate index (-0 is
// taken as +0, so equal scores compare as equal, as floats do)
__device__ __forceinline__ uint64_t sel_key(float x, int i) {
  return ((uint64_t)float_key(x == 0.f ? 0.f : x) << 32) | (uint32_t)~(uint32_t)i;
}

// Threshold path of the selection (the common case): a bound t0 that at
// least k' candidates reach, the candidates at or above it listed in LDS,
// and those ranked exactly by (score desc, id asc).
//  (1) Bound.  Each thread takes the maximum of its own keys and the lanes of
//      a wavefront are grouped by G = 4, 2 or 1 (k' <= 32, <= 64, more);
//      the 256 / G group maxima (DPP maxima within each group) are pooled in
//      LDS.  Each group maximum is a key of its own, so the k'-th largest of
//      the pool is reached by at least k' candidates.  Every wavefront finds
//      it in the pool on its own (no second barrier): a radix select over the
//      top 16 bits of the order-preserving integer form of the scores, with
//      one ballot count per bit, gives the k'-th largest 16-bit prefix P, and
//      t0 is the smallest score with prefix P (so t0 <= the pool's k'-th
//      largest).
//  (2) List.  Each wavefront writes its candidates >= t0, as packed keys and
//      pages, into its own LDS list in (u, lane) order (positions from one
//      ballot per u, no atomics): the four lists one after the other are in
//      candidate order.
//  (3) Rank.  Thread (lane, wavefront w) counts, for the listed candidates e
//      = lane, lane + 64, ..., how many keys of list w are larger; the four
//      partial counts sum to e's rank.
// Three barriers.  Returns false (every thread alike) when more than
// kThreads candidates reach the bound or a list would overflow; the caller
// then runs the bucket path.  On true, the listed candidates are
// L.fkey / L.fpg (n of them, see sel_listed) and their partial ranks
// L.prank[e]; the rank of e is below k' exactly when it is chosen, and its
// output position is 1 + the chosen candidates listed before it.
template <int KPT>
__device__ __forceinline__ int select_threshold_rank(const DecodeArgs& a, int nb, const SelectKeys<KPT>& k,
                                                     SelectLds& L) {
  const int nc = nb - 2;
  const int kp = a.top_k - 2;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // (1) the bound
  using Mask = typename std::conditional<(KPT <= 32), uint32_t, uint64_t>::type;
  Mask valid = 0;
  float mt = -INFINITY;
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const bool in = SelectKeys<KPT>::cand(u) < nc;
    valid |= (Mask)in << u;
    mt = fmaxf(mt, in ? k.x[u] : -INFINITY);
  }
  const int gsh = kp <= 32 ? 2 : (kp <= 64 ? 1 : 0);  // log2 of the group size
  float gm = mt;
  if (gsh >= 1) gm = fmaxf(gm, dpp_f<kDppXor1>(gm, gm));
  if (gsh >= 2) gm = fmaxf(gm, dpp_f<kDppXor2>(gm, gm));
  if ((lane & ((1 << gsh) - 1)) == 0) L.pool[threadIdx.x >> gsh] = gm;
  __syncthreads();
  // the k'-th largest 16-bit key prefix of the pool (Q pooled values per lane)
  auto radix = [&](auto qc) {
    constexpr int Q = decltype(qc)::value;
    uint32_t pk[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) pk[q] = float_key(L.pool[lane + 64 * q]) >> 16;
    uint32_t pre = 0;
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t cand = pre | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < Q; ++q) cnt += __popcll(__ballot(pk[q] >= cand));
      if (cnt >= kp) pre = cand;
    }
    return pre;
  };
  const uint32_t pre = gsh == 2 ? radix(std::integral_constant<int, 1>{})
                                : (gsh == 1 ? radix(std::integral_constant<int, 2>{})
                                            : radix(std::integral_constant<int, 4>{}));
  // the smallest score whose key has prefix pre (-inf at or below the prefix
  // of -inf, whose smallest key would be a NaN pattern)
  const uint32_t key0 = pre << 16;
  const float t0 = key0 <= float_key(-INFINITY) ? -INFINITY
                                                 : __uint_as_float((key0 & 0x80000000u) ? (key0 & 0x7fffffffu) : ~key0);
  // (2) this wavefront's list, in (u, lane) order = candidate order; the
  // entries past the capacity are dropped and the count decides below
  int tot = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const bool in = ((valid >> u) & 1) && k.x[u] >= t0;
    const uint64_t m = __ballot(in);
    const int pos = tot + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (in && pos < kFastCap) {
      L.fkey[wv][pos] = sel_key(k.x[u], SelectKeys<KPT>::cand(u));
      L.fpg[wv][pos] = k.pg[u];
    }
    tot += __popcll(m);
  }
  if (tot <= kFastCap && lane < 2) L.fkey[wv][tot + lane] = 0;  // smaller than every key: never beats one
  if (lane == 0) L.s_fcnt[wv] = tot;
  __syncthreads();
  const int c0 = L.s_fcnt[0], c1 = L.s_fcnt[1], c2 = L.s_fcnt[2], c3 = L.s_fcnt[3];
  const int n = (c0 + c1) + (c2 + c3);
  // (fewer than k' only if the scores are not ordered, e.g. NaN: the bucket path decides)
  if (max(max(c0, c1), max(c2, c3)) > kFastCap || n > kThreads || n < kp) return 0;
  // (3) partial ranks against list wv
  const int cw = wv == 0 ? c0 : (wv == 1 ? c1 : (wv == 2 ? c2 : c3));
  for (int e = lane; e < n; e += 64) {
    const int r = e < c0 ? 0 : (e < c0 + c1 ? 1 : (e < c0 + c1 + c2 ? 2 : 3));
    const int o = e - (r > 0 ? c0 : 0) - (r > 1 ? c1 : 0) - (r > 2 ? c2 : 0);
    const uint64_t key = L.fkey[r][o];
    int rank = 0;
    for (int v = 0; v < cw; v += 2) {
      const ulonglong2 y = *reinterpret_cast<const ulonglong2*>(&L.fkey[wv][v]);
      rank += (y.x > key) + (y.y > key);
    }
    reinterpret_cast<int*>(&L.prank[e])[wv] = rank;
  }
  __syncthreads();
  return n;
}

// listed candidate e of the threshold path: its candidate index and page
__device__ __forceinline__ void sel_listed(const SelectLds& L, int e, int& i, int& pg) {
  const int c0 = L.s_fcnt[0], c1 = L.s_fcnt[1], c2 = L.s_fcnt[2];
  const int r = e < c0 ? 0 : (e < c0 + c1 ? 1 : (e < c0 + c1 + c2 ? 2 : 3));
  const int o = e - (r > 0 ? c0 : 0) - (r > 1 ? c1 : 0) - (r > 2 ? c2 : 0);
  i = (int)~(uint32_t)L.fkey[r][o];
  pg = L.fpg[r][o];
}

// Pass m of the chosen candidates in list order, for one wavefront: listed
// candidate e = 64 m + lane is chosen when its rank is below k'; its output
// position is 1 + base + the chosen lanes below it.  Returns the chosen
// lanes of the pass.
__device__ __forceinline__ uint64_t sel_chosen_pass(const SelectLds& L, int n, int kp, int m, bool& chosen) {
  const int e = 64 * m + (threadIdx.x & 63);
  chosen = false;
  if (e < n) {
    const int4 pr = L.prank[e];
    chosen = (pr.x + pr.y) + (pr.z + pr.w) < kp;
  }
  return __ballot(chosen);
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
__device__ __forceinline__ void select_bucket(const DecodeArgs& a, int nb, const SelectKeys<KPT>& k, SelectLds& L,
                                              Emit&& emit) {
  using Mask = typename std::conditional<(KPT <= 32), uint32_t, uint64_t>::type;
  const int nc = nb - 2;
  const int kp = a.top_k - 2;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  Mask memb = 0, above = 0;  // bit u: key u still in the threshold bucket / already taken
#pragma unroll
  for (int u = 0; u < KPT; ++u) memb |= (Mask)(SelectKeys<KPT>::cand(u) < nc) << u;
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
      for (int u = 0; u < KPT; ++u) c += ((memb >> u) & 1) && (SelectKeys<KPT>::cand(u) < mid);
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
      low |= (((memb >> u) & 1) && SelectKeys<KPT>::cand(u) < lo) ? ((Mask)1 << u) : (Mask)0;
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
      const int i = SelectKeys<KPT>::cand(u);
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

// The selection of one (b, g): the sink and the current block alone when
// top_k = 2, else the threshold path, or the bucket path when the threshold
// path declines.  Requires nb > top_k and the keys of select_load; every
// thread of the workgroup must call it.  For each output position pos in
// [0, top_k), exactly one thread calls emit(pos, block id, page id).
template <int KPT, typename Emit>
__device__ __forceinline__ void select_core(const DecodeArgs& a, int nb, const SelectKeys<KPT>& k, SelectLds& L,
                                            Emit&& emit) {
  const int kp = a.top_k - 2;
  if (threadIdx.x == 0) emit(0, 0, k.pg_sink);
  if (threadIdx.x == kThreads - 1) emit(kp + 1, nb - 1, k.pg_cur);
  if (kp == 0) return;
  const int n = select_threshold_rank<KPT>(a, nb, k, L);
  if (n > 0) {
    // wavefront 0 takes the listed candidates in passes of 64, in list
    // (= candidate) order, and emits the chosen ones at their positions
    if (threadIdx.x < 64) {
      int base = 1;
      for (int m = 0; 64 * m < n; ++m) {
        bool chosen;
        const uint64_t mask = sel_chosen_pass(L, n, kp, m, chosen);
        if (chosen) {
          int i, pg;
          sel_listed(L, 64 * m + threadIdx.x, i, pg);
          emit(base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u)),
               i + 1, pg);
        }
        base += __popcll(mask);
      }
    }
    return;
  }
  select_bucket<KPT>(a, nb, k, L, [&](int pos, int id, int pg) {
    if (pos > 0 && pos <= kp) emit(pos, id, pg);  // the sink and the current block are out already
  });
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

// The block at position `slot` of the ascending selection of (b, g) and its
// page (uniform over the workgroup), for a kernel whose workgroups each take
// one slot: the sink and the current block directly; otherwise every
// wavefront finds its slot in the threshold path's chosen list on its own
// (passes of 64 listed candidates in candidate order, counting the chosen
// ones, until the pass holding the slot-th chosen candidate), or the bucket
// path hands it over in LDS.  Every thread of the workgroup must call it;
// brow is b's block-table row.
template <int KPT>
__device__ __forceinline__ void select_slot(const DecodeArgs& a, const int32_t* block_table, int max_blocks, int brow,
                                            int nb, int slot, const SelectKeys<KPT>& k, SelectLds& L, int& j,
                                            int& page) {
  const int kp = a.top_k - 2;
  if (nb <= a.top_k) {
    j = slot < nb ? slot : -1;
    page = j >= 0 ? block_table[(size_t)brow * max_blocks + j] : -1;
  } else if (slot == 0) {  // the sink
    j = 0;
    page = k.pg_sink;
  } else if (slot == kp + 1) {  // the current block
    j = nb - 1;
    page = k.pg_cur;
  } else if (const int n = select_threshold_rank<KPT>(a, nb, k, L)) {
    const int lane = threadIdx.x & 63;
    int base = 1, src = -1, m = 0;
    for (; 64 * m < n; ++m) {
      bool chosen;
      const uint64_t mask = sel_chosen_pass(L, n, kp, m, chosen);
      const int cnt = __popcll(mask);
      if (slot < base + cnt) {
        // the (slot - base)-th set bit of the mask
        const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        src = __ffsll((unsigned long long)__ballot(chosen && pos == slot)) - 1;
        break;
      }
      base += cnt;
    }
    int i_, pg_;
    sel_listed(L, min(64 * m + lane, n - 1), i_, pg_);
    j = __builtin_amdgcn_readlane(i_ + 1, src);
    page = __builtin_amdgcn_readlane(pg_, src);
  } else {
    select_bucket<KPT>(a, nb, k, L, [&](int pos, int id, int pg) {
      if (pos == slot) {
        L.s_j = id;
        L.s_page = pg;
      }
    });
    __syncthreads();
    j = L.s_j;
    page = L.s_page;
  }
}

}  // namespace
}  // namespace spla
