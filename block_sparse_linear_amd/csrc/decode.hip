// spla_decode kernels.
//
//   k_score    log-domain second-order Taylor block score of every candidate
//              block, summed over the query heads of a KV group
//              (SPLA Technical Summary 2.1, score formula with the diagonal
//              covariance of its implementation paragraph)
//   k_select   top-(top_k - 2) candidates per (sequence, KV head) by radix
//              select over the scores, plus the sink and the current block
//   k_attend   one selected block per workgroup: exact softmax partials
//              (max, sum, sum p v) and the linear-attention partials
//              (sum w v, sum w, w = phi(q).phi(k)) from the same K/V tile
//              (Technical Summary 2.2: o_tilde from the blocks already loaded)
//   k_combine  merge of the partials, o_bar = phi(q)^T S_all, o_rla = o_bar -
//              o_tilde, D = phi(q).z_all - sum w, o = o_sparse + g_h o_rla
#include "append_items.h"

namespace spla {

namespace {

__device__ __forceinline__ int n_blocks(const DecodeArgs& a, int b) { return (a.lens[b] + a.bk - 1) / a.bk; }

// ============================================================== score
// grid (score_tiles, G, B); lane = block within a 64-block tile, the four
// wavefronts split the channels and meet in LDS.  Every wavefront issues its
// query loads and then all of its statistics loads before the first wait.
template <bool BF16, int R, int D>
__device__ void score_tile(const DecodeArgs& a, const int t, const int g, const int b) {
  constexpr int NC4 = D / 16;  // channel quartets per wavefront
  constexpr int CW = D / 4;    // channels per wavefront
  constexpr int QPL = (R * CW + 63) / 64;  // query elements per lane
  __shared__ float4 qs[4][R][CW / 4];
  __shared__ float4 q2s[4][R][CW / 4];
  __shared__ float red[4][2 * R][kTile];
  const int nb = n_blocks(a, b);
  if (nb <= a.top_k) return;  // every block is selected, nothing to rank
  const int j0 = t * kTile;
  if (j0 > nb - 2) return;
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
    qv[i] = load_elem<BF16>(a.q, ((size_t)b * a.H + g * R + h) * D + w * CW + c);
  }
  // statistics of the tile: 64 blocks x this wavefront's channels
  const float4* mean4 = reinterpret_cast<const float4*>(a.blk_mean);
  const float4* var4 = reinterpret_cast<const float4*>(a.blk_var);
  const size_t base = (((size_t)b * a.G + g) * a.n_tiles + t) * (size_t)(D / 4) * kTile + (size_t)(w * NC4) * kTile + lane;
  float4 m[NC4], v[NC4];
#pragma unroll
  for (int i = 0; i < NC4; ++i) m[i] = mean4[base + (size_t)i * kTile];
#pragma unroll
  for (int i = 0; i < NC4; ++i) v[i] = var4[base + (size_t)i * kTile];
  // keep every load above this point: the whole tile is in flight before the
  // first use
  __builtin_amdgcn_sched_barrier(0);
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
    const float ls = dd * a.inv_sqrt_d + __logf(1.f + fmaxf(vv, 0.f) * half_inv_d);
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
      a.lg[((size_t)b * a.G + g) * (size_t)(a.n_tiles * kTile) + j] = cand ? lg : -INFINITY;
      if (a.lg_out && cand) a.lg_out[((size_t)b * a.G + g) * a.max_blocks + j] = lg;
    }
  }
}

template <bool BF16, int R, int D>
__global__ __launch_bounds__(kThreads) void k_score(const DecodeArgs a) {
  score_tile<BF16, R, D>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Fused decode step, first launch: the scorer's tiles (flat, first) and the
// append of this step's token for every sequence.  The two are independent:
// the scorer reads statistics of candidate blocks 1..nb-2 only, all completed
// by earlier appends, and neither pages nor S_all.
template <bool BF16, int R, int D>
__global__ __launch_bounds__(kThreads) void k_step_score(const StepArgs a) {
  const DecodeArgs& dc = a.dec;
  const int nsc = dc.score_tiles * dc.G * dc.B;
  int item = blockIdx.x;
  if (item < nsc) {
    const int t = item % dc.score_tiles;
    const int g = (item / dc.score_tiles) % dc.G;
    const int b = item / (dc.score_tiles * dc.G);
    score_tile<BF16, R, D>(dc, t, g, b);
    return;
  }
  item -= nsc;
  const int chunks = D / (1024 / D);
  if (item < a.s_items) {
    const int per = dc.G * chunks;
    const int b = item / per;
    const int rem = item - b * per;
    const AppendEntry E{b, 1, dc.lens[b] - 1, b};
    append_state_rows<BF16>(a.st, E, rem / chunks, rem % chunks);
    return;
  }
  item -= a.s_items;
  if (item < dc.B) {
    const AppendEntry E{item, 1, dc.lens[item] - 1, item};
    append_page_rows<BF16>(a.st, E, 0);
    return;
  }
  item -= dc.B;
  if (item < a.n_stat * dc.G) {
    const int b = a.stat_seq[item / dc.G];
    const AppendEntry E{b, 1, dc.lens[b] - 1, b};
    append_block_stats<BF16>(a.st, E, dc.lens[b] / dc.bk - 1, item % dc.G);
  }
}

// ============================================================== select
constexpr int kSelMax = kMaxBlocksPerSeq - 2;  // candidates per (b, g) the selector handles
constexpr int kSelLevels = 12;   // bucket refinement levels
constexpr int kSelRank = 256;    // threshold-bucket size ranked exactly

// bucket of x at one refinement level: monotone non-decreasing in x
__device__ __forceinline__ int sel_bucket(float x, float lo, float scale) {
  const float f = (x - lo) * scale;
  return f >= 255.f ? 255 : (f <= 0.f ? 0 : (int)f);
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// append the entries flagged in bit u of `flags` (u < KPT) of every lane of a
// wavefront to an LDS list with one atomic per wavefront; slot[u] receives the
// entry's position (or -1)
template <int KPT>
__device__ __forceinline__ void wave_append(uint64_t flags, int* counter, int (&slot)[KPT]) {
  int total = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) total += __popcll(__ballot((flags >> u) & 1));
  if (total == 0) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) slot[u] = -1;
    return;
  }
  int base = 0;
  if ((threadIdx.x & 63) == 0) base = atomicAdd(counter, total);
  base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const bool f = (flags >> u) & 1;
    const uint64_t m = __ballot(f);
    slot[u] = f ? base + lanes_below(m) : -1;
    base += __popcll(m);
  }
}

// grid (G, B).  Bucket select over the scores held in registers (KPT per
// thread, candidate i = thread + 256 u): the scores are binned into 256
// buckets spread over [min, max] of the remaining candidates; every
// candidate in a bucket above the one holding the k'-th largest is taken, and
// that bucket is refined the same way until it holds at most kSelRank
// candidates (then ranked exactly by (score desc, id asc)) or only equal
// scores (then taken by ascending id).  The bucket index is a monotone function
// of the score, so the result is the exact top k'.  The chosen ids are sorted
// by a rank count and written ascending with their page ids.
template <int KPT>
__global__ __launch_bounds__(kThreads) void k_select(const DecodeArgs a) {
  __shared__ int hist[4][256];  // one histogram per wavefront
  __shared__ float s_mn[4], s_mx[4];
  __shared__ int s_cnt[4];
  __shared__ int s_bt, s_above, s_n, s_nm;
  // lists padded with sentinels so the rank counts read them four at a time
  __shared__ __attribute__((aligned(16))) float mkey[kSelRank];
  __shared__ __attribute__((aligned(16))) int midx[kSelRank];
  __shared__ __attribute__((aligned(16))) int slist[256];
  __shared__ int spage[256];      // page of slist[i]
  __shared__ int mpage[kSelRank];  // page of midx[i]
  const int g = blockIdx.x, b = blockIdx.y;
  const int nb = n_blocks(a, b);
  int32_t* out = a.sel + ((size_t)b * a.G + g) * a.top_k;
  int32_t* out2 = a.sel_out ? a.sel_out + ((size_t)b * a.G + g) * a.top_k : nullptr;
  int32_t* pages = a.sel_page + ((size_t)b * a.G + g) * a.top_k;
  const int32_t* btab = a.block_table + (size_t)b * a.max_blocks;
  if (nb <= a.top_k) {
    for (int s = threadIdx.x; s < a.top_k; s += kThreads) {
      out[s] = s < nb ? s : -1;
      if (out2) out2[s] = s < nb ? s : -1;
      pages[s] = s < nb ? btab[s] : -1;
    }
    return;
  }
  const int nc = nb - 2;
  const int kp = a.top_k - 2;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float* row = a.lg + ((size_t)b * a.G + g) * (size_t)(a.n_tiles * kTile) + 1;  // row[i] = LG(i + 1)
  // scores and page ids of this thread's candidates (the pages ride along so
  // the output needs no dependent lookup), plus the sink's and current's pages
  float x[KPT];
  int pg[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int i = min((int)threadIdx.x + u * kThreads, nc - 1);  // clamped, masked by memb below
    x[u] = row[i];
    pg[u] = btab[i + 1];
  }
  const int pg_sink = btab[0], pg_cur = btab[nb - 1];
  uint64_t memb = 0, above = 0;  // bit u: key u still in the threshold bucket / already taken
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if ((int)threadIdx.x + u * kThreads < nc) memb |= 1ull << u;
  if (threadIdx.x == 0) {
    s_n = 0;
    s_nm = 0;
  }
  mkey[threadIdx.x] = -INFINITY;
  midx[threadIdx.x] = 0x7fffffff;
  slist[threadIdx.x] = 0x7fffffff;
  int need = kp;
  bool equal_mode = false;
  for (int lev = 0;; ++lev) {
    float mn = INFINITY, mx = -INFINITY;
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      if (memb >> u & 1) {
        mn = fminf(mn, x[u]);
        mx = fmaxf(mx, x[u]);
        ++cnt;
      }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    cnt = wave_sum_i(cnt);
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[q][threadIdx.x] = 0;
    if (lane == 0) {
      s_mn[wv] = mn;
      s_mx[wv] = mx;
      s_cnt[wv] = cnt;
    }
    __syncthreads();
    mn = fminf(fminf(s_mn[0], s_mn[1]), fminf(s_mn[2], s_mn[3]));
    mx = fmaxf(fmaxf(s_mx[0], s_mx[1]), fmaxf(s_mx[2], s_mx[3]));
    cnt = (s_cnt[0] + s_cnt[1]) + (s_cnt[2] + s_cnt[3]);
    if (cnt <= kSelRank) break;
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
      bkt[u] = sel_bucket(x[u], mn, scale);
      if (memb >> u & 1) atomicAdd(&hist[wv][bkt[u]], 1);
    }
    __syncthreads();
    if (wv == 0) {
      int c[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int bin = 255 - 4 * lane - q;
        c[q] = (hist[0][bin] + hist[1][bin]) + (hist[2][bin] + hist[3][bin]);
        sum += c[q];
      }
      int run = wave_incl_scan_i(sum) - sum;  // keys in buckets above this lane's
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (run < need && run + c[q] >= need) {
          s_bt = 255 - 4 * lane - q;
          s_above = run;
        }
        run += c[q];
      }
    }
    __syncthreads();
    const int bt = s_bt;
    need -= s_above;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      if (memb >> u & 1) {
        if (bkt[u] > bt) above |= 1ull << u;
        if (bkt[u] != bt) memb &= ~(1ull << u);
      }
    }
  }
  // taken so far: every key above a threshold bucket
  {
    int slot[KPT];
    wave_append<KPT>(above, &s_n, slot);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      if (slot[u] >= 0) {
        slist[slot[u]] = threadIdx.x + u * kThreads;
        spage[slot[u]] = pg[u];
      }
    }
  }
  if (!equal_mode) {
    // the final bucket (<= kSelRank candidates): exact rank by (score desc, id asc)
    {
      int slot[KPT];
      wave_append<KPT>(memb, &s_nm, slot);
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        if (slot[u] >= 0) {
          mkey[slot[u]] = x[u];
          midx[slot[u]] = threadIdx.x + u * kThreads;
          mpage[slot[u]] = pg[u];
        }
      }
    }
    __syncthreads();
    const int nm = s_nm;
    bool take = false;
    int my = 0, mypg = 0;
    if ((int)threadIdx.x < nm) {
      const float xv = mkey[threadIdx.x];
      my = midx[threadIdx.x];
      mypg = mpage[threadIdx.x];
      int rank = 0;
#pragma unroll 4
      for (int v = 0; v < nm; v += 4) {
        const float4 y = *reinterpret_cast<const float4*>(&mkey[v]);
        const int4 iy = *reinterpret_cast<const int4*>(&midx[v]);
        rank += (y.x > xv) || (y.x == xv && iy.x < my);
        rank += (y.y > xv) || (y.y == xv && iy.y < my);
        rank += (y.z > xv) || (y.z == xv && iy.z < my);
        rank += (y.w > xv) || (y.w == xv && iy.w < my);
      }
      take = rank < need;
    }
    int slot1[1];
    wave_append<1>(take ? 1ull : 0ull, &s_n, slot1);
    if (slot1[0] >= 0) {
      slist[slot1[0]] = my;
      spage[slot1[0]] = mypg;
    }
  } else {
    // equal scores: the `need` smallest ids among the members; find the id
    // bound by bisection on counts
    int lo = 0, hi = nc;  // smallest X with #members(id < X) >= need
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      int c = 0;
#pragma unroll
      for (int u = 0; u < KPT; ++u) c += (memb >> u & 1) && ((int)threadIdx.x + u * kThreads < mid);
      c = wave_sum_i(c);
      __syncthreads();
      if (lane == 0) s_cnt[wv] = c;
      __syncthreads();
      c = (s_cnt[0] + s_cnt[1]) + (s_cnt[2] + s_cnt[3]);
      if (c >= need) hi = mid; else lo = mid + 1;
    }
    uint64_t low = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      if ((memb >> u & 1) && (int)threadIdx.x + u * kThreads < lo) low |= 1ull << u;
    int slot[KPT];
    wave_append<KPT>(low, &s_n, slot);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      if (slot[u] >= 0) {
        slist[slot[u]] = threadIdx.x + u * kThreads;
        spage[slot[u]] = pg[u];
      }
    }
  }
  __syncthreads();
  // ascending order by a rank count over the kp chosen ids
  if ((int)threadIdx.x < kp) {
    const int v = slist[threadIdx.x];
    int pos = 0;
#pragma unroll 4
    for (int u = 0; u < kp; u += 4) {
      const int4 y = *reinterpret_cast<const int4*>(&slist[u]);
      pos += (y.x < v) + (y.y < v) + (y.z < v) + (y.w < v);
    }
    out[1 + pos] = v + 1;
    if (out2) out2[1 + pos] = v + 1;
    pages[1 + pos] = spage[threadIdx.x];
  } else if ((int)threadIdx.x == kp) {
    out[0] = 0;
    if (out2) out2[0] = 0;
    pages[0] = pg_sink;
  } else if ((int)threadIdx.x == kp + 1) {
    out[kp + 1] = nb - 1;
    if (out2) out2[kp + 1] = nb - 1;
    pages[kp + 1] = pg_cur;
  }
}

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
  const int page = a.block_table[(size_t)b * a.max_blocks + j];
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
  const int rec = 2 * d + kPartHdr;
#pragma unroll
  for (int k = 0; k < npair; ++k) {
    const int p = grp + k * ngrp;
    if (p < 2 * R) {
      const int h = p < R ? p : p - R;
      float* dst = a.part + (((size_t)b * a.H + g * R + h) * a.top_k + slot) * rec + kPartHdr + (p < R ? 0 : d);
      dst[c] = acc[k];
    }
  }
  if (threadIdx.x < R) {
    const int h = threadIdx.x;
    float* dst = a.part + (((size_t)b * a.H + g * R + h) * a.top_k + slot) * rec;
    dst[0] = s_m[h];
    dst[1] = s_l[h];
    dst[2] = s_sw[h];
    dst[3] = 0.f;
  }
}

// ============================================================== attend (MFMA)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (round to nearest even, hardware conversion)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo_f(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi_f(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  c, 0, 0, 0);
}

__device__ __forceinline__ float phi_fast(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// phi of 8 packed bf16 values rounded to bf16
__device__ __forceinline__ uint4 phi_bf16(const uint4& raw) {
  const uint32_t in[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = pack_bf16(phi_fast(bf16_lo_f(in[k])), phi_fast(bf16_hi_f(in[k])));
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// phi of 8 packed bf16 values split into bf16 hi + lo parts (hi + lo carries
// phi to ~2^-16 relative)
__device__ __forceinline__ void phi_hilo(const uint4& raw, uint4& hi, uint4& lo) {
  const uint32_t in[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float f0 = phi_fast(bf16_lo_f(in[k])), f1 = phi_fast(bf16_hi_f(in[k]));
    h[k] = pack_bf16(f0, f1);
    l[k] = pack_bf16(f0 - bf16_lo_f(h[k]), f1 - bf16_hi_f(h[k]));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// grid (top_k, G, B): one selected block of one (b, g) per workgroup, all R
// query heads of the group, bf16 K/V.  Matrix cores do both contractions:
//   (1) logits s = q.k and linear weights w = phi(q).phi(k) of the block's
//       tokens: rows of the 16-row A operand are the R queries and the R
//       phi(q) (bf16 hi/lo split), B is the K tile read straight from the
//       page plus phi(K) hi/lo computed in registers; wavefront w takes 16
//       (Bk = 64) or 32 (Bk = 128) tokens;
//   (2) sum_t p_t v_t and sum_t w_t v_t: rows of A are p and w (hi/lo split,
//       from LDS), B is the V tile staged transposed in LDS; wavefront w
//       takes a quarter of the value channels.
// Softmax max / sums cross the wavefronts through LDS (two barriers).
template <int R, int D, int BK>
__global__ __launch_bounds__(kThreads) void k_attend_mfma(const DecodeArgs a) {
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

  const int slot = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64, l16 = lane % 16, lg4 = lane / 16;
  // queries first: they do not depend on the selection
  const int m = l16;  // A-operand row of this lane in product (1)
  const int hq = m < R ? m : ((m >= WB && m < WB + R) ? m - WB : -1);
  uint4 qraw[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    // unconditional load of a valid row; rows that hold no query are masked
    // when the A operands are formed
    qraw[ks] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                               ((size_t)b * a.H + g * R + max(hq, 0)) * D + 32 * ks + 8 * lg4);
  }
  const size_t srow = ((size_t)b * a.G + g) * a.top_k + slot;
  int j, page;
  if (a.sel_in) {
    j = a.sel_in[srow];
    page = (j >= 0 && j < a.max_blocks) ? a.block_table[(size_t)b * a.max_blocks + j] : -1;
  } else {
    j = a.sel[srow];
    page = a.sel_page[srow];
  }
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
    uint4 hi, lo;
    phi_hilo(qraw[ks], hi, lo);
    aq[ks] = make_uint4(qraw[ks].x & mq, qraw[ks].y & mq, qraw[ks].z & mq, qraw[ks].w & mq);
    afh[ks] = make_uint4(hi.x & mw, hi.y & mw, hi.z & mw, hi.w & mw);
    afl[ks] = make_uint4(lo.x & mw, lo.y & mw, lo.z & mw, lo.w & mw);
  }

  // ---- product (1): logits and linear weights of this wavefront's tokens
  f32x4_t c1[NT1W];
#pragma unroll
  for (int nt = 0; nt < NT1W; ++nt) {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      // phi(k) in bf16 (its rounding is independent per token and averages
      // out of o_tilde); phi(q) keeps hi + lo (shared by every token)
      const uint4 fk = phi_bf16(kraw[nt][ks]);
      c = mfma_bf16(aq[ks], kraw[nt][ks], c);
      c = mfma_bf16(afh[ks], fk, c);
      c = mfma_bf16(afl[ks], fk, c);
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

// ============================================================== combine
// grid (D/32, G, B): one 32-channel slice of the R heads of (b, g).  Merges
// the per-block partials (softmax rescaling by exp(m_s - m) / L), contracts
// phi(q) with the slice's S_all columns (o_bar) and, in slice 0, with z_all
// (the normaliser D), and writes o = o_sparse + g_h (o_bar - o_tilde).
// Item = (kind, head, channel quartet) of the slice; the slots are split over
// SG thread groups whose float4 sums meet in LDS.  Every global load is
// issued before the first wait.
template <bool BF16, int R, int D>
__global__ __launch_bounds__(kThreads) void k_combine(const DecodeArgs a) {
  constexpr int CS = 32;                 // channels per workgroup
  constexpr int RG = kThreads / CS;      // row groups of the S contraction
  constexpr int RPG = D / RG;            // rows per group
  constexpr int NIT = 2 * R * (CS / 4);  // float4 items
  constexpr int SG = kThreads / NIT;     // slot groups
  constexpr int SPT = 16;                // slots per thread per load batch
  constexpr int HPW = (R + 3) / 4;       // heads per wavefront (header pass)
  constexpr int SPL = 4;                 // slots per lane in the header pass (top_k <= 256)
  constexpr int QPT = (R * D + kThreads - 1) / kThreads;
  __shared__ float fq[R][D];
  __shared__ float wsl[R][256];          // exp(m_s - m) / L per head and slot (0 for unused slots)
  __shared__ int valid[256];
  __shared__ float obr[RG][R][CS];
  __shared__ float4 red4[SG][NIT];
  __shared__ float s_sw[R], s_dz[R];
  const int cc = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nb = n_blocks(a, b);
  const bool covers_all = nb <= a.top_k;
  const int top_k = a.top_k;
  const int32_t* srow = (a.sel_in ? a.sel_in : a.sel) + ((size_t)b * a.G + g) * top_k;
  const int rec = 2 * D + kPartHdr;
  const float* P0 = a.part + ((size_t)b * a.H + g * R) * top_k * (size_t)rec;
  const int c0 = cc * CS;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  // ---- loads
  const int sc = threadIdx.x % CS, rg = threadIdx.x / CS;
  const float* S = a.s_all + ((size_t)b * a.G + g) * D * (size_t)D + (size_t)(rg * RPG) * D + c0 + sc;
  float sv[RPG];
#pragma unroll
  for (int x = 0; x < RPG; ++x) sv[x] = S[(size_t)x * D];
  float qv[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = threadIdx.x + k * kThreads;
    qv[k] = load_elem<BF16>(a.q, ((size_t)b * a.H + g * R) * D + min(i, R * D - 1));
  }
  float zv[(D + 63) / 64];
#pragma unroll
  for (int k = 0; k < (D + 63) / 64; ++k) zv[k] = a.z_all[((size_t)b * a.G + g) * D + lane + 64 * k];
  int vs[SPL];
#pragma unroll
  for (int u = 0; u < SPL; ++u) {
    const int s = lane + 64 * u;
    const int v = srow[min(s, top_k - 1)];
    vs[u] = s < top_k ? v : -1;
  }
  float hm[HPW][SPL], hl[HPW][SPL], hs[HPW][SPL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = min(w + 4 * hh, R - 1);
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int s = min(lane + 64 * u, top_k - 1);
      const float* P = P0 + ((size_t)h * top_k + s) * rec;
      hm[hh][u] = P[0];
      hl[hh][u] = P[1];
      hs[hh][u] = P[2];
    }
  }
  const int it = threadIdx.x % NIT, sg = threadIdx.x / NIT;
  const int kind = it / (R * CS / 4), ih = (it / (CS / 4)) % R, c4 = it % (CS / 4);
  const float* PD = P0 + (size_t)ih * top_k * rec + kPartHdr + (kind ? D : 0) + c0 + 4 * c4;
  float4 dv[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int s = sg + SG * u;
    dv[u] = *reinterpret_cast<const float4*>(PD + (size_t)min(s, top_k - 1) * rec);
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- phi(q), validity, merge weights and phi(q).z per head
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = threadIdx.x + k * kThreads;
    if (i < R * D) fq[i / D][i % D] = phi_f(qv[k]);
  }
  if (w == 0) {
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int s = lane + 64 * u;
      if (s < top_k) valid[s] = (vs[u] >= 0 && vs[u] < nb) ? 1 : 0;
    }
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = w + 4 * hh;
    if (h >= R) continue;
    bool ok[SPL];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      ok[u] = vs[u] >= 0 && vs[u] < nb;
      if (ok[u]) m = fmaxf(m, hm[hh][u]);
    }
    m = wave_max(m);
    float l = 0.f, sw = 0.f, e[SPL];
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      e[u] = ok[u] ? expf(hm[hh][u] - m) : 0.f;
      l = fmaf(e[u], ok[u] ? hl[hh][u] : 0.f, l);
      sw += ok[u] ? hs[hh][u] : 0.f;
    }
    l = wave_sum(l);
    sw = wave_sum(sw);
    const float inv_l = 1.f / l;
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int s = lane + 64 * u;
      if (s < top_k) wsl[h][s] = e[u] * inv_l;
    }
    float dz = 0.f;
    if (cc == 0) {
#pragma unroll
      for (int k = 0; k < (D + 63) / 64; ++k) dz = fmaf(fq[h][lane + 64 * k], zv[k], dz);
      dz = wave_sum(dz);
    }
    if (lane == 0) {
      s_sw[h] = sw;
      s_dz[h] = dz;
    }
  }
  // o_bar partial sums over this thread's rows
  {
    float ob[R];
#pragma unroll
    for (int h = 0; h < R; ++h) ob[h] = 0.f;
#pragma unroll
    for (int x = 0; x < RPG; ++x) {
#pragma unroll
      for (int h = 0; h < R; ++h) ob[h] = fmaf(fq[h][rg * RPG + x], sv[x], ob[h]);
    }
#pragma unroll
    for (int h = 0; h < R; ++h) obr[rg][h][sc] = ob[h];
  }
  __syncthreads();
  // ---- this thread's slots of its item
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int u0 = 0; sg + SG * u0 < top_k; u0 += SPT) {
    if (u0 > 0) {
#pragma unroll
      for (int u = 0; u < SPT; ++u) {
        const int s = sg + SG * (u0 + u);
        dv[u] = *reinterpret_cast<const float4*>(PD + (size_t)min(s, top_k - 1) * rec);
      }
    }
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int s = sg + SG * (u0 + u);
      if (s >= top_k || !valid[s]) continue;  // unused slot: its record holds stale data
      const float wt = kind == 0 ? wsl[ih][s] : 1.f;
      acc.x = fmaf(wt, dv[u].x, acc.x);
      acc.y = fmaf(wt, dv[u].y, acc.y);
      acc.z = fmaf(wt, dv[u].z, acc.z);
      acc.w = fmaf(wt, dv[u].w, acc.w);
    }
  }
  red4[sg][it] = acc;
  __syncthreads();
  // ---- finalise: thread = (head, channel quartet), both kinds from LDS
  if ((int)threadIdx.x < R * CS / 4) {
    const int h = threadIdx.x / (CS / 4), q4 = threadIdx.x % (CS / 4);
    float4 os = make_float4(0.f, 0.f, 0.f, 0.f), ot = os;
#pragma unroll
    for (int k = 0; k < SG; ++k) {
      const float4 x0 = red4[k][h * (CS / 4) + q4];
      const float4 x1 = red4[k][R * CS / 4 + h * (CS / 4) + q4];
      os.x += x0.x; os.y += x0.y; os.z += x0.z; os.w += x0.w;
      ot.x += x1.x; ot.y += x1.y; ot.z += x1.z; ot.w += x1.w;
    }
    float orl[4] = {0.f, 0.f, 0.f, 0.f};
    if (!covers_all) {
      const float otv[4] = {ot.x, ot.y, ot.z, ot.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float obar = 0.f;
#pragma unroll
        for (int q = 0; q < RG; ++q) obar += obr[q][h][4 * q4 + e];
        orl[e] = obar - otv[e];
      }
    }
    const size_t oi = ((size_t)b * a.H + g * R + h) * D + c0 + 4 * q4;
    const float gh = a.gate[g * R + h];
    *reinterpret_cast<float4*>(a.out + oi) =
        make_float4(fmaf(gh, orl[0], os.x), fmaf(gh, orl[1], os.y), fmaf(gh, orl[2], os.z), fmaf(gh, orl[3], os.w));
    if (a.o_sparse_out) *reinterpret_cast<float4*>(a.o_sparse_out + oi) = os;
    if (a.o_rla_out) *reinterpret_cast<float4*>(a.o_rla_out + oi) = make_float4(orl[0], orl[1], orl[2], orl[3]);
  }
  if (cc == 0 && (int)threadIdx.x < top_k && a.sel_out)
    a.sel_out[((size_t)b * a.G + g) * top_k + threadIdx.x] = srow[threadIdx.x];
  if (cc == 0 && (int)threadIdx.x < R && a.d_rla_out) {
    const int h = threadIdx.x;
    a.d_rla_out[(size_t)b * a.H + g * R + h] = covers_all ? 0.f : s_dz[h] - s_sw[h];
  }
}

}  // namespace

// each launcher returns the status of its own launch (hipLaunchKernel /
// hipExtLaunchKernel report it directly, so an error left behind by an
// unrelated earlier HIP call is never attributed to it)
#define SPLA_DISPATCH_D(D_, ...)                                     \
  switch (D_) {                                                     \
    case 64: { constexpr int DD = 64; return __VA_ARGS__; }         \
    case 128: { constexpr int DD = 128; return __VA_ARGS__; }       \
    default: return hipErrorInvalidValue;                           \
  }
#define SPLA_DISPATCH_RD(R_, D_, ...)                                         \
  switch (R_) {                                                              \
    case 1: { constexpr int RR = 1; SPLA_DISPATCH_D(D_, __VA_ARGS__) }       \
    case 2: { constexpr int RR = 2; SPLA_DISPATCH_D(D_, __VA_ARGS__) }       \
    case 4: { constexpr int RR = 4; SPLA_DISPATCH_D(D_, __VA_ARGS__) }       \
    case 8: { constexpr int RR = 8; SPLA_DISPATCH_D(D_, __VA_ARGS__) }       \
    default: return hipErrorInvalidValue;                                    \
  }

hipError_t launch_score(const DecodeArgs& a, bool bf16, const Launch& l) {
  const dim3 grid(a.score_tiles, a.G, a.B);
  if (a.score_tiles == 0) return hipSuccess;
  if (bf16) SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_score<true, RR, DD>, grid, l, a))
  SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_score<false, RR, DD>, grid, l, a))
}

hipError_t launch_step_score(const StepArgs& a, bool bf16, const Launch& l) {
  const dim3 grid(a.dec.score_tiles * a.dec.G * a.dec.B + a.s_items + a.dec.B + a.n_stat * a.dec.G);
  if (bf16) SPLA_DISPATCH_RD(a.dec.r, a.dec.d, launch_kernel(k_step_score<true, RR, DD>, grid, l, a))
  SPLA_DISPATCH_RD(a.dec.r, a.dec.d, launch_kernel(k_step_score<false, RR, DD>, grid, l, a))
}

// keys-per-thread sizes compiled for the selector: the smallest one that
// holds the longest sequence's candidates is launched
template <int... Ks>
struct SelectSizes {};

template <int K, int... Ks>
hipError_t launch_select_sized(const DecodeArgs& a, const Launch& l, int nc, SelectSizes<K, Ks...>) {
  if (nc <= K * kThreads) return launch_kernel(k_select<K>, dim3(a.G, a.B), l, a);
  if constexpr (sizeof...(Ks) == 0) {
    return hipErrorInvalidValue;
  } else {
    return launch_select_sized(a, l, nc, SelectSizes<Ks...>{});
  }
}

hipError_t launch_select(const DecodeArgs& a, const Launch& l) {
  int nc = 0;  // candidates of the longest sequence that has more blocks than top_k
  for (int b = 0; b < a.B; ++b) {
    const int nb = (a.lens[b] + a.bk - 1) / a.bk;
    if (nb > a.top_k) nc = max(nc, nb - 2);
  }
  return launch_select_sized(a, l, nc, SelectSizes<1, 2, 3, 4, 6, 8, 9, 10, 12, 16, 20, 24, 32, 40, 48, 64>{});
}

hipError_t launch_attend(const DecodeArgs& a, bool bf16, const Launch& l) {
  const dim3 grid(a.top_k, a.G, a.B);
  if (!bf16) SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_attend<false, RR, DD>, grid, l, a))
  if (a.bk == 64) SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_attend_mfma<RR, DD, 64>, grid, l, a))
  SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_attend_mfma<RR, DD, 128>, grid, l, a))
}

hipError_t launch_combine(const DecodeArgs& a, bool bf16, const Launch& l) {
  const dim3 grid(a.d / 32, a.G, a.B);
  if (bf16) SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_combine<true, RR, DD>, grid, l, a))
  SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_combine<false, RR, DD>, grid, l, a))
}

}  // namespace spla
