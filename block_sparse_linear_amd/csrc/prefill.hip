// Block-centric attend of a prefill group (bf16 K/V, matrix cores).  The
// group's m virtual queries select up to top_k blocks each; a block chosen by
// several of them is read once per work item of up to kPfQ queries instead of
// once per (query, slot).  Three launches:
//   k_pf_bucket  files every (query, slot) under its block: lists[g][j][cap]
//   k_pf_items   turns the non-empty lists into work items (KV head, block,
//                page, up to kPfQ query codes) and clears the counts
//   k_pf_attend  one item per workgroup: the block's K tile in registers
//                (with phi(K) hi / lo), its V tile transposed in LDS, the
//                item's queries staged in LDS, then the queries in batches
//                of 16 / R through the decode attend's products (16 A rows
//                = (query, head) pairs) and partial records
// A query code is vq * 256 + slot.
#include "attend_mfma.h"

namespace spla {

namespace {

// max of two floats below +inf (finite logits or the -inf of an empty row) in
// one instruction, the median of x, y and the largest float: fmaxf first quiets
// signalling NaNs, one more instruction per operand that comes from LDS or
// another lane, and the median with +inf is folded back into fmaxf
__device__ __forceinline__ float max_nn(float x, float y) { return __builtin_amdgcn_fmed3f(x, y, 3.402823466e38f); }
__device__ __forceinline__ float row16_max_nn(float v) {
  v = max_nn(v, dpp_f<kDppXor1>(v, v));
  v = max_nn(v, dpp_f<kDppXor2>(v, v));
  v = max_nn(v, dpp_f<kDppRowHalfMirror>(v, v));
  return max_nn(v, dpp_f<kDppRowMirror>(v, v));
}

// grid (ceil(G * max_blocks / 256)): the per-block counts start at zero
__global__ __launch_bounds__(kThreads) void k_pf_clear(int32_t* cnt, int32_t n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) cnt[i] = 0;
}

// grid (ceil(m top_k / 256), G): thread = (query vq, slot s), the slots of
// consecutive queries side by side (a workgroup per query would leave all but
// top_k of its threads idle)
__global__ __launch_bounds__(kThreads) void k_pf_bucket(const int32_t* sel, int32_t* cnt, int32_t* lists,
                                                         int32_t* n_items, int32_t m, int32_t G, int32_t top_k,
                                                         int32_t max_blocks, int32_t cap) {
  const int flat = blockIdx.x * kThreads + threadIdx.x, g = blockIdx.y;
  if (flat == 0 && g == 0) *n_items = 0;
  if (flat >= m * top_k) return;
  const int vq = flat / top_k, s = flat - vq * top_k;
  const int j = sel[((size_t)vq * G + g) * top_k + s];
  if (j < 0 || j >= max_blocks) return;
  const size_t cell = (size_t)g * max_blocks + j;
  const int idx = atomicAdd(&cnt[cell], 1);  // < cap: a query selects a block at most once
  if (idx < cap) lists[cell * cap + idx] = vq * 256 + s;
}

// grid (ceil(max_blocks / 256), G): thread = block j; items of kPfQ codes
__global__ __launch_bounds__(kThreads) void k_pf_items(int32_t* cnt, const int32_t* lists, int4* items,
                                                        int32_t* n_items, const int32_t* block_table, int32_t G,
                                                        int32_t max_blocks, int32_t cap, int32_t max_items) {
  const int j = blockIdx.x * kThreads + threadIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x % 64;
  const size_t cell = (size_t)g * max_blocks + j;
  const int c = j < max_blocks ? min(cnt[cell], cap) : 0;
  const int nch = (c + kPfQ - 1) / kPfQ;
  // places in the item list: one atomic per workgroup (nearly every block has
  // items, and atomics on the one counter queue at the cache), the
  // wavefronts' totals through LDS
  __shared__ int s_wsum[kThreads / 64], s_base;
  const int w = threadIdx.x / 64;
  const int incl = wave_incl_scan_i(nch);
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
#pragma unroll
    for (int k = 0; k < kThreads / 64; ++k) tot += s_wsum[k];
    s_base = tot > 0 ? atomicAdd(n_items, tot) : 0;
  }
  __syncthreads();
  int base = s_base + incl - nch;
  for (int k = 0; k < w; ++k) base += s_wsum[k];
  if (c == 0) return;
  const int page = block_table[j];
  for (int i = 0; i < nch && base + i < max_items; ++i) {  // max_items bounds the sum of nch
    const int n = min(kPfQ, c - i * kPfQ);
    int code[kPfQ];
#pragma unroll
    for (int e = 0; e < kPfQ; ++e) code[e] = e < n ? lists[cell * cap + i * kPfQ + e] : 0;
    int4* it = items + (size_t)(base + i) * kPfItemInts / 4;
    it[0] = make_int4(g, j, n, page);
#pragma unroll
    for (int e = 0; e < kPfQ; e += 4) it[1 + e / 4] = make_int4(code[e], code[e + 1], code[e + 2], code[e + 3]);
  }
  cnt[cell] = 0;
}

// one work item per workgroup (grid: an upper bound of the item count).  A
// batch of QB = 16 / R queries fills the 16 rows of the A operands: product
// (1) forms the logits from the q rows and the linear weights from the
// phi(q) hi / lo rows (separate accumulators), the softmax max and sums meet
// across the wavefronts in LDS (one exchange per batch), and product (2)
// takes the batch's p and w rows (hi / lo, 64 rows) against the V tile.  Each
// row has its own causal limit (its query's length).
template <int R, int D, int BK>
__global__ __launch_bounds__(kThreads) void k_pf_attend(const int4* items, const int32_t* n_items,
                                                         const DecodeArgs a) {
  constexpr int NKS = D / 32;              // k-steps per channel block
  constexpr int NT1W = BK / 64;            // 16-token tiles per wavefront
  constexpr int QB = 16 / R;               // queries per batch: A rows (query, head) = 16
  constexpr int NT2W = D / 64;             // 16-channel tiles per wavefront
  constexpr int MT2 = 4;                   // row tiles of product (2): hi/lo rows of p and w of 16 rows
  constexpr int KS2 = BK / 32;             // token k-steps of product (2)
  constexpr int VS = BK + 8;               // row stride (elements) of the transposed V tile
  // p / w rows: stride BK + 8 elements, odd (lo) rows shifted by 4 more words
  // into their pad and rows 8 u .. 8 u + 7 by 16 u words (the shifts only
  // grow, so rows never overlap), so that the 32 words one ds_write_b32 of a
  // half-wavefront stores (lane groups 0-1 or 2-3, hi and lo rows, 8 token
  // pairs) fall in 32 different banks.  Three workgroups still fit a CU's LDS
  // at 4 x 128.
  constexpr int PS = BK + 8;
  auto pw_row = [](int row) { return row * PS + 8 * (row & 1) + 32 * (row >> 3); };
  constexpr int NV = BK * D / (16 * kThreads);  // token-pair x 8-channel pieces per thread
  constexpr int QE = R * 3 * D;            // staged elements per query: raw q, phi(q) hi, lo per head
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VS];
  __shared__ __attribute__((aligned(16))) uint16_t pw[MT2 * 16 * PS + 8 + 32 * (MT2 * 2 - 1)];
  __shared__ __attribute__((aligned(16))) uint16_t qs[kPfQ * QE];
  __shared__ float s_max[4][16], s_l[4][16], s_sw[4][16];
  __shared__ int s_code[kPfQ];
  __shared__ int s_len[kPfQ];     // length of each query's sequence prefix (its causal limit)
  __shared__ size_t s_dst[16];    // partial record index of each A row of the current batch
  // the item (the array holds max_items records, so any workgroup may read
  // its own) and the count, in one round trip
  const int4* itp = items + (size_t)blockIdx.x * kPfItemInts / 4;
  const int* codes = reinterpret_cast<const int*>(itp) + 4;  // kPfQ codes (0 past n)
  const int4 hd = itp[0];
  const int my_code = codes[min((int)threadIdx.x, kPfQ - 1)];  // first of all vector loads
  __builtin_amdgcn_sched_barrier(0);
  SPLA_SCALARS_READY("s"(a.q), "s"(a.phq), "s"(a.H), "s"(a.k_pages), "s"(a.v_pages), "s"(a.G), "s"(a.num_pages));
  if ((int)blockIdx.x >= *n_items) return;
  const int g = hd.x, j = hd.y, n = hd.z, page = hd.w;
  if (page < 0 || page >= a.num_pages) {
    if (threadIdx.x == 0) atomicOr(a.err, kErrPage);
    return;
  }
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64, l16 = lane % 16, lg4 = lane / 16;
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.k_pages) + ((size_t)page * a.G + g) * BK * D;
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(a.v_pages) + ((size_t)page * a.G + g) * BK * D;
  // ---- every global load first: K operands, V pieces, the item's queries
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
  // the codes through LDS (each piece needs the code of its own query), then
  // the item's queries: q and phi(q) hi / lo, staged for every query of the loop
  if (threadIdx.x < kPfQ) {
    s_code[threadIdx.x] = my_code;
    s_len[threadIdx.x] = a.lens[my_code >> 8];
  }
  __syncthreads();
  constexpr int QPT = (kPfQ * QE / 8 + kThreads - 1) / kThreads;  // 8-element pieces per thread
  static_assert(QPT <= 12, "at most 12 staged query pieces per thread");
  // piece i of this thread: q (kind 0) or phi(q) hi / lo (kind 1, 2) of head h
  // of the item's query e, 8 channels; pieces past the end repeat the last
  auto pidx = [&](int i) { return min((int)threadIdx.x + kThreads * i, kPfQ * QE / 8 - 1); };
  // the code of each piece's query first (a code past n is 0: query 0, read
  // and unused), then every load; named registers, not arrays (an array here
  // ends up in scratch)
  auto code_of = [&](int i) { return s_code[pidx(i) / (QE / 8)]; };
  const int k0 = code_of(0), k1 = QPT > 1 ? code_of(1) : 0, k2 = QPT > 2 ? code_of(2) : 0;
  const int k3 = QPT > 3 ? code_of(3) : 0, k4 = QPT > 4 ? code_of(4) : 0, k5 = QPT > 5 ? code_of(5) : 0;
  const int k6 = QPT > 6 ? code_of(6) : 0, k7 = QPT > 7 ? code_of(7) : 0, k8 = QPT > 8 ? code_of(8) : 0;
  const int k9 = QPT > 9 ? code_of(9) : 0, k10 = QPT > 10 ? code_of(10) : 0, k11 = QPT > 11 ? code_of(11) : 0;
  const uint16_t* qbase = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* fbase = a.phq;
  const int H = a.H;
  auto piece = [&](int i, int cd) {
    const int rem = pidx(i) % (QE / 8);
    const int h = rem / (3 * D / 8), rem2 = rem % (3 * D / 8);
    const int kind = rem2 / (D / 8), c8 = rem2 % (D / 8);
    const size_t row = (size_t)(cd >> 8) * H + g * R + h;
    const uint16_t* src = kind == 0 ? qbase + row * D : fbase + (row * 2 + (kind - 1)) * D;
    return *reinterpret_cast<const uint4*>(src + 8 * c8);
  };
  const uint4 q0 = piece(0, k0);
  const uint4 q1 = QPT > 1 ? piece(1, k1) : q0, q2 = QPT > 2 ? piece(2, k2) : q0, q3 = QPT > 3 ? piece(3, k3) : q0;
  const uint4 q4 = QPT > 4 ? piece(4, k4) : q0, q5 = QPT > 5 ? piece(5, k5) : q0, q6 = QPT > 6 ? piece(6, k6) : q0;
  const uint4 q7 = QPT > 7 ? piece(7, k7) : q0, q8 = QPT > 8 ? piece(8, k8) : q0, q9 = QPT > 9 ? piece(9, k9) : q0;
  const uint4 q10 = QPT > 10 ? piece(10, k10) : q0, q11 = QPT > 11 ? piece(11, k11) : q0;
  __builtin_amdgcn_sched_barrier(0);
  SPLA_SCALARS_READY("s"(a.bk), "s"(a.top_k), "s"(a.part), "s"(a.part_hdr), "s"(a.inv_sqrt_d), "s"(a.H), "s"(a.B));
  // rows of the tile past the group's last token: never attended, zeroed so
  // that 0 x (stale data) cannot make NaN
  const int nvalid = min(BK, a.lens[a.B - 1] - j * BK);
  {
    // clamped like the loads: a repeated piece rewrites the same value
    uint4* qd = reinterpret_cast<uint4*>(qs);
    auto put = [&](int i, const uint4& v) { qd[min((int)threadIdx.x + kThreads * i, kPfQ * QE / 8 - 1)] = v; };
    put(0, q0);
    if (QPT > 1) put(1, q1);
    if (QPT > 2) put(2, q2);
    if (QPT > 3) put(3, q3);
    if (QPT > 4) put(4, q4);
    if (QPT > 5) put(5, q5);
    if (QPT > 6) put(6, q6);
    if (QPT > 7) put(7, q7);
    if (QPT > 8) put(8, q8);
    if (QPT > 9) put(9, q9);
    if (QPT > 10) put(10, q10);
    if (QPT > 11) put(11, q11);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = threadIdx.x + kThreads * i;
    const int tp = idx % (BK / 2), cg = idx / (BK / 2);
    const bool v0 = 2 * tp < nvalid, v1 = 2 * tp + 1 < nvalid;
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
  // phi(K) of the tile as bf16 hi + lo, once for every query
  uint4 fkh[NT1W][NKS], fkl[NT1W][NKS];
#pragma unroll
  for (int nt = 0; nt < NT1W; ++nt)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) phi_bf16_split(kraw[nt][ks], fkh[nt][ks], fkl[nt][ks]);
  __syncthreads();
  const float inv_sqrt_d = a.inv_sqrt_d;
  const int rec = 2 * D;
  // batches of QB queries: row r = 4 lg4 + i of a result tile is (query
  // b0 + r / R, head r % R); the A operand row of this lane is l16
  const int eh = l16 % R, ee = l16 / R;
  for (int b0 = 0; b0 < n; b0 += QB) {
    const int nb = min(QB, n - b0);
    // ---- A operands of product (1): q rows and phi(q) hi / lo rows of the
    // batch.  Rows past its end repeat its last query: a result row depends on
    // its own A row only, and those rows are never stored.
    const uint16_t* qe = qs + min(b0 + ee, n - 1) * QE + eh * 3 * D;
    uint4 aq[NKS], afh[NKS], afl[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      aq[ks] = *reinterpret_cast<const uint4*>(qe + 0 * D + 32 * ks + 8 * lg4);
      afh[ks] = *reinterpret_cast<const uint4*>(qe + 1 * D + 32 * ks + 8 * lg4);
      afl[ks] = *reinterpret_cast<const uint4*>(qe + 2 * D + 32 * ks + 8 * lg4);
    }
    if ((int)threadIdx.x < 16) {
      const int r = threadIdx.x, e = r / R, h = r % R;
      const int cd = s_code[min(b0 + e, n - 1)];
      s_dst[r] = ((size_t)(cd >> 8) * a.H + g * R + h) * a.top_k + (cd & 255);
    }
    // ---- product (1): logits s = q.k and linear weights w = phi(q).phi(k) of this wavefront's tokens
    f32x4_t cs[NT1W], cw[NT1W];
#pragma unroll
    for (int nt = 0; nt < NT1W; ++nt) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f}, d2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        c = mfma_bf16(aq[ks], kraw[nt][ks], c);
        d2 = mfma_bf16(afh[ks], fkh[nt][ks], d2);
        d2 = mfma_bf16(afl[ks], fkh[nt][ks], d2);
        d2 = mfma_bf16(afh[ks], fkl[nt][ks], d2);
      }
      cs[nt] = c;
      cw[nt] = d2;
    }
    // causal limit of each of this lane's four rows (its query's own length)
    int ntok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * lg4 + i;
      ntok[i] = min(BK, s_len[min(b0 + r / R, n - 1)] - j * BK);
    }
    float mloc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int nt = 0; nt < NT1W; ++nt) {
      const int tok = (w * NT1W + nt) * 16 + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tok < ntok[i]) mloc[i] = max_nn(mloc[i], cs[nt][i] * inv_sqrt_d);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) mloc[i] = row16_max_nn(mloc[i]);
    if (l16 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s_max[w][4 * lg4 + i] = mloc[i];
    }
    __syncthreads();
    // ---- p = exp(s - m) and w, split hi/lo, into the rows of product (2):
    // row pair 2 (kind 16 + r) (hi) and + 1 (lo), kind 0 = p, 1 = w.  The
    // lanes of a token pair (2 u, 2 u + 1) trade values so that each stores
    // whole words: the even lane the hi row's word of both tokens, the odd
    // lane the lo row's.
    const bool odd = l16 & 1;
    float lsum[4] = {0.f, 0.f, 0.f, 0.f}, wsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * lg4 + i;
      const float mh = max_nn(max_nn(s_max[0][r], s_max[1][r]), max_nn(s_max[2][r], s_max[3][r]));
#pragma unroll
      for (int nt = 0; nt < NT1W; ++nt) {
        const int tok = (w * NT1W + nt) * 16 + l16;
        const bool valid = tok < ntok[i];
        const float px = valid ? __expf(cs[nt][i] * inv_sqrt_d - mh) : 0.f;
        const float wx = valid ? cw[nt][i] : 0.f;
        lsum[i] += px;
        wsum[i] += wx;
        // residuals below the bf16 hi parts; the even lane sends its residual,
        // the odd lane its value
        const float pr = px - bf16_lo_f(pack_bf16(px, 0.f));
        const float wr = wx - bf16_lo_f(pack_bf16(wx, 0.f));
        const float ps = odd ? px : pr, ws = odd ? wx : wr;
        const float pn = dpp_f<kDppXor1>(ps, ps), wn = dpp_f<kDppXor1>(ws, ws);
        // even: hi(t), hi(t + 1); odd: lo(t - 1), lo(t)
        const uint32_t pword = odd ? pack_bf16(pn, pr) : pack_bf16(px, pn);
        const uint32_t wword = odd ? pack_bf16(wn, wr) : pack_bf16(wx, wn);
        const int col = tok & ~1;
        *reinterpret_cast<uint32_t*>(&pw[pw_row(2 * r + odd) + col]) = pword;
        *reinterpret_cast<uint32_t*>(&pw[pw_row(2 * (16 + r) + odd) + col]) = wword;
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
        s_l[w][4 * lg4 + i] = lsum[i];
        s_sw[w][4 * lg4 + i] = wsum[i];
      }
    }
    __syncthreads();
    // ---- product (2) and the partial records of the batch's (query, slot) pairs
#pragma unroll
    for (int nt2 = 0; nt2 < NT2W; ++nt2) {
      const int ch = (w * NT2W + nt2) * 16 + l16;
#pragma unroll
      for (int mt = 0; mt < MT2; ++mt) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS2; ++ks) {
          const uint4 av = *reinterpret_cast<const uint4*>(&pw[pw_row(mt * 16 + l16) + 32 * ks + 8 * lg4]);
          const uint4 bv = *reinterpret_cast<const uint4*>(&vt[ch * VS + 32 * ks + 8 * lg4]);
          c = mfma_bf16(av, bv, c);
        }
        // lane group lg4 holds rows 4 lg4 .. 4 lg4 + 3 of tile mt: pairs
        // pi0 = 8 mt + 2 lg4 (hi + lo in c[0], c[1]) and pi0 + 1 (c[2], c[3])
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int pi = 8 * mt + 2 * lg4 + e2;
          const int kind = pi / 16, r = pi % 16;
          if (r / R < nb) a.part[s_dst[r] * rec + (kind ? D : 0) + ch] = c[2 * e2] + c[2 * e2 + 1];
        }
      }
    }
    if ((int)threadIdx.x < 16) {
      const int r = threadIdx.x;
      if (r / R < nb) {
        *reinterpret_cast<float4*>(a.part_hdr + s_dst[r] * kPartHdr) =
            make_float4(max_nn(max_nn(s_max[0][r], s_max[1][r]), max_nn(s_max[2][r], s_max[3][r])),
                        (s_l[0][r] + s_l[1][r]) + (s_l[2][r] + s_l[3][r]),
                        (s_sw[0][r] + s_sw[1][r]) + (s_sw[2][r] + s_sw[3][r]), 0.f);
      }
    }
    __syncthreads();  // s_max / pw / s_l are rewritten by the next batch
  }
}

}  // namespace

hipError_t launch_pf_clear(const PfBuffers& pb, int G, int max_blocks, const Launch& l) {
  const int n = G * max_blocks;
  return launch_kernel(k_pf_clear, dim3((n + kThreads - 1) / kThreads), l, pb.cnt, n);
}

hipError_t launch_pf_attend(const DecodeArgs& a, const PfBuffers& pb, const Launch& l) {
  hipError_t e = launch_kernel(k_pf_bucket, dim3((a.B * a.top_k + kThreads - 1) / kThreads, a.G), l, a.sel, pb.cnt,
                               pb.lists, pb.n_items, a.B, a.G, a.top_k, a.max_blocks, pb.cap);
  if (e != hipSuccess) return e;
  e = launch_kernel(k_pf_items, dim3((a.max_blocks + kThreads - 1) / kThreads, a.G), l, pb.cnt,
                    static_cast<const int32_t*>(pb.lists), pb.items, pb.n_items, a.block_table, a.G, a.max_blocks,
                    pb.cap, pb.max_items);
  if (e != hipSuccess) return e;
  const dim3 grid(pb.max_items);
  if (a.bk == 64)
    SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_pf_attend<RR, DD, 64>, grid, l,
                                             static_cast<const int4*>(pb.items), static_cast<const int32_t*>(pb.n_items), a))
  SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_pf_attend<RR, DD, 128>, grid, l,
                                           static_cast<const int4*>(pb.items), static_cast<const int32_t*>(pb.n_items), a))
}

}  // namespace spla
