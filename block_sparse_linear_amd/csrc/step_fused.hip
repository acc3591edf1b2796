// One-kernel decode step for small batches (bf16 K/V, Bk = 64, Taylor
// score): the work of the step's first two kernels -- the one-token append,
// the block scores, the S_all update with its o_bar partials (SPLA Technical
// Summary 2.1 and 2.2), then the selection and attend + correct of every slot
// (2.1 and 2.2) -- in one launch.  The combine stays a kernel of its own.
//
// Every dependency of a step lies inside one (sequence, KV head) pair: the
// pair's selection needs all of its tile scores, its attend needs the
// selection, phi(q) from the state rows and, for the current block, the page
// row of the new token.  So each pair runs on one XCD and hands its results
// over in that XCD's L2:
//   - workgroups go to the XCDs in turn by linear id, from wherever the
//     previous dispatch left off, so ids equal modulo 8 share an XCD; pair
//     p takes ids = p (mod 8);
//   - producers (score tiles, S_all row chunks, the append) come first in
//     linear order; each one, once its stores are in the L2, bumps its pair's
//     counter there;
//   - attend workgroups come after every producer; each issues its loads
//     that need nothing from the producers (page ids of the candidates, the
//     queries), then waits until its pair's counter reaches the number of
//     producers, polling it with an atomic that is performed in the L2.
// An attend workgroup waits only on workgroups with smaller linear ids, which
// are dispatched before it and never wait themselves, so the waits end
// whatever the residency.  The wait is also bounded: past kSpinLimit polls it
// sets an error bit and goes on.  The pair's last attend workgroup to pass its
// wait (a second counter) puts both counters back to zero for the next call.
#include "attend_mfma.h"
#include "score_parts.h"
#include "select_core.h"
#include "xcd_sync.h"

namespace spla {

namespace {

template <int R, int D>
union StepLds {
  ProducerLds<true, R, D> prod;
  SelectLds sel;
};

// 1-D grid of 8 * pp * (np + top_k) workgroups, pp = ceil(B G / 8) pairs per
// id residue, np = score_tiles + d * d / 1024 + 1 producers per pair.  Id =
// 8 i + r: i < pp np is producer i % np of pair r + 8 (i / np); the rest are
// the attend workgroups, slot i' % top_k of pair r + 8 (i' / top_k), i' = i -
// pp np.  Pairs past B G exit at once.
template <int KPT, int R, int D>
__global__ __launch_bounds__(kThreads) void k_step_fused(const float* mean, const float* var, const void* q,
                                                          int32_t n_tiles, int32_t G, int32_t H, int32_t tiles_all,
                                                          int32_t score_tiles, int32_t pp, const StepArgs a) {
  constexpr int kChunks = D / (1024 / D);  // S_all row chunks per pair
  __shared__ StepLds<R, D> L;
  const DecodeArgs& dc = a.dec;
  const int r = blockIdx.x & 7, i = blockIdx.x >> 3;
  const int np = score_tiles + kChunks + 1;
  if (i < pp * np) {
    // ---- producer
    const int jp = i / np, role = i - jp * np;
    const int bgi = r + 8 * jp;
    if (bgi >= dc.B * G) return;
    const int b = bgi / G, g = bgi - b * G;
    if (role < score_tiles) {
      const ScorePre p{mean, var, q, n_tiles, G, H, tiles_all};
      score_tile<true, R, D, true>(dc, role, g, b, p, L.prod.score);
    } else if (role < score_tiles + kChunks) {
      state_rows<true, R, D, true>(dc, a.st, b, g, role - score_tiles, L.prod.state);
    } else {
      const int T = dc.lens[b];  // after the append
      const AppendEntry E{b, 1, T - 1, b};
      append_page_row_head<true>(a.st, E, g);
      if (T % dc.bk == 0) append_block_stats<true, D>(a.st, E, T / dc.bk - 1, g, L.prod.stats);
    }
    step_signal(dc.step_ctr + (size_t)bgi * kStepCtrStride);
    return;
  }
  // ---- attend: slot `slot` of pair bgi
  const int i2 = i - pp * np;
  const int jp = i2 / dc.top_k, slot = i2 - jp * dc.top_k;
  const int bgi = r + 8 * jp;
  if (bgi >= dc.B * G) return;
  const int b = bgi / G, g = bgi - b * G;
  int32_t* ctr = dc.step_ctr + (size_t)bgi * kStepCtrStride;
  // what needs nothing from the producers: the candidates' page ids and the
  // queries
  SelectKeys<KPT> k;
  select_load_pages<KPT>(dc.block_table, n_tiles, dc.max_blocks, b, k);
  QOps<R, D> qo;
  load_qops_q<R, D>(q, H, g, b, qo);
  SPLA_SCALARS_READY("s"(dc.lens[b]), "s"(dc.bk), "s"(dc.top_k), "s"(dc.sel), "s"(dc.k_pages), "s"(dc.v_pages),
                     "s"(dc.part), "s"(dc.part_hdr), "s"(dc.num_pages), "s"(dc.inv_sqrt_d), "s"(dc.lg), "s"(dc.phq));
  step_wait(ctr, np, dc.err);
  select_load_scores<KPT>(dc.lg, n_tiles, dc.max_blocks, G, g, b, k);
  load_qops_phi<R, D>(dc.phq, H, g, b, qo);
  // the pair's attend count, and (slot 0) the producers' XCD mask: every
  // producer counted here must have run on this XCD, else its stores may
  // sit in another XCD's L2.  Issued after the loads above, so that their
  // results (vector memory returns in order) do not wait for these atomics
  // on the pair's contended line; both are checked at the end.
  int arrived = 0, mask = 0;
  if (threadIdx.x == 0) {
    if (slot == 0) {
      int zero;
      asm volatile("v_mov_b32 %0, 0" : "=v"(zero));  // an or of a known zero would become a load
      mask = __hip_atomic_fetch_or(ctr + 2, zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      // the mask has arrived before this workgroup counts itself in below:
      // until then the pair's last attend workgroup cannot have cleared it
      asm volatile("" ::"v"(mask));
    }
    arrived = __hip_atomic_fetch_add(ctr + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) + 1;
  }
  const int nb = n_blocks(dc, b);
  select_pages<KPT>(dc.block_table, dc.max_blocks, b, nb, k);
  int j, page;
  select_slot<KPT>(dc, dc.block_table, dc.max_blocks, b, nb, slot, k, L.sel, j, page);
  // the combine reads the selection to tell used slots from unused ones
  if (threadIdx.x == 0) dc.sel[((size_t)b * G + g) * dc.top_k + slot] = j;
  attend_block_mfma<R, D, 64>(dc, slot, g, b, j, page, qo);
  if (threadIdx.x == 0) {
    if (arrived > dc.top_k) atomicOr(dc.err, kErrStepArrive);
    if (slot == 0 && mask != (1 << xcc_id())) atomicOr(dc.err, kErrStepXcd);
    if (arrived == dc.top_k) {  // every attend workgroup of the pair is past its wait
      ctr[0] = 0;
      ctr[1] = 0;
      ctr[2] = 0;
    }
  }
}

template <int K, int... Ks>
hipError_t launch_step_fused_sized(const StepArgs& a, const Launch& l, int nc, SelectSizes<K, Ks...>) {
  const DecodeArgs& d = a.dec;
  if (nc <= K * kThreads) {
    const int chunks = d.d / (1024 / d.d);
    const int pp = (d.B * d.G + 7) / 8;
    const dim3 grid(8 * pp * (d.score_tiles + chunks + 1 + d.top_k));
    SPLA_DISPATCH_RD(d.r, d.d, launch_kernel(k_step_fused<K, RR, DD>, grid, l, d.blk_mean, d.blk_var, d.q,
                                             d.n_tiles, d.G, d.H, d.tiles_all, d.score_tiles, pp, a))
  }
  if constexpr (sizeof...(Ks) == 0) {
    return hipErrorInvalidValue;
  } else {
    return launch_step_fused_sized(a, l, nc, SelectSizes<Ks...>{});
  }
}

}  // namespace

bool step_fused_supported(const DecodeArgs& a, bool bf16) {
  return select_attend_supported(a, bf16) && a.score_form == kScoreTaylor && a.B * a.G <= kStepPairs &&
         a.step_ctr != nullptr;
}

hipError_t launch_step_fused(const StepArgs& a, const Launch& l) {
  if (!step_fused_supported(a.dec, true)) return hipErrorInvalidValue;
  return launch_step_fused_sized(a, l, max_candidates(a.dec), SelectSizes<1, 2, 4, 6, 9, 12, 16>{});
}

}  // namespace spla
