// Fused select + attend (bf16 K/V, Bk = 64).  Every workgroup of (b, g) runs
// the selection of (b, g) itself, with the same select_core as the
// stand-alone selector over the scorer's group log scores, and then attends
// the block at its own slot of the ascending selection.  The selection is
// computed top_k times instead of being handed over through memory: idle
// compute is traded for one kernel boundary and one dependent global round
// trip, which is what the latency-bound small-batch decode pays for.
//
// The grid puts the workgroups of a (b, g) on one XCD (workgroups go to the
// XCDs in turn by linear id, and the ids of a (b, g) are equal modulo 8), so
// the (b, g)'s score row, block-table row and queries, which each of them
// reads, come from that XCD's L2 after the first reader.
//
// MERGE: more workgroups per (b, g), after its attend workgroups in linear
// order, merge their partial records into the outputs (SPLA Technical
// Summary 2.2 and 2.3: o_sparse, o_rla = o_bar - o_tilde, the gated sum) in
// place of the combine kernel: each is the combine kernel's workgroup for one
// 32-channel slice of one query head, running the same code.  It loads the
// first kernel's o_bar / phi(q).z row-chunk partials first, then waits until
// every attend workgroup of the pair has its record in the L2, and reads the
// records from there.
#include "attend_mfma.h"
#include "select_core.h"
#include "combine_body.h"

namespace spla {

namespace {

// merge workgroups per (b, g): one per 32-channel slice of each query head
template <int R, int D>
constexpr int kMergeGroups = R * (D / 32);

template <int R, int D>
union SelectAttendLds {
  SelectLds sel;
  CombineLds<R, D, kRlaPlain, false, false> merge;
};

// grid (8 (top_k + MERGE R D / 32), ceil(B G / 8)): workgroup (x, y) takes
// slot x / 8 of pair (b, g) = 8 y + x % 8, so the linear ids of a pair are
// equal modulo 8 (the dispatcher hands the XCDs consecutive linear ids in
// turn, from wherever the previous dispatch left off); slots top_k and up are
// the pair's merge workgroups, one per 32-channel slice of each query head,
// after all of its attend workgroups in linear order; the pairs past B G
// exit at once
template <int KPT, int R, int D, bool MERGE>
__global__ __launch_bounds__(kThreads) void k_select_attend(const float* lg, const int32_t* block_table,
                                                             const void* q, const uint16_t* phq, int32_t n_tiles,
                                                             int32_t max_blocks, int32_t G, int32_t H,
                                                             const DecodeArgs a) {
  __shared__ SelectAttendLds<R, D> U;
  const int slot = blockIdx.x >> 3;
  const int bgi = (blockIdx.y << 3) + (blockIdx.x & 7);
  const int b = bgi / G, g = bgi - b * G;
  if (b >= a.B) return;
  if constexpr (MERGE) {
    if (slot >= a.top_k) {
      // the combine kernel's workgroup for slice cc of query head g R + h,
      // after a wait for the pair's records
      const int m = slot - a.top_k, h = m / (D / 32), cc = m % (D / 32);
      const CombineWait wt{a.step_ctr + (size_t)bgi * kStepCtrStride, a.top_k, kMergeGroups<R, D>, m == 0,
                           a.rla_form == kRlaNormalized};
      combine_slice<R, D, kRlaPlain, false, false>(a.part, a.part_hdr, a.obar_part, a.dz_part, a.sel, G, H, a.top_k,
                                                   a, cc, g * R + h, b, U.merge, wt);
      return;
    }
  }
  // every load that does not depend on the selection goes out first, from
  // the leading kernel arguments alone: the scores and page ids it ranks and
  // the queries
  SelectKeys<KPT> k;
  select_load<KPT>(lg, block_table, n_tiles, max_blocks, G, g, b, b, k);
  QOps<R, D> qo;
  load_qops<R, D>(q, phq, H, g, b, qo);
  SPLA_SCALARS_READY("s"(a.lens[b]), "s"(a.bk), "s"(a.top_k), "s"(a.sel), "s"(a.k_pages), "s"(a.v_pages),
                     "s"(a.part), "s"(a.part_hdr), "s"(a.num_pages), "s"(a.inv_sqrt_d));
  const int nb = n_blocks(a, b);
  select_pages<KPT>(block_table, max_blocks, b, nb, k);
  int j, page;
  select_slot<KPT>(a, block_table, max_blocks, b, nb, slot, k, U.sel, j, page);
  // the combine reads the selection to tell used slots from unused ones
  if (threadIdx.x == 0) a.sel[((size_t)b * a.G + g) * a.top_k + slot] = j;
  attend_block_mfma<R, D, 64>(a, slot, g, b, j, page, qo);
  // the record and the selection are in the L2: the pair's merge workgroups
  // may read them
  if constexpr (MERGE) step_signal(a.step_ctr + (size_t)bgi * kStepCtrStride);
}

template <bool MERGE, int K, int... Ks>
hipError_t launch_select_attend_sized(const DecodeArgs& a, const Launch& l, int nc, SelectSizes<K, Ks...>) {
  if (nc <= K * kThreads) {
    const int merges = MERGE ? a.r * (a.d / 32) : 0;
    const dim3 grid(8 * (a.top_k + merges), (a.B * a.G + 7) / 8);
    SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_select_attend<K, RR, DD, MERGE>, grid, l, a.lg, a.block_table,
                                             a.q, a.phq, a.n_tiles, a.max_blocks, a.G, a.H, a))
  }
  if constexpr (sizeof...(Ks) == 0) {
    return hipErrorInvalidValue;
  } else {
    return launch_select_attend_sized<MERGE>(a, l, nc, SelectSizes<Ks...>{});
  }
}

constexpr int kFusedMaxKpt = 16;  // largest keys-per-thread size compiled for the fused kernel

}  // namespace

bool select_attend_supported(const DecodeArgs& a, bool bf16) {
  return bf16 && a.bk == 64 && !a.sel_in && max_candidates(a) <= kFusedMaxKpt * kThreads && !a.virtual_queries;
}

bool select_attend_merge_supported(const DecodeArgs& a) {
  return a.rla_form != kRlaRms && a.B * a.H < kCombineWholeHeads && a.B * a.G <= kStepPairs &&
         a.step_ctr != nullptr && !a.virtual_queries;
}

hipError_t launch_select_attend(const DecodeArgs& a, const Launch& l, bool merge) {
  using Sizes = SelectSizes<1, 2, 4, 6, 9, 12, 16>;
  if (merge) {
    if (!select_attend_merge_supported(a)) return hipErrorInvalidValue;
    return launch_select_attend_sized<true>(a, l, max_candidates(a), Sizes{});
  }
  return launch_select_attend_sized<false>(a, l, max_candidates(a), Sizes{});
}

}  // namespace spla
