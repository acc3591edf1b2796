// Fused select + attend (bf16 K/V, Bk = 64), grid (top_k, G, B).  Every
// workgroup of (b, g) runs the selection of (b, g) itself, with the same
// select_core as the stand-alone selector over the scorer's group log scores,
// and then attends the block at its own slot of the ascending selection.  The
// selection is computed top_k times instead of being handed over through
// memory: idle compute is traded for one kernel boundary and one dependent
// global round trip, which is what the latency-bound small-batch decode pays
// for.
#include "attend_mfma.h"
#include "select_core.h"

namespace spla {

namespace {

template <int KPT, int R, int D>
__global__ __launch_bounds__(kThreads) void k_select_attend(const float* lg, const int32_t* block_table,
                                                             const void* q, const uint16_t* phq, int32_t n_tiles,
                                                             int32_t max_blocks, int32_t G, int32_t H,
                                                             const DecodeArgs a) {
  __shared__ SelectLds L;
  __shared__ int s_j, s_page;
  const int slot = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  // every load that does not depend on the selection goes out first, from
  // the leading kernel arguments alone: the scores and page ids it ranks and
  // the queries
  SelectKeys<KPT> k;
  select_load<KPT>(lg, block_table, n_tiles, max_blocks, G, g, b, b, k);
  uint4 qraw[D / 32], fh[D / 32], fl[D / 32];
  load_q_mfma<R, D>(q, phq, H, g, b, qraw, fh, fl);
  SPLA_SCALARS_READY("s"(a.lens[b]), "s"(a.bk), "s"(a.top_k), "s"(a.sel), "s"(a.k_pages), "s"(a.v_pages),
                     "s"(a.part), "s"(a.num_pages), "s"(a.inv_sqrt_d));
  const int nb = n_blocks(a, b);
  select_pages<KPT>(block_table, max_blocks, b, nb, k);
  int j, page;
  if (nb <= a.top_k) {
    j = slot < nb ? slot : -1;
    page = j >= 0 ? block_table[(size_t)b * max_blocks + j] : -1;
  } else {
    select_core<KPT>(a, nb, k, L, [&](int pos, int id, int pg) {
      if (pos == slot) {
        s_j = id;
        s_page = pg;
      }
    });
    __syncthreads();
    j = s_j;
    page = s_page;
  }
  // the combine reads the selection to tell used slots from unused ones
  if (threadIdx.x == 0) a.sel[((size_t)b * a.G + g) * a.top_k + slot] = j;
  attend_block_mfma<R, D, 64>(a, slot, g, b, j, page, qraw, fh, fl);
}

template <int K, int... Ks>
hipError_t launch_select_attend_sized(const DecodeArgs& a, const Launch& l, int nc, SelectSizes<K, Ks...>) {
  if (nc <= K * kThreads) {
    const dim3 grid(a.top_k, a.G, a.B);
    SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_select_attend<K, RR, DD>, grid, l, a.lg, a.block_table, a.q,
                                             a.phq, a.n_tiles, a.max_blocks, a.G, a.H, a))
  }
  if constexpr (sizeof...(Ks) == 0) {
    return hipErrorInvalidValue;
  } else {
    return launch_select_attend_sized(a, l, nc, SelectSizes<Ks...>{});
  }
}

constexpr int kFusedMaxKpt = 16;  // largest keys-per-thread size compiled for the fused kernel

}  // namespace

bool select_attend_supported(const DecodeArgs& a, bool bf16) {
  return bf16 && a.bk == 64 && !a.sel_in && max_candidates(a) <= kFusedMaxKpt * kThreads;
}

hipError_t launch_select_attend(const DecodeArgs& a, const Launch& l) {
  return launch_select_attend_sized(a, l, max_candidates(a), SelectSizes<1, 2, 4, 6, 9, 12, 16>{});
}

}  // namespace spla
