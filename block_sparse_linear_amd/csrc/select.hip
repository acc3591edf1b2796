// Stand-alone selector: grid (G, B), one (sequence, KV head) per workgroup;
// writes the ascending selection and its page ids for the attend kernel.
// VQ: the batch is the virtual queries of one sequence's prefill chunk, which
// all read block-table row 0 (the pointer addresses that sequence's row).
#include "select_core.h"

namespace spla {

namespace {

template <int KPT, bool VQ>
__global__ __launch_bounds__(kThreads) void k_select(const float* lg, const int32_t* block_table, int32_t n_tiles,
                                                      int32_t max_blocks, int32_t G, const DecodeArgs a) {
  __shared__ SelectLds L;
  const int g = blockIdx.x, b = blockIdx.y;
  const int brow = VQ ? 0 : b;
  SelectKeys<KPT> k;
  select_load<KPT>(lg, block_table, n_tiles, max_blocks, G, g, b, brow, k);  // first: needs no other argument
  SPLA_SCALARS_READY("s"(a.lens[b]), "s"(a.bk), "s"(a.top_k), "s"(a.sel), "s"(a.sel_out), "s"(a.sel_page));
  const int nb = n_blocks(a, b);
  select_pages<KPT>(block_table, max_blocks, brow, nb, k);
  const size_t row = ((size_t)b * a.G + g) * a.top_k;
  int32_t* out = a.sel + row;
  int32_t* out2 = a.sel_out ? a.sel_out + row : nullptr;
  int32_t* pages = a.sel_page + row;
  if (nb <= a.top_k) {
    const int32_t* btab = a.block_table + (size_t)brow * a.max_blocks;
    for (int s = threadIdx.x; s < a.top_k; s += kThreads) {
      out[s] = s < nb ? s : -1;
      if (out2) out2[s] = s < nb ? s : -1;
      pages[s] = s < nb ? btab[s] : -1;
    }
    return;
  }
  select_core<KPT>(a, nb, k, L, [&](int pos, int id, int page) {
    out[pos] = id;
    if (out2) out2[pos] = id;
    pages[pos] = page;
  });
}

template <bool VQ, int K, int... Ks>
hipError_t launch_select_sized(const DecodeArgs& a, const Launch& l, int nc, SelectSizes<K, Ks...>) {
  if (nc <= K * kThreads)
    return launch_kernel(k_select<K, VQ>, dim3(a.G, a.B), l, a.lg, a.block_table, a.n_tiles, a.max_blocks, a.G, a);
  if constexpr (sizeof...(Ks) == 0) {
    return hipErrorInvalidValue;
  } else {
    return launch_select_sized<VQ>(a, l, nc, SelectSizes<Ks...>{});
  }
}

using SelectorSizes = SelectSizes<1, 2, 3, 4, 6, 8, 9, 10, 12, 16, 20, 24, 32, 40, 48, 64>;

}  // namespace

hipError_t launch_select(const DecodeArgs& a, const Launch& l) {
  if (a.virtual_queries) return launch_select_sized<true>(a, l, max_candidates(a), SelectorSizes{});
  return launch_select_sized<false>(a, l, max_candidates(a), SelectorSizes{});
}

}  // namespace spla
