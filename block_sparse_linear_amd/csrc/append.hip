// spla_append_kv kernel: page write and block statistics of completed blocks
// (SPLA Technical Summary 2.1); the global linear-attention state part of an
// append is k_state_add (fp32 matrix cores).
//
// One launch covers up to kMaxAppendEntries (sequence, rows) entries.  The
// grid is a flat list of two kinds of workgroups:
//   [0, page_items)                     page copy of up to page_tok appended tokens
//   [page_items, +stat_items)           mean / population variance of one block
//                                       completed by this append, one KV head
// The two kinds touch disjoint memory: statistics read tokens older than the
// append from the pages (written by earlier launches) and the new tokens from
// k_new, never the page rows this launch writes.
#include "decode_common.h"

namespace spla {

namespace {

__device__ __forceinline__ int find_entry(const int32_t* prefix, int n, int item) {
  int e = 0;
  while (e + 1 < n && prefix[e + 1] <= item) ++e;
  return e;
}

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_append(const AppendArgs a) {
  int item = blockIdx.x;
  if (item < a.page_items) {
    const int e = find_entry(a.page_prefix, a.n_entries, item);
    append_page_rows<BF16>(a.st, a.e[e], (item - a.page_prefix[e]) * a.page_tok, a.page_tok);
    return;
  }
  item -= a.page_items;
  if (item < a.stat_items) {
    const int e = find_entry(a.stat_prefix, a.n_entries, item);
    const int local = item - a.stat_prefix[e];
    __shared__ BlockStatsLds<BF16> L;
    append_block_stats<BF16, D>(a.st, a.e[e], a.e[e].t0 / a.st.bk + local / a.st.G, local % a.st.G, L);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, bool bf16, const Launch& l) {
  const int n = a.page_items + a.stat_items;
  if (n == 0) return hipSuccess;
  if (bf16) SPLA_DISPATCH_D(a.st.d, launch_kernel(k_append<true, DD>, dim3(n), l, a))
  SPLA_DISPATCH_D(a.st.d, launch_kernel(k_append<false, DD>, dim3(n), l, a))
}

}  // namespace spla
