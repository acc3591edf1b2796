// Block scorer: log-domain second-order Taylor score of every candidate block,
// summed over the query heads of a KV group (SPLA Technical Summary 2.1, score
// formula with the diagonal covariance of its implementation paragraph), and
// the fused decode-step kernel that also carries the one-token append.
#include "score_parts.h"

namespace spla {

namespace {

// spla_decode, first launch, grid (score_tiles + D * D / 1024, G, B): for
// each (b, g) the scorer's tiles, then the o_bar partials of the S_all row
// chunks.
template <bool BF16, int R, int D, bool TAYLOR>
__global__ __launch_bounds__(kThreads) void k_score(const float* mean, const float* var, const void* q,
                                                     int32_t n_tiles, int32_t G, int32_t H, int32_t tiles_all,
                                                     int32_t score_tiles, const StepArgs a) {
  const int x = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (x < score_tiles) {
    __shared__ ScoreTileLds<R, D> L;
    const ScorePre p{mean, var, q, n_tiles, G, H, tiles_all};
    score_tile<BF16, R, D, TAYLOR>(a.dec, x, g, b, p, L);
    return;
  }
  __shared__ StateRowsLds<R, D> L;
  SPLA_SCALARS_READY("s"(a.st.s_all), "s"(a.st.z_all), "s"(a.dec.obar_part), "s"(a.dec.dz_part));
  state_rows<BF16, R, D, false>(a.dec, a.st, b, g, x - score_tiles, L);
}

// Fused decode step, first launch, grid (score_tiles + D * D / (1024 CPW) +
// 1, G, B): for each (b, g), the scorer's tiles, then the S_all / z_all
// update of this step's token in row chunks, CPW chunks a workgroup (with
// their o_bar partials), then the token's page row and the statistics of the
// block it completes.  The two
// parts are independent: the scorer reads statistics of candidate blocks
// 1..nb-2 only, all completed by earlier appends, and neither pages nor
// S_all.
template <bool BF16, int R, int D, bool TAYLOR, int CPW, bool STREAM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_step_score(const float* mean, const float* var, const void* q,
                                                          int32_t n_tiles, int32_t G, int32_t H, int32_t tiles_all,
                                                          int32_t score_tiles, const StepArgs a) {
  constexpr int kGroups = D / (1024 / D) / CPW;  // S_all row-chunk workgroups per (b, g)
  __shared__ ProducerLds<BF16, R, D> L;
  const DecodeArgs& dc = a.dec;
  const int x = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (x < score_tiles) {
    const ScorePre p{mean, var, q, n_tiles, G, H, tiles_all};
    score_tile<BF16, R, D, TAYLOR>(dc, x, g, b, p, L.score);
    return;
  }
  SPLA_SCALARS_READY("s"(dc.bk), "s"(a.st.k_new), "s"(a.st.v_new), "s"(a.st.s_all), "s"(a.st.z_all),
                     "s"(dc.obar_part), "s"(dc.dz_part), "s"(a.st.block_table), "s"(a.st.k_pages),
                     "s"(a.st.v_pages));
  if (x < score_tiles + kGroups) {
    state_rows<BF16, R, D, true, CPW, STREAM>(dc, a.st, b, g, (x - score_tiles) * CPW, L.state);
    return;
  }
  const int T = dc.lens[b];  // after the append
  const AppendEntry E{b, 1, T - 1, b};
  append_page_row_head<BF16>(a.st, E, g);
  if (T % dc.bk == 0) append_block_stats<BF16, D>(a.st, E, T / dc.bk - 1, g, L.stats);
}

template <bool TAYLOR>
hipError_t launch_score_form(const StepArgs& a, bool bf16, const Launch& l) {
  const DecodeArgs& d = a.dec;
  const int chunks = d.d / (1024 / d.d);
  const dim3 grid(d.score_tiles + chunks, d.G, d.B);
  if (bf16)
    SPLA_DISPATCH_RD(d.r, d.d, launch_kernel(k_score<true, RR, DD, TAYLOR>, grid, l, d.blk_mean, d.blk_var,
                                             d.q, d.n_tiles, d.G, d.H, d.tiles_all, d.score_tiles, a))
  SPLA_DISPATCH_RD(d.r, d.d, launch_kernel(k_score<false, RR, DD, TAYLOR>, grid, l, d.blk_mean, d.blk_var,
                                           d.q, d.n_tiles, d.G, d.H, d.tiles_all, d.score_tiles, a))
}

template <bool TAYLOR, int CPW, bool STREAM>
hipError_t launch_step_score_cpw(const StepArgs& a, bool bf16, const Launch& l) {
  const int groups = a.dec.d / (1024 / a.dec.d) / CPW;
  const dim3 grid(a.dec.score_tiles + groups + 1, a.dec.G, a.dec.B);
  const DecodeArgs& d = a.dec;
  if (bf16)
    SPLA_DISPATCH_RD(d.r, d.d, launch_kernel(k_step_score<true, RR, DD, TAYLOR, CPW, STREAM>, grid, l, d.blk_mean,
                                             d.blk_var, d.q, d.n_tiles, d.G, d.H, d.tiles_all, d.score_tiles, a))
  SPLA_DISPATCH_RD(d.r, d.d, launch_kernel(k_step_score<false, RR, DD, TAYLOR, CPW, STREAM>, grid, l, d.blk_mean,
                                           d.blk_var, d.q, d.n_tiles, d.G, d.H, d.tiles_all, d.score_tiles, a))
}

// (b, g) pairs from which the S_all rows are read and written past the
// caches (non-temporal): at 16 x 8 and 64 x 8 pairs the decode step took 62.5
// and 165 us that way against 64.8 and 173 us, at 8 pairs (B = 1) 19.5
// against 19.4 us
constexpr int kStreamStatePairs = 128;

// the S_all row chunks four to a workgroup from kStateGroupPairs (b, g)
// pairs on: at 64 sequences x 8 KV heads the first kernel takes 56 us
// instead of 63 us that way, while at 128 pairs and fewer the single-chunk
// workgroups are faster (the longer state workgroups end the kernel)
template <bool TAYLOR>
hipError_t launch_step_score_form(const StepArgs& a, bool bf16, const Launch& l) {
  const int pairs = a.dec.B * a.dec.G;
  if (pairs >= kStateGroupPairs) return launch_step_score_cpw<TAYLOR, 4, true>(a, bf16, l);
  if (pairs >= kStreamStatePairs) return launch_step_score_cpw<TAYLOR, 1, true>(a, bf16, l);
  return launch_step_score_cpw<TAYLOR, 1, false>(a, bf16, l);
}

}  // namespace

hipError_t launch_score(const StepArgs& a, bool bf16, const Launch& l) {
  if (a.dec.virtual_queries) return hipErrorInvalidValue;  // a prefill group is scored by k_pf_score
  return a.dec.score_form == kScoreMean ? launch_score_form<false>(a, bf16, l) : launch_score_form<true>(a, bf16, l);
}

hipError_t launch_step_score(const StepArgs& a, bool bf16, const Launch& l) {
  return a.dec.score_form == kScoreMean ? launch_step_score_form<false>(a, bf16, l)
                                        : launch_step_score_form<true>(a, bf16, l);
}

}  // namespace spla
