// Combine: merge of the per-block partials of one query head, o_bar =
// phi(q)^T S_all from the row-chunk partials of the first kernel, o_rla =
// o_bar - o_tilde, D = phi(q).z_all - sum w, o = o_sparse + g_h * branch
// (SPLA Technical Summary 2.2, IO-efficient formulation; 2.3, hybrid
// strategy).  The branch is o_rla itself, o_rla / D (linear attention over
// the unselected tokens with its normaliser, the kernelised form of the Baidu
// Cloud sparse-attention article, section 7), or gamma * o_rla / rms(o_rla)
// (the RMS norm of the RLA output, Technical Summary 2.3).
#include "combine_body.h"

namespace spla {

namespace {

// grid (D / CS, H, B): one CS-channel slice of one query head (the whole
// head for the RMS form, whose norm runs over all D channels, and with
// WHOLE).  Item = (kind, channel quartet) with kind 0 the softmax numerators
// (weighted by exp(m_s - m) / L) and kind 1 the linear-attention sums; the
// slots are split over kThreads / (2 CS / 4) slot groups whose float4 sums
// meet in LDS.  Every global load is issued before the first wait; the
// leading arguments address all of them.
// ONE: a single o_bar / phi(q).z partial per head (chunked prefill) instead
// of the first kernel's D * D / 1024 row-chunk partials.
// WHOLE: a workgroup takes a whole head (as ONE and the RMS form always do)
// instead of a 32-channel slice: with many (b, h) pairs there are workgroups
// enough, and each head's merge-weight pass and fixed costs are paid once
// instead of D / 32 times (with 2048 pairs the combine takes 9.6 us instead of
// 27 us); with few pairs the slices give the parallelism.
template <int R, int D, int FORM, bool ONE, bool WHOLE>
__global__ __launch_bounds__(kThreads) void k_combine(const float* part, const float* part_hdr, const float* obar_part,
                                                       const float* dz_part, const int32_t* sel, int32_t G, int32_t H,
                                                       int32_t top_k, const DecodeArgs a) {
  __shared__ CombineLds<R, D, FORM, ONE, WHOLE> L;
  combine_slice<R, D, FORM, ONE, WHOLE>(part, part_hdr, obar_part, dz_part, sel, G, H, top_k, a, blockIdx.x,
                                        blockIdx.y, blockIdx.z, L, CombineWait{nullptr, 0, 0, false, false});
}

template <int FORM>
hipError_t launch_combine_form(const DecodeArgs& a, const Launch& l) {
  const bool whole = FORM == kRlaRms || a.obar_one || a.B * a.H >= kCombineWholeHeads;
  const dim3 grid(whole ? 1 : a.d / 32, a.H, a.B);
  const int32_t* sel = a.sel_in ? a.sel_in : a.sel;
  if (a.obar_one)
    SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_combine<RR, DD, FORM, true, true>, grid, l, a.part, a.part_hdr,
                                             a.obar_part, a.dz_part, sel, a.G, a.H, a.top_k, a))
  if (whole)
    SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_combine<RR, DD, FORM, false, true>, grid, l, a.part, a.part_hdr,
                                             a.obar_part, a.dz_part, sel, a.G, a.H, a.top_k, a))
  SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_combine<RR, DD, FORM, false, false>, grid, l, a.part, a.part_hdr,
                                           a.obar_part, a.dz_part, sel, a.G, a.H, a.top_k, a))
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, const Launch& l) {
  switch (a.rla_form) {
    case kRlaPlain: return launch_combine_form<kRlaPlain>(a, l);
    case kRlaNormalized: return launch_combine_form<kRlaNormalized>(a, l);
    case kRlaRms: return launch_combine_form<kRlaRms>(a, l);
  }
  return hipErrorInvalidValue;
}

}  // namespace spla
