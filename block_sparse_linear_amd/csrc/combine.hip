// Combine: merge of the per-block partials of one query head, o_bar =
// phi(q)^T S_all from the row-chunk partials of the first kernel, o_rla =
// o_bar - o_tilde, D = phi(q).z_all - sum w, o = o_sparse + g_h o_rla (SPLA
// Technical Summary 2.2, IO-efficient formulation; 2.3, hybrid strategy).
#include "decode_common.h"

namespace spla {

namespace {

// grid (D / 32, H, B): one 32-channel slice of one query head.  Item =
// (kind, channel quartet) with kind 0 the softmax numerators (weighted by
// exp(m_s - m) / L) and kind 1 the linear-attention sums; the slots are split
// over 16 slot groups whose float4 sums meet in LDS.  Every global load is
// issued before the first wait; the leading arguments address all of them.
template <bool BF16, int R, int D>
__global__ __launch_bounds__(kThreads) void k_combine(const float* part, const float* obar_part, const float* dz_part,
                                                       const int32_t* sel, int32_t G, int32_t H, int32_t top_k,
                                                       const DecodeArgs a) {
  constexpr int CS = 32;                 // channels per workgroup
  constexpr int NQ = CS / 4;             // channel quartets
  constexpr int NIT = 2 * NQ;            // float4 items (kind, quartet)
  constexpr int SG = kThreads / NIT;     // slot groups
  constexpr int SPT = 4;                 // slots per thread per load batch
  constexpr int SPL = 4;                 // slots per lane in the header pass (top_k <= 256)
  constexpr int CHUNKS = D / (1024 / D); // o_bar partials per head
  __shared__ float wsl[256];             // exp(m_s - m) / L (0 for unused slots)
  __shared__ int valid[256];
  __shared__ float4 obp[CHUNKS][NQ];
  __shared__ float dzp[CHUNKS];
  __shared__ float4 red4[SG][NIT];
  __shared__ float s_sw;
  const int cc = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int g = hq / R, h = hq % R;
  const size_t bg = (size_t)b * G + g;
  const int32_t* srow = sel + bg * top_k;
  const int rec = 2 * D + kPartHdr;
  const float* P0 = part + ((size_t)b * H + hq) * top_k * (size_t)rec;
  const int c0 = cc * CS;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  // ---- loads (slot indices clamped into range, masked afterwards)
  int vs[SPL];
  float hm[SPL], hl[SPL], hs[SPL];
#pragma unroll
  for (int u = 0; u < SPL; ++u) {
    const int s = min(lane + 64 * u, top_k - 1);
    vs[u] = srow[s];
    const float* P = P0 + (size_t)s * rec;
    hm[u] = P[0];
    hl[u] = P[1];
    hs[u] = P[2];
  }
  const int it = threadIdx.x % NIT, sg = threadIdx.x / NIT;
  const int kind = it / NQ, q4 = it % NQ;
  const float* PD = P0 + kPartHdr + (kind ? D : 0) + c0 + 4 * q4;
  float4 dv[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u)
    dv[u] = *reinterpret_cast<const float4*>(PD + (size_t)min(sg + SG * u, top_k - 1) * rec);
  const int ob_rc = min((int)threadIdx.x / NQ, CHUNKS - 1), ob_q4 = threadIdx.x % NQ;
  const float4 obv =
      reinterpret_cast<const float4*>(obar_part)[((bg * CHUNKS + ob_rc) * R + h) * (D / 4) + c0 / 4 + ob_q4];
  const float dzv = dz_part[(bg * CHUNKS + min((int)threadIdx.x, CHUNKS - 1)) * R + h];
  __builtin_amdgcn_sched_barrier(0);
  // the rest of the arguments, while the loads are in flight
  SPLA_SCALARS_READY("s"(a.lens[b]), "s"(a.bk), "s"(a.gate), "s"(a.out), "s"(a.o_sparse_out), "s"(a.o_rla_out),
                     "s"(a.d_rla_out), "s"(a.sel_out));
  const int nb = n_blocks(a, b);
  const bool covers_all = nb <= top_k;
  // ---- merge weights of the slots (wavefront 0), o_bar / D partials to LDS
  if (w == 0) {
    bool ok[SPL];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      ok[u] = lane + 64 * u < top_k && vs[u] >= 0 && vs[u] < nb;
      m = fmaxf(m, ok[u] ? hm[u] : -INFINITY);
    }
    m = wave_max(m);
    float l = 0.f, sw = 0.f, e[SPL];
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      e[u] = ok[u] ? expf(hm[u] - m) : 0.f;
      l = fmaf(e[u], ok[u] ? hl[u] : 0.f, l);
      sw += ok[u] ? hs[u] : 0.f;
    }
    l = wave_sum(l);
    sw = wave_sum(sw);
    const float inv_l = 1.f / l;
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int s = lane + 64 * u;
      if (s < top_k) {
        wsl[s] = e[u] * inv_l;
        valid[s] = ok[u] ? 1 : 0;
      }
    }
    if (lane == 0) s_sw = sw;
  }
  if ((int)threadIdx.x < CHUNKS * NQ) obp[ob_rc][ob_q4] = obv;
  if ((int)threadIdx.x < CHUNKS) dzp[threadIdx.x] = dzv;
  __syncthreads();
  // ---- this thread's slots of its item
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int u0 = 0; sg + SG * u0 < top_k; u0 += SPT) {
    if (u0 > 0) {
#pragma unroll
      for (int u = 0; u < SPT; ++u)
        dv[u] = *reinterpret_cast<const float4*>(PD + (size_t)min(sg + SG * (u0 + u), top_k - 1) * rec);
    }
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int s = sg + SG * (u0 + u);
      if (s >= top_k || !valid[s]) continue;  // unused slot: its record holds stale data
      const float wt = kind == 0 ? wsl[s] : 1.f;
      acc.x = fmaf(wt, dv[u].x, acc.x);
      acc.y = fmaf(wt, dv[u].y, acc.y);
      acc.z = fmaf(wt, dv[u].z, acc.z);
      acc.w = fmaf(wt, dv[u].w, acc.w);
    }
  }
  red4[sg][it] = acc;
  __syncthreads();
  // ---- finalise: thread = channel quartet, both kinds from LDS
  if ((int)threadIdx.x < NQ) {
    const int qq = threadIdx.x;
    float4 os = make_float4(0.f, 0.f, 0.f, 0.f), ot = os;
#pragma unroll
    for (int k = 0; k < SG; ++k) {
      const float4 x0 = red4[k][qq];
      const float4 x1 = red4[k][NQ + qq];
      os.x += x0.x; os.y += x0.y; os.z += x0.z; os.w += x0.w;
      ot.x += x1.x; ot.y += x1.y; ot.z += x1.z; ot.w += x1.w;
    }
    float4 ob = obp[0][qq];
#pragma unroll
    for (int rc = 1; rc < CHUNKS; ++rc) {
      const float4 t = obp[rc][qq];
      ob.x += t.x; ob.y += t.y; ob.z += t.z; ob.w += t.w;
    }
    const float4 orl = covers_all ? make_float4(0.f, 0.f, 0.f, 0.f)
                                  : make_float4(ob.x - ot.x, ob.y - ot.y, ob.z - ot.z, ob.w - ot.w);
    const size_t oi = ((size_t)b * H + hq) * D + c0 + 4 * qq;
    const float gh = a.gate[hq];
    *reinterpret_cast<float4*>(a.out + oi) =
        make_float4(fmaf(gh, orl.x, os.x), fmaf(gh, orl.y, os.y), fmaf(gh, orl.z, os.z), fmaf(gh, orl.w, os.w));
    if (a.o_sparse_out) *reinterpret_cast<float4*>(a.o_sparse_out + oi) = os;
    if (a.o_rla_out) *reinterpret_cast<float4*>(a.o_rla_out + oi) = orl;
  }
  if (cc == 0 && (int)threadIdx.x == NQ && a.d_rla_out) {
    float dz = dzp[0];
#pragma unroll
    for (int rc = 1; rc < CHUNKS; ++rc) dz += dzp[rc];
    a.d_rla_out[(size_t)b * H + hq] = covers_all ? 0.f : dz - s_sw;
  }
  if (cc == 0 && h == 0 && a.sel_out)
    for (int s = threadIdx.x; s < top_k; s += kThreads) a.sel_out[bg * top_k + s] = srow[s];
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, bool bf16, const Launch& l) {
  const dim3 grid(a.d / 32, a.H, a.B);
  const int32_t* sel = a.sel_in ? a.sel_in : a.sel;
  if (bf16)
    SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_combine<true, RR, DD>, grid, l, a.part, a.obar_part, a.dz_part, sel,
                                             a.G, a.H, a.top_k, a))
  SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_combine<false, RR, DD>, grid, l, a.part, a.obar_part, a.dz_part, sel,
                                           a.G, a.H, a.top_k, a))
}

}  // namespace spla
