// Combine: merge of the per-block partials, o_bar = phi(q)^T S_all,
// o_rla = o_bar - o_tilde, D = phi(q).z_all - sum w, o = o_sparse + g_h o_rla
// (SPLA Technical Summary 2.2, IO-efficient formulation; 2.3, hybrid
// strategy).
#include "decode_common.h"

namespace spla {

namespace {

// ============================================================== combine
// grid (D/32, G, B): one 32-channel slice of the R heads of (b, g).  Merges
// the per-block partials (softmax rescaling by exp(m_s - m) / L), contracts
// phi(q) with the slice's S_all columns (o_bar) and, in slice 0, with z_all
// (the normaliser D), and writes o = o_sparse + g_h (o_bar - o_tilde).
// Item = (kind, head, channel quartet) of the slice; the slots are split over
// SG thread groups whose float4 sums meet in LDS.  Every global load is
// issued before the first wait.
template <bool BF16, int R, int D>
__global__ __launch_bounds__(kThreads) void k_combine(const float* s_all, const void* q, const float* z_all,
                                                       const float* part, const int32_t* sel, int32_t G, int32_t H,
                                                       int32_t top_k, const DecodeArgs a) {
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
  // (sel is the selection the attend kernel used: the caller's override or
  // the selector's; the leading arguments address every first load)
  const int32_t* srow = sel + ((size_t)b * G + g) * top_k;
  const int rec = 2 * D + kPartHdr;
  const float* P0 = part + ((size_t)b * H + g * R) * top_k * (size_t)rec;
  const int c0 = cc * CS;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  // ---- loads
  const int sc = threadIdx.x % CS, rg = threadIdx.x / CS;
  const float* S = s_all + ((size_t)b * G + g) * D * (size_t)D + (size_t)(rg * RPG) * D + c0 + sc;
  float sv[RPG];
#pragma unroll
  for (int x = 0; x < RPG; ++x) sv[x] = S[(size_t)x * D];
  float qv[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = threadIdx.x + k * kThreads;
    qv[k] = load_elem<BF16>(q, ((size_t)b * H + g * R) * D + min(i, R * D - 1));
  }
  float zv[(D + 63) / 64];
#pragma unroll
  for (int k = 0; k < (D + 63) / 64; ++k) zv[k] = z_all[((size_t)b * G + g) * D + lane + 64 * k];
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
  // the rest of the arguments, while the loads are in flight
  SPLA_SCALARS_READY("s"(a.lens[b]), "s"(a.bk), "s"(a.gate), "s"(a.out), "s"(a.o_sparse_out), "s"(a.o_rla_out),
                     "s"(a.d_rla_out), "s"(a.sel_out));
  const int nb = n_blocks(a, b);
  const bool covers_all = nb <= top_k;
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
    const size_t oi = ((size_t)b * H + g * R + h) * D + c0 + 4 * q4;
    const float gh = a.gate[g * R + h];
    *reinterpret_cast<float4*>(a.out + oi) =
        make_float4(fmaf(gh, orl[0], os.x), fmaf(gh, orl[1], os.y), fmaf(gh, orl[2], os.z), fmaf(gh, orl[3], os.w));
    if (a.o_sparse_out) *reinterpret_cast<float4*>(a.o_sparse_out + oi) = os;
    if (a.o_rla_out) *reinterpret_cast<float4*>(a.o_rla_out + oi) = make_float4(orl[0], orl[1], orl[2], orl[3]);
  }
  if (cc == 0 && (int)threadIdx.x < top_k && a.sel_out)
    a.sel_out[((size_t)b * G + g) * top_k + threadIdx.x] = srow[threadIdx.x];
  if (cc == 0 && (int)threadIdx.x < R && a.d_rla_out) {
    const int h = threadIdx.x;
    a.d_rla_out[(size_t)b * H + g * R + h] = covers_all ? 0.f : s_dz[h] - s_sw[h];
  }
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, bool bf16, const Launch& l) {
  const dim3 grid(a.d / 32, a.G, a.B);
  const int32_t* sel = a.sel_in ? a.sel_in : a.sel;
  if (bf16)
    SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_combine<true, RR, DD>, grid, l, a.s_all, a.q, a.z_all, a.part, sel,
                                             a.G, a.H, a.top_k, a))
  SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_combine<false, RR, DD>, grid, l, a.s_all, a.q, a.z_all, a.part, sel,
                                           a.G, a.H, a.top_k, a))
}


}  // namespace spla
