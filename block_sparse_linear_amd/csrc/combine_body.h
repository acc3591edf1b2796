// Combine: merge of the per-block partials of one query head, o_bar =
// phi(q)^T S_all from the row-chunk partials of the first kernel, o_rla =
// o_bar - o_tilde, D = phi(q).z_all - sum w, o = o_sparse + g_h * branch
// (SPLA Technical Summary 2.2, IO-efficient formulation; 2.3, hybrid
// strategy).  The branch is o_rla itself, o_rla / D (linear attention over
// the unselected tokens with its normaliser, the kernelised form of the Baidu
// Cloud sparse-attention article, section 7), or gamma * o_rla / rms(o_rla)
// (the RMS norm of the RLA output, Technical Summary 2.3).
#pragma once

#include "xcd_sync.h"

namespace spla {
namespace {

// slices and slot groups of a combine workgroup
template <int D, int FORM, bool ONE, bool WHOLE>
struct CombineShape {
  static constexpr int CS = (FORM == kRlaRms || ONE || WHOLE) ? D : 32;  // channels per workgroup
  static constexpr int NQ = CS / 4;                                      // channel quartets
  static constexpr int NIT = 2 * NQ;                                     // float4 items (kind, quartet)
  static constexpr int SG = kThreads / NIT;                              // slot groups
  static constexpr int CHUNKS = ONE ? 1 : D / (1024 / D);                // o_bar partials per head
};

template <int R, int D, int FORM, bool ONE, bool WHOLE>
struct CombineLds {
  using T = CombineShape<D, FORM, ONE, WHOLE>;
  float wsl[256];  // exp(m_s - m) / L (0 for unused slots)
  int valid[256];
  float4 obp[T::CHUNKS][T::NQ];
  float dzp[T::CHUNKS];
  float4 red4[T::SG][T::NIT];
  float s_sw;
};

// In the fused select + attend kernel a combine workgroup runs after the
// pair's attend workgroups in the same launch and first waits for their
// records (ctr: the pair's counter line, target: its attend workgroups);
// `waiters` merge workgroups share the line, and `checker` reads its XCD mask.
// normalized: the normalised RLA form (its FORM is the plain one there).
struct CombineWait {
  int32_t* ctr;
  int target, waiters;
  bool checker, normalized;
};

__device__ __forceinline__ void combine_wait(const CombineWait& wt, uint32_t* err) {
  step_wait(wt.ctr, wt.target, err);
  if (threadIdx.x == 0) {
    if (wt.checker) {
      // every attend workgroup counted here ran on this XCD; read before this
      // workgroup counts itself in, so the line cannot have been cleared yet
      const int mask = step_mask(wt.ctr);
      if (mask != (1 << xcc_id())) atomicOr(err, kErrStepXcd);
      asm volatile("" ::"v"(mask));
    }
    const int arrived = __hip_atomic_fetch_add(wt.ctr + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) + 1;
    if (arrived == wt.waiters) {  // every merge workgroup is past its wait: clear the line for the next call
      wt.ctr[0] = 0;
      wt.ctr[1] = 0;
      wt.ctr[2] = 0;
    }
  }
}

// 16 bytes of a partial record, read once per call: past the caches
// (non-temporal) for the whole-head decode combine of many (b, h) pairs
// (with 16 x 32 and 64 x 32 heads the combine took 5.1 and 9.6 us that way
// against 5.2 and 9.9 us)
template <bool STREAM>
__device__ __forceinline__ float4 load_rec4(const float* p) {
  if constexpr (STREAM) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    const v4f x = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
  } else {
    return *reinterpret_cast<const float4*>(p);
  }
}

template <int R, int D, int FORM, bool ONE, bool WHOLE>
__device__ __forceinline__ void combine_slice(const float* part, const float* part_hdr, const float* obar_part,
                                              const float* dz_part, const int32_t* sel, int32_t G, int32_t H,
                                              int32_t top_k, const DecodeArgs& a, int cc, int hq, int b,
                                              CombineLds<R, D, FORM, ONE, WHOLE>& L, const CombineWait& wt) {
  using T = CombineShape<D, FORM, ONE, WHOLE>;
  constexpr int CS = T::CS, NQ = T::NQ, NIT = T::NIT, SG = T::SG, CHUNKS = T::CHUNKS;
  constexpr int SPT = 4;                        // slots per thread per load batch
  constexpr int SPL = 4;                        // slots per lane in the header pass (top_k <= 256)
  constexpr int OBN = (CHUNKS * NQ + kThreads - 1) / kThreads;  // o_bar partial float4s per thread
  static_assert(OBN <= 2, "at most two o_bar partial loads per thread");
  auto& wsl = L.wsl;
  auto& valid = L.valid;
  auto& obp = L.obp;
  auto& dzp = L.dzp;
  auto& red4 = L.red4;
  auto& s_sw = L.s_sw;
  const int g = hq / R, h = hq % R;
  const size_t bg = (size_t)b * G + g;
  const int32_t* srow = sel + bg * top_k;
  const int rec = 2 * D;
  const float* P0 = part + ((size_t)b * H + hq) * top_k * (size_t)rec;
  const float4* PH = reinterpret_cast<const float4*>(part_hdr) + ((size_t)b * H + hq) * top_k;  // this head's headers
  const int c0 = cc * CS;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  // ---- loads (slot indices clamped into range, masked afterwards): the
  // first kernel's o_bar / phi(q).z partials first, then (after the wait,
  // when there is one) the selection, the headers and the records
  auto obar_at = [&](int i) {  // o_bar partial float4 i of this slice (clamped)
    i = min(i, CHUNKS * NQ - 1);
    return reinterpret_cast<const float4*>(obar_part)[((bg * CHUNKS + i / NQ) * R + h) * (D / 4) + c0 / 4 + i % NQ];
  };
  const float4 obv0 = obar_at(threadIdx.x);
  const float4 obv1 = OBN > 1 ? obar_at(threadIdx.x + kThreads) : obv0;
  const float dzv = dz_part[(bg * CHUNKS + min((int)threadIdx.x, CHUNKS - 1)) * R + h];
  if (wt.ctr) combine_wait(wt, a.err);
  int vs[SPL];
  float hm[SPL], hl[SPL], hs[SPL];
#pragma unroll
  for (int u = 0; u < SPL; ++u) {
    const int s = min(lane + 64 * u, top_k - 1);
    vs[u] = srow[s];
    const float4 hd = PH[s];
    hm[u] = hd.x;
    hl[u] = hd.y;
    hs[u] = hd.z;
  }
  const int it = threadIdx.x % NIT, sg = threadIdx.x / NIT;
  const int kind = it / NQ, q4 = it % NQ;
  const float* PD = P0 + (kind ? D : 0) + c0 + 4 * q4;
  float4 dv[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u)
    dv[u] = load_rec4<WHOLE && !ONE>(PD + (size_t)min(sg + SG * u, top_k - 1) * rec);
  __builtin_amdgcn_sched_barrier(0);
  // the rest of the arguments, while the loads are in flight
  float4 gm = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (FORM == kRlaRms) {
    SPLA_SCALARS_READY("s"(a.lens[b]), "s"(a.bk), "s"(a.gate), "s"(a.out), "s"(a.o_sparse_out), "s"(a.o_rla_out),
                       "s"(a.d_rla_out), "s"(a.sel_out), "s"(a.rla_gamma), "s"(a.rla_eps));
    gm = reinterpret_cast<const float4*>(a.rla_gamma + (size_t)hq * D)[min(lane, NQ - 1)];
  } else {
    SPLA_SCALARS_READY("s"(a.lens[b]), "s"(a.bk), "s"(a.gate), "s"(a.out), "s"(a.o_sparse_out), "s"(a.o_rla_out),
                       "s"(a.d_rla_out), "s"(a.sel_out));
  }
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
  if ((int)threadIdx.x < CHUNKS * NQ) obp[threadIdx.x / NQ][threadIdx.x % NQ] = obv0;
  if (OBN > 1 && (int)threadIdx.x + kThreads < CHUNKS * NQ)
    obp[(threadIdx.x + kThreads) / NQ][(threadIdx.x + kThreads) % NQ] = obv1;
  if ((int)threadIdx.x < CHUNKS) dzp[threadIdx.x] = dzv;
  __syncthreads();
  // ---- this thread's slots of its item
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int u0 = 0; sg + SG * u0 < top_k; u0 += SPT) {
    if (u0 > 0) {
#pragma unroll
      for (int u = 0; u < SPT; ++u)
        dv[u] = load_rec4<WHOLE && !ONE>(PD + (size_t)min(sg + SG * (u0 + u), top_k - 1) * rec);
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
  // D = phi(q).z_all - sum w of this head (0 when every block is selected)
  auto d_rla = [&]() {
    float dz = dzp[0];
#pragma unroll
    for (int rc = 1; rc < CHUNKS; ++rc) dz += dzp[rc];
    return covers_all ? 0.f : dz - s_sw;
  };
  // ---- finalise: lane = channel quartet of wavefront 0, both kinds from LDS
  if (w == 0) {
    const int qq = min(lane, NQ - 1);
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
    float4 br = orl;  // the branch in its output form
    if (FORM == kRlaNormalized || wt.normalized) {
      const float dh = d_rla();
      const float inv = covers_all ? 0.f : 1.f / dh;
      br = make_float4(orl.x * inv, orl.y * inv, orl.z * inv, orl.w * inv);
    } else if constexpr (FORM == kRlaRms) {
      float ss = lane < NQ ? orl.x * orl.x + orl.y * orl.y + orl.z * orl.z + orl.w * orl.w : 0.f;
      ss = wave_sum(ss);  // over the head's D channels
      const float inv = covers_all ? 0.f : 1.f / sqrtf(ss * (1.f / D) + a.rla_eps);
      br = make_float4(gm.x * orl.x * inv, gm.y * orl.y * inv, gm.z * orl.z * inv, gm.w * orl.w * inv);
    }
    if (lane < NQ) {
      const size_t oi = ((size_t)b * H + hq) * D + c0 + 4 * lane;
      const float gh = a.gate[hq];
      *reinterpret_cast<float4*>(a.out + oi) =
          make_float4(fmaf(gh, br.x, os.x), fmaf(gh, br.y, os.y), fmaf(gh, br.z, os.z), fmaf(gh, br.w, os.w));
      if (a.o_sparse_out) *reinterpret_cast<float4*>(a.o_sparse_out + oi) = os;
      if (a.o_rla_out) *reinterpret_cast<float4*>(a.o_rla_out + oi) = orl;
    }
  }
  if (cc == 0 && (int)threadIdx.x == 64 && a.d_rla_out) a.d_rla_out[(size_t)b * H + hq] = d_rla();
  if (cc == 0 && h == 0 && a.sel_out)
    for (int s = threadIdx.x; s < top_k; s += kThreads) a.sel_out[bg * top_k + s] = srow[s];
}

}  // namespace
}  // namespace spla
