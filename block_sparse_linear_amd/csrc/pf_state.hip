// Linear-attention side of a chunked-prefill group on the matrix cores.  The
// virtual query of token t of the group needs o_bar_t = phi(q_t)^T S_t and
// phi(q_t).z_t with S_t, z_t the state after token t (SPLA Technical Summary
// 2.2, at every position):
//   phi(q_t)^T S_t = phi(q_t)^T S_0 + sum_{i <= t} (phi(q_t) . phi(k_i)) v_i,
//   phi(q_t).z_t  = phi(q_t).z_0  + sum_{i <= t}  phi(q_t) . phi(k_i),
// with S_0, z_0 the state before the group.  Over a group these are matrix
// products: phi(Q) S_0, the causal weights W = phi(Q) phi(K)^T (i <= t) and
// W V, all in fp32 on the 16x16x4 fp32 matrix cores.  The kernel writes one
// o_bar / phi(q).z partial per (token, KV head, query head) (the combine of a
// prefill group sums one chunk) and phi(q) as bf16 hi / lo for the attend.
#include "decode_common.h"

namespace spla {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// N consecutive values from element `off` of a bf16 or fp32 array, as fp32
// (N a multiple of 4; off a multiple of 4, and of 8 for bf16 runs of 8 or more)
template <bool BF16, int N>
__device__ __forceinline__ void load_run(const void* p, size_t off, float (&out)[N]) {
  if constexpr (BF16 && N % 8 == 0) {
    const uint4* s = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + off);
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      const uint4 u = s[i];
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        out[8 * i + 2 * e] = bf16_lo_f(wd[e]);
        out[8 * i + 2 * e + 1] = bf16_hi_f(wd[e]);
      }
    }
  } else if constexpr (BF16) {
    static_assert(N % 4 == 0, "bf16 runs of whole 8-byte pieces");
    const uint2* s = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + off);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint2 u = s[i];
      out[4 * i] = bf16_lo_f(u.x);
      out[4 * i + 1] = bf16_hi_f(u.x);
      out[4 * i + 2] = bf16_lo_f(u.y);
      out[4 * i + 3] = bf16_hi_f(u.y);
    }
  } else {
    const float4* s = reinterpret_cast<const float4*>(static_cast<const float*>(p) + off);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const float4 u = s[i];
      out[4 * i] = u.x;
      out[4 * i + 1] = u.y;
      out[4 * i + 2] = u.z;
      out[4 * i + 3] = u.w;
    }
  }
}

// grid (ceil(m / 16), G, R): token tile a (tokens 16 a .. 16 a + 15 of the
// group), KV head g, query head h.  Operands of the 16x16x4 products: lane
// (kk = lane / 16, l16 = lane % 16) gives A row l16 and B column l16 at k
// slot kk.  Contractions over the head dim take channel x = kk * KS + ks at
// k-step ks (each lane's channels contiguous); output columns are value
// channels y = CPL * l16 + c of column tile c (each lane's columns
// contiguous).  The four wavefronts split the work: wavefront w takes k-steps
// w KSW .. w KSW + KSW - 1 of phi(q)^T S_0 and the group's token tiles j = w,
// w + 4, ... up to a (W = phi(q) phi(k)^T over the whole head dim, then W V);
// their partial sums meet in LDS.  W goes from the result layout (rows =
// tokens t) to the A layout through a wavefront-private LDS tile (LDS
// operations of one wavefront complete in order).  The next token tile's keys
// and values are loaded while the current one is multiplied.
template <bool BF16, int R, int D>
__global__ __launch_bounds__(kThreads) void k_pf_state(const void* q, const void* k_new, const void* v_new,
                                                        const float* s_all, const float* z_all, float* obar,
                                                        float* dz, uint16_t* phq, int32_t m, int32_t G, int32_t H) {
  constexpr int KS = D / 4;    // k-steps over the head dim
  constexpr int KSW = KS / 4;  // of them per wavefront in phi(q)^T S_0
  constexpr int CPL = D / 16;  // output column tiles (columns per lane)
  __shared__ float wt[4][16][17];                        // W tile of each wavefront
  __shared__ __attribute__((aligned(16))) float red[4][16][D];  // partial o_bar rows of each wavefront
  __shared__ float rsum[4][16];                          // partial sum_i W[t][i] of each wavefront
  __shared__ float sdz[16];                              // phi(q_t).z_0
  const int a = blockIdx.x, g = blockIdx.y, h = blockIdx.z;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64, l16 = lane % 16, kk = lane / 16;
  const int t0 = 16 * a;
  const int tq = min(t0 + l16, m - 1);  // A row token (rows past the group repeat the last token, never stored)
  const int hq = g * R + h;
  const float* S = s_all + (size_t)g * D * D;

  // ---- A: phi(q) of token tq, channels kk KS .. kk KS + KS - 1
  float fq[KS];
  load_run<BF16, KS>(q, ((size_t)tq * H + hq) * D + kk * KS, fq);
  // this wavefront's first token tile of keys and values
  float fk[KS], vr[4][CPL];
  auto load_kv = [&](int j) {
    load_run<BF16, KS>(k_new, ((size_t)min(16 * j + l16, m - 1) * G + g) * D + kk * KS, fk);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      load_run<BF16, CPL>(v_new, ((size_t)min(16 * j + 4 * ks + kk, m - 1) * G + g) * D + CPL * l16, vr[ks]);
  };
  if (w <= a) load_kv(w);
  // this wavefront's rows of S_0
  float sr[KSW][CPL];
#pragma unroll
  for (int u = 0; u < KSW; ++u) load_run<false, CPL>(S, (size_t)(kk * KS + w * KSW + u) * D + CPL * l16, sr[u]);
#pragma unroll
  for (int i = 0; i < KS; ++i) fq[i] = phi_f(fq[i]);
  if (w == 0) {
    // phi(q) as bf16 hi + lo for the attend (hi + lo carries phi to ~2^-16 relative)
    if (t0 + l16 < m) {
      uint16_t* dst = phq + ((size_t)tq * H + hq) * 2 * D + kk * KS;
#pragma unroll
      for (int i = 0; i < KS; i += 2) {
        const uint32_t hi = pack_bf16(fq[i], fq[i + 1]);
        const uint32_t lo = pack_bf16(fq[i] - bf16_lo_f(hi), fq[i + 1] - bf16_hi_f(hi));
        *reinterpret_cast<uint32_t*>(dst + i) = hi;
        *reinterpret_cast<uint32_t*>(dst + D + i) = lo;
      }
    }
    // phi(q_t).z_0: this lane's channels, then the four k slots
    float zv[KS];
    load_run<false, KS>(z_all + (size_t)g * D, kk * KS, zv);
    float sz = 0.f;
#pragma unroll
    for (int i = 0; i < KS; ++i) sz = fmaf(fq[i], zv[i], sz);
    sz += __shfl_xor(sz, 16);
    sz += __shfl_xor(sz, 32);
    if (kk == 0) sdz[l16] = sz;
  }

  // ---- phi(q)^T S_0 over this wavefront's k-steps
  f32x4_t acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < KSW; ++u)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = mfma_f32(fq[w * KSW + u], sr[u][c], acc[c]);

  // ---- the group's tokens i <= t: this wavefront's token tiles
  float wsum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = w; j <= a; j += 4) {
    float fkc[KS], vc[4][CPL];
#pragma unroll
    for (int i = 0; i < KS; ++i) fkc[i] = phi_f(fk[i]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int c = 0; c < CPL; ++c) vc[ks][c] = vr[ks][c];
    if (j + 4 <= a) load_kv(j + 4);
    f32x4_t wc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) wc = mfma_f32(fq[ks], fkc[ks], wc);
    // lane holds W[t = t0 + 4 kk + r][i = 16 j + l16]; zero where i > t or past the group
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ti = t0 + 4 * kk + r, ii = 16 * j + l16;
      const float wv = (ii <= ti && ii < m) ? wc[r] : 0.f;
      wsum[r] += wv;
      wt[w][4 * kk + r][l16] = wv;
    }
    // o += W V: A[t = l16][i = 4 ks + kk], B[i][y] = v_i[y]
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float av = wt[w][l16][4 * ks + kk];
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = mfma_f32(av, vc[ks][c], acc[c]);
    }
  }

  // ---- partial sums of the wavefronts meet in LDS: lane holds rows 4 kk + r, columns CPL l16 ..
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float ws = row16_sum(wsum[r]);
#pragma unroll
    for (int c = 0; c < CPL; c += 4)
      *reinterpret_cast<float4*>(&red[w][4 * kk + r][CPL * l16 + c]) =
          make_float4(acc[c][r], acc[c + 1][r], acc[c + 2][r], acc[c + 3][r]);
    if (l16 == 0) rsum[w][4 * kk + r] = ws;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * (D / 4); e += kThreads) {
    const int tl = e / (D / 4), y4 = e % (D / 4);
    const int t = t0 + tl;
    if (t >= m) continue;
    const float4 x0 = *reinterpret_cast<const float4*>(&red[0][tl][4 * y4]);
    const float4 x1 = *reinterpret_cast<const float4*>(&red[1][tl][4 * y4]);
    const float4 x2 = *reinterpret_cast<const float4*>(&red[2][tl][4 * y4]);
    const float4 x3 = *reinterpret_cast<const float4*>(&red[3][tl][4 * y4]);
    *reinterpret_cast<float4*>(obar + (((size_t)t * G + g) * R + h) * D + 4 * y4) =
        make_float4((x0.x + x1.x) + (x2.x + x3.x), (x0.y + x1.y) + (x2.y + x3.y), (x0.z + x1.z) + (x2.z + x3.z),
                    (x0.w + x1.w) + (x2.w + x3.w));
  }
  if ((int)threadIdx.x < 16) {
    const int t = t0 + threadIdx.x;
    if (t < m)
      dz[((size_t)t * G + g) * R + h] =
          sdz[threadIdx.x] + ((rsum[0][threadIdx.x] + rsum[1][threadIdx.x]) + (rsum[2][threadIdx.x] + rsum[3][threadIdx.x]));
  }
}

// Appended tokens into the state: S_all[seq][g] += phi(K)^T V and
// z_all[seq][g] += sum_t phi(k_t) over the n tokens of each append entry
// (SPLA Technical Summary 2.2), fp32 on the 16x16x4 fp32 matrix cores.  grid
// (D / 16, G, entries): rows x of a 16-row tile of S (A rows = key channels,
// B columns = value channels y = CPL * l16 + c, k = tokens t = 4 ks + kk);
// wavefront w takes k-steps w, w + 4, ... and the four partial tiles meet in
// LDS before the one read-modify-write of S.  A single token adds its exact
// products phi(k[x]) v[y] (the other terms are zeros), so a one-token append
// rounds like the decode step's fused append.
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_state_add(const AppendArgs a) {
  constexpr int CPL = D / 16;
  __shared__ __attribute__((aligned(16))) float red[4][16][D];
  __shared__ float zr[4][16];
  const AppendEntry& E = a.e[blockIdx.z];
  const int xt = blockIdx.x, g = blockIdx.y, G = a.st.G, m = E.n;
  if (m <= 0) return;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64, l16 = lane % 16, kk = lane / 16;
  const int x = 16 * xt + l16;  // A row: key channel
  const int nks = (m + 3) / 4;
  f32x4_t acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float zs = 0.f;
  for (int ks = w; ks < nks; ks += 4) {
    const int t = 4 * ks + kk;
    const size_t row = ((size_t)(E.row + min(t, m - 1)) * G + g) * D;
    const float kx = load_elem<BF16>(a.st.k_new, row + x);
    float vr[CPL];
    load_run<BF16, CPL>(a.st.v_new, row + CPL * l16, vr);
    const float fk = t < m ? phi_f(kx) : 0.f;
    zs += fk;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = mfma_f32(fk, vr[c], acc[c]);
  }
  zs += __shfl_xor(zs, 16);
  zs += __shfl_xor(zs, 32);
  // lane holds rows 4 kk + r of the tile, columns CPL l16 ..
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < CPL; c += 4)
      *reinterpret_cast<float4*>(&red[w][4 * kk + r][CPL * l16 + c]) =
          make_float4(acc[c][r], acc[c + 1][r], acc[c + 2][r], acc[c + 3][r]);
  if (kk == 0) zr[w][l16] = zs;
  __syncthreads();
  float* S = a.st.s_all + (((size_t)E.seq * G + g) * D + 16 * xt) * D;
  for (int e = threadIdx.x; e < 16 * (D / 4); e += kThreads) {
    const int xl = e / (D / 4), y4 = e % (D / 4);
    const float4 x0 = *reinterpret_cast<const float4*>(&red[0][xl][4 * y4]);
    const float4 x1 = *reinterpret_cast<const float4*>(&red[1][xl][4 * y4]);
    const float4 x2 = *reinterpret_cast<const float4*>(&red[2][xl][4 * y4]);
    const float4 x3 = *reinterpret_cast<const float4*>(&red[3][xl][4 * y4]);
    float4* dst = reinterpret_cast<float4*>(S + (size_t)xl * D) + y4;
    const float4 o = *dst;
    *dst = make_float4(o.x + ((x0.x + x1.x) + (x2.x + x3.x)), o.y + ((x0.y + x1.y) + (x2.y + x3.y)),
                       o.z + ((x0.z + x1.z) + (x2.z + x3.z)), o.w + ((x0.w + x1.w) + (x2.w + x3.w)));
  }
  if ((int)threadIdx.x < 16)
    a.st.z_all[((size_t)E.seq * G + g) * D + 16 * xt + threadIdx.x] +=
        (zr[0][threadIdx.x] + zr[1][threadIdx.x]) + (zr[2][threadIdx.x] + zr[3][threadIdx.x]);
}

}  // namespace

// the state part of an append: every entry of a (its k_new / v_new rows from
// E.row on, [rows][G][d]) into S_all / z_all of its sequence
hipError_t launch_state_add(const AppendArgs& a, bool bf16, const Launch& l) {
  if (a.n_entries <= 0) return hipSuccess;
  const dim3 grid(a.st.d / 16, a.st.G, a.n_entries);
  if (bf16) {
    SPLA_DISPATCH_D(a.st.d, launch_kernel(k_state_add<true, DD>, grid, l, a))
  }
  SPLA_DISPATCH_D(a.st.d, launch_kernel(k_state_add<false, DD>, grid, l, a))
}

// a.B tokens of one sequence (virtual queries) whose state rows the pointers
// address; k_new / v_new: the group's tokens [a.B][G][d]
hipError_t launch_pf_state(const DecodeArgs& a, bool bf16, const void* k_new, const void* v_new, const Launch& l) {
  if (!a.virtual_queries) return hipErrorInvalidValue;
  const dim3 grid((a.B + 15) / 16, a.G, a.r);
  if (bf16)
    SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_pf_state<true, RR, DD>, grid, l, a.q, k_new, v_new, a.s_all, a.z_all,
                                             a.obar_part, a.dz_part, a.phq, a.B, a.G, a.H))
  SPLA_DISPATCH_RD(a.r, a.d, launch_kernel(k_pf_state<false, RR, DD>, grid, l, a.q, k_new, v_new, a.s_all, a.z_all,
                                           a.obar_part, a.dz_part, a.phq, a.B, a.G, a.H))
}

}  // namespace spla
