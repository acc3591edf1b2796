// spla_decode kernels.
//
//   k_score    log-domain second-order Taylor block score of every candidate
//              block, summed over the query heads of a KV group
//              (SPLA Technical Summary 2.1, score formula with the diagonal
//              covariance of its implementation paragraph)
//   k_select   top-(top_k - 2) candidates per (sequence, KV head) by radix
//              select over the scores, plus the sink and the current block
//   k_attend   one selected block per workgroup: exact softmax partials
//              (max, sum, sum p v) and the linear-attention partials
//              (sum w v, sum w, w = phi(q).phi(k)) from the same K/V tile
//              (Technical Summary 2.2: o_tilde from the blocks already loaded)
//   k_combine  merge of the partials, o_bar = phi(q)^T S_all, o_rla = o_bar -
//              o_tilde, D = phi(q).z_all - sum w, o = o_sparse + g_h o_rla
#include "spla_common.h"

namespace spla {

namespace {

__device__ __forceinline__ int n_blocks(const DecodeArgs& a, int b) { return (a.lens[b] + a.bk - 1) / a.bk; }

// ============================================================== score
// grid (score_tiles, G, B); lane = block within a 64-block tile, the four
// wavefronts split the channels and meet in LDS.
template <bool BF16, int R, int D>
__global__ __launch_bounds__(kThreads) void k_score(const DecodeArgs a) {
  __shared__ float qs[R][D];
  __shared__ float q2s[R][D];
  __shared__ float red[4][2 * R][kTile];
  const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nb = n_blocks(a, b);
  if (nb <= a.top_k) return;  // every block is selected, nothing to rank
  const int j0 = t * kTile;
  if (j0 > nb - 2) return;
  constexpr int d = D;
  for (int i = threadIdx.x; i < R * d; i += kThreads) {
    const int h = i / d, c = i - h * d;
    const float v = load_elem<BF16>(a.q, ((size_t)b * a.H + g * R + h) * d + c);
    qs[h][c] = v;
    q2s[h][c] = v * v;
  }
  __syncthreads();
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  constexpr int nc4 = d / 16;  // channel quartets per wavefront
  const float4* mean4 = reinterpret_cast<const float4*>(a.blk_mean);
  const float4* var4 = reinterpret_cast<const float4*>(a.blk_var);
  const size_t base = (((size_t)b * a.G + g) * a.n_tiles + t) * (size_t)(d / 4) * kTile;
  float dot[R], qv[R];
#pragma unroll
  for (int h = 0; h < R; ++h) dot[h] = qv[h] = 0.f;
  float4 m[nc4], v[nc4];
#pragma unroll
  for (int i = 0; i < nc4; ++i) {
    const size_t o = base + (size_t)(w * nc4 + i) * kTile + lane;
    m[i] = mean4[o];
    v[i] = var4[o];
  }
#pragma unroll
  for (int i = 0; i < nc4; ++i) {
    {
      const int c = (w * nc4 + i) * 4;
#pragma unroll
      for (int h = 0; h < R; ++h) {
        const float4 q = *reinterpret_cast<const float4*>(&qs[h][c]);
        const float4 q2 = *reinterpret_cast<const float4*>(&q2s[h][c]);
        dot[h] = fmaf(q.x, m[i].x, dot[h]);
        dot[h] = fmaf(q.y, m[i].y, dot[h]);
        dot[h] = fmaf(q.z, m[i].z, dot[h]);
        dot[h] = fmaf(q.w, m[i].w, dot[h]);
        qv[h] = fmaf(q2.x, v[i].x, qv[h]);
        qv[h] = fmaf(q2.y, v[i].y, qv[h]);
        qv[h] = fmaf(q2.z, v[i].z, qv[h]);
        qv[h] = fmaf(q2.w, v[i].w, qv[h]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < R; ++h) {
    red[w][h][lane] = dot[h];
    red[w][R + h][lane] = qv[h];
  }
  __syncthreads();
  if (w != 0) return;
  const int j = j0 + lane;
  if (j < 1 || j > nb - 2) return;
  const float half_inv_d = 0.5f / (float)d;
  float ls[R];
  float mx = -INFINITY;
#pragma unroll
  for (int h = 0; h < R; ++h) {
    const float dd = red[0][h][lane] + red[1][h][lane] + red[2][h][lane] + red[3][h][lane];
    const float vv = red[0][R + h][lane] + red[1][R + h][lane] + red[2][R + h][lane] + red[3][R + h][lane];
    ls[h] = dd * a.inv_sqrt_d + log1pf(fmaxf(vv, 0.f) * half_inv_d);
    mx = fmaxf(mx, ls[h]);
  }
  float lg = ls[0];
  if (R > 1) {
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < R; ++h) s += expf(ls[h] - mx);
    lg = mx + logf(s);
  }
  a.lg[((size_t)b * a.G + g) * (size_t)(a.n_tiles * kTile) + j] = lg;
  if (a.lg_out) a.lg_out[((size_t)b * a.G + g) * a.max_blocks + j] = lg;
}

// ============================================================== select
__device__ __forceinline__ int block_excl_scan(int v, int* tmp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int add = 0;
  for (int i = 0; i < w; ++i) add += tmp[i];
  __syncthreads();
  return x - v + add;
}

// grid (G, B).  Finds the exact key tau of the k'-th largest LG by four 8-bit
// radix passes (LDS histograms), then keeps every candidate with key > tau and
// the lowest-id candidates with key == tau.
__global__ __launch_bounds__(kThreads) void k_select(const DecodeArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ int s_digit, s_gt;
  __shared__ int tmp[4];
  const int g = blockIdx.x, b = blockIdx.y;
  const int nb = n_blocks(a, b);
  int32_t* out = a.sel + ((size_t)b * a.G + g) * a.top_k;
  int32_t* out2 = a.sel_out ? a.sel_out + ((size_t)b * a.G + g) * a.top_k : nullptr;
  if (nb <= a.top_k) {
    for (int s = threadIdx.x; s < a.top_k; s += kThreads) {
      out[s] = s < nb ? s : -1;
      if (out2) out2[s] = s < nb ? s : -1;
    }
    return;
  }
  const int nc = nb - 2;
  const int kp = a.top_k - 2;
  const float* L = a.lg + ((size_t)b * a.G + g) * (size_t)(a.n_tiles * kTile) + 1;  // L[i] = LG(i + 1)
  const int per = (nc + kThreads - 1) / kThreads;
  const int i0 = min(nc, (int)threadIdx.x * per), i1 = min(nc, i0 + per);
  uint32_t prefix = 0, mask = 0;
  int krem = kp;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[threadIdx.x] = 0;
    __syncthreads();
    for (int i = i0; i < i1; ++i) {
      const uint32_t key = float_key(L[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      uint32_t c[4];
      int sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hist[255 - 4 * lane - q];
        sum += (int)c[q];
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      int run = incl - sum;  // keys in higher bins than this lane's
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (run < krem && run + (int)c[q] >= krem) {
          s_digit = 255 - 4 * lane - q;
          s_gt = run;
        }
        run += (int)c[q];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_digit << shift;
    mask |= 255u << shift;
    krem -= s_gt;
    __syncthreads();
  }
  const uint32_t tau = prefix;
  int my_eq = 0;
  for (int i = i0; i < i1; ++i) my_eq += float_key(L[i]) == tau;
  const int eq_before = block_excl_scan(my_eq, tmp);
  int my_sel = 0, seen = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = float_key(L[i]);
    if (key > tau) {
      ++my_sel;
    } else if (key == tau) {
      if (eq_before + seen < krem) ++my_sel;
      ++seen;
    }
  }
  int pos = 1 + block_excl_scan(my_sel, tmp);
  seen = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = float_key(L[i]);
    bool take = false;
    if (key > tau) {
      take = true;
    } else if (key == tau) {
      take = eq_before + seen < krem;
      ++seen;
    }
    if (take) {
      out[pos] = i + 1;
      if (out2) out2[pos] = i + 1;
      ++pos;
    }
  }
  if (threadIdx.x == 0) {
    out[0] = 0;
    out[kp + 1] = nb - 1;
    if (out2) {
      out2[0] = 0;
      out2[kp + 1] = nb - 1;
    }
  }
}

// ============================================================== attend
// grid (top_k, G, B): one selected block of one (b, g) per workgroup, all R
// query heads of the group.  Tokens in chunks of 64: K chunk staged in LDS as
// fp32, lane = token for the two dot products, then thread = value channel for
// the weighted sums (V read straight from the page, coalesced along d).
template <bool BF16, int R, int D>
__global__ __launch_bounds__(kThreads) void k_attend(const DecodeArgs a) {
  constexpr int KS = D + 1;  // padded row stride of the K chunk (floats)
  __shared__ float ks[64 * KS];
  __shared__ float qs[R][D];
  __shared__ float fq[R][D];
  __shared__ float red[4][2 * R][64];
  __shared__ float pw[2 * R][64];  // p (softmax numerators) then w (linear weights)
  __shared__ float sf[R];          // rescale of the running sums for this chunk
  __shared__ float s_m[R], s_l[R], s_sw[R];
  const int slot = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  constexpr int d = D;
  const int bk = a.bk;
  const int32_t* selp = a.sel_in ? a.sel_in : a.sel;
  const int j = selp[((size_t)b * a.G + g) * a.top_k + slot];
  if (j < 0) return;
  const int T = a.lens[b];
  const int nb = n_blocks(a, b);
  if (j >= nb) {
    if (threadIdx.x == 0) atomicOr(a.err, kErrSel);
    return;
  }
  const int page = a.block_table[(size_t)b * a.max_blocks + j];
  if (page < 0 || page >= a.num_pages) {
    if (threadIdx.x == 0) atomicOr(a.err, kErrPage);
    return;
  }
  const int ntok = min(bk, T - j * bk);
  for (int i = threadIdx.x; i < R * d; i += kThreads) {
    const int h = i / d, c = i - h * d;
    const float v = load_elem<BF16>(a.q, ((size_t)b * a.H + g * R + h) * d + c);
    qs[h][c] = v;
    fq[h][c] = phi_f(v);
  }
  if (threadIdx.x < R) {
    s_m[threadIdx.x] = -INFINITY;
    s_l[threadIdx.x] = 0.f;
    s_sw[threadIdx.x] = 0.f;
  }
  const size_t page_base = (((size_t)page * a.G + g) * bk) * d;
  // per-thread accumulators: value channel c, pairs (kind, head) strided by the group count
  constexpr int ngrp = kThreads / d;
  constexpr int npair = (2 * R + ngrp - 1) / ngrp;
  const int c = threadIdx.x % d;
  const int grp = threadIdx.x / d;
  float acc[npair];
#pragma unroll
  for (int k = 0; k < npair; ++k) acc[k] = 0.f;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  constexpr int cq = d / 4;  // channels per wavefront in the dot phase
  for (int c0 = 0; c0 < ntok; c0 += 64) {
    const int n = min(64, ntok - c0);
    __syncthreads();
    // stage K chunk (n x d) as fp32
    for (int i = threadIdx.x; i < n * (d / 4); i += kThreads) {
      const int tok = i / (d / 4), q4 = i - tok * (d / 4);
      const float4 k4 = load4<BF16>(a.k_pages, page_base + (size_t)(c0 + tok) * d + q4 * 4);
      float* dst = &ks[tok * KS + q4 * 4];
      dst[0] = k4.x;
      dst[1] = k4.y;
      dst[2] = k4.z;
      dst[3] = k4.w;
    }
    __syncthreads();
    float sp[R], wp[R];
#pragma unroll
    for (int h = 0; h < R; ++h) sp[h] = wp[h] = 0.f;
    if (lane < n) {
      for (int cc = w * cq; cc < (w + 1) * cq; ++cc) {
        const float kv = ks[lane * KS + cc];
        const float fk = phi_f(kv);
#pragma unroll
        for (int h = 0; h < R; ++h) {
          sp[h] = fmaf(qs[h][cc], kv, sp[h]);
          wp[h] = fmaf(fq[h][cc], fk, wp[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < R; ++h) {
      red[w][h][lane] = sp[h];
      red[w][R + h][lane] = wp[h];
    }
    __syncthreads();
    // softmax bookkeeping: wavefront w handles heads w, w+4
    for (int h = w; h < R; h += 4) {
      float s = -INFINITY, wv = 0.f;
      if (lane < n) {
        s = (red[0][h][lane] + red[1][h][lane] + red[2][h][lane] + red[3][h][lane]) * a.inv_sqrt_d;
        wv = red[0][R + h][lane] + red[1][R + h][lane] + red[2][R + h][lane] + red[3][R + h][lane];
      }
      const float mc = wave_max(s);
      const float m_old = s_m[h];
      const float m_new = fmaxf(m_old, mc);
      const float p = lane < n ? expf(s - m_new) : 0.f;
      const float ps = wave_sum(p);
      const float ws = wave_sum(wv);
      pw[h][lane] = p;
      pw[R + h][lane] = wv;
      if (lane == 0) {
        const float scale = expf(m_old - m_new);  // 0 on the first chunk
        sf[h] = scale;
        s_l[h] = s_l[h] * scale + ps;
        s_m[h] = m_new;
        s_sw[h] += ws;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < npair; ++k) {
      const int p = grp + k * ngrp;
      if (p < 2 * R) {
        const bool is_sm = p < R;
        float x = is_sm ? acc[k] * sf[p] : acc[k];
        const float* wt = pw[p];
        for (int i = 0; i < n; ++i) {
          const float v = load_elem<BF16>(a.v_pages, page_base + (size_t)(c0 + i) * d + c);
          x = fmaf(wt[i], v, x);
        }
        acc[k] = x;
      }
    }
  }
  __syncthreads();
  const int rec = 2 * d + kPartHdr;
#pragma unroll
  for (int k = 0; k < npair; ++k) {
    const int p = grp + k * ngrp;
    if (p < 2 * R) {
      const int h = p < R ? p : p - R;
      float* dst = a.part + (((size_t)b * a.H + g * R + h) * a.top_k + slot) * rec + kPartHdr + (p < R ? 0 : d);
      dst[c] = acc[k];
    }
  }
  if (threadIdx.x < R) {
    const int h = threadIdx.x;
    float* dst = a.part + (((size_t)b * a.H + g * R + h) * a.top_k + slot) * rec;
    dst[0] = s_m[h];
    dst[1] = s_l[h];
    dst[2] = s_sw[h];
    dst[3] = 0.f;
  }
}

// ============================================================== combine
// grid (G, B): merge the slot partials of the R heads of (b, g), contract
// phi(q) with S_all and z_all, write o (and the optional outputs).
template <bool BF16, int R, int D>
__global__ __launch_bounds__(kThreads) void k_combine(const DecodeArgs a) {
  constexpr int ngrp = kThreads / D;
  __shared__ float fq[R][D];
  __shared__ float wsl[R][256];  // per-slot softmax weight exp(m_s - m) / L
  __shared__ float s_sw[R];
  __shared__ float obr[ngrp][R][D];
  __shared__ float s_dz[R];
  __shared__ int valid[256];
  const int g = blockIdx.x, b = blockIdx.y;
  constexpr int d = D;
  const int nb = n_blocks(a, b);
  const bool covers_all = nb <= a.top_k;
  const int32_t* selp = a.sel_in ? a.sel_in : a.sel;
  const int32_t* srow = selp + ((size_t)b * a.G + g) * a.top_k;
  for (int s = threadIdx.x; s < a.top_k; s += kThreads) {
    const int j = srow[s];
    valid[s] = (j >= 0 && j < nb) ? 1 : 0;
    if (a.sel_out) a.sel_out[((size_t)b * a.G + g) * a.top_k + s] = j;
  }
  for (int i = threadIdx.x; i < R * d; i += kThreads) {
    const int h = i / d, c = i - h * d;
    fq[h][c] = phi_f(load_elem<BF16>(a.q, ((size_t)b * a.H + g * R + h) * d + c));
  }
  __syncthreads();
  const int rec = 2 * d + kPartHdr;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int h = w; h < R; h += 4) {
    const float* P = a.part + ((size_t)b * a.H + g * R + h) * a.top_k * (size_t)rec;
    float m = -INFINITY;
    for (int s = lane; s < a.top_k; s += 64)
      if (valid[s]) m = fmaxf(m, P[(size_t)s * rec]);
    m = wave_max(m);
    float l = 0.f, sw = 0.f;
    for (int s = lane; s < a.top_k; s += 64) {
      if (valid[s]) {
        const float e = expf(P[(size_t)s * rec] - m);
        wsl[h][s] = e;
        l += e * P[(size_t)s * rec + 1];
        sw += P[(size_t)s * rec + 2];
      } else {
        wsl[h][s] = 0.f;
      }
    }
    l = wave_sum(l);
    sw = wave_sum(sw);
    const float inv_l = 1.f / l;
    for (int s = lane; s < a.top_k; s += 64) wsl[h][s] *= inv_l;
    // phi(q) . z_all
    float dz = 0.f;
    const float* z = a.z_all + ((size_t)b * a.G + g) * d;
    for (int c = lane; c < d; c += 64) dz = fmaf(fq[h][c], z[c], dz);
    dz = wave_sum(dz);
    if (lane == 0) {
      s_sw[h] = sw;
      s_dz[h] = dz;
    }
  }
  // o_bar = phi(q)^T S: thread = column, rows split over ngrp thread groups
  {
    const int c = threadIdx.x % d, grp = threadIdx.x / d;
    const float* S = a.s_all + ((size_t)b * a.G + g) * d * (size_t)d;
    constexpr int rows = d / ngrp;
    float ob[R];
#pragma unroll
    for (int h = 0; h < R; ++h) ob[h] = 0.f;
    for (int x = grp * rows; x < (grp + 1) * rows; ++x) {
      const float sv = S[(size_t)x * d + c];
#pragma unroll
      for (int h = 0; h < R; ++h) ob[h] = fmaf(fq[h][x], sv, ob[h]);
    }
#pragma unroll
    for (int h = 0; h < R; ++h) obr[grp][h][c] = ob[h];
  }
  __syncthreads();
  // finalize: thread -> (h, c)
  for (int i = threadIdx.x; i < R * d; i += kThreads) {
    const int h = i / d, c = i - h * d;
    const float* P = a.part + ((size_t)b * a.H + g * R + h) * a.top_k * (size_t)rec;
    float os = 0.f, ot = 0.f;
    for (int s = 0; s < a.top_k; ++s) {
      if (!valid[s]) continue;
      const float* ps = P + (size_t)s * rec + kPartHdr;
      os = fmaf(wsl[h][s], ps[c], os);
      ot += ps[d + c];
    }
    float orla = 0.f, drla = 0.f;
    if (!covers_all) {
      float obar = 0.f;
#pragma unroll
      for (int q = 0; q < ngrp; ++q) obar += obr[q][h][c];
      orla = obar - ot;
      drla = s_dz[h] - s_sw[h];
    }
    const size_t oi = ((size_t)b * a.H + g * R + h) * d + c;
    a.out[oi] = os + a.gate[g * R + h] * orla;
    if (a.o_sparse_out) a.o_sparse_out[oi] = os;
    if (a.o_rla_out) a.o_rla_out[oi] = orla;
    if (a.d_rla_out && c == 0) a.d_rla_out[(size_t)b * a.H + g * R + h] = drla;
  }
}

}  // namespace

#define SPLA_DISPATCH_D(D_, ...)                                 \
  switch (D_) {                                                 \
    case 64: { constexpr int DD = 64; __VA_ARGS__; } break;     \
    case 128: { constexpr int DD = 128; __VA_ARGS__; } break;   \
    default: return hipErrorInvalidValue;                       \
  }
#define SPLA_DISPATCH_RD(R_, D_, ...)                                        \
  switch (R_) {                                                             \
    case 1: { constexpr int RR = 1; SPLA_DISPATCH_D(D_, __VA_ARGS__) } break; \
    case 2: { constexpr int RR = 2; SPLA_DISPATCH_D(D_, __VA_ARGS__) } break; \
    case 4: { constexpr int RR = 4; SPLA_DISPATCH_D(D_, __VA_ARGS__) } break; \
    case 8: { constexpr int RR = 8; SPLA_DISPATCH_D(D_, __VA_ARGS__) } break; \
    default: return hipErrorInvalidValue;                                   \
  }

hipError_t launch_score(const DecodeArgs& a, bool bf16, hipStream_t s) {
  dim3 grid(a.score_tiles, a.G, a.B);
  if (a.score_tiles == 0) return hipSuccess;
  if (bf16) {
    SPLA_DISPATCH_RD(a.r, a.d, (k_score<true, RR, DD><<<grid, kThreads, 0, s>>>(a)))
  } else {
    SPLA_DISPATCH_RD(a.r, a.d, (k_score<false, RR, DD><<<grid, kThreads, 0, s>>>(a)))
  }
  return hipGetLastError();
}

hipError_t launch_select(const DecodeArgs& a, hipStream_t s) {
  k_select<<<dim3(a.G, a.B), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_attend(const DecodeArgs& a, bool bf16, hipStream_t s) {
  dim3 grid(a.top_k, a.G, a.B);
  if (bf16) {
    SPLA_DISPATCH_RD(a.r, a.d, (k_attend<true, RR, DD><<<grid, kThreads, 0, s>>>(a)))
  } else {
    SPLA_DISPATCH_RD(a.r, a.d, (k_attend<false, RR, DD><<<grid, kThreads, 0, s>>>(a)))
  }
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs& a, bool bf16, hipStream_t s) {
  dim3 grid(a.G, a.B);
  if (bf16) {
    SPLA_DISPATCH_RD(a.r, a.d, (k_combine<true, RR, DD><<<grid, kThreads, 0, s>>>(a)))
  } else {
    SPLA_DISPATCH_RD(a.r, a.d, (k_combine<false, RR, DD><<<grid, kThreads, 0, s>>>(a)))
  }
  return hipGetLastError();
}

}  // namespace spla
