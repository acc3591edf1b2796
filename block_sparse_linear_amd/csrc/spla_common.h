// Internal definitions shared by the SPLA HIP kernels and the host ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
#include <utility>

namespace spla {

constexpr int kMaxBatch = 256;
constexpr int kMaxBlocksPerSeq = 16386;  // the selector ranks at most 16384 candidates in LDS
constexpr int kMaxAppendEntries = 64;  // entries per append launch (host splits larger calls)
constexpr int kTile = 64;              // blocks per statistics tile (= wavefront width)
constexpr int kThreads = 256;          // threads per workgroup of every kernel
constexpr int kPartHdr = 4;  // floats of a partial record's header: m, l, sum_w, pad
// (b, h) pairs from which a combine workgroup takes a whole head (fewer: a
// 32-channel slice each)
constexpr int kCombineWholeHeads = 256;
// (b, g) pairs from which the first kernel of a decode step takes four S_all
// row chunks per workgroup instead of one
constexpr int kStateGroupPairs = 512;

// block score forms (spla_score_form)
constexpr int kScoreTaylor = 0, kScoreMean = 1;

// output forms of the RLA branch (spla_rla_form)
constexpr int kRlaPlain = 0, kRlaNormalized = 1, kRlaRms = 2;

// error word bits (workspace bytes [0, 4))
constexpr uint32_t kErrPage = 1u;
constexpr uint32_t kErrSel = 2u;
// one-kernel step: a wait ran out (4), a producer count above its target at
// a wait (8), more attend workgroups past their wait than slots (16), a
// pair's producers not all on the attend workgroup's XCD (32)
constexpr uint32_t kErrStepWait = 4u, kErrStepCount = 8u, kErrStepArrive = 16u, kErrStepXcd = 32u;

// counters of the one-kernel decode step: one 128-byte line per (sequence,
// KV head) pair (count of finished producer workgroups, count of attend
// workgroups past their wait), at workspace bytes [256, 256 + 128 kStepPairs);
// each call leaves them at zero
constexpr int kStepPairs = 256;
constexpr int kStepCtrStride = 32;  // int32 per pair
constexpr size_t kStepCtrOffset = 256;

struct AppendEntry {
  int32_t seq;  // sequence id
  int32_t n;    // rows appended
  int32_t t0;   // length before the append
  int32_t row;  // first row of this entry in k_new / v_new
};

struct DecodeArgs {
  const void* q;
  const float* gate;
  float* out;
  const void* k_pages;
  const void* v_pages;
  const int32_t* block_table;
  const float* blk_mean;
  const float* blk_var;
  const float* s_all;
  const float* z_all;
  float* lg;        // workspace [B][G][NT*64]
  int32_t* sel;     // workspace [B][G][top_k] selected block ids
  int32_t* sel_page;  // workspace [B][G][top_k] their page ids
  float* part;      // workspace [B][H][top_k][2d]: a slot's partial acc[d], o_tilde[d] (line-aligned)
  float* part_hdr;  // workspace [B][H][top_k][kPartHdr]: its m, l, sum_w, pad (a head's headers contiguous)
  float* obar_part;  // workspace [B][G][d * d / 1024][R][d]: phi(q)^T S_all over one chunk of S rows
  float* dz_part;    // workspace [B][G][d * d / 1024][R]: phi(q).z_all over the same rows
  int32_t obar_one;  // 1: one o_bar / phi(q).z partial per head ([B][G][R][d], [B][G][R]) instead
  uint16_t* phq;     // workspace [B][H][2][d]: phi(q) as bf16 hi, then the bf16 rounding of the rest
  uint32_t* err;    // workspace error word
  int32_t* step_ctr;  // workspace counters of the one-kernel step (kStepPairs lines)
  const int32_t* sel_in;
  int32_t* sel_out;
  float* lg_out;
  float* o_sparse_out;
  float* o_rla_out;
  float* d_rla_out;
  const float* rla_gamma;  // [H][d] scale of the RMS-normalised RLA branch
  float rla_eps;
  int32_t rla_form;        // spla_rla_form
  int32_t score_form;      // spla_score_form
  int32_t virtual_queries;  // 1: the batch is the tokens of one sequence's prefill chunk (state pointers
                            // address that sequence; every b reads its row 0 of statistics, state, block table)
  int32_t B, H, G, d, r, bk, top_k, max_blocks, num_pages, n_tiles;
  int32_t score_tiles;  // grid.x of the scorer
  int32_t tiles_all;    // score tiles that every sequence of the batch has
  float inv_sqrt_d;
  int32_t lens[kMaxBatch];
};

// where the state lives (device pointers) and its dimensions
struct StateRefs {
  const void* k_new;
  const void* v_new;
  void* k_pages;
  void* v_pages;
  const int32_t* block_table;
  float* blk_mean;
  float* blk_var;
  float* s_all;
  float* z_all;
  uint32_t* err;
  int32_t G, d, bk, max_blocks, num_pages, n_tiles;
};

struct AppendArgs {
  StateRefs st;
  int32_t n_entries;
  int32_t page_items;  // page-copy workgroups
  int32_t page_tok;    // appended tokens per page-copy workgroup (append_page_tokens)
  int32_t stat_items;  // block-statistics workgroups
  int32_t page_prefix[kMaxAppendEntries + 1];
  int32_t stat_prefix[kMaxAppendEntries + 1];
  AppendEntry e[kMaxAppendEntries];
};

// tokens per page-copy workgroup: as many as give every thread one 16-byte
// piece of k (and one of v), at least one
inline int append_page_tokens(int G, int d, bool bf16) {
  const int per_tok = G * d * (bf16 ? 2 : 4) / 16;
  return per_tok >= kThreads ? 1 : kThreads / per_tok;
}

// fused decode step: append one token to every sequence (row b of k_new /
// v_new is sequence b) inside the scorer's launch, then the usual decode
struct StepArgs {
  DecodeArgs dec;      // lens: after the append
  StateRefs st;
};

// where a kernel is launched; with start / stop set, the launch goes through
// hipExtLaunchKernel, which stamps the two events with the kernel's own begin
// and end times (the dispatch packet's timestamps)
struct Launch {
  hipStream_t s = nullptr;
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// launch a kernel with 256-thread workgroups; returns this launch's status.
// Kernels on the decode path take, ahead of their argument struct, the few
// scalars and pointers their first memory accesses need: the library is
// built with kernel-argument preloading, so those arrive in SGPRs at wave
// start instead of through a scalar load from the argument buffer.
template <typename Kernel, typename Tuple, size_t... I>
inline hipError_t launch_tuple(Kernel kernel, dim3 grid, const Launch& l, Tuple& vals, std::index_sequence<I...>) {
  void* argv[] = {static_cast<void*>(&std::get<I>(vals))...};
  const void* f = reinterpret_cast<const void*>(kernel);
  if (l.start || l.stop) return hipExtLaunchKernel(f, grid, dim3(kThreads), argv, 0, l.s, l.start, l.stop, 0);
  return hipLaunchKernel(f, grid, dim3(kThreads), argv, 0, l.s);
}

template <typename... P, typename... A>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, const Launch& l, const A&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<std::decay_t<P>...> vals(args...);  // each argument in the kernel's own parameter type
  return launch_tuple(kernel, grid, l, vals, std::index_sequence_for<P...>{});
}

// host-side launchers (defined next to their kernels)
hipError_t launch_append(const AppendArgs& a, bool bf16, const Launch& l);
hipError_t launch_score(const StepArgs& a, bool bf16, const Launch& l);  // st: no new k / v
hipError_t launch_select(const DecodeArgs& a, const Launch& l);
hipError_t launch_attend(const DecodeArgs& a, bool bf16, const Launch& l);
hipError_t launch_combine(const DecodeArgs& a, const Launch& l);
hipError_t launch_step_score(const StepArgs& a, bool bf16, const Launch& l);
// chunked prefill, block-centric attend (bf16): per-block lists of the
// group's (query, slot) pairs and the work items made from them
constexpr int kPfQ = 8;           // queries per work item
constexpr int kPfItemInts = 16;   // g, j, n, page, kPfQ codes, padding
struct PfBuffers {
  int32_t* cnt;      // [G][max_blocks] (query, slot) pairs per block
  int32_t* lists;    // [G][max_blocks][cap] codes vq * 256 + slot
  int4* items;       // [max_items][kPfItemInts / 4]
  int32_t* n_items;  // items of the current group
  int32_t cap;       // queries per group (list capacity per block)
  int32_t max_items;
};
hipError_t launch_pf_clear(const PfBuffers& pb, int G, int max_blocks, const Launch& l);
hipError_t launch_pf_attend(const DecodeArgs& a, const PfBuffers& pb, const Launch& l);
// chunked prefill: the chunk's own tokens added into the o_bar / phi(q).z
// partials of its virtual queries (k_new / v_new address the chunk's first row)
hipError_t launch_pf_score(const DecodeArgs& a, bool bf16, const Launch& l);
hipError_t launch_pf_state(const DecodeArgs& a, bool bf16, const void* k_new, const void* v_new, const Launch& l);
hipError_t launch_state_add(const AppendArgs& a, bool bf16, const Launch& l);
// exact group log mass of every candidate block (a dense pass over the keys)
hipError_t launch_block_mass(const DecodeArgs& a, bool bf16, float* lgx, int max_cand, const Launch& l);
// fused select + attend: supported for bf16 K/V, block size 64, no selection
// override and at most 16 * 256 candidates per sequence
bool select_attend_supported(const DecodeArgs& a, bool bf16);
// merge: the fused kernel also merges each (b, g)'s records in place of the
// combine kernel (plain and normalised RLA forms, B * H < kCombineWholeHeads,
// B * G <= kStepPairs)
bool select_attend_merge_supported(const DecodeArgs& a);
hipError_t launch_select_attend(const DecodeArgs& a, const Launch& l, bool merge);
// one-kernel decode step (append + scores + o_bar partials, then select +
// attend, with waits inside one XCD): where the fused select + attend is
// supported, with the Taylor score and at most kStepPairs (b, g) pairs
bool step_fused_supported(const DecodeArgs& a, bool bf16);
hipError_t launch_step_fused(const StepArgs& a, const Launch& l);

// ------------------------------------------------------------ device helpers
// the XCD (accelerator complex die) the calling wavefront runs on
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(x));
  return x;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// phi(x) = elu(x) + 1
__device__ __forceinline__ float phi_f(float x) { return x > 0.f ? x + 1.f : expf(x); }

// scalar element i of a K/V/q array
template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
  if constexpr (BF16) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

// four consecutive elements starting at i (i % 4 == 0)
template <bool BF16>
__device__ __forceinline__ float4 load4(const void* p, size_t i) {
  if constexpr (BF16) {
    uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p) + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
  }
}

// ----------------------------------------------------- cross-lane (DPP) ops
// DPP moves run on the VALU with a few cycles of latency, unlike the LDS
// crossbar behind __shfl_*.  Controls (GFX9 encoding): quad_perm, row_shr:n,
// row_mirror, row_half_mirror, row_bcast:15, row_bcast:31.
constexpr int kDppXor1 = 0xb1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;         // quad_perm [2,3,0,1]
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr3 = 0x113;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf, bool BOUND_CTRL = false>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, BANK_MASK, BOUND_CTRL));
}
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf, bool BOUND_CTRL = false>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, BANK_MASK, BOUND_CTRL);
}

// reductions over each 16-lane row; every lane of the row gets the result
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v, v));
  v = fmaxf(v, dpp_f<kDppXor2>(v, v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v, v));
  v = fmaxf(v, dpp_f<kDppRowMirror>(v, v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppXor1>(0.f, v);
  v += dpp_f<kDppXor2>(0.f, v);
  v += dpp_f<kDppRowHalfMirror>(0.f, v);
  v += dpp_f<kDppRowMirror>(0.f, v);
  return v;
}

// full 64-lane reductions, result returned in every lane
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, dpp_f<kDppRowBcast15, 0xa>(-INFINITY, v));
  v = fmaxf(v, dpp_f<kDppRowBcast31, 0xc>(-INFINITY, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_min(float v) {
  v = -v;
  return -wave_max(v);
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += dpp_f<kDppRowBcast15, 0xa>(0.f, v);
  v += dpp_f<kDppRowBcast31, 0xc>(0.f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<kDppXor1>(0, v);
  v += dpp_i<kDppXor2>(0, v);
  v += dpp_i<kDppRowHalfMirror>(0, v);
  v += dpp_i<kDppRowMirror>(0, v);
  v += dpp_i<kDppRowBcast15, 0xa>(0, v);
  v += dpp_i<kDppRowBcast31, 0xc>(0, v);
  return __builtin_amdgcn_readlane(v, 63);
}
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ int wave_incl_scan_i(int v) {
  int t = v + dpp_i<kDppRowShr1, 0xf, 0xf, true>(0, v);
  t += dpp_i<kDppRowShr2, 0xf, 0xf, true>(0, v);
  t += dpp_i<kDppRowShr3, 0xf, 0xf, true>(0, v);
  t += dpp_i<kDppRowShr4, 0xf, 0xe>(0, t);
  t += dpp_i<kDppRowShr8, 0xf, 0xc>(0, t);
  t += dpp_i<kDppRowBcast15, 0xa>(0, t);
  t += dpp_i<kDppRowBcast31, 0xc>(0, t);
  return t;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (round to nearest even, hardware conversion)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo_f(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi_f(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// order-preserving map float -> uint32 (larger float -> larger key)
__device__ __forceinline__ uint32_t float_key(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace spla
