// Internal definitions shared by the SPLA HIP kernels and the host ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spla {

constexpr int kMaxBatch = 256;
constexpr int kMaxAppendEntries = 64;  // entries per append launch (host splits larger calls)
constexpr int kTile = 64;              // blocks per statistics tile (= wavefront width)
constexpr int kThreads = 256;          // threads per workgroup of every kernel
constexpr int kPartHdr = 4;            // m, l, sum_w, pad ahead of acc[d], o_tilde[d]

// error word bits (workspace bytes [0, 4))
constexpr uint32_t kErrPage = 1u;
constexpr uint32_t kErrSel = 2u;

struct AppendEntry {
  int32_t seq;  // sequence id
  int32_t n;    // rows appended
  int32_t t0;   // length before the append
  int32_t row;  // first row of this entry in k_new / v_new
};

struct AppendArgs {
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
  int32_t n_entries;
  int32_t s_items;     // state-update workgroups (n_entries * G * d / rows_per_item)
  int32_t page_items;  // page-copy workgroups
  int32_t stat_items;  // block-statistics workgroups
  int32_t page_prefix[kMaxAppendEntries + 1];
  int32_t stat_prefix[kMaxAppendEntries + 1];
  AppendEntry e[kMaxAppendEntries];
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
  int32_t* sel;     // workspace [B][G][top_k]
  float* part;      // workspace [B][H][top_k][2d + kPartHdr]
  uint32_t* err;    // workspace error word
  const int32_t* sel_in;
  int32_t* sel_out;
  float* lg_out;
  float* o_sparse_out;
  float* o_rla_out;
  float* d_rla_out;
  int32_t B, H, G, d, r, bk, top_k, max_blocks, num_pages, n_tiles;
  int32_t score_tiles;  // grid.x of the scorer
  float inv_sqrt_d;
  int32_t lens[kMaxBatch];
};

// host-side launchers (defined next to their kernels)
hipError_t launch_append(const AppendArgs& a, bool bf16, hipStream_t s);
hipError_t launch_score(const DecodeArgs& a, bool bf16, hipStream_t s);
hipError_t launch_select(const DecodeArgs& a, hipStream_t s);
hipError_t launch_attend(const DecodeArgs& a, bool bf16, hipStream_t s);
hipError_t launch_combine(const DecodeArgs& a, bool bf16, hipStream_t s);

// ------------------------------------------------------------ device helpers
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

// 64-wide wavefront reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// order-preserving map float -> uint32 (larger float -> larger key)
__device__ __forceinline__ uint32_t float_key(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace spla
