// Host side of the C ABI declared in include/spla.h: configuration checks,
// the host mirror of sequence lengths, workspace layout and kernel launches.
#include <math.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "../../include/spla.h"
#include "spla_common.h"

using namespace spla;

struct spla_handle {
  spla_config cfg{};
  int r = 0;
  int n_tiles = 0;
  bool bound = false;
  spla_buffers buf{};
  std::vector<int32_t> lens;
  hipError_t last_hip = hipSuccess;  // status of the last launch that failed
  int32_t fused_select = -1;         // SPLA_TUNE_FUSED_SELECT
  int32_t step_kernel = -1;          // SPLA_TUNE_STEP_KERNEL
  int32_t fused_merge = -1;          // SPLA_TUNE_FUSED_MERGE
  int32_t rla_form = SPLA_RLA_PLAIN;  // output form of the RLA branch
  const float* rla_gamma = nullptr;
  float rla_eps = 0.f;
  int32_t score_form = SPLA_SCORE_TAYLOR;  // block score the selection ranks
  // workspace layout (bytes)
  size_t off_lg = 0, off_sel = 0, off_page = 0, off_part = 0, off_phdr = 0, off_obar = 0, off_dz = 0, off_phq = 0;
  size_t ws_bytes = 0;
};

// offsets (bytes) of the per-query decode scratch in a workspace sized for nq
// queries: the handle's own workspace (nq = batch) or a prefill workspace
// (nq = virtual queries of one chunk)
struct WsLayout {
  size_t lg, sel, page, part, phdr, obar, dz, phq, bytes;
};

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

WsLayout ws_layout(const spla_config& c, int n_tiles, size_t nq) {
  const size_t H = c.n_q_heads, G = c.n_kv_heads, d = c.head_dim, k = c.top_k;
  WsLayout w;
  // error word + spare, then the counters of the one-kernel step at the same
  // offset in every layout (each call leaves them at zero)
  size_t off = kStepCtrOffset + (size_t)kStepPairs * kStepCtrStride * sizeof(int32_t);
  w.lg = off;
  off = align256(off + nq * G * (size_t)n_tiles * kTile * sizeof(float));
  w.sel = off;
  off = align256(off + nq * G * k * sizeof(int32_t));
  w.page = off;
  off = align256(off + nq * G * k * sizeof(int32_t));
  w.part = off;
  off = align256(off + nq * H * k * 2 * d * sizeof(float));
  w.phdr = off;
  off = align256(off + nq * H * k * kPartHdr * sizeof(float));
  const size_t chunks = d * d / 1024;  // S_all row chunks per (query, KV head)
  w.obar = off;
  off = align256(off + nq * G * chunks * (H / G) * d * sizeof(float));
  w.dz = off;
  off = align256(off + nq * G * chunks * (H / G) * sizeof(float));
  w.phq = off;
  off = align256(off + nq * H * 2 * d * sizeof(uint16_t));
  w.bytes = off;
  return w;
}

// a prefill workspace for groups of `chunk` tokens: the per-query scratch of
// ws_layout, then the block-centric attend's per-block lists and work items
struct PfLayout {
  WsLayout q;
  size_t cnt, lists, items, n_items, bytes;
  int32_t max_items;
};

PfLayout pf_layout(const spla_config& c, int n_tiles, int chunk) {
  PfLayout p;
  p.q = ws_layout(c, n_tiles, chunk);
  const size_t G = c.n_kv_heads, MB = c.max_blocks_per_seq, k = c.top_k;
  const size_t pairs = (size_t)chunk * k;  // (query, slot) pairs per KV head
  p.max_items = (int32_t)(G * ((pairs + kPfQ - 1) / kPfQ + (pairs < MB ? pairs : MB)));
  size_t off = p.q.bytes;
  p.cnt = off;
  off = align256(off + G * MB * sizeof(int32_t));
  p.lists = off;
  off = align256(off + G * MB * (size_t)chunk * sizeof(int32_t));
  p.items = off;
  off = align256(off + (size_t)p.max_items * kPfItemInts * sizeof(int32_t));
  p.n_items = off;
  off = align256(off + sizeof(int32_t));
  p.bytes = off;
  return p;
}

void layout(spla_handle* h) {
  const WsLayout w = ws_layout(h->cfg, h->n_tiles, h->cfg.batch);
  h->off_lg = w.lg;
  h->off_sel = w.sel;
  h->off_page = w.page;
  h->off_part = w.part;
  h->off_phdr = w.phdr;
  h->off_obar = w.obar;
  h->off_dz = w.dz;
  h->off_phq = w.phq;
  h->ws_bytes = w.bytes;
}

template <typename T>
T* ws_ptr(const spla_handle* h, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(h->buf.workspace) + off);
}

// base of the per-call scratch (score rows, selections, partial records,
// o_bar partials, phi(q)) of a decode: the bound workspace, or the static
// scratch of spla_decode_step_noalloc.  The sticky error word always stays in
// bytes [0, 4) of the bound workspace, where callers read it.
void fill_decode_args(const spla_handle* h, const void* q, const float* gate, float* out,
                      const spla_decode_aux* aux, DecodeArgs* a, char* scratch_base);

spla_status fill_decode_args(const spla_handle* h, const void* q, const float* gate, float* out,
                             const spla_decode_aux* aux, DecodeArgs* a) {
  fill_decode_args(h, q, gate, out, aux, a, static_cast<char*>(h->buf.workspace));
  return SPLA_OK;
}

void fill_decode_args(const spla_handle* h, const void* q, const float* gate, float* out,
                      const spla_decode_aux* aux, DecodeArgs* a, char* scratch_base) {
  const spla_config& c = h->cfg;
  memset(a, 0, sizeof(*a));
  a->q = q;
  a->gate = gate;
  a->out = out;
  a->k_pages = h->buf.k_pages;
  a->v_pages = h->buf.v_pages;
  a->block_table = h->buf.block_table;
  a->blk_mean = h->buf.blk_mean;
  a->blk_var = h->buf.blk_var;
  a->s_all = h->buf.s_all;
  a->z_all = h->buf.z_all;
  a->lg = reinterpret_cast<float*>(scratch_base + h->off_lg);
  a->sel = reinterpret_cast<int32_t*>(scratch_base + h->off_sel);
  a->sel_page = reinterpret_cast<int32_t*>(scratch_base + h->off_page);
  a->part = reinterpret_cast<float*>(scratch_base + h->off_part);
  a->part_hdr = reinterpret_cast<float*>(scratch_base + h->off_phdr);
  a->obar_part = reinterpret_cast<float*>(scratch_base + h->off_obar);
  a->dz_part = reinterpret_cast<float*>(scratch_base + h->off_dz);
  a->phq = reinterpret_cast<uint16_t*>(scratch_base + h->off_phq);
  a->step_ctr = reinterpret_cast<int32_t*>(scratch_base + kStepCtrOffset);
  a->err = ws_ptr<uint32_t>(h, 0);
  if (aux) {
    a->sel_in = aux->sel_in;
    a->sel_out = aux->sel_idx;
    a->lg_out = aux->lg;
    a->o_sparse_out = aux->o_sparse;
    a->o_rla_out = aux->o_rla;
    a->d_rla_out = aux->d_rla;
  }
  a->rla_form = h->rla_form;
  a->rla_gamma = h->rla_gamma;
  a->rla_eps = h->rla_eps;
  a->score_form = h->score_form;
  a->B = c.batch;
  a->H = c.n_q_heads;
  a->G = c.n_kv_heads;
  a->d = c.head_dim;
  a->r = h->r;
  a->bk = c.block_size;
  a->top_k = c.top_k;
  a->max_blocks = c.max_blocks_per_seq;
  a->num_pages = c.num_pages;
  a->n_tiles = h->n_tiles;
  a->inv_sqrt_d = (float)(1.0 / sqrt((double)c.head_dim));
  int max_tiles = 0, min_tiles = 1 << 30;
  for (int b = 0; b < c.batch; ++b) {
    a->lens[b] = h->lens[b];
    const int nb = (h->lens[b] + c.block_size - 1) / c.block_size;
    const int tiles = nb > c.top_k ? (nb - 2) / kTile + 1 : 0;  // tiles holding candidates 1..nb-2
    if (tiles > max_tiles) max_tiles = tiles;
    if (tiles < min_tiles) min_tiles = tiles;
  }
  a->score_tiles = max_tiles;
  a->tiles_all = min_tiles;
}

void fill_state_refs(const spla_handle* h, const void* k_new, const void* v_new, StateRefs* st) {
  const spla_config& c = h->cfg;
  st->k_new = k_new;
  st->v_new = v_new;
  st->k_pages = h->buf.k_pages;
  st->v_pages = h->buf.v_pages;
  st->block_table = h->buf.block_table;
  st->blk_mean = h->buf.blk_mean;
  st->blk_var = h->buf.blk_var;
  st->s_all = h->buf.s_all;
  st->z_all = h->buf.z_all;
  st->err = ws_ptr<uint32_t>(h, 0);
  st->G = c.n_kv_heads;
  st->d = c.head_dim;
  st->bk = c.block_size;
  st->max_blocks = c.max_blocks_per_seq;
  st->num_pages = c.num_pages;
  st->n_tiles = h->n_tiles;
}

// validation shared by spla_decode and spla_decode_step
spla_status check_decode_args(const spla_handle* h, const void* q, const float* gate, float* out,
                              const spla_decode_aux* aux) {
  if (!q || !gate || !out) return SPLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(gate) || !aligned16(out)) return SPLA_ERR_ALIGNMENT;
  if (aux) {
    const void* ap[] = {aux->sel_idx, aux->lg, aux->o_sparse, aux->o_rla, aux->d_rla, aux->sel_in};
    for (const void* p : ap)
      if (p && !aligned16(p)) return SPLA_ERR_ALIGNMENT;
    if (aux->kernel_events && aux->n_kernel_events < 0) return SPLA_ERR_INVALID_ARG;
  }
  (void)h;
  return SPLA_OK;
}

// launch descriptors of the kernels of one call, in launch order: the i-th
// kernel carries kernel_events[2i] / [2i+1] as its begin / end events
struct LaunchSeq {
  hipStream_t st = nullptr;
  void* const* ev = nullptr;
  int nev = 0, k = 0;
  LaunchSeq(hipStream_t s, const spla_decode_aux* aux) : st(s) {
    if (aux && aux->kernel_events) {
      ev = aux->kernel_events;
      nev = aux->n_kernel_events;
    }
  }
  Launch next() {
    Launch l;
    l.s = st;
    if (k < nev) {
      l.start = reinterpret_cast<hipEvent_t>(ev[2 * k]);
      l.stop = reinterpret_cast<hipEvent_t>(ev[2 * k + 1]);
    }
    ++k;
    return l;
  }
};

// record a failed launch on the handle
spla_status hip_fail(spla_handle* h, hipError_t e) {
  h->last_hip = e;
  return SPLA_ERR_HIP;
}

// (sequence, KV head) pairs up to which the automatic choice fuses the
// selector into the attend kernel: there the decode is a chain of latency-
// bound launches and removing one pays for the selection being recomputed
// by every attend workgroup
constexpr int kAutoFusedPairs = 64;

bool use_fused_select(const spla_handle* h, const DecodeArgs& a, bool bf16) {
  if (h->fused_select == 0 || !select_attend_supported(a, bf16)) return false;
  return h->fused_select == 1 || a.B * a.G <= kAutoFusedPairs;
}

// the fused select + attend also merges the records (no combine kernel), on
// request: at B = 1, 128K context, GQA 32/8 the kernel then takes 13.1 us
// against 9.4 + 4.0 us with the combine kernel, and the step 20.7 against
// 20.5 us (its merge workgroups see the attends done about as late as the
// next kernel would start)
bool use_fused_merge(const spla_handle* h, const DecodeArgs& a) {
  return h->fused_merge == 1 && select_attend_merge_supported(a);
}

// the one-kernel step: on request, where the fused select + attend applies
// (automatic keeps the separate kernels: at B = 1, 128K context, GQA 32/8 it
// takes 16.2 us against 5.7 + 9.3 us for the two kernels it replaces, since
// its attend workgroups run the same dependent chain after the scores)
bool use_step_fused(const spla_handle* h, const DecodeArgs& a, bool bf16) {
  return h->step_kernel == 1 && use_fused_select(h, a, bf16) && step_fused_supported(a, bf16);
}

// the kernels one call launches, in order (SPLA_KERNEL_*); the single source
// of truth for both the launches and spla_launch_plan
int decode_plan(const spla_handle* h, const DecodeArgs& a, int32_t call, int32_t* k) {
  const bool bf16 = h->cfg.kv_dtype == SPLA_BF16;
  int n = 0;
  if (call == SPLA_CALL_DECODE_STEP && use_step_fused(h, a, bf16)) {
    k[n++] = SPLA_KERNEL_STEP_FUSED;
    k[n++] = SPLA_KERNEL_COMBINE;
    return n;
  }
  // the first kernel also forms the phi(q)^T S_all partials the combine needs,
  // so it runs even when there is nothing to score
  k[n++] = call == SPLA_CALL_DECODE_STEP ? SPLA_KERNEL_STEP_SCORE : SPLA_KERNEL_SCORE;
  if (call == SPLA_CALL_DECODE_SEL_IN) {
    k[n++] = SPLA_KERNEL_ATTEND;
  } else if (use_fused_select(h, a, bf16)) {
    k[n++] = SPLA_KERNEL_SELECT_ATTEND;
    if (use_fused_merge(h, a)) return n;  // it merges the records itself
  } else {
    k[n++] = SPLA_KERNEL_SELECT;
    k[n++] = SPLA_KERNEL_ATTEND;
  }
  k[n++] = SPLA_KERNEL_COMBINE;
  return n;
}

constexpr int kMaxPlan = 4;

// launch a plan; sa.dec are the decode arguments, sa.st the state (with the
// step's k / v for spla_decode_step)
hipError_t run_plan(const spla_handle* h, const StepArgs& sa, const int32_t* plan, int n, LaunchSeq& ls) {
  const bool bf16 = h->cfg.kv_dtype == SPLA_BF16;
  const DecodeArgs& a = sa.dec;
  // a fused select + attend without a combine after it merges the records
  bool merge = true;
  for (int i = 0; i < n; ++i) merge = merge && plan[i] != SPLA_KERNEL_COMBINE;
  for (int i = 0; i < n; ++i) {
    const Launch l = ls.next();
    hipError_t e = hipErrorInvalidValue;
    switch (plan[i]) {
      case SPLA_KERNEL_SCORE: e = launch_score(sa, bf16, l); break;
      case SPLA_KERNEL_STEP_SCORE: e = launch_step_score(sa, bf16, l); break;
      case SPLA_KERNEL_SELECT: e = launch_select(a, l); break;
      case SPLA_KERNEL_ATTEND: e = launch_attend(a, bf16, l); break;
      case SPLA_KERNEL_SELECT_ATTEND: e = launch_select_attend(a, l, merge); break;
      case SPLA_KERNEL_STEP_FUSED: e = launch_step_fused(sa, l); break;
      case SPLA_KERNEL_COMBINE: e = launch_combine(a, l); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// the lengths the decode part of a step sees: after its one-token append
void fill_step_args(spla_handle* h, const void* k_new, const void* v_new, const void* q, const float* gate,
                    float* out, const spla_decode_aux* aux, StepArgs* a, char* scratch_base = nullptr) {
  const spla_config& c = h->cfg;
  memset(a, 0, sizeof(*a));
  for (int b = 0; b < c.batch; ++b) h->lens[b] += 1;
  fill_decode_args(h, q, gate, out, aux, &a->dec,
                   scratch_base ? scratch_base : static_cast<char*>(h->buf.workspace));
  fill_state_refs(h, k_new, v_new, &a->st);
  for (int b = 0; b < c.batch; ++b) h->lens[b] -= 1;
}

// ------------------------------------------------ static scratch (no-alloc)
// The per-call scratch of spla_decode_step_noalloc: one array per GPU that
// the library runs on, held until the process ends.  Host code never uses
// the array's name as an address (on the host it is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = size_t(SPLA_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of the scratch on the device that runs `stream` (the
// current device for the null stream), looked up with that device current
hipError_t noalloc_scratch(hipStream_t stream, char** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream) {
    hipDevice_t sd = 0;
    if ((e = hipStreamGetDevice(stream, &sd)) != hipSuccess) return e;
    dev = sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* spla_status_str(spla_status st) {
  switch (st) {
    case SPLA_OK: return "ok";
    case SPLA_ERR_INVALID_ARG: return "invalid argument";
    case SPLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SPLA_ERR_CAPACITY: return "capacity exceeded";
    case SPLA_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case SPLA_ERR_HIP: return "HIP launch failed";
    case SPLA_ERR_STATE: return "handle not bound";
    case SPLA_ERR_SCRATCH: return "per-call scratch larger than the library's static scratch";
  }
  return "unknown status";
}

int32_t spla_abi_version(void) { return SPLA_ABI_VERSION; }

int32_t spla_last_hip_error(const spla_handle* h, const char** name) {
  const hipError_t e = h ? h->last_hip : hipSuccess;
  if (name) *name = hipGetErrorName(e);
  return (int32_t)e;
}

spla_status spla_create(const spla_config* cfg, spla_handle** out) {
  if (!cfg || !out) return SPLA_ERR_INVALID_ARG;
  *out = nullptr;
  const spla_config& c = *cfg;
  if (c.batch < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.head_dim < 1 || c.block_size < 1 ||
      c.top_k < 1 || c.max_blocks_per_seq < 1 || c.num_pages < 1)
    return SPLA_ERR_INVALID_ARG;
  if (c.batch > kMaxBatch) return SPLA_ERR_UNSUPPORTED;
  if (c.head_dim != 64 && c.head_dim != 128) return SPLA_ERR_UNSUPPORTED;
  if (c.block_size != 64 && c.block_size != 128) return SPLA_ERR_UNSUPPORTED;
  if (c.n_q_heads % c.n_kv_heads) return SPLA_ERR_UNSUPPORTED;
  const int r = c.n_q_heads / c.n_kv_heads;
  if (r != 1 && r != 2 && r != 4 && r != 8) return SPLA_ERR_UNSUPPORTED;
  if (c.top_k < 2 || c.top_k > 256) return SPLA_ERR_UNSUPPORTED;
  if (c.max_blocks_per_seq > kMaxBlocksPerSeq) return SPLA_ERR_UNSUPPORTED;
  if (c.kv_dtype != SPLA_F32 && c.kv_dtype != SPLA_BF16) return SPLA_ERR_UNSUPPORTED;
  spla_handle* h = new (std::nothrow) spla_handle();
  if (!h) return SPLA_ERR_INVALID_ARG;
  h->cfg = c;
  h->r = r;
  h->n_tiles = (c.max_blocks_per_seq + kTile - 1) / kTile;
  h->lens.assign(c.batch, 0);
  layout(h);
  *out = h;
  return SPLA_OK;
}

void spla_destroy(spla_handle* h) { delete h; }

size_t spla_workspace_bytes(const spla_handle* h) { return h ? h->ws_bytes : 0; }

size_t spla_stats_floats(const spla_handle* h) {
  if (!h) return 0;
  const spla_config& c = h->cfg;
  return (size_t)c.batch * c.n_kv_heads * h->n_tiles * kTile * c.head_dim;
}

spla_status spla_bind(spla_handle* h, const spla_buffers* b, const int32_t* lens_host) {
  if (!h || !b) return SPLA_ERR_INVALID_ARG;
  const void* ptrs[] = {b->k_pages, b->v_pages, b->block_table, b->blk_mean, b->blk_var,
                        b->s_all, b->z_all, b->workspace};
  for (const void* p : ptrs)
    if (!p) return SPLA_ERR_INVALID_ARG;
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPLA_ERR_ALIGNMENT;
  if (b->workspace_bytes < h->ws_bytes) return SPLA_ERR_INVALID_ARG;
  const spla_config& c = h->cfg;
  const int64_t cap = (int64_t)c.max_blocks_per_seq * c.block_size;
  if (lens_host) {
    for (int i = 0; i < c.batch; ++i)
      if (lens_host[i] < 0 || lens_host[i] > cap) return SPLA_ERR_INVALID_ARG;
  }
  h->buf = *b;
  for (int i = 0; i < c.batch; ++i) h->lens[i] = lens_host ? lens_host[i] : 0;
  h->bound = true;
  return SPLA_OK;
}

spla_status spla_get_lens(const spla_handle* h, int32_t* lens_host) {
  if (!h || !lens_host) return SPLA_ERR_INVALID_ARG;
  for (int i = 0; i < h->cfg.batch; ++i) lens_host[i] = h->lens[i];
  return SPLA_OK;
}

spla_status spla_append_kv(spla_handle* h, int32_t n_seqs, const int32_t* seq_ids_host,
                           const int32_t* n_new_host, const void* k_new, const void* v_new,
                           void* stream) {
  if (!h) return SPLA_ERR_INVALID_ARG;
  if (!h->bound) return SPLA_ERR_STATE;
  const spla_config& c = h->cfg;
  if (n_seqs < 0 || n_seqs > c.batch) return SPLA_ERR_INVALID_ARG;
  if (n_seqs == 0) return SPLA_OK;
  if (!seq_ids_host || !n_new_host) return SPLA_ERR_INVALID_ARG;
  const int64_t cap = (int64_t)c.max_blocks_per_seq * c.block_size;
  std::vector<char> seen(c.batch, 0);
  int64_t total = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int s = seq_ids_host[i];
    if (s < 0 || s >= c.batch || seen[s]) return SPLA_ERR_INVALID_ARG;
    seen[s] = 1;
    if (n_new_host[i] < 0) return SPLA_ERR_INVALID_ARG;
    total += n_new_host[i];
  }
  for (int i = 0; i < n_seqs; ++i)
    if ((int64_t)h->lens[seq_ids_host[i]] + n_new_host[i] > cap) return SPLA_ERR_CAPACITY;
  if (total == 0) return SPLA_OK;
  if (total > (int64_t)INT32_MAX / (c.n_kv_heads * c.head_dim)) return SPLA_ERR_INVALID_ARG;
  if (!k_new || !v_new) return SPLA_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return SPLA_ERR_ALIGNMENT;

  const bool bf16 = c.kv_dtype == SPLA_BF16;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  AppendArgs a;
  memset(&a, 0, sizeof(a));
  fill_state_refs(h, k_new, v_new, &a.st);
  const size_t es = bf16 ? 2 : 4;
  const size_t row_bytes = (size_t)c.n_kv_heads * c.head_dim * es;
  int64_t row = 0;
  // launches of at most kMaxAppendEntries entries; the rows of one launch
  // start at its first entry's row
  for (int i0 = 0; i0 < n_seqs; i0 += kMaxAppendEntries) {
    const int ne = n_seqs - i0 < kMaxAppendEntries ? n_seqs - i0 : kMaxAppendEntries;
    a.st.k_new = static_cast<const char*>(k_new) + row * row_bytes;
    a.st.v_new = static_cast<const char*>(v_new) + row * row_bytes;
    a.n_entries = ne;
    a.page_tok = append_page_tokens(c.n_kv_heads, c.head_dim, bf16);
    int lrow = 0, pp = 0, sp = 0;
    for (int e = 0; e < ne; ++e) {
      const int s = seq_ids_host[i0 + e];
      const int n = n_new_host[i0 + e];
      const int t0 = h->lens[s];
      a.e[e].seq = s;
      a.e[e].n = n;
      a.e[e].t0 = t0;
      a.e[e].row = lrow;
      a.page_prefix[e] = pp;
      a.stat_prefix[e] = sp;
      pp += (n + a.page_tok - 1) / a.page_tok;
      sp += ((t0 + n) / c.block_size - t0 / c.block_size) * c.n_kv_heads;
      lrow += n;
    }
    a.page_prefix[ne] = pp;
    a.stat_prefix[ne] = sp;
    a.page_items = pp;
    a.stat_items = sp;
    hipError_t e = launch_append(a, bf16, Launch{st, nullptr, nullptr});
    if (e == hipSuccess) e = launch_state_add(a, bf16, Launch{st, nullptr, nullptr});
    if (e != hipSuccess) return hip_fail(h, e);
    row += lrow;
  }
  for (int i = 0; i < n_seqs; ++i) h->lens[seq_ids_host[i]] += n_new_host[i];
  return SPLA_OK;
}

spla_status spla_decode(spla_handle* h, const void* q, const float* gate, float* out,
                        const spla_decode_aux* aux, void* stream) {
  if (!h) return SPLA_ERR_INVALID_ARG;
  if (!h->bound) return SPLA_ERR_STATE;
  const spla_status vs = check_decode_args(h, q, gate, out, aux);
  if (vs != SPLA_OK) return vs;
  const spla_config& c = h->cfg;
  for (int b = 0; b < c.batch; ++b)
    if (h->lens[b] <= 0) return SPLA_ERR_INVALID_ARG;
  StepArgs sa;
  memset(&sa, 0, sizeof(sa));
  fill_decode_args(h, q, gate, out, aux, &sa.dec);
  fill_state_refs(h, nullptr, nullptr, &sa.st);
  int32_t plan[kMaxPlan];
  const int n = decode_plan(h, sa.dec, sa.dec.sel_in ? SPLA_CALL_DECODE_SEL_IN : SPLA_CALL_DECODE, plan);
  LaunchSeq ls(reinterpret_cast<hipStream_t>(stream), aux);
  const hipError_t e = run_plan(h, sa, plan, n, ls);
  return e == hipSuccess ? SPLA_OK : hip_fail(h, e);
}

spla_status spla_decode_step(spla_handle* h, const void* k_new, const void* v_new, const void* q, const float* gate,
                             float* out, const spla_decode_aux* aux, void* stream) {
  if (!h) return SPLA_ERR_INVALID_ARG;
  if (!h->bound) return SPLA_ERR_STATE;
  const spla_status vs = check_decode_args(h, q, gate, out, aux);
  if (vs != SPLA_OK) return vs;
  if (aux && aux->sel_in) return SPLA_ERR_INVALID_ARG;
  if (!k_new || !v_new) return SPLA_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return SPLA_ERR_ALIGNMENT;
  const spla_config& c = h->cfg;
  const int64_t cap = (int64_t)c.max_blocks_per_seq * c.block_size;
  for (int b = 0; b < c.batch; ++b)
    if ((int64_t)h->lens[b] + 1 > cap) return SPLA_ERR_CAPACITY;
  StepArgs a;
  fill_step_args(h, k_new, v_new, q, gate, out, aux, &a);
  int32_t plan[kMaxPlan];
  const int n = decode_plan(h, a.dec, SPLA_CALL_DECODE_STEP, plan);
  LaunchSeq ls(reinterpret_cast<hipStream_t>(stream), aux);
  const hipError_t e = run_plan(h, a, plan, n, ls);
  // the mirror advances once the append is enqueued (the first kernel)
  if (e != hipSuccess && ls.k <= 1) return hip_fail(h, e);
  for (int b = 0; b < c.batch; ++b) h->lens[b] += 1;
  return e == hipSuccess ? SPLA_OK : hip_fail(h, e);
}

spla_status spla_decode_step_noalloc(spla_handle* h, const void* k_new, const void* v_new, const void* q,
                                     const float* gate, float* out, const spla_decode_aux* aux, void* stream) {
  if (!h) return SPLA_ERR_INVALID_ARG;
  if (!h->bound) return SPLA_ERR_STATE;
  const spla_status vs = check_decode_args(h, q, gate, out, aux);
  if (vs != SPLA_OK) return vs;
  if (aux && aux->sel_in) return SPLA_ERR_INVALID_ARG;
  if (!k_new || !v_new) return SPLA_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return SPLA_ERR_ALIGNMENT;
  const spla_config& c = h->cfg;
  const int64_t cap = (int64_t)c.max_blocks_per_seq * c.block_size;
  for (int b = 0; b < c.batch; ++b)
    if ((int64_t)h->lens[b] + 1 > cap) return SPLA_ERR_CAPACITY;
  if (h->ws_bytes > kNoAllocScratchBytes) return SPLA_ERR_SCRATCH;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* base = nullptr;
  const hipError_t es = noalloc_scratch(st, &base);
  if (es != hipSuccess) return hip_fail(h, es);
  StepArgs a;
  fill_step_args(h, k_new, v_new, q, gate, out, aux, &a, base);
  int32_t plan[kMaxPlan];
  const int n = decode_plan(h, a.dec, SPLA_CALL_DECODE_STEP, plan);
  LaunchSeq ls(st, aux);
  const hipError_t e = run_plan(h, a, plan, n, ls);
  if (e != hipSuccess && ls.k <= 1) return hip_fail(h, e);
  for (int b = 0; b < c.batch; ++b) h->lens[b] += 1;
  return e == hipSuccess ? SPLA_OK : hip_fail(h, e);
}

spla_status spla_set_tuning(spla_handle* h, int32_t key, int32_t value) {
  if (!h) return SPLA_ERR_INVALID_ARG;
  switch (key) {
    case SPLA_TUNE_FUSED_SELECT:
      if (value < -1 || value > 1) return SPLA_ERR_INVALID_ARG;
      h->fused_select = value;
      return SPLA_OK;
    case SPLA_TUNE_STEP_KERNEL:
      if (value < -1 || value > 1) return SPLA_ERR_INVALID_ARG;
      h->step_kernel = value;
      return SPLA_OK;
    case SPLA_TUNE_FUSED_MERGE:
      if (value < -1 || value > 1) return SPLA_ERR_INVALID_ARG;
      h->fused_merge = value;
      return SPLA_OK;
  }
  return SPLA_ERR_INVALID_ARG;
}

size_t spla_prefill_workspace_bytes(const spla_handle* h, int32_t chunk) {
  if (!h || chunk < 1 || chunk > kMaxBatch) return 0;
  return pf_layout(h->cfg, h->n_tiles, chunk).bytes;
}

spla_status spla_prefill(spla_handle* h, int32_t seq, int32_t n, const void* k_new, const void* v_new, const void* q,
                         const float* gate, float* out, int32_t* sel_idx, float* lg, void* workspace,
                         size_t workspace_bytes,
                         void* stream) {
  if (!h) return SPLA_ERR_INVALID_ARG;
  if (!h->bound) return SPLA_ERR_STATE;
  const spla_config& c = h->cfg;
  if (seq < 0 || seq >= c.batch || n < 0) return SPLA_ERR_INVALID_ARG;
  if (n == 0) return SPLA_OK;
  if (!k_new || !v_new || !q || !gate || !out || !workspace) return SPLA_ERR_INVALID_ARG;
  const void* ptrs[] = {k_new, v_new, q, gate, out, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPLA_ERR_ALIGNMENT;
  if ((sel_idx && !aligned16(sel_idx)) || (lg && !aligned16(lg))) return SPLA_ERR_ALIGNMENT;
  if ((int64_t)h->lens[seq] + n > (int64_t)c.max_blocks_per_seq * c.block_size) return SPLA_ERR_CAPACITY;
  if ((int64_t)n > (int64_t)INT32_MAX / (c.n_q_heads * c.head_dim)) return SPLA_ERR_INVALID_ARG;
  int chunk = kMaxBatch;  // virtual queries per launch: the most the workspace holds
  while (chunk > 0 && pf_layout(c, h->n_tiles, chunk).bytes > workspace_bytes) --chunk;
  if (chunk == 0) return SPLA_ERR_INVALID_ARG;
  const PfLayout pl = pf_layout(c, h->n_tiles, chunk);
  const WsLayout& wl = pl.q;
  const bool bf16 = c.kv_dtype == SPLA_BF16;
  const size_t es = bf16 ? 2 : 4;
  const size_t G = c.n_kv_heads, H = c.n_q_heads, d = c.head_dim;
  const size_t stats_row = G * (size_t)h->n_tiles * kTile * d;  // floats of one sequence's statistics
  const Launch l{reinterpret_cast<hipStream_t>(stream), nullptr, nullptr};
  char* wsb = static_cast<char*>(workspace);
  PfBuffers pb;
  pb.cnt = reinterpret_cast<int32_t*>(wsb + pl.cnt);
  pb.lists = reinterpret_cast<int32_t*>(wsb + pl.lists);
  pb.items = reinterpret_cast<int4*>(wsb + pl.items);
  pb.n_items = reinterpret_cast<int32_t*>(wsb + pl.n_items);
  pb.cap = chunk;
  pb.max_items = pl.max_items;
  if (bf16) {
    const hipError_t e = launch_pf_clear(pb, c.n_kv_heads, c.max_blocks_per_seq, l);
    if (e != hipSuccess) return hip_fail(h, e);
  }
  for (int c0 = 0; c0 < n; c0 += chunk) {
    const int m = n - c0 < chunk ? n - c0 : chunk;
    const int t0 = h->lens[seq];
    const char* kc = static_cast<const char*>(k_new) + (size_t)c0 * G * d * es;
    const char* vc = static_cast<const char*>(v_new) + (size_t)c0 * G * d * es;
    // (1) the chunk's pages and the statistics of the blocks it completes
    AppendArgs ap;
    memset(&ap, 0, sizeof(ap));
    fill_state_refs(h, kc, vc, &ap.st);
    ap.n_entries = 1;
    ap.e[0] = AppendEntry{seq, m, t0, 0};
    ap.page_prefix[0] = ap.stat_prefix[0] = 0;
    ap.page_tok = append_page_tokens(c.n_kv_heads, c.head_dim, bf16);
    ap.page_items = ap.page_prefix[1] = (m + ap.page_tok - 1) / ap.page_tok;
    ap.stat_items = ap.stat_prefix[1] = ((t0 + m) / c.block_size - t0 / c.block_size) * c.n_kv_heads;
    hipError_t e = launch_append(ap, bf16, l);
    if (e != hipSuccess) return hip_fail(h, e);
    // (2) every token of the chunk decoded as a virtual query of this
    // sequence, against the state before the chunk
    DecodeArgs a;
    fill_decode_args(h, static_cast<const char*>(q) + (size_t)c0 * H * d * es, gate, out + (size_t)c0 * H * d,
                     nullptr, &a);
    a.B = m;
    a.virtual_queries = 1;
    a.sel_out = sel_idx ? sel_idx + (size_t)c0 * G * c.top_k : nullptr;
    a.lg_out = lg ? lg + (size_t)c0 * G * c.max_blocks_per_seq : nullptr;
    a.block_table = h->buf.block_table + (size_t)seq * c.max_blocks_per_seq;
    a.blk_mean = h->buf.blk_mean + (size_t)seq * stats_row;
    a.blk_var = h->buf.blk_var + (size_t)seq * stats_row;
    a.s_all = h->buf.s_all + (size_t)seq * G * d * d;
    a.z_all = h->buf.z_all + (size_t)seq * G * d;
    a.lg = reinterpret_cast<float*>(wsb + wl.lg);
    a.sel = reinterpret_cast<int32_t*>(wsb + wl.sel);
    a.sel_page = reinterpret_cast<int32_t*>(wsb + wl.page);
    a.part = reinterpret_cast<float*>(wsb + wl.part);
    a.part_hdr = reinterpret_cast<float*>(wsb + wl.phdr);
    a.obar_part = reinterpret_cast<float*>(wsb + wl.obar);
    a.dz_part = reinterpret_cast<float*>(wsb + wl.dz);
    a.phq = reinterpret_cast<uint16_t*>(wsb + wl.phq);
    int max_tiles = 0, min_tiles = 1 << 30;
    for (int i = 0; i < m; ++i) {
      a.lens[i] = t0 + i + 1;
      const int nb = (a.lens[i] + c.block_size - 1) / c.block_size;
      const int tiles = nb > c.top_k ? (nb - 2) / kTile + 1 : 0;
      if (tiles > max_tiles) max_tiles = tiles;
      if (tiles < min_tiles) min_tiles = tiles;
    }
    a.score_tiles = max_tiles;
    a.tiles_all = min_tiles;
    // the group's block scores, then phi(q_t)^T S_t and phi(q_t).z_t in one
    // partial per head (state before the group plus its own tokens up to t)
    // and phi(q), all on the matrix cores
    if (a.score_tiles > 0 && (e = launch_pf_score(a, bf16, l)) != hipSuccess) return hip_fail(h, e);
    if ((e = launch_pf_state(a, bf16, kc, vc, l)) != hipSuccess) return hip_fail(h, e);
    a.obar_one = 1;
    if ((e = launch_select(a, l)) != hipSuccess) return hip_fail(h, e);
    // bf16: every selected block read once per item of up to kPfQ queries
    if ((e = bf16 ? launch_pf_attend(a, pb, l) : launch_attend(a, bf16, l)) != hipSuccess) return hip_fail(h, e);
    if ((e = launch_combine(a, l)) != hipSuccess) return hip_fail(h, e);
    // (3) the chunk's tokens into S_all / z_all: phi(K)^T V on the matrix cores
    AppendArgs as;
    memset(&as, 0, sizeof(as));
    fill_state_refs(h, kc, vc, &as.st);
    as.n_entries = 1;
    as.e[0] = AppendEntry{seq, m, t0, 0};
    if ((e = launch_state_add(as, bf16, l)) != hipSuccess) return hip_fail(h, e);
    h->lens[seq] = t0 + m;
  }
  return SPLA_OK;
}

spla_status spla_set_score_form(spla_handle* h, int32_t form) {
  if (!h || (form != SPLA_SCORE_TAYLOR && form != SPLA_SCORE_MEAN)) return SPLA_ERR_INVALID_ARG;
  h->score_form = form;
  return SPLA_OK;
}

spla_status spla_block_mass(spla_handle* h, const void* q, float* lgx, void* stream) {
  if (!h) return SPLA_ERR_INVALID_ARG;
  if (!h->bound) return SPLA_ERR_STATE;
  if (!q || !lgx) return SPLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(lgx)) return SPLA_ERR_ALIGNMENT;
  const spla_config& c = h->cfg;
  for (int b = 0; b < c.batch; ++b)
    if (h->lens[b] <= 0) return SPLA_ERR_INVALID_ARG;
  DecodeArgs a;
  fill_decode_args(h, q, nullptr, nullptr, nullptr, &a);
  int max_cand = 0;
  for (int b = 0; b < c.batch; ++b) {
    const int nb = (h->lens[b] + c.block_size - 1) / c.block_size;
    if (nb - 2 > max_cand) max_cand = nb - 2;
  }
  if (max_cand == 0) return SPLA_OK;
  const hipError_t e = launch_block_mass(a, c.kv_dtype == SPLA_BF16, lgx, max_cand,
                                         Launch{reinterpret_cast<hipStream_t>(stream), nullptr, nullptr});
  return e == hipSuccess ? SPLA_OK : hip_fail(h, e);
}

spla_status spla_set_rla_output(spla_handle* h, int32_t form, const float* gamma, float eps) {
  if (!h) return SPLA_ERR_INVALID_ARG;
  switch (form) {
    case SPLA_RLA_PLAIN:
    case SPLA_RLA_NORMALIZED:
      h->rla_form = form;
      h->rla_gamma = nullptr;
      h->rla_eps = 0.f;
      return SPLA_OK;
    case SPLA_RLA_RMSNORM:
      if (!gamma || !(eps > 0.f) || !isfinite(eps)) return SPLA_ERR_INVALID_ARG;
      if (!aligned16(gamma)) return SPLA_ERR_ALIGNMENT;
      h->rla_form = form;
      h->rla_gamma = gamma;
      h->rla_eps = eps;
      return SPLA_OK;
  }
  return SPLA_ERR_INVALID_ARG;
}

int32_t spla_launch_plan(const spla_handle* h, int32_t call, int32_t* kernels, int32_t cap) {
  if (!h || call < SPLA_CALL_DECODE || call > SPLA_CALL_DECODE_STEP) return -1;
  spla_handle* hh = const_cast<spla_handle*>(h);  // lengths are restored before returning
  int32_t plan[kMaxPlan];
  int n;
  if (call == SPLA_CALL_DECODE_STEP) {
    StepArgs a;
    fill_step_args(hh, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, &a);
    n = decode_plan(h, a.dec, call, plan);
  } else {
    DecodeArgs a;
    fill_decode_args(h, nullptr, nullptr, nullptr, nullptr, &a);
    n = decode_plan(h, a, call, plan);
  }
  for (int i = 0; i < n && i < cap; ++i)
    if (kernels) kernels[i] = plan[i];
  return n;
}

}  // extern "C"
