/*
 * spla.h -- C ABI of the SPLA (Block Sparse Plus Linear Attention) decode
 * step on one AMD Instinct MI355X (gfx950).
 *
 * Method (arXiv 2601.22379, "SPLA: Block Sparse Plus Linear Attention for
 * Long Context Modeling"; gist.science Technical Summary):
 *   - every KV block keeps first/second order key statistics (mean and the
 *     diagonal of the covariance), Technical Summary section 2.1;
 *   - a decode query scores each block with the second-order Taylor
 *     estimate exp(q_hat.mean) (1 + 1/2 q_hat^T diag(var) q_hat) of the
 *     block's attention mass, q_hat = q / sqrt(d) (section 2.1, score);
 *   - the top_k blocks (sink block 0 and the current block always among
 *     them) get exact softmax attention (sections 1 and 2);
 *   - the rest ("long tail") enters through Residual Linear Attention in its
 *     subtraction form o_rla = o_bar - o_tilde: o_bar = phi(q)^T S_all from a
 *     running state over all tokens, o_tilde = phi(q)^T sum_sel phi(k) v^T
 *     from the K/V tiles already loaded for exact attention, so unselected
 *     blocks are never read (section 2.2, IO-efficient formulation);
 *   - o = o_sparse + g_h * o_rla with a per-query-head gate g_h; phi(x) =
 *     elu(x) + 1 (section 2.3 leaves both open; they are fixed parameters of
 *     this library).
 *
 * Two calls do the work: spla_append_kv (update K/V pages, block statistics
 * and S_all / z_all) and spla_decode (score -> top-k -> attend + correct ->
 * combine).  A decode step is spla_append_kv of the step's token for every
 * sequence followed by spla_decode (the token attends to itself).
 *
 * Conventions
 *   - Every device buffer is allocated and owned by the caller.  The library
 *     owns only the host handle (a copy of the configuration, the buffer
 *     pointers and a host mirror of the sequence lengths).  It never
 *     allocates or frees device memory and never synchronises a stream.
 *   - Work is enqueued on the caller's stream (a hipStream_t passed as
 *     void*; NULL = the null stream).  Outputs are valid when the stream
 *     reaches that point.  Kernel launch parameters (grid sizes, lengths)
 *     come from the host mirror, so a captured HIP graph replays exactly the
 *     step it recorded.
 *   - Validation happens on the host before anything is enqueued.  On any
 *     error status nothing is enqueued and nothing (the mirror included)
 *     changes, except SPLA_ERR_HIP, which reports a failed launch.
 *   - Device pointers must be 16-byte aligned.
 *   - One handle must not be used from two host threads at once; distinct
 *     handles are independent.  Calls on one handle are ordered by the
 *     caller's stream(s): use one stream per handle or order them yourself.
 *   - Layouts are row-major, index order as written.
 *
 * Buffer layouts (B = batch, H = n_q_heads, G = n_kv_heads, d = head_dim,
 * Bk = block_size, MB = max_blocks_per_seq, NT = ceil(MB / 64)):
 *   k_pages, v_pages  [num_pages][G][Bk][d] kv_dtype.  One page holds one
 *                     block (Bk consecutive tokens) of one sequence, all KV
 *                     heads.
 *   block_table       [B][MB] int32: page id of block j of sequence b.
 *                     Filled by the caller for every block a sequence will
 *                     reach; an id outside [0, num_pages) is never
 *                     dereferenced: the access is skipped and bit 0 of the
 *                     workspace error word is set.
 *   blk_mean, blk_var [B][G][NT][d/4][64][4] float32: statistics of block j,
 *                     channel c of (b, g) live at
 *                     ((((b*G + g)*NT + j/64)*(d/4) + c/4)*64 + j%64)*4 + c%4.
 *                     (64 blocks side by side per channel quartet, so the
 *                     scorer reads them with whole-wavefront vector loads.)
 *                     Only blocks completed by an append are written.
 *   s_all             [B][G][d][d] float32: S[b][g][x][y] = sum_t phi(k_t[x]) v_t[y].
 *   z_all             [B][G][d] float32:    z[b][g][x]    = sum_t phi(k_t[x]).
 *   workspace         spla_workspace_bytes() bytes, zero-filled by the
 *                     caller once before the first call.  Bytes [0, 4) hold
 *                     a sticky uint32 error word (bit 0: out-of-range page
 *                     id, bit 1: a selected block id outside the sequence,
 *                     bits 2-4: a one-kernel step's counters out of step, see
 *                     SPLA_TUNE_STEP_KERNEL); the rest is scratch: bytes
 *                     [256, 33024) are the one-kernel step's counters, which
 *                     every call leaves at zero, the rest the library clears
 *                     itself.
 *                     A fresh state needs s_all, z_all zero-filled.
 */
#ifndef SPLA_H
#define SPLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPLA_ABI_VERSION 2

typedef enum {
    SPLA_OK = 0,
    SPLA_ERR_INVALID_ARG = 1,  /* null/out-of-range argument, empty sequence at decode */
    SPLA_ERR_UNSUPPORTED = 2,  /* configuration outside the supported set */
    SPLA_ERR_CAPACITY = 3,     /* append would exceed max_blocks_per_seq * block_size */
    SPLA_ERR_ALIGNMENT = 4,    /* a device pointer is not 16-byte aligned */
    SPLA_ERR_HIP = 5,          /* a kernel launch failed (see spla_last_hip_error) */
    SPLA_ERR_STATE = 6,        /* call before spla_bind */
    SPLA_ERR_SCRATCH = 7       /* per-call scratch above SPLA_NOALLOC_SCRATCH_BYTES (no-alloc call) */
} spla_status;

typedef enum { SPLA_F32 = 0, SPLA_BF16 = 1 } spla_dtype;

/* Supported: 1 <= batch <= 256; head_dim in {64, 128}; block_size in {64,
 * 128}; n_q_heads = r * n_kv_heads with r in {1, 2, 4, 8}; 2 <= top_k <= 256;
 * 1 <= max_blocks_per_seq <= 16386 (1M tokens at block 64, 2M at 128); num_pages >= 1; kv_dtype F32 or BF16
 * (K, V and q share it).  Anything else returns SPLA_ERR_UNSUPPORTED. */
typedef struct {
    int32_t batch;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t top_k;              /* blocks kept per (sequence, KV head), sink and current included */
    int32_t max_blocks_per_seq;
    int32_t num_pages;
    int32_t kv_dtype;           /* spla_dtype */
} spla_config;

typedef struct {               /* device pointers, all caller-owned */
    void *k_pages;
    void *v_pages;
    const int32_t *block_table;
    float *blk_mean;
    float *blk_var;
    float *s_all;
    float *z_all;
    void *workspace;
    size_t workspace_bytes;
} spla_buffers;

typedef struct {               /* optional outputs / test hook of spla_decode; NULL = unused */
    int32_t *sel_idx;          /* out [B][G][top_k] selected block ids, ascending, -1 padded */
    float *lg;                 /* out [B][G][MB] group log score LG(j) of candidate blocks
                                  1..nb-2 (other entries untouched); written only when
                                  nb > top_k, the case where a choice is made */
    float *o_sparse;           /* out [B][H][d] exact attention over the selected blocks */
    float *o_rla;              /* out [B][H][d] o_bar - o_tilde (0 when every block is selected) */
    float *d_rla;              /* out [B][H] phi(q).(z_all - z_sel) (0 when every block is selected) */
    const int32_t *sel_in;     /* in  [B][G][top_k]: use these block ids (ascending, -1 padded,
                                  each < nb) instead of scoring + top-k */
    void *const *kernel_events;  /* in: hipEvent_t[2 * n], created by the caller; when set, the i-th
                                  kernel this call launches (i < n) is launched with
                                  hipExtLaunchKernel and kernel_events[2i] / [2i+1] take the
                                  kernel's own begin / end timestamps (either may be NULL), for
                                  per-kernel timing.  Not for use under stream capture.  Launch
                                  order: as spla_launch_plan reports it. */
    int32_t n_kernel_events;   /* n: entries of kernel_events / 2 */
} spla_decode_aux;

typedef struct spla_handle spla_handle;

/* Validate cfg and create a handle (host only, no HIP call). */
spla_status spla_create(const spla_config *cfg, spla_handle **out);
void spla_destroy(spla_handle *h);

/* Sizes the caller allocates: workspace bytes; floats of blk_mean (= of
 * blk_var). */
size_t spla_workspace_bytes(const spla_handle *h);
size_t spla_stats_floats(const spla_handle *h);

/* Attach the caller's buffers and the current sequence lengths (host array
 * of batch entries; NULL = all zero).  The buffers must already hold the
 * state of those lengths (all zero for an empty state).  Host only. */
spla_status spla_bind(spla_handle *h, const spla_buffers *b, const int32_t *lens_host);

/* Append n_new_host[i] tokens to sequence seq_ids_host[i] for i < n_seqs
 * (distinct ids).  k_new, v_new: device [sum n_new][G][d] kv_dtype, the
 * rows of entry i following those of entry i-1.  Writes the rows into the
 * pages (via block_table), adds phi(k) v^T and phi(k) to s_all and z_all,
 * and writes blk_mean / blk_var of every block the append completes
 * (population variance, two passes).  Technical Summary 2.1 (statistics)
 * and 2.2 (global linear-attention state). */
spla_status spla_append_kv(spla_handle *h, int32_t n_seqs, const int32_t *seq_ids_host,
                           const int32_t *n_new_host, const void *k_new, const void *v_new,
                           void *stream);

/* Decode one query token per sequence.  q: device [B][H][d] kv_dtype;
 * gate: device [H] float32; out: device [B][H][d] float32 receives
 * o = o_sparse + gate[h] * o_rla (o_rla in the output form set by
 * spla_set_rla_output; plain by default).  Query head h uses KV head h / (H/G).
 * Every sequence must be non-empty (SPLA_ERR_INVALID_ARG otherwise).
 * Selection per (b, g): nb = ceil(T/Bk); if nb <= top_k every block;
 * otherwise blocks 0 and nb-1 plus the top_k-2 candidates 1..nb-2 with the
 * largest LG(j) = log sum_h exp(q_hat_h.mean_j + log1p(1/2 sum_c
 * q_hat_hc^2 var_jc)), ties to the smaller id.  aux may be NULL. */
spla_status spla_decode(spla_handle *h, const void *q, const float *gate, float *out,
                        const spla_decode_aux *aux, void *stream);

/* One decode step as a single call: spla_append_kv of one token for every
 * sequence (k_new, v_new: device [B][G][d] kv_dtype, row b = sequence b)
 * followed by spla_decode, with the same results.  The append runs inside
 * the scorer's launch (the scorer reads statistics of blocks completed by
 * earlier appends only), so the step takes one kernel launch less.
 * aux->sel_in is not accepted here (SPLA_ERR_INVALID_ARG).  If a launch
 * after the first fails, the append has been enqueued and the mirror
 * advances; if the first fails, nothing changes. */
spla_status spla_decode_step(spla_handle *h, const void *k_new, const void *v_new, const void *q,
                             const float *gate, float *out, const spla_decode_aux *aux, void *stream);

/* For callers that cannot allocate device memory at call time (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * spla_decode_step with the per-call scratch (group log scores, selections,
 * partial records, phi(q)^T S_all partials, phi(q)) taken from one static
 * device array of the library instead of the bound workspace.  It allocates
 * nothing and calls no allocating routine; arguments, results, validation
 * and the sticky error word (bytes [0, 4) of the bound workspace, which is
 * otherwise not touched) are those of spla_decode_step.
 *   - The array holds SPLA_NOALLOC_SCRATCH_BYTES (64 MiB); a handle whose
 *     spla_workspace_bytes() exceeds it gets SPLA_ERR_SCRATCH, with nothing
 *     enqueued.
 *   - Each GPU the library runs on holds its own copy until the process
 *     ends.  Its device address is looked up on the first call on that GPU
 *     (with the GPU of `stream` made current for the lookup); make that
 *     first call outside stream capture.
 *   - Every call on one GPU shares that GPU's array and it keeps the last
 *     call's contents (every part is written before it is read, so nothing
 *     needs clearing).  Calls that overlap on one GPU -- on two streams, or
 *     from two handles -- race on it: order them on one stream. */
#define SPLA_NOALLOC_SCRATCH_BYTES (64u << 20)
spla_status spla_decode_step_noalloc(spla_handle *h, const void *k_new, const void *v_new, const void *q,
                                     const float *gate, float *out, const spla_decode_aux *aux,
                                     void *stream);

/* Copy the host mirror of the sequence lengths (batch entries). */
spla_status spla_get_lens(const spla_handle *h, int32_t *lens_host);

const char *spla_status_str(spla_status st);

/* Tuning switches (host only, per handle; results are bitwise identical
 * whatever the setting).
 *   SPLA_TUNE_FUSED_SELECT: -1 automatic (default: fused for at most 64
 *   (sequence, KV head) pairs), 0 = the stand-alone selector kernel, 1 = the
 *   fused select + attend kernel whenever it supports the call (bf16 K/V,
 *   block_size 64, no sel_in, at most 4096 candidate blocks per sequence).
 *   The fused kernel recomputes the selection of a (sequence, KV head) in
 *   every attend workgroup of that pair instead of handing it over through
 *   memory, which saves one launch per decode.
 *   SPLA_TUNE_STEP_KERNEL: 1 = spla_decode_step runs its append, scores,
 *   o_bar partials, selection and attend in one kernel wherever the fused
 *   select + attend runs, the score form is the Taylor score and
 *   B * n_kv_heads <= 256; -1 automatic (default) and 0 = the separate
 *   kernels (automatic keeps them: they are as fast or faster).  The
 *   one-kernel step hands each (sequence, KV head) pair's scores over to its
 *   attend workgroups inside the kernel, through counters at workspace bytes
 *   [256, 33024) that every call leaves at zero (the workspace starts
 *   zero-filled); a wait that runs out sets bit 2 of the error word, a
 *   counter found above its target bit 3, an attend count above top_k bit 4.
 *   SPLA_TUNE_FUSED_MERGE: 1 = where the fused select + attend runs with the
 *   plain or normalised RLA form and B * n_q_heads < 256, it also merges each
 *   (sequence, KV head) pair's partial records into the outputs (the combine
 *   kernel's workgroups for the pair's heads, in the same launch, waiting for
 *   the pair's attend workgroups through the same workspace counters and
 *   error bits as the one-kernel step) and no combine kernel runs; -1
 *   automatic (default) and 0 = the combine kernel (automatic keeps it: it is
 *   as fast or faster).
 * SPLA_ERR_INVALID_ARG for an unknown key or value. */
typedef enum { SPLA_TUNE_FUSED_SELECT = 0, SPLA_TUNE_STEP_KERNEL = 1, SPLA_TUNE_FUSED_MERGE = 2 } spla_tune_key;
spla_status spla_set_tuning(spla_handle *h, int32_t key, int32_t value);

/* Output form of the residual-linear-attention branch in o = o_sparse +
 * gate[h] * branch (per handle, host only; applies to spla_decode and
 * spla_decode_step from the next call on).  aux->o_rla and aux->d_rla keep
 * reporting o_rla and D themselves in every form.  The branch is 0 in every
 * form when the selection covers every token.
 *   SPLA_RLA_PLAIN       o_rla (the default).
 *   SPLA_RLA_NORMALIZED  o_rla / D.  By the subtraction form (Technical
 *                        Summary 2.2) o_rla and D are the numerator and the
 *                        normaliser of linear attention over the unselected
 *                        tokens, so this is that attention normalised, the
 *                        kernelised form phi(Q)(phi(K)^T V) / phi(Q)(phi(K)^T 1)
 *                        (Baidu Cloud sparse-attention article, section 7).
 *   SPLA_RLA_RMSNORM     gamma[h][c] * o_rla[c] / sqrt(mean_c o_rla[c]^2 + eps)
 *                        over the head_dim channels of each query head: the
 *                        RMS norm of the RLA output whose scale is the
 *                        method's only added parameter (Technical Summary
 *                        2.3).  gamma: device [H][d] float32, caller-owned,
 *                        read at every decode (keep it alive and unchanged
 *                        while the handle uses it); eps > 0 and finite.
 * gamma and eps are ignored (and forgotten) for the other forms.
 * SPLA_ERR_INVALID_ARG for an unknown form, a NULL gamma or a bad eps with
 * SPLA_RLA_RMSNORM; SPLA_ERR_ALIGNMENT for a misaligned gamma.  On error
 * the handle keeps its previous form. */
typedef enum { SPLA_RLA_PLAIN = 0, SPLA_RLA_NORMALIZED = 1, SPLA_RLA_RMSNORM = 2 } spla_rla_form;
spla_status spla_set_rla_output(spla_handle *h, int32_t form, const float *gamma, float eps);

/* Chunked prefill of one sequence: append the n tokens k_new, v_new (device
 * [n][G][d] kv_dtype) to sequence seq and write, for each new token t, the
 * output its query q[t] (device [n][H][d] kv_dtype) gets as a decode at its
 * own position: out[t] (device [n][H][d] float32) equals what spla_append_kv
 * of token t alone followed by a spla_decode of q[t] would give that
 * sequence (Technical Summary 2.1-2.3 applied at every position; the token
 * attends to itself and to every earlier token, causally inside its own
 * block).  Other sequences are untouched.  The handle's output form and
 * score form apply.  sel_idx (optional, device [n][G][top_k] int32) receives
 * every token's selected block ids, ascending, -1 padded; lg (optional,
 * device [n][G][max_blocks_per_seq] float32, 16-byte aligned) every token's
 * group log score of each of its candidate blocks 1 .. nb-2 (the other
 * entries untouched), as spla_decode_aux.lg does for a decode.
 * workspace: device scratch of workspace_bytes >= spla_prefill_workspace_bytes
 * (h, 1), caller-owned; the call processes up to 256 tokens per group of
 * launches, as many as the workspace holds (spla_prefill_workspace_bytes(h,
 * c) bytes hold c), and its contents are undefined afterwards.  It may not
 * be the handle's own workspace.  Each group appends its tokens' pages and
 * block statistics, decodes its tokens against the state before the group
 * (adding the group's own earlier tokens to the linear-attention sums), then
 * adds the group to S_all / z_all.  With bf16 K/V the group's attention is
 * block-centric: the (token, slot) pairs are filed under the blocks they
 * selected (lists in the workspace) and each selected block's tiles are read
 * once per 8 tokens that chose it.
 * Errors as for spla_append_kv (capacity, alignment, seq out of range);
 * n = 0 does nothing.  On SPLA_ERR_HIP the state of sequence seq is
 * undefined (part of the tokens may be in it). */
size_t spla_prefill_workspace_bytes(const spla_handle *h, int32_t chunk);
spla_status spla_prefill(spla_handle *h, int32_t seq, int32_t n, const void *k_new, const void *v_new,
                         const void *q, const float *gate, float *out, int32_t *sel_idx, float *lg,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Block score the selection ranks (per handle, host only; from the next
 * decode on).
 *   SPLA_SCORE_TAYLOR  the second-order Taylor score (default; Technical
 *                      Summary 2.1).
 *   SPLA_SCORE_MEAN    its first-order term q_hat . mean alone: the
 *                      mean-pooling heuristic the second-order selection is
 *                      compared with (Technical Summary 3).  It reads no
 *                      variances.  aux->lg then reports this score.
 * SPLA_ERR_INVALID_ARG for an unknown form. */
typedef enum { SPLA_SCORE_TAYLOR = 0, SPLA_SCORE_MEAN = 1 } spla_score_form;
spla_status spla_set_score_form(spla_handle *h, int32_t form);

/* Exact attention mass of every candidate block, for measuring how well a
 * block score ranks blocks: lgx[b][g][j] = log sum_h (1/Bk) sum_{i in j}
 * exp(q_hat_h . k_i) for j in 1 .. nb-2 (the other entries untouched), with
 * the heads h of KV head g and q_hat = q / sqrt(d) (Technical Summary 2.1:
 * the block's integrated probability mass, which the Taylor score
 * estimates; per-token mean form, summed over the group like the score).
 * q: device [B][H][d] kv_dtype; lgx: device [B][G][MB] float32.  It reads
 * every key of every candidate block (a dense pass, not part of a decode)
 * and changes no state.  Every sequence must be non-empty
 * (SPLA_ERR_INVALID_ARG); an out-of-range page id sets bit 0 of the error
 * word and leaves that block's entry untouched. */
spla_status spla_block_mass(spla_handle *h, const void *q, float *lgx, void *stream);

/* The kernels the next call of kind `call` on this handle would launch, in
 * launch order (the order of spla_decode_aux.kernel_events), from the
 * current lengths and tuning.  Writes min(n, cap) entries of kernels
 * (SPLA_KERNEL_*) and returns n (at most 4), or -1 for a NULL handle or an
 * unknown call. */
typedef enum {
    SPLA_KERNEL_SCORE = 1,         /* block scorer (spla_decode) */
    SPLA_KERNEL_STEP_SCORE = 2,    /* one-token append + block scorer (spla_decode_step) */
    SPLA_KERNEL_SELECT = 3,        /* stand-alone top-k selector */
    SPLA_KERNEL_ATTEND = 4,        /* attend + correct over the selector's blocks */
    SPLA_KERNEL_SELECT_ATTEND = 5, /* fused select + attend + correct (+ the merge when no combine follows) */
    SPLA_KERNEL_COMBINE = 6,       /* merge, o_bar, o_rla, D, gate */
    SPLA_KERNEL_STEP_FUSED = 7     /* append + scores + o_bar partials + select + attend (spla_decode_step) */
} spla_kernel;
typedef enum {
    SPLA_CALL_DECODE = 0,          /* spla_decode without sel_in */
    SPLA_CALL_DECODE_SEL_IN = 1,   /* spla_decode with sel_in */
    SPLA_CALL_DECODE_STEP = 2      /* spla_decode_step */
} spla_call;
int32_t spla_launch_plan(const spla_handle *h, int32_t call, int32_t *kernels, int32_t cap);

/* The hipError_t of the last launch on this handle that failed (0 = none)
 * and, if name is non-NULL, its name (hipGetErrorName; static storage).  A
 * call that returned SPLA_ERR_HIP leaves its launch's code here. */
int32_t spla_last_hip_error(const spla_handle *h, const char **name);
int32_t spla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPLA_H */
