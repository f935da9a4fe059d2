/*
 * attn.h -- C ABI of libattn: attention forward on AMD Instinct MI355X (gfx950).
 *
 * Two operations, each with a host-only argument check that makes no HIP call:
 *
 *   attn_fwd            multi-head scaled dot-product attention forward over
 *                       dense [B, H, S, D] tensors, computed as a tiled
 *                       online-softmax recurrence.
 *   attn_paged_decode   one decode query per sequence against a paged KV
 *                       pool, split over the key dimension, with the partial
 *                       results merged through their log-sum-exp.
 *
 * What is computed follows two pages: the kernel-contract page
 * ("fuel-reference-backend -- attention kernel contracts", sections
 * attention_naive, attention_flash and attention_paged_naive) and the
 * derivation page ("gfx942 unified attention, from the math up", sections 1-5
 * and 8).  For query row i of head h (KV head g = h / (Hq / Hkv)):
 *
 *   i'  = i + Sk - Sq                        bottom-right aligned position
 *   s_j = softmax_scale * (q_i . k_j)
 *   s_j = softcap * tanh(s_j / softcap)      if softcap > 0
 *   s_j = s_j + alibi[h] * (j - i')          if alibi != NULL
 *   key j is admissible iff 0 <= j < Sk, (!causal || j <= i'),
 *         (window_left  < 0 || j >= i' - window_left),
 *         (window_right < 0 || j <= i' + window_right)
 *   out_i = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m) over admissible j
 *           (m = max admissible s_j), and out_i = 0 if no key is admissible.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is DEVICE memory owned by the caller and borrowed
 *     only for the work enqueued by the call.  The library allocates nothing,
 *     frees nothing and keeps no state between calls.
 *   - Tensors are contiguous, row-major, zero-offset, 16-byte aligned.  Views
 *     with other strides must be materialised by the caller.
 *   - q, k, v (or the pools) and out share one element type (dtype); out has
 *     the shape and dtype of q.  ALiBi slopes are always float32 [Hq].
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream).  A non-OK status means nothing was enqueued, except
 *     ATTN_ERR_HIP, which reports a launch failure.
 *   - Results are bitwise reproducible for identical inputs and parameters
 *     (no atomics in any reduction, fixed reduction orders).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_dtype {
  ATTN_F32 = 0,
  ATTN_F16 = 1,
  ATTN_BF16 = 2,
  ATTN_F64 = 3   /* dense forward only (kernel-contract page: F64 accepted) */
} attn_dtype_t;

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,         /* a required pointer is NULL                          */
  ATTN_ERR_DTYPE = 2,        /* dtype is not an attn_dtype_t value                  */
  ATTN_ERR_SHAPE = 3,        /* a size is negative, inconsistent or too large       */
  ATTN_ERR_GQA = 4,          /* Hkv == 0 or Hq is not a multiple of Hkv             */
  ATTN_ERR_HEAD_DIM = 5,     /* D not built for the dtype (see attn_fwd_params_t)   */
  ATTN_ERR_PARAM = 6,        /* scale/softcap/window/split parameter out of range   */
  ATTN_ERR_ALIGN = 7,        /* a pointer is not 16-byte aligned                    */
  ATTN_ERR_ALIAS = 8,        /* out overlaps an input or the workspace              */
  ATTN_ERR_WORKSPACE = 9,    /* workspace missing or smaller than required          */
  ATTN_ERR_UNSUPPORTED = 10, /* allowed by the contract but not built here          */
  ATTN_ERR_HIP = 11          /* the HIP runtime reported an error at launch         */
} attn_status_t;

/* Parameters of attn_fwd (kernel-contract page, attention_naive: the
 * FlashAttn parameter set -- scale, causal flag, optional left/right window,
 * optional softcap). */
typedef struct attn_fwd_params {
  int64_t B;             /* batch                                               */
  int64_t Hq;            /* query heads; a multiple of Hkv                      */
  int64_t Hkv;           /* key/value heads                                     */
  int64_t Sq;            /* query length (0 allowed: nothing to do)             */
  int64_t Sk;            /* key length (0 allowed: output is all zero); one    *
                          * head's K (Sk * D * element size) must be < 2 GiB    */
  int64_t D;             /* head dim: 64, 128 or 256 for F16/BF16 (matrix      *
                          * cores); 32, 64, 128 or 256 for F32/F64 (vector     *
                          * ALU); the same for the backward                    */
  int32_t dtype;         /* attn_dtype_t of q, k, v and out                     */
  int32_t causal;        /* nonzero: bottom-right causal mask                   */
  int64_t window_left;   /* -1: unbounded; else keys j >= i' - window_left      */
  int64_t window_right;  /* -1: unbounded; else keys j <= i' + window_right     */
  float softmax_scale;   /* finite, >= 0 (1/sqrt(D) is the usual value)         */
  float softcap;         /* 0: off; > 0: s <- softcap * tanh(s / softcap)       */
  int64_t k_len;         /* live key prefix length, read only when has_k_len    */
  int32_t has_k_len;     /* 0: every one of the Sk keys is live (a zeroed      *
                          * struct means this).  Else the kernel-contract      *
                          * page's k_len parameter of attention_naive: k_len   *
                          * in 0..Sk, only keys j < k_len exist, and the call  *
                          * equals one on k[:, :, :k_len] and v[:, :, :k_len]  *
                          * (queries align bottom-right to the live length,    *
                          * i' = i + k_len - Sq) while k and v keep their      *
                          * [B, Hkv, Sk, D] layout; keys j >= k_len are never  *
                          * read.  The backward entry points require 0.        */
} attn_fwd_params_t;

/* Host-only validation of an attn_fwd call (no HIP call is made).
 *   q     [B, Hq, Sq, D]   dtype
 *   k, v  [B, Hkv, Sk, D]  dtype
 *   alibi [Hq] float32 or NULL
 *   out   [B, Hq, Sq, D]   dtype; must not overlap q, k, v or alibi.
 * A pointer may be NULL only when its tensor has no elements. */
attn_status_t attn_fwd_check(const void* q, const void* k, const void* v,
                             const float* alibi, const void* out,
                             const attn_fwd_params_t* p);

/* Attention forward: validates as attn_fwd_check, then enqueues the kernel
 * for p->dtype and p->D on `stream` and returns.  F16/BF16 compute both
 * matmuls on the matrix cores with float32 accumulation (the softmax weights
 * enter the second matmul rounded to the input dtype); F32 and F64 compute in
 * their own precision throughout, on the vector ALU. */
attn_status_t attn_fwd(const void* q, const void* k, const void* v,
                       const float* alibi, void* out,
                       const attn_fwd_params_t* p, void* stream);

/* Host-only validation of an attn_fwd_lse call: as attn_fwd_check, plus
 *   lse   [B, Hq, Sq] float32 (for every dtype, F64 included), 4-byte
 *         aligned, overlapping no input and not out; NULL only when
 *         B * Hq * Sq == 0. */
attn_status_t attn_fwd_lse_check(const void* q, const void* k, const void* v,
                                 const float* alibi, const void* out,
                                 const float* lse, const attn_fwd_params_t* p);

/* Attention forward that also writes, for every query row, the natural-log
 * log-sum-exp of its transformed admissible scores, ln(sum_j exp(s_j)), or
 * -infinity for a row with no admissible key.  This is the row state the
 * online recurrence ends with (derivation page, section 3: m + log l) and
 * the input the backward pass of the kernel-contract page
 * (attention_flash_backward) needs from the forward.  Validates as
 * attn_fwd_lse_check, then enqueues the same kernel as attn_fwd. */
attn_status_t attn_fwd_lse(const void* q, const void* k, const void* v,
                           const float* alibi, void* out, float* lse,
                           const attn_fwd_params_t* p, void* stream);

/* Parameters of attn_paged_decode (kernel-contract page, attention_paged_naive:
 * the PagedAttn parameter set -- scale, block size, optional softcap -- plus
 * the number of key-dimension splits of the decode path, derivation page
 * section 8). */
typedef struct attn_paged_params {
  int64_t B;                   /* sequences                                      */
  int64_t Hq;                  /* query heads; a multiple of Hkv                 */
  int64_t Hkv;                 /* key/value heads                                */
  int64_t D;                   /* head dim: 64, 128 or 256 (F16/BF16); 32, 64,
                                  128 or 256 (F32/F64)                           */
  int64_t num_blocks;          /* physical blocks in each pool                   */
  int64_t block_size;          /* tokens per block (>= 1)                        */
  int64_t max_blocks_per_seq;  /* columns of block_table                         */
  int32_t dtype;               /* attn_dtype_t of q, pools and out: F16/BF16 on
                                  the matrix cores, F32/F64 on the vector ALU
                                  (one workgroup per (sequence, head); the
                                  workspace is then not touched)                 */
  int32_t num_splits;          /* key-dimension splits per sequence, 1..256,
                                  or 0: chosen by the library from the shape
                                  (about 1024 work items of (sequence, KV
                                  head, 16-query-head chunk, split), 4096
                                  from 256 groups up, with at least 256
                                  tokens of block-table capacity per split).
                                  A tuning value: with at least one group
                                  per compute unit but fewer than 4 items
                                  per compute unit, each group is split over
                                  the waves of one workgroup instead         */
  float softmax_scale;         /* finite, >= 0                                   */
  float softcap;               /* 0: off; > 0: softcap * tanh(s / softcap)       */
} attn_paged_params_t;

/* Bytes of device workspace attn_paged_decode needs for these parameters
 * (0 if the parameters are invalid).  The workspace holds, per (sequence,
 * query head, split), a float32 partial output [D] and its log-sum-exp. */
size_t attn_paged_decode_workspace_size(const attn_paged_params_t* p);

/* Host-only validation of an attn_paged_decode call (no HIP call is made).
 *   q            [B, Hq, 1, D]                         dtype
 *   k_pool,v_pool[num_blocks, block_size, Hkv, D]       dtype
 *   block_table  [B, max_blocks_per_seq] int32: physical block of logical
 *                block n of sequence b; entries past the last live block are
 *                never read.
 *   seq_lens     [B] int32: live keys of sequence b (the query sits at
 *                position seq_lens[b] - 1 and sees every live key).
 *   alibi        [Hq] float32 or NULL (ALiBi distance is k_pos - (seq_len-1))
 *   out          [B, Hq, 1, D] dtype
 *   workspace    >= attn_paged_decode_workspace_size(p) bytes
 *   error_flag   NULL or one device int32. */
attn_status_t attn_paged_decode_check(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      const float* alibi, const void* out,
                                      const void* workspace, size_t workspace_bytes,
                                      const int32_t* error_flag,
                                      const attn_paged_params_t* p);

/* Paged split-KV decode: validates as attn_paged_decode_check, then enqueues
 * the kernels on `stream` and returns.  For block sizes that are multiples of
 * 16: a persistent kernel whose per-wave workers write per-split partials for
 * the merge kernel (B <= 2048, unless there are at least as many (sequence,
 * KV head, 16-query-head chunk) groups as compute units and either D = 256
 * or fewer than 4 group-split items per compute unit); or a persistent kernel
 * with one workgroup per compute unit that spreads each group over its waves,
 * merges them in LDS and writes out directly, the workspace untouched (that
 * case, and 2048 < B <= 4096 with max_blocks_per_seq * block_size > 1024).
 * Otherwise,
 * and for other block sizes, a partial kernel (one workgroup per sequence, KV
 * head and split) and the merge kernel.  The result is the same up to
 * rounding order in every form.
 * Device-side errors do not fault:
 * a seq_len outside [0, max_blocks_per_seq * block_size] is clamped into that
 * range and a block_table entry outside [0, num_blocks) masks its keys; both
 * store 1 to *error_flag when error_flag is not NULL (the flag is never
 * cleared by the library).  A sequence with no live key outputs zeros. */
attn_status_t attn_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const float* alibi, void* out,
                                void* workspace, size_t workspace_bytes,
                                int32_t* error_flag,
                                const attn_paged_params_t* p, void* stream);

/* Bytes of the device-resident workspace behind attn_paged_decode_noalloc
 * (one copy per GPU the library runs on, held until the process ends). */
#define ATTN_DECODE_SCRATCH_BYTES (32u << 20)

/* attn_paged_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, validation, kernels and results (bitwise) as
 * attn_paged_decode, except that no workspace is passed: the split forms
 * keep their partials in a file-scope device array of
 * ATTN_DECODE_SCRATCH_BYTES bytes inside the library.  A call whose
 * attn_paged_decode_workspace_size(p) exceeds that returns
 * ATTN_ERR_WORKSPACE before anything is launched.  The library allocates
 * nothing and calls no allocating routine here; on the first call on a
 * device it looks up that device's copy of the array (hipGetSymbolAddress;
 * ATTN_ERR_HIP if that fails).  Every call on one GPU shares that GPU's
 * array, whatever the stream: calls that overlap in time on one GPU race on
 * it, so callers serialise them (one stream, or events).  Nothing in the
 * array needs clearing between calls: every call writes each partial it
 * reads. */
attn_status_t attn_paged_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        const float* alibi, void* out, int32_t* error_flag,
                                        const attn_paged_params_t* p, void* stream);

/* Parameters of attn_paged_prefill: variable-length prefill over the paged
 * pool (kernel-contract page, attention_paged_naive, with the packed query
 * layout of the derivation page, section 5: queries [total_q, Hq, D] with a
 * cu_seqlens_q prefix sum, per-sequence key lengths in seq_lens). */
typedef struct attn_varlen_params {
  int64_t B;                   /* sequences                                      */
  int64_t Hq;                  /* query heads; a multiple of Hkv                 */
  int64_t Hkv;                 /* key/value heads                                */
  int64_t D;                   /* head dim: 64, 128 or 256 (F16/BF16); 32, 64,
                                  128 or 256 (F32/F64)                           */
  int64_t total_q;             /* rows of q and out                              */
  int64_t max_seqlen_q;        /* >= cu_seqlens_q[b+1] - cu_seqlens_q[b] for all b */
  int64_t num_blocks;          /* physical blocks in each pool                   */
  int64_t block_size;          /* tokens per block: a multiple of 64 for F16/BF16,
                                  any for F32/F64                                */
  int64_t max_blocks_per_seq;  /* columns of block_table                         */
  int32_t dtype;               /* attn_dtype_t of q, pools and out               */
  int32_t causal;              /* nonzero: key t admissible iff t <= i'          */
  int64_t window_left;         /* -1: unbounded; else keys t >= i' - window_left */
  int64_t window_right;        /* -1: unbounded; else keys t <= i' + window_right*/
  float softmax_scale;         /* finite, >= 0                                   */
  float softcap;               /* 0: off; > 0: softcap * tanh(s / softcap)       */
} attn_varlen_params_t;

/* Host-only validation of an attn_paged_prefill call (no HIP call is made).
 *   q             [total_q, Hq, D]                      dtype
 *   k_pool,v_pool [num_blocks, block_size, Hkv, D]      dtype
 *   block_table   [B, max_blocks_per_seq] int32
 *   seq_lens      [B] int32: live keys of sequence b
 *   cu_seqlens_q  [B + 1] int32: sequence b owns query rows
 *                 cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1; row i of it sits
 *                 at position i' = seq_lens[b] - Sq_b + i (bottom-right)
 *   alibi         [Hq] float32 or NULL (ALiBi distance t - i')
 *   out           [total_q, Hq, D] dtype
 *   error_flag    NULL or one device int32.
 * For F16/BF16 (matrix cores) block_size must be a multiple of 64
 * (ATTN_ERR_UNSUPPORTED otherwise); F32/F64 run on the vector ALU, computing
 * in that type throughout, with any block size. */
attn_status_t attn_paged_prefill_check(const void* q, const void* k_pool, const void* v_pool,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       const int32_t* cu_seqlens_q, const float* alibi,
                                       const void* out, const int32_t* error_flag,
                                       const attn_varlen_params_t* p);

/* Variable-length prefill (or chunked prefill) over the paged pool:
 * validates as attn_paged_prefill_check, then enqueues one kernel on `stream`
 * and returns.  Rows of out outside every sequence are not written.
 * Device-side errors do not fault: a prefix sum outside [0, total_q] or a
 * sequence longer than max_seqlen_q is clamped, a seq_len outside
 * [0, max_blocks_per_seq * block_size] is clamped, and a block_table entry
 * outside [0, num_blocks) masks its keys; each stores 1 to *error_flag when
 * error_flag is not NULL.  A row with no admissible key outputs zeros. */
attn_status_t attn_paged_prefill(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* cu_seqlens_q, const float* alibi, void* out,
                                 int32_t* error_flag, const attn_varlen_params_t* p,
                                 void* stream);

/* ---- backward (kernel-contract page, attention_flash_backward) ----------
 * Gradients of attn_fwd with respect to q, k and v for the upstream gradient
 * dout of its output, by recompute: the entry point re-runs the forward
 * softmax of every row (its log-sum-exp and dout . out land in the
 * workspace), then forms dV += P^T dO, dP = dO V^T, dS = (dP - rowsum(P dP))
 * P (times 1 - tanh^2(s_pre / softcap) with a softcap), dQ = scale dS K and
 * dK = scale dS^T Q.  dk and dv are [B, Hkv, Sk, D], summed over the query
 * heads of each KV head's group; dq is [B, Hq, Sq, D].  A row with no
 * admissible key contributes nothing.  F16/BF16 with head dims 64/128/256 run
 * on the matrix cores (float32 accumulation, P and dS rounded to the input dtype
 * as matmul operands); F32/F64 with head dims 32 to 256 on the vector ALU,
 * computing in that type throughout.  Deterministic: no atomics, fixed
 * order. */

/* Workspace bytes attn_bwd needs for p, 0 for an invalid p: for F16/BF16,
 * 8 * B * Hq * Sq for the forward's row statistics plus float32 partial
 * dK/dV when the key blocks' work is split (the split depends only on p);
 * for F32/F64, two values of the element type per query row. */
size_t attn_bwd_workspace_size(const attn_fwd_params_t* p);

/* Host-only validation of an attn_bwd call (no HIP call is made).
 *   q, dout    [B, Hq, Sq, D]   dtype
 *   k, v       [B, Hkv, Sk, D]  dtype
 *   alibi      [Hq] float32 or NULL
 *   dq         [B, Hq, Sq, D]   dtype
 *   dk, dv     [B, Hkv, Sk, D]  dtype
 *   workspace  >= attn_bwd_workspace_size(p) bytes, 16-byte aligned.
 * The outputs and the workspace overlap no input and no other output.  The
 * rules of attn_fwd_check apply to p, q, k, v and alibi. */
attn_status_t attn_bwd_check(const void* q, const void* k, const void* v, const void* dout,
                             const float* alibi, const void* dq, const void* dk,
                             const void* dv, const void* workspace, size_t workspace_bytes,
                             const attn_fwd_params_t* p);

/* Attention backward: validates as attn_bwd_check, then enqueues three
 * kernels on `stream` (the forward's row statistics, dK/dV, dQ) and returns.
 * The workspace is scratch for the duration of the call; its contents
 * afterwards are unspecified. */
attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* dout,
                       const float* alibi, void* dq, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, const attn_fwd_params_t* p, void* stream);

/* Host-only validation of an attn_bwd_lse call (no HIP call is made): the
 * rules of attn_bwd_check, and
 *   out  [B, Hq, Sq, D] dtype    the output attn_fwd_lse returned for q, k, v,
 *                                alibi and p;
 *   lse  [B, Hq, Sq] float32     its natural-log LSE (-inf for a row without
 *                                keys), 4-byte aligned;
 * both required when B * Hq * Sq > 0, both read only, neither overlapping
 * dq, dk, dv or the workspace. */
attn_status_t attn_bwd_lse_check(const void* q, const void* k, const void* v, const void* out,
                                 const float* lse, const void* dout, const float* alibi,
                                 const void* dq, const void* dk, const void* dv,
                                 const void* workspace, size_t workspace_bytes,
                                 const attn_fwd_params_t* p);

/* The gradients of attn_bwd (kernel-contract page, attention_flash_backward)
 * for a caller that kept the forward's output and LSE (attn_fwd_lse): S and P
 * are still recomputed per key block as in attn_bwd, but the two per-row
 * quantities that attn_bwd gets by re-running the forward -- the softmax
 * normaliser and sum_j P dP = dO . O -- come from lse and from the rounded
 * out, so that pass is skipped.  Same workspace, outputs and determinism as
 * attn_bwd; the gradients agree with attn_bwd's to rounding (dO . O from the
 * rounded output here, from the float32 accumulator there).  F32/F64
 * recompute the statistics in the element type as attn_bwd does (out and
 * lse are validated but not read), so their gradients equal attn_bwd's. */
attn_status_t attn_bwd_lse(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, const void* dout, const float* alibi, void* dq,
                           void* dk, void* dv, void* workspace, size_t workspace_bytes,
                           const attn_fwd_params_t* p, void* stream);

/* Static string naming a status code. */
const char* attn_status_str(attn_status_t status);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
