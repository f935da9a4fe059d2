// launch.h -- internal interface between the C ABI (attn_api.cpp) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Dense forward problem, sizes narrowed to int after validation.
struct FwdProblem {
  const void* q;
  const void* k;
  const void* v;
  const float* alibi;  // [Hq] float32 or nullptr
  void* out;
  float* lse;     // [B, Hq, Sq] float32 natural-log LSE of each row, or nullptr
  // backward support (matrix-core path): with dout [B, Hq, Sq, D], stats
  // [B, Hq, Sq] of float pairs (log2-unit LSE, +inf without keys; dO . O)
  const void* dout = nullptr;
  float* stats = nullptr;
  int B, Hq, Hkv, Sq, Sk, D;
  int causal;
  int wl, wr;     // window; -1 = unbounded (already clamped to the useful range)
  float scale;    // softmax scale
  float softcap;  // 0 = off
};

// Variable-length prefill over the paged pool (queries packed by a prefix sum).
struct PagedPrefillProblem {
  const void* q;          // [total_q, Hq, D]
  const void* k_pool;     // [num_blocks, block_size, Hkv, D]
  const void* v_pool;
  const int32_t* block_table;   // [B, max_blocks]
  const int32_t* seq_lens;      // [B] live keys
  const int32_t* cu_seqlens_q;  // [B + 1]
  const float* alibi;
  void* out;              // [total_q, Hq, D]
  int32_t* error_flag;
  int B, Hq, Hkv, D, total_q, max_sq;
  int num_blocks, block_size, max_blocks;
  int causal;
  int wl, wr;             // -1 = unbounded (already clamped to the useful range)
  float scale, softcap;
};

// Paged decode problem.
struct DecodeProblem {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const float* alibi;
  void* out;
  float* ws_o;    // [B, Hq, splits, D] float32 partial outputs
  float* ws_lse;  // [B, Hq, splits] float32 log-sum-exp (natural log)
  int32_t* error_flag;
  int B, Hq, Hkv, D;
  int num_blocks, block_size, max_blocks;
  int splits;
  float scale;
  float softcap;
};

// Backward (matrix-core path): dQ, dK, dV from Q, K, V, dO and the forward's
// per-row statistics.
struct BwdProblem {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;     // [B, Hq, Sq, D]
  const float* alibi;   // [Hq] float32 or nullptr
  const float* stats;   // [B, Hq, Sq] float pairs written by the forward (FwdProblem::stats)
  void* dq;             // [B, Hq, Sq, D]
  void* dk;             // [B, Hkv, Sk, D]
  void* dv;
  int B, Hq, Hkv, Sq, Sk, D;
  int causal;
  int wl, wr;
  float scale;
  float softcap;
};

// 0 = F32, 1 = F16, 2 = BF16 (attn_dtype_t).
hipError_t launch_fwd_mfma(const FwdProblem& p, int dtype, hipStream_t stream);
hipError_t launch_fwd_valu(const FwdProblem& p, bool f64, hipStream_t stream);
hipError_t launch_paged_prefill(const PagedPrefillProblem& p, int dtype, hipStream_t stream);
hipError_t launch_paged_decode(const DecodeProblem& p, int dtype, hipStream_t stream);
hipError_t launch_bwd_mfma(const BwdProblem& p, int dtype, hipStream_t stream);

}  // namespace attn
