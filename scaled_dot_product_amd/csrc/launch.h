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
  int B, Hq, Hkv, Sq, Sk, D;  // Sk: live keys (the k_len prefix when one is given)
  int kv_stride = 0;          // keys between consecutive (sequence, KV head) slices of k and v (>= Sk)
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
  // dK/dV work split: a 128-key block's (head, 32-query tile) items are cut
  // into chunks of chunk_items; a block of more than one chunk sums float32
  // partials (`partials`, max_chunks slots per block) in a second pass
  int chunk_items, max_chunks;
  float* partials;
};

// Items (query heads x 32-query tiles) that see key block kb of 128 keys.
inline int bwd_kv_items(int kb, int Sq, int Sk, int group, int causal, int wl, int wr) {
  const bool has_hi = causal || wr >= 0;
  const int dmax = causal ? 0 : wr;  // causal: j <= i' (a right window cannot widen it)
  const int off = Sk - Sq;
  const int k0 = kb * 128;
  const int k_last = (k0 + 128 < Sk ? k0 + 128 : Sk) - 1;
  if (k_last < k0) return 0;
  int q_lo = has_hi ? k0 - dmax - off : 0;
  if (q_lo < 0) q_lo = 0;
  int q_hi = wl >= 0 ? k_last + wl - off + 1 : Sq;
  if (q_hi > Sq) q_hi = Sq;
  if (q_hi <= q_lo) return 0;
  const int nt = (q_hi + 31) / 32 - q_lo / 32;
  return nt * group;
}

// Chunk size (items per dK/dV workgroup) and the most chunks any key block
// needs.  The dK/dV workgroups run one per compute unit, so they go through
// the chip in rounds of kBwdSlots, and a round lasts about as long as its
// largest chunk.  For one and for two rounds the smallest chunk size whose
// workgroups fit is found by bisection (the workgroup count falls as the
// chunk grows); the smaller (rounds x size) wins, ties going to the larger
// chunk (fewer float32 partials to sum).  Work that needs more than two
// rounds of whole key blocks is not split at all.  Chunks hold at least 16
// items.  More rounds of smaller chunks lose in practice (each workgroup pays
// its K/V loads and its partial): a sweep of fixed chunk sizes on causal
// 2048-, 4096- and 8192-token GQA backwards, a non-causal 1024-token one and
// a D = 64 one put the best size at the one that fills two rounds (or one,
// for the non-causal shape), and this rule picks it on all five.
constexpr long long kBwdSlots = 256;   // dK/dV workgroups resident at once (one per CU of the chip)
constexpr int kBwdMaxRounds = 2;
inline void bwd_chunking(int B, int Hkv, int Hq, int Sq, int Sk, int D, int causal, int wl, int wr,
                         int* chunk_items, int* max_chunks) {
  const int group = Hkv > 0 ? Hq / Hkv : 0;
  const int nkb = (Sk + 127) / 128;
  const long long copies = (long long)B * Hkv * (D > 128 ? 2 : 1);  // workgroups per chunk
  int most = 0;
  for (int kb = 0; kb < nkb; ++kb) {
    const int n = bwd_kv_items(kb, Sq, Sk, group, causal, wl, wr);
    most = n > most ? n : most;
  }
  if (most == 0) {
    *chunk_items = 16;
    *max_chunks = 1;
    return;
  }
  auto workgroups = [&](long long L) {
    long long w = 0;
    for (int kb = 0; kb < nkb; ++kb) {
      const int n = bwd_kv_items(kb, Sq, Sk, group, causal, wl, wr);
      w += (n + L - 1) / L;
    }
    return w * copies;
  };
  long long best_L = most, best_cost = -1;
  for (int r = 1; r <= kBwdMaxRounds; ++r) {
    const long long cap = r * kBwdSlots;
    long long L;
    if (workgroups(most) > cap) {
      L = most;  // even whole blocks take more rounds
    } else {
      long long lo = 16, hi = most;  // smallest L in [16, most] with workgroups(L) <= cap
      if (lo > hi) lo = hi;
      while (lo < hi) {
        const long long mid = (lo + hi) / 2;
        if (workgroups(mid) <= cap) hi = mid;
        else lo = mid + 1;
      }
      L = lo;
    }
    const long long rounds = (workgroups(L) + kBwdSlots - 1) / kBwdSlots;
    const long long cost = rounds * L;
    if (best_cost < 0 || cost < best_cost || (cost == best_cost && L > best_L)) {
      best_cost = cost;
      best_L = L;
    }
  }
  *chunk_items = (int)best_L;
  *max_chunks = (int)((most + best_L - 1) / best_L);
}

// 0 = F32, 1 = F16, 2 = BF16 (attn_dtype_t).
hipError_t launch_fwd_mfma(const FwdProblem& p, int dtype, hipStream_t stream);
hipError_t launch_fwd_valu(const FwdProblem& p, bool f64, hipStream_t stream);
// Vector-ALU paged forward (F32/F64): packed queries with a prefix sum, or,
// with cu_seqlens_q == nullptr, one query per sequence (row b: decode).
hipError_t launch_paged_valu(const PagedPrefillProblem& p, bool f64, hipStream_t stream);
hipError_t launch_paged_prefill(const PagedPrefillProblem& p, int dtype, hipStream_t stream);
hipError_t launch_paged_decode(const DecodeProblem& p, int dtype, hipStream_t stream);
// Device address of the current device's copy of the allocation-free decode
// workspace (ATTN_DECODE_SCRATCH_BYTES), or nullptr if it cannot be found.
void* decode_scratch();
hipError_t launch_bwd_mfma(const BwdProblem& p, int dtype, hipStream_t stream);
// Vector-ALU backward (F32/F64): `stats` holds two values of the element type
// per query row; the chunking fields of p are not used.
hipError_t launch_bwd_valu(const BwdProblem& p, bool f64, void* stats, hipStream_t stream);
// Backward row statistics (BwdProblem::stats) from a saved forward: out and
// dout [rows, D] of the dtype, lse [rows] float32 natural-log LSE.
hipError_t launch_bwd_rowstats(const void* out, const void* dout, const float* lse, float* stats,
                               long long rows, int D, int dtype, hipStream_t stream);

}  // namespace attn
