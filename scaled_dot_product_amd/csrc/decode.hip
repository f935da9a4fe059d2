// decode.hip -- paged-KV split-KV decode: partial pass + log-sum-exp merge.
//
// What is computed is the kernel-contract page's attention_paged_naive
// ("fuel-reference-backend -- attention kernel contracts"): the key at logical
// position t of sequence b lives in block block_table[b, t / block_size], slot
// t % block_size, of a [num_blocks, block_size, Hkv, D] pool; the single decode
// query sits at seq_len - 1 and so sees every live key (derivation page,
// section 4).  The key dimension is split across workgroups and the partial
// results are combined afterwards (derivation page, section 8); the combine
// re-bases each part to a common max exactly as the section-3 recurrence
// re-bases tiles.
//
// Three forms, chosen by the launcher:
//   * fused persistent (block_size % 16 == 0, B <= 256, at least one
//     (sequence, KV head, 16-head chunk) group per compute unit): one
//     workgroup per compute unit walks whole groups; its waves stream equal
//     token chunks of a group and merge them through LDS, writing the output;
//   * split persistent (block_size % 16 == 0, B <= 256, smaller batches):
//     every wave walks (split, group) items and writes a partial per item,
//     combined by the merge kernel;
//   * partial kernel (any block size or batch): one workgroup per (split,
//     group), then the merge kernel.
// Common to all: both products run on the matrix cores with the query heads
// of the KV head as the N dimension (up to 16, padded):
//     S^T = K Q^T    16x16x32, gathered key rows as the A operand straight
//                    from the pool (64 contiguous bytes per 4 lanes);
//     O^T += V^T P^T 16x16x16, where the S^T accumulator (4 tokens of one
//                    head per lane) is already the P^T operand and V^T comes
//                    from a per-wave LDS block through the transpose read.
// Every lane therefore owns one head: softmax state, rescale and output need
// no cross-lane reduction except the block max over 4 lane groups.  Loads run
// two 16-token blocks ahead.  When every 16-token block lies inside one KV
// block (block_size % 16 == 0) the physical block of a whole block is one
// wave-uniform value: a wave reads the page ids of its next 63 blocks in one
// load and broadcasts them with readlane, and the loads go through a buffer
// descriptor whose size ends at the chunk's last live token (later rows read
// as zero, no branches).  Other block sizes translate every token separately.
// Sequences are taken longest first (each workgroup ranks the lengths
// itself).  Partials are the normalised o[D] and its natural-log LSE per
// (sequence, head, split) in the caller's workspace; the merge kernel takes 4
// d per thread, combines the splits in fixed order and casts to the input
// type.
#include <limits.h>

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kTB = 16;         // tokens per block
constexpr int kRankMax = 2048;  // batches up to this size (and the LDS it fits) go longest-first
constexpr int kPageWindow = 63; // blocks per page-id window: <= 64 lanes, a multiple of the ring size
constexpr float kRescaleGap = 8.0f;

struct DecArgs {
  const void* q;
  const void* kp;
  const void* vp;
  const int32_t* table;
  const int32_t* lens;
  const float* alibi;
  float* ws_o;
  float* ws_lse;
  void* out;      // [B, Hq, D] (the fused persistent form writes it directly)
  int32_t* err;
  int B, Hq, Hkv, group, hchunks, num_blocks, bs, maxb, splits;
  int softcap;
  float c_score;  // log2(e) * scale; with softcap 2 * log2(e) * scale / cap
  float c_cap;    // log2(e) * cap
};

// max / sum of x over lanes l, l^16, l^32, l^48 (the four lane groups).
__device__ __forceinline__ float groups_max(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __builtin_fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
  return halves_max(x);
}
__device__ __forceinline__ float groups_sum(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
  return halves_sum(x);
}

template <typename T>
__device__ __forceinline__ floatx4 mma16x16x16(u32x2 a, u32x2 b, floatx4 c);
template <>
__device__ __forceinline__ floatx4 mma16x16x16<__bf16>(u32x2 a, u32x2 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ floatx4 mma16x16x16<_Float16>(u32x2 a, u32x2 b, floatx4 c) {
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                               __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// XOR swizzle of the 16-byte chunk of V row r in the per-wave LDS block, so
// that the transpose reads (4 rows x 2 chunks per 16 lanes) hit distinct banks.
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D >= 128 ? ((r & 7) << 1) : (((r >> 1) & 3) << 1);
}

// Block copies are issued as global -> LDS copies in inline asm, so that the
// compiler neither counts them nor inserts waits of its own (they have no
// register result): the loop below keeps a fixed number of copies in flight
// and waits, with wait_vmem_le, for exactly the ones it is about to read.
// The K/V pool is read once per decode, so the copies are non-temporal.
__device__ __forceinline__ void asm_dma16(__amdgpu_buffer_rsrc_t rs, uint32_t lds_addr, int voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :: "s"(m0), "v"(voff), "s"(rs) : "memory", "m0");
}
// Waits until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// XOR swizzle of the 16-byte chunk of K row r in the per-wave LDS block, so
// that the operand reads (16 rows, one chunk each, per 16 lanes) hit distinct
// banks.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D >= 128 ? (r & 15) : ((r >> 1) & 7);
}

template <typename T, int D, int PF, bool UNIFORM, int NW>
__global__ __launch_bounds__(64 * NW) void decode_partial_kernel(DecArgs a) {
  constexpr int kWaves = NW;
  constexpr int kThreads = 64 * NW;
  using E = Elem<T>;
  constexpr int KS = D / 32;          // 16x16x32 steps of S^T over d
  constexpr int NCH = D / 8;          // 16-byte chunks per row
  constexpr int ROWS = 64 / NCH;      // rows per copy instruction (1 KiB each)
  constexpr int CPB = kTB / ROWS;     // copy instructions per block and tensor
  constexpr int DB = D / 16;          // 16-row blocks of O^T
  constexpr int NS = PF + 1;          // blocks in the prefetch ring
  constexpr int SLOT = kTB * NCH;     // 16-byte chunks of one K (or V) block
  constexpr int LOADS = 2 * CPB;      // vector-memory operations per block
  static_assert(NS == 3 && kPageWindow % NS == 0, "ring slots must follow the unroll index");
  static_assert(2 * SLOT * 16 >= 16 * D * 4, "two K slots hold the wave totals");
  constexpr int RANK_MAX = kWaves * SLOT * 4 < kRankMax ? kWaves * SLOT * 4 : kRankMax;  // ints in kring2
  // Per wave: rings of NS K blocks and NS V blocks (row-major, swizzled
  // chunks), one LDS object per slot so that the slot being filled is never
  // confused with the one being read.  Afterwards K slots 0 and 1 hold the
  // wave's totals (heads 0-7 and 8-15).
  __shared__ u32x4 kring0[kWaves][SLOT], kring1[kWaves][SLOT], kring2[kWaves][SLOT];
  __shared__ u32x4 vring0[kWaves][SLOT], vring1[kWaves][SLOT], vring2[kWaves][SLOT];
  __shared__ float m_lds[kWaves][16];
  __shared__ float l_lds[kWaves][16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4, hl = lane & 15;
  const int split = blockIdx.x;

  // ---- sequence of this workgroup: the blockIdx.z-th longest (ties by index),
  // so that the dispatcher issues the longest splits first and the short ones
  // fill the tail.  The ranks are a permutation of 0..B-1.
  int b = blockIdx.z;
  if (a.B <= RANK_MAX) {
    int* lens_lds = reinterpret_cast<int*>(kring2);  // free until the main loop
    __shared__ int s_seq;
    for (int i = tid; i < a.B; i += kThreads) lens_lds[i] = a.lens[i];
    __syncthreads();
    for (int i = tid; i < a.B; i += kThreads) {
      const int li = lens_lds[i];
      int r = 0;
      for (int j = 0; j < a.B; ++j) {
        const int lj = lens_lds[j];
        r += (lj > li || (lj == li && j < i)) ? 1 : 0;
      }
      if (r == (int)blockIdx.z) s_seq = i;
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(s_seq);
  }
  const int kvh = blockIdx.y / a.hchunks, hc = blockIdx.y - kvh * a.hchunks;
  const int h0 = kvh * a.group + hc * 16;
  const int nh = min(16, a.group - hc * 16);

  // live length, clamped into the table's capacity (flagged when outside)
  const int cap = a.maxb * a.bs;
  int ctx = __builtin_amdgcn_readfirstlane(a.lens[b]);  // one value per workgroup
  if (ctx < 0 || ctx > cap) {
    if (a.err && tid == 0) *a.err = 1;
    ctx = ctx < 0 ? 0 : cap;
  }
  const int per = (ctx + a.splits - 1) / a.splits;
  const int chunk = (per + kTB - 1) / kTB * kTB;
  const int t0 = min(ctx, split * chunk);
  const int t1 = min(ctx, t0 + chunk);
  const int nblk = (t1 - t0 + kTB - 1) / kTB;
  const int nj = wave < nblk ? (nblk - wave + kWaves - 1) / kWaves : 0;  // this wave's blocks

  // Q^T as the B operand: lane -> head hl, d = 32 ks + 8 g .. +7
  const T* Qb = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.Hq + h0) * D;
  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = hl < nh ? load16(Qb + hl * D + 32 * ks + 8 * g) : zero_u32x4();
  const float slope_l2 = (a.alibi && hl < nh) ? a.alibi[h0 + hl] * kLog2e : 0.f;
  const float qpos = (float)(ctx - 1);

  floatx4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_part = 0.f;

  const size_t tok_stride = (size_t)a.Hkv * D;  // elements between consecutive slots
  const T* Kp = reinterpret_cast<const T*>(a.kp) + (size_t)kvh * D;
  const T* Vp = reinterpret_cast<const T*>(a.vp) + (size_t)kvh * D;
  const int32_t* trow = a.table + (size_t)b * a.maxb;
  const int crow = lane / NCH, cch = lane % NCH;  // copy layout: chunk cch of rows crow + ROWS i

  int page_reg = 0;  // lane j: physical block of this wave's block (window + j)
  auto load_pages = [&](int j0) {
    const int j = j0 + lane;
    page_reg = j < nj ? trow[(t0 + kTB * (wave + kWaves * j)) / a.bs] : 0;
  };
  auto kslot = [&](int u) -> u32x4* { return u == 0 ? kring0[wave] : (u == 1 ? kring1[wave] : kring2[wave]); };
  auto vslot = [&](int u) -> u32x4* { return u == 0 ? vring0[wave] : (u == 1 ? vring1[wave] : vring2[wave]); };
  // 32-bit LDS address of a slot chunk (folds to scalar arithmetic)
  auto lds_addr = [](const u32x4* p) { return (uint32_t)(uintptr_t)(const ATTN_LDS void*)p; };

  bool bad_page = false;  // a table entry outside the pool was met (wave-uniform)
  uint32_t valid[NS];     // per ring slot: bit t = token t of the block is live
  // Issues the copies of block j (window-relative index jw for its page id)
  // into ring slot u.  A block that is not `live` (past this window) is
  // padding: it keeps the ring rotating, but its copies read nothing.
  auto fetch = [&](int u, int j, int jw, bool live) {
    const int tb = __builtin_amdgcn_readfirstlane(t0 + kTB * (wave + kWaves * j));
    const int nvalid = live ? min(kTB, t1 - tb) : 0;
    u32x4* ks_ = kslot(u);
    u32x4* vs_ = vslot(u);
    if constexpr (UNIFORM) {
      const int phys = __builtin_amdgcn_readlane(page_reg, live ? jw : 0);
      const bool ok = nvalid > 0 && (unsigned)phys < (unsigned)a.num_blocks;
      bad_page |= nvalid > 0 && !ok;
      const long long row0 = ok ? ((long long)phys * a.bs + (tb % a.bs)) * (long long)tok_stride : 0;
      const long long bytes = ok ? (long long)nvalid * tok_stride * sizeof(T) : 0;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kp + row0, bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vp + row0, bytes);
#pragma unroll
      for (int i = 0; i < CPB; ++i) {
        const int r = crow + ROWS * i;
        asm_dma16(rk, lds_addr(ks_ + i * 64), (int)((r * tok_stride + 8 * (cch ^ swz_k<D>(r))) * sizeof(T)));
        asm_dma16(rv, lds_addr(vs_ + i * 64), (int)((r * tok_stride + 8 * (cch ^ swz_v<D>(r))) * sizeof(T)));
      }
      valid[u] = ok ? (nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u)) : 0u;
    } else {
      // per-token translation: any block size (synchronous staging)
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < CPB; ++i) {
        const int r = crow + ROWS * i;
        const int t = tb + r;
        long long row = -1;
        if (live && t < t1) {
          const int page = t / a.bs;
          const int phys = trow[page];
          if ((unsigned)phys < (unsigned)a.num_blocks)
            row = ((long long)phys * a.bs + (t - page * a.bs)) * (long long)tok_stride;
          else if (a.err)
            *a.err = 1;
        }
        ks_[r * NCH + (cch ^ swz_k<D>(r))] = row >= 0 ? load16(Kp + row + 8 * cch) : zero_u32x4();
        vs_[r * NCH + (cch ^ swz_v<D>(r))] = row >= 0 ? load16(Vp + row + 8 * cch) : zero_u32x4();
        // row crow + ROWS i is live iff its chunk-0 lane (lane crow * NCH) found it
        const uint64_t m = __builtin_amdgcn_ballot_w64(row >= 0 && cch == 0);
#pragma unroll
        for (int rr = 0; rr < ROWS; ++rr)
          bits |= ((m >> (rr * NCH)) & 1ull) ? (1u << (rr + ROWS * i)) : 0u;
      }
      valid[u] = bits;
    }
  };

  auto compute = [&](int u, int j) {
    const int tb = t0 + kTB * (wave + kWaves * j);
    // Every block is followed by exactly PF fetches (padding included), so this
    // block's copies have landed once at most PF * LOADS operations remain.
    if constexpr (UNIFORM) wait_vmem_le<PF * LOADS>();
    const u32x4* ks_ = kslot(u);
    const T* vs = reinterpret_cast<const T*>(vslot(u));
    // S^T = K Q^T: A operand lane (g, hl) = K row hl, d = 32 ks + 8 g .. +7
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s = E::mma16(ks_[hl * NCH + ((4 * ks + g) ^ swz_k<D>(hl))], qf[ks], s);
    // s[r]: head hl, token 4 g + r
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = s[r];
      if (a.softcap) {
        const float ex = fast_exp2(x * a.c_score);
        x = a.c_cap - 2.f * a.c_cap * fast_rcp(1.f + ex);
      } else {
        x *= a.c_score;
      }
      const int tok = 4 * g + r;
      x = __builtin_fmaf(slope_l2, (float)(tb + tok) - qpos, x);
      s[r] = ((valid[u] >> tok) & 1u) ? x : kNegInf;
      mx = __builtin_fmaxf(mx, s[r]);
    }
    mx = groups_max(mx);
    const bool need = mx > m_run + kRescaleGap;
    if (wave_any(need)) {
      const float alpha = need ? fast_exp2(m_run - mx) : 1.f;
      m_run = need ? mx : m_run;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    const uint32_t p01 = E::pack2(fast_exp2(s[0] - m_use), fast_exp2(s[1] - m_use));
    const uint32_t p23 = E::pack2(fast_exp2(s[2] - m_use), fast_exp2(s[3] - m_use));
    l_part = E::dot2(p01, E::kOnePair, l_part);
    l_part = E::dot2(p23, E::kOnePair, l_part);
    const u32x2 pf = {p01, p23};
    // O^T += V^T P^T: A operand lane (g, hl) = V[4 g + 0..3][16 db + hl]
    const int tr_row = 4 * g + (hl >> 2);
    const int sw = swz_v<D>(tr_row);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 16 * db + 4 * (hl & 3);
      const u32x2 va = lds_read_tr16(vs + tr_row * D + ((col >> 3) ^ sw) * 8 + (col & 7));
      o[db] = mma16x16x16<T>(va, pf, o[db]);
    }
  };

  // ---- main loop: PF blocks in flight ahead of the one being computed, in
  // windows of kPageWindow blocks (one page-id load per window).
  for (int c0 = 0; c0 < nj; c0 += kPageWindow) {
    const int cn = min(kPageWindow, nj - c0);
    if constexpr (UNIFORM) load_pages(c0);
#pragma unroll
    for (int p = 0; p < PF; ++p) fetch(p, c0 + p, p, p < cn);
    for (int j0 = 0; j0 < cn; j0 += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int jw = j0 + u;  // window-relative
        const int jf = jw + PF;
        fetch((u + PF) % NS, c0 + jf, jf, jf < cn);
        if (jw < cn) compute(u, c0 + jw);
      }
    }
  }
  wait_vmem_le<0>();  // padding copies into the slots reused below have landed
  if (bad_page && a.err && lane == 0) *a.err = 1;

  // ---- wave totals: l over the 4 lane groups; o is already complete per lane
  const float l = groups_sum(l_part);
  float* ow = reinterpret_cast<float*>(hl < 8 ? kring0[wave] : kring1[wave]) + (hl & 7) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) *reinterpret_cast<floatx4*>(ow + 16 * db + 4 * g) = o[db];
  if (g == 0) {
    m_lds[wave][hl] = m_run;
    l_lds[wave][hl] = l;
  }
  __syncthreads();

  // ---- merge the 4 waves, write the split's normalised output and LSE
  for (int idx = tid; idx < nh * D; idx += kThreads) {
    const int hh = idx / D, d = idx - hh * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = __builtin_fmaxf(M, m_lds[w][hh]);
    float ov = 0.f, lse = kNegInf;
    if (M != kNegInf) {
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = fast_exp2(m_lds[w][hh] - M);
        const float* tw = reinterpret_cast<const float*>(hh < 8 ? kring0[w] : kring1[w]);
        num = __builtin_fmaf(wt, tw[(hh & 7) * D + d], num);
        den = __builtin_fmaf(wt, l_lds[w][hh], den);
      }
      if (den > 0.f) {
        ov = num / den;
        lse = (M + __log2f(den)) * kLn2;
      }
    }
    const size_t slot = ((size_t)b * a.Hq + h0 + hh) * a.splits + split;
    a.ws_o[slot * D + d] = ov;
    if (d == 0) a.ws_lse[slot] = lse;
  }
}

// Four transpose reads of LDS (byte addresses a[0..3]) in one asm statement that
// also waits for them: the compiler does not see these reads, so it adds no
// wait of its own for the copies still landing in the other ring slots, and
// every output is written when the statement ends.
__device__ __forceinline__ void lds_tr4(u32x2 (&v)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

// Persistent form for block sizes that are multiples of kTB.  The grid fills
// the chip once (8 waves per compute unit, the rate at which the pool streams
// best) and every wave is an independent worker over whole work items, item =
// (split, KV head, head chunk, sequence), taken in order of decreasing
// sequence length (ties by index) and dealt in snake order (round k: wave w
// takes rank k W + w, or k W + W - 1 - w on odd rounds) so that each wave's
// total is close to the mean; within a sequence the items go split-major, so
// waves running side by side read the same token rows.
// Per block the K rows go straight into registers in the A-operand layout and
// the V rows into the wave's 3-slot LDS ring (two blocks ahead).  A worker
// ends an item by storing its normalised partial and LSE from registers and
// goes straight on with the next item, whose Q and first page ids it loaded
// one item earlier: no wave waits for its stores to be acknowledged, and no
// item starts cold.  Every load and copy is one the compiler counts, so its
// waits are exact; only the V transpose reads are inline asm, after an
// explicit wait for that block's copies.
//
// Fused form (FUSED; the launcher picks it when there are at least as many
// (sequence, KV head, head chunk) groups as compute units but few items per
// compute unit, or for long contexts above the split form's batch limit): the
// worker is the whole workgroup and the item is a group; wave w streams the
// w-th of NW equal token chunks of the group, and at the group's end the NW
// partial states meet in the waves' ring slots and the workgroup writes the
// output itself (the same re-basing to a common max as the merge kernel), so
// there is neither a workspace round trip nor a second launch.
// Batches are ordered longest-first: up to kOrdMax sequences by counting, above
// that by a sort, up to kOrdMaxSplit (split form) or kOrdMaxFused (fused form:
// one workgroup per compute unit, so more LDS) sequences.
constexpr int kOrdMax = 256;
constexpr int kOrdMaxSplit = 2048;
constexpr int kOrdMaxFused = 4096;   // (a 12-bit sequence index in the sort key)
constexpr int kStreamWaves = 4;
template <bool FUSED, int D>
constexpr int stream_waves() { return FUSED ? (D <= 128 ? 8 : 4) : kStreamWaves; }

template <typename T, int D, bool FUSED>
__global__ __launch_bounds__((64 * stream_waves<FUSED, D>())) void decode_stream_kernel(DecArgs a) {
  using E = Elem<T>;
  constexpr int NW = stream_waves<FUSED, D>();
  constexpr int KS = D / 32;          // 16x16x32 steps of S^T over d
  constexpr int NCH = D / 8;          // 16-byte chunks per row
  constexpr int ROWS = 64 / NCH;      // rows per V copy instruction
  constexpr int CPB = kTB / ROWS;     // V copy instructions per block
  constexpr int DB = D / 16;          // 16-row blocks of O^T
  constexpr int PF = 2;
  constexpr int NS = PF + 1;
  constexpr int SLOT = kTB * NCH;
  static_assert(NS == 3 && kPageWindow % NS == 0 && DB % 4 == 0, "ring and read batches");
  __shared__ u32x4 vring0[NW][SLOT], vring1[NW][SLOT], vring2[NW][SLOT];
  constexpr int ORD = FUSED ? kOrdMaxFused : kOrdMaxSplit;
  __shared__ int ord[ORD], lens_lds[ORD];
  __shared__ float2 ml_x[FUSED ? NW : 1][16];  // fused: per wave and head, (max, sum)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, hl = lane & 15;

  // ---- ord[r] = the r-th longest sequence, ties by index (the launcher
  // guarantees B <= ORD); the lengths stay in LDS so that no item start waits
  // on a global load.  Up to kOrdMax sequences each thread counts the longer
  // ones (B^2 / threads steps); above that a bitonic sort of packed keys in
  // ord (log2(n) (log2(n) + 1) / 2 passes over n = B rounded up to a power of
  // two).  Either way every workgroup derives the same order.
  const bool big = a.B > kOrdMax;
  int npow = 1;
  while (big && npow < a.B) npow <<= 1;
  unsigned* key = reinterpret_cast<unsigned*>(ord);
  for (int i = tid; i < (big ? npow : a.B); i += 64 * NW) {
    const int l = i < a.B ? a.lens[i] : 0;
    if (i < a.B) lens_lds[i] = l;
    // length (clamped to 20 bits) descending, then index ascending, as one
    // ascending unsigned key; padding sorts last
    if (big)
      key[i] = i < a.B ? ((0xFFFFFu - (unsigned)min(max(l, 0), 0xFFFFF)) << 12) | (unsigned)i : 0xFFFFFFFFu;
  }
  __syncthreads();
  if (!big) {
    for (int i = tid; i < a.B; i += 64 * NW) {
      const int li = lens_lds[i];
      int r = 0;
      for (int j = 0; j < a.B; ++j) {
        const int lj = lens_lds[j];
        r += (lj > li || (lj == li && j < i)) ? 1 : 0;
      }
      ord[r] = i;
    }
  } else {
    for (int k = 2; k <= npow; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int p = tid; p < npow / 2; p += 64 * NW) {
          const int lo = ((p & ~(j - 1)) << 1) | (p & (j - 1));   // bit j clear; partner lo + j
          const unsigned x = key[lo], y = key[lo + j];
          if ((x > y) == ((lo & k) == 0)) {
            key[lo] = y;
            key[lo + j] = x;
          }
        }
        __syncthreads();
      }
    for (int r = tid; r < a.B; r += 64 * NW) ord[r] = (int)(key[r] & 0xFFFu);
  }
  __syncthreads();

  const int nhc = a.Hkv * a.hchunks;
  const int splits = FUSED ? 1 : a.splits;
  const int per_seq = nhc * splits;
  const int n_items = a.B * per_seq;
  const int W = FUSED ? gridDim.x : gridDim.x * NW;    // workers
  const int gw = FUSED ? blockIdx.x : blockIdx.x * NW + wave;
  const size_t tok_stride = (size_t)a.Hkv * D;
  const int crow = lane / NCH, cch = lane % NCH;
  const int cap = a.maxb * a.bs;
  auto vslot = [&](int u) -> u32x4* { return u == 0 ? vring0[wave] : (u == 1 ? vring1[wave] : vring2[wave]); };
  auto lds_addr = [](const void* p) { return (uint32_t)(uintptr_t)(const ATTN_LDS void*)p; };
  bool bad_page = false, bad_len = false;

  // ---- the k-th item of this wave (wave-uniform fields)
  struct Item { int b, kvh, h0, nh, split, ctx, t0, t1, nj; };
  auto item_of = [&](int k, Item& it) -> bool {
    const int base = k * W;
    if (base >= n_items) return false;
    const int r = base + ((k & 1) ? (W - 1 - gw) : gw);
    if (r >= n_items) return false;
    const int sr = r / per_seq;
    const int rem = r - sr * per_seq;
    it.split = rem / nhc;
    const int y = rem - it.split * nhc;
    it.b = __builtin_amdgcn_readfirstlane(ord[sr]);
    it.kvh = y / a.hchunks;
    const int hc = y - it.kvh * a.hchunks;
    it.h0 = it.kvh * a.group + hc * 16;
    it.nh = min(16, a.group - hc * 16);
    int ctx = __builtin_amdgcn_readfirstlane(lens_lds[it.b]);
    if (ctx < 0 || ctx > cap) {
      bad_len = true;
      ctx = ctx < 0 ? 0 : cap;
    }
    it.ctx = ctx;
    const int parts = FUSED ? NW : a.splits;
    const int per = (ctx + parts - 1) / parts;
    const int chunk = (per + kTB - 1) / kTB * kTB;
    it.t0 = min(ctx, (FUSED ? wave : it.split) * chunk);
    it.t1 = min(ctx, it.t0 + chunk);
    it.nj = (it.t1 - it.t0 + kTB - 1) / kTB;
    return true;
  };
  // Q of an item as the B operand (lane: head hl, d = 32 ks + 8 g .. + 7) and
  // the physical blocks of its blocks c0 .. c0 + 62 (lane j: block c0 + j)
  auto load_q = [&](const Item& it, u32x4 (&q)[KS], float& slope) {
    const T* Qb = reinterpret_cast<const T*>(a.q) + ((size_t)it.b * a.Hq + it.h0) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      q[ks] = hl < it.nh ? load16(Qb + hl * D + 32 * ks + 8 * g) : zero_u32x4();
    slope = (a.alibi && hl < it.nh) ? a.alibi[it.h0 + hl] * kLog2e : 0.f;
  };
  auto load_pages = [&](const Item& it, int c0) -> int {
    const int j = c0 + lane;
    return j < it.nj ? a.table[(size_t)it.b * a.maxb + (it.t0 + kTB * j) / a.bs] : 0;
  };

  Item cur, nxt;
  bool have = item_of(0, cur);
  // the fused form ends every item with two barriers: it loads an item's Q
  // and page ids when it starts it; the split form loads them one item ahead
  bool have_nxt = !FUSED && have && item_of(1, nxt);
  u32x4 qf[KS], qn[KS];
  int page_reg = 0, page_nxt = 0;
  float slope_l2 = 0.f, slope_nxt = 0.f;
  if (have) {
    load_q(cur, qf, slope_l2);
    page_reg = load_pages(cur, 0);
  }
  if (have_nxt) {
    load_q(nxt, qn, slope_nxt);
    page_nxt = load_pages(nxt, 0);
  }

  u32x4 kr[NS][KS];   // K rows of ring slot u
  uint32_t valid[NS]; // per ring slot: bit t = token t of the block is live
  for (int k = 0; have; ++k) {
    const float qpos = (float)(cur.ctx - 1);
    floatx4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_part = 0.f;
    const T* Kp = reinterpret_cast<const T*>(a.kp) + (size_t)cur.kvh * D;
    const T* Vp = reinterpret_cast<const T*>(a.vp) + (size_t)cur.kvh * D;

    // Copies of block j (window-relative jw for its page id) into ring slot u,
    // non-temporal (the pool is read once);
    // a block that is not `live` is padding: it keeps every block followed by
    // exactly PF fetches, but reads nothing.
    auto fetch = [&](int u, int j, int jw, bool live) {
      const int tb = __builtin_amdgcn_readfirstlane(cur.t0 + kTB * j);
      const int nvalid = live ? min(kTB, cur.t1 - tb) : 0;
      const int phys = __builtin_amdgcn_readlane(page_reg, live ? jw : 0);
      const bool ok = nvalid > 0 && (unsigned)phys < (unsigned)a.num_blocks;
      bad_page |= nvalid > 0 && !ok;
      const long long row0 = ok ? ((long long)phys * a.bs + (tb % a.bs)) * (long long)tok_stride : 0;
      const long long bytes = ok ? (long long)nvalid * tok_stride * sizeof(T) : 0;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kp + row0, bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vp + row0, bytes);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kr[u][ks] = __builtin_amdgcn_raw_buffer_load_b128(
            rk, (int)((hl * tok_stride + 32 * ks + 8 * g) * sizeof(T)), 0, kLoadStream);
      u32x4* vs_ = vslot(u);
#pragma unroll
      for (int i = 0; i < CPB; ++i) {
        const int r = crow + ROWS * i;
        dma16<kLoadStream>(rv, vs_ + i * 64, (int)((r * tok_stride + 8 * (cch ^ swz_v<D>(r))) * sizeof(T)));
      }
      valid[u] = ok ? (nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u)) : 0u;
    };

    auto compute = [&](int u, int j) {
      const int tb = cur.t0 + kTB * j;
      const T* vs = reinterpret_cast<const T*>(vslot(u));
      // S^T = K Q^T: A operand lane (g, hl) = K row hl, d = 32 ks + 8 g .. + 7
      floatx4 sv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sv = E::mma16(kr[u][ks], qf[ks], sv);
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = sv[r];
        if (a.softcap) {
          const float ex = fast_exp2(x * a.c_score);
          x = a.c_cap - 2.f * a.c_cap * fast_rcp(1.f + ex);
        } else {
          x *= a.c_score;
        }
        const int tok = 4 * g + r;
        x = __builtin_fmaf(slope_l2, (float)(tb + tok) - qpos, x);
        sv[r] = ((valid[u] >> tok) & 1u) ? x : kNegInf;
        mx = __builtin_fmaxf(mx, sv[r]);
      }
      mx = groups_max(mx);
      const bool need = mx > m_run + kRescaleGap;
      if (wave_any(need)) {
        const float alpha = need ? fast_exp2(m_run - mx) : 1.f;
        m_run = need ? mx : m_run;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
      const float m_use = m_run == kNegInf ? 0.f : m_run;
      const uint32_t p01 = E::pack2(fast_exp2(sv[0] - m_use), fast_exp2(sv[1] - m_use));
      const uint32_t p23 = E::pack2(fast_exp2(sv[2] - m_use), fast_exp2(sv[3] - m_use));
      l_part = E::dot2(p01, E::kOnePair, l_part);
      l_part = E::dot2(p23, E::kOnePair, l_part);
      const u32x2 pf = {p01, p23};
      // O^T += V^T P^T: A operand lane (g, hl) = V[4 g + 0..3][16 db + hl];
      // this block's V copies have landed once at most PF later fetches (KS
      // loads + CPB copies each) remain in flight
      wait_vmem_le<PF * (KS + CPB)>();
      const int tr_row = 4 * g + (hl >> 2);
      const int sw = swz_v<D>(tr_row);
#pragma unroll
      for (int d4 = 0; d4 < DB; d4 += 4) {
        uint32_t ad[4];
        u32x2 va[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = 16 * (d4 + q) + 4 * (hl & 3);
          ad[q] = lds_addr(vs + tr_row * D + ((col >> 3) ^ sw) * 8 + (col & 7));
        }
        lds_tr4(va, ad);
#pragma unroll
        for (int q = 0; q < 4; ++q) o[d4 + q] = mma16x16x16<T>(va[q], pf, o[d4 + q]);
      }
    };

    for (int c0 = 0; c0 < cur.nj; c0 += kPageWindow) {
      const int cn = min(kPageWindow, cur.nj - c0);
      // items of more than one window: the next window's page ids load
      // while this one streams
      int page_win = 0;
      if (c0 + kPageWindow < cur.nj) page_win = load_pages(cur, c0 + kPageWindow);
#pragma unroll
      for (int p = 0; p < PF; ++p) fetch(p, c0 + p, p, p < cn);
      for (int j0 = 0; j0 < cn; j0 += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          const int jw = j0 + u;
          const int jf = jw + PF;
          fetch((u + PF) % NS, c0 + jf, jf, jf < cn);
          if (jw < cn) compute(u, c0 + jw);
        }
      }
      page_reg = page_win;
    }

    // ---- this item's partial: o / l and its LSE, per head (lane group g
    // holds d = 16 db + 4 g .. + 3)
    const float l = groups_sum(l_part);
    if constexpr (FUSED) {
      // every copy into this wave's ring has landed; heads 0..7 go to slot 0,
      // heads 8..15 to slot 1 (8 rows of D floats each)
      wait_vmem();
      float* ex = reinterpret_cast<float*>(hl < 8 ? vring0[wave] : vring1[wave]) + (hl & 7) * D + 4 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<floatx4*>(ex + 16 * db) = o[db];
      if (g == 0) ml_x[wave][hl] = float2{m_run, l};
      __syncthreads();
      constexpr int TPH = D / 4;             // threads per head, 4 d each
      constexpr int HPP = 64 * NW / TPH;     // heads per pass
      const int d4 = (tid % TPH) * 4;
      for (int h = tid / TPH; h < cur.nh; h += HPP) {
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float2 s = ml_x[w][h];
          M = s.y > 0.f ? __builtin_fmaxf(M, s.x) : M;
        }
        floatx4 num = {0.f, 0.f, 0.f, 0.f};
        float den = 0.f;
        if (M != kNegInf) {
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const float2 s = ml_x[w][h];
            if (s.y > 0.f) {
              const float c = fast_exp2(s.x - M);
              const float* src = reinterpret_cast<const float*>(h < 8 ? vring0[w] : vring1[w]) + (h & 7) * D + d4;
              const floatx4 v = *reinterpret_cast<const floatx4*>(src);
#pragma unroll
              for (int e = 0; e < 4; ++e) num[e] = __builtin_fmaf(c, v[e], num[e]);
              den = __builtin_fmaf(c, s.y, den);
            }
          }
        }
        const float inv = den > 0.f ? 1.f / den : 0.f;
        const u32x2 w2 = {E::pack2(num[0] * inv, num[1] * inv), E::pack2(num[2] * inv, num[3] * inv)};
        *reinterpret_cast<u32x2*>(reinterpret_cast<T*>(a.out) + ((size_t)cur.b * a.Hq + cur.h0 + h) * D + d4) = w2;
      }
      __syncthreads();  // the ring slots are free again
    } else if (hl < cur.nh) {
      const size_t slot = ((size_t)cur.b * a.Hq + cur.h0 + hl) * a.splits + cur.split;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* dst = a.ws_o + slot * D + 4 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        floatx4 w = o[db];
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] *= inv;
        *reinterpret_cast<floatx4*>(dst + 16 * db) = w;
      }
      if (g == 0) a.ws_lse[slot] = l > 0.f ? (m_run + __log2f(l)) * kLn2 : kNegInf;
    }

    // ---- next item.  Fused form: load its Q and page ids now.  Split form:
    // they arrived long ago; start those of the one after it.
    if constexpr (FUSED) {
      have = item_of(k + 1, cur);
      if (have) {
        load_q(cur, qf, slope_l2);
        page_reg = load_pages(cur, 0);
      }
      continue;
    }
    have = have_nxt;
    if (have) {
      cur = nxt;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = qn[ks];
      page_reg = page_nxt;
      slope_l2 = slope_nxt;
      have_nxt = item_of(k + 2, nxt);
      if (have_nxt) {
        load_q(nxt, qn, slope_nxt);
        page_nxt = load_pages(nxt, 0);
      }
    }
  }
  wait_vmem();  // no copy may still be writing this workgroup's LDS at exit
  if ((bad_page || bad_len) && a.err && lane == 0) *a.err = 1;
}

struct MergeArgs {
  const float* ws_o;
  const float* ws_lse;
  void* out;
  int splits;
  int nbh;  // B * Hq
};

// One thread per 4 consecutive d of one (sequence, head); a workgroup covers
// 256 / (D / 4) heads.  Every split's LSE and partial are loaded up front and
// combined in split order.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(MergeArgs a) {
  using E = Elem<T>;
  constexpr int TPH = D / 4;      // threads per (sequence, head)
  constexpr int HPW = 256 / TPH;  // (sequence, head) pairs per workgroup
  const int t = threadIdx.x;
  const size_t bh = (size_t)blockIdx.x * HPW + t / TPH;
  if (bh >= (size_t)a.nbh) return;
  const int d4 = (t % TPH) * 4;
  const float* lse = a.ws_lse + bh * a.splits;
  const float* o = a.ws_o + bh * a.splits * D + d4;
  float M = kNegInf;
#pragma unroll 8
  for (int s = 0; s < a.splits; ++s) M = __builtin_fmaxf(M, lse[s]);
  floatx4 r = {0.f, 0.f, 0.f, 0.f};
  if (M != kNegInf) {
    floatx4 num = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
#pragma unroll 8
    for (int s = 0; s < a.splits; ++s) {
      const float w = expf(lse[s] - M);
      const floatx4 v = *reinterpret_cast<const floatx4*>(o + (size_t)s * D);
#pragma unroll
      for (int c = 0; c < 4; ++c) num[c] = __builtin_fmaf(w, v[c], num[c]);
      den += w;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) r[c] = num[c] / den;
  }
  u32x2 w2 = {E::pack2(r[0], r[1]), E::pack2(r[2], r[3])};
  *reinterpret_cast<u32x2*>(reinterpret_cast<T*>(a.out) + bh * D + d4) = w2;
}

#ifndef ATTN_DECODE_WAVES
#define ATTN_DECODE_WAVES 2
#endif

// Compute units of the current device (queried once per device).
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0
                   ? n : 256;
  }
  return cus[dev];
}

template <typename T, int D>
hipError_t launch_typed(const DecodeProblem& p, const DecArgs& a, hipStream_t stream) {
  constexpr int NW = ATTN_DECODE_WAVES;
  const dim3 grid(p.splits, p.Hkv * a.hchunks, p.B);
  const long long groups = (long long)p.B * p.Hkv * a.hchunks;
  const int cus = device_cus();
  const long long items = groups * p.splits;
  const long long cap = (long long)p.max_blocks * p.block_size;
  const bool uniform = p.block_size % kTB == 0;
  // The split form's independent per-wave workers stream best once there
  // are at least 4 items per compute unit; with fewer, a group is better
  // spread over the waves of a workgroup (the fused form).  At head dim 256
  // the split form runs one 4-wave workgroup per compute unit and the fused
  // form is the faster whenever it has a group per compute unit (B = 64 x
  // 512..8192 tokens: 352 vs 364 us; 128..1024: 60.5 vs 77.4 us).  Above the
  // split form's ordering limit the fused form serves long contexts; short
  // ones (capacity of at most 1024 tokens) go to the partial kernel, whose
  // many small workgroups hide the latency of items this short.
  const bool split_form =
      uniform && p.B <= kOrdMaxSplit && (groups < cus || (D <= 128 && items >= 4LL * cus));
  const bool fused_form = uniform && !split_form && groups >= cus && p.B <= kOrdMaxFused &&
                          (p.B <= kOrdMaxSplit || cap > 1024);
  if (fused_form) {
    // fused persistent form: one workgroup per compute unit (it fills the
    // unit's registers), the output written directly
    constexpr int FW = stream_waves<true, D>();
    hipLaunchKernelGGL((decode_stream_kernel<T, D, true>), dim3((unsigned)cus), dim3(64 * FW), 0, stream, a);
    return hipGetLastError();
  }
  if (split_form) {
    // persistent: as many 4-wave workgroups as are resident at once (two per
    // compute unit, one at head dim 256), never more than there are items
    const long long per_cu = D <= 128 ? 2 : 1;  // head dim 256: one wave per SIMD
    const long long wgs = std::min<long long>((items + kStreamWaves - 1) / kStreamWaves, per_cu * cus);
    hipLaunchKernelGGL((decode_stream_kernel<T, D, false>), dim3((unsigned)wgs), dim3(64 * kStreamWaves), 0,
                       stream, a);
  } else if (uniform)
    hipLaunchKernelGGL((decode_partial_kernel<T, D, 2, true, NW>), grid, dim3(64 * NW), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_partial_kernel<T, D, 2, false, NW>), grid, dim3(64 * NW), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MergeArgs m{p.ws_o, p.ws_lse, p.out, p.splits, p.B * p.Hq};
  constexpr int HPW = 256 / (D / 4);
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((p.B * p.Hq + HPW - 1) / HPW), dim3(256), 0,
                     stream, m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode(const DecodeProblem& p, int dtype, hipStream_t stream) {
  DecArgs a;
  a.q = p.q;
  a.kp = p.k_pool;
  a.vp = p.v_pool;
  a.table = p.block_table;
  a.lens = p.seq_lens;
  a.alibi = p.alibi;
  a.ws_o = p.ws_o;
  a.ws_lse = p.ws_lse;
  a.out = p.out;
  a.err = p.error_flag;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.group = p.Hq / p.Hkv;
  a.hchunks = (a.group + 15) / 16;
  a.num_blocks = p.num_blocks;
  a.bs = p.block_size;
  a.maxb = p.max_blocks;
  a.splits = p.splits;
  a.softcap = p.softcap > 0.f;
  a.c_score = a.softcap ? 2.f * kLog2e * p.scale / p.softcap : kLog2e * p.scale;
  a.c_cap = kLog2e * p.softcap;
  if (dtype == 2)
    return p.D == 256 ? launch_typed<__bf16, 256>(p, a, stream)
         : p.D == 128 ? launch_typed<__bf16, 128>(p, a, stream) : launch_typed<__bf16, 64>(p, a, stream);
  return p.D == 256 ? launch_typed<_Float16, 256>(p, a, stream)
       : p.D == 128 ? launch_typed<_Float16, 128>(p, a, stream) : launch_typed<_Float16, 64>(p, a, stream);
}

}  // namespace attn
