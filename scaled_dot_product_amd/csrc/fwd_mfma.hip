// fwd_mfma.hip -- attention forward for bf16 / f16 on the gfx950 matrix cores.
//
// Computes what the kernel-contract page ("fuel-reference-backend -- attention
// kernel contracts", attention_naive / attention_flash) defines, with the
// streaming softmax of the derivation page ("gfx942 unified attention, from the
// math up", section 3) and its causal tile early exit (section 4).
//
// Compiled once per (element type, head dim): ATTN_ELEM is __bf16 or _Float16,
// ATTN_D is 64, 128 or 256, ATTN_TAG names the exported launcher.  At head dim
// 256 the Q fragments and the O accumulator alone take 192 VGPRs: one wave
// per SIMD, one workgroup per compute unit (128 KiB of K/V tiles), and no key
// split (it would need twice the tiles).
//
// Mapping onto CDNA4 (designed for gfx950, not taken from the gfx942 design):
//   * A workgroup of 4 waves owns 128 query rows of one (batch, head); each
//     wave owns 32 rows.  Key/value tiles of 64 keys are staged in LDS
//     (double-buffered, one barrier per tile) and shared by the 4 waves.
//   * Scores are computed transposed, S^T = K Q^T, on the 32x32x16 matrix
//     instruction: K (LDS, row-major, XOR-swizzled 16-byte chunks) is the A
//     operand, this wave's Q rows (registers, loaded once) are the B operand.
//     In the 32x32 accumulator layout a lane then holds 16 keys of ONE query,
//     so row reductions are in-lane plus a single cross-half swap.
//   * Softmax runs in log2 units (exp2); the running max is raised only when a
//     tile's max exceeds it by more than 2^8, which keeps every weight <= 256
//     and skips the rescale of the output in almost every tile.  The final
//     o / l is independent of the reference value, so the result is the same
//     recurrence (the derivation page notes the streaming form is exact).
//   * The weights, rounded to the input type, are already laid out as the B
//     operand of O^T = V^T P^T; V^T comes from row-major V in LDS through the
//     gfx950 LDS transpose read.  The output accumulator therefore also has
//     one query per lane, matching the softmax state.
//   * K fragments are read from LDS kKPF MFMAs ahead of their use, the first
//     ones before the softmax of the previous tile.
//   * The output is staged through LDS and written as whole rows with
//     non-temporal stores.
//   * Tiles wholly outside a wave's admissible key range are skipped (causal
//     and window early exit, per wave); masks are evaluated only on tiles that
//     straddle a mask boundary.
//   * Workgroups are issued heaviest-first under a causal mask, and the heads
//     of one dispatch round are dealt to the 8 XCDs in contiguous runs so that
//     the query heads sharing a KV head run on the same L2.
#include <limits.h>

#include "device_common.h"
#include "launch.h"

#ifndef ATTN_ELEM
#define ATTN_ELEM __bf16
#define ATTN_D 128
#define ATTN_TAG bf16_d128
#endif

#define ATTN_CAT2(a, b) a##b
#define ATTN_CAT(a, b) ATTN_CAT2(a, b)

namespace attn {
namespace {

constexpr int kBN = 64;            // keys per tile
constexpr int kNW = 4;             // waves per workgroup
constexpr int kQW = 32;            // query rows per wave
constexpr int kBM = kNW * kQW;     // query rows per workgroup
constexpr int kThreads = kNW * 64;
constexpr float kRescaleGap = 8.0f;  // log2 units: weights stay <= 2^8

enum : int { F_MASK = 1, F_SOFTCAP = 2, F_ALIBI = 4, F_PAGED = 8, F_SPLIT = 16 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alibi;
  void* out;    // nullptr: the output is not stored
  float* lse;   // per-row log-sum-exp (natural log), or nullptr
  // backward support: with dout, stats[row] = (lse in log2 units, or +inf for
  // a row without keys; sum_d dO * O from the float32 accumulator)
  const void* dout;
  float* stats;
  int Sq, Sk, Hq, Hkv, group, nbh, nqb;
  int kv_stride;  // dense: keys between consecutive (sequence, KV head) slices of k and v
  int heavy_first;
  // paged, variable-length form (F_PAGED): queries packed [total_q, Hq, D]
  // with a prefix sum, K/V in a [num_blocks, bs, Hkv, D] pool
  const int32_t* table;   // [B, maxb] physical block of each logical block
  const int32_t* kv_lens; // [B] live keys of each sequence
  const int32_t* cu_q;    // [B + 1] query row prefix sum
  int32_t* err;           // device error flag or nullptr
  int maxb, bs, num_blocks, total_q, max_sq;
  int wl;       // left window, -1 = unbounded
  int has_hi;   // is j - i' bounded above?
  int dmax;     // that bound (causal and/or right window)
  float c_score;  // log2(e) * scale; with softcap 2 * log2(e) * scale / cap
  float c_cap;    // log2(e) * cap
};

// XOR swizzles of the 16-byte chunk index, chosen so that the matrix-operand
// reads of K (16 rows, one chunk each) and the transpose reads of V (4 rows x
// 2-4 chunks per 16/32 lanes) hit distinct LDS banks.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D >= 128 ? (r & 15) : ((r >> 1) & 7);
}
// (the same for rows r and r + 8, which the transpose read of one step pairs)
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 256 ? ((r & 7) << 2) : (D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2));
}

// Key offset (within a 64-key tile, without the lane-half term 4*g) of
// accumulator element r of score block kb, from the 32x32 accumulator layout:
// element r of lane l is row 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ constexpr int key_of(int kb, int r) {
  return 32 * kb + 8 * (r >> 2) + (r & 3);
}

// Per-wave state of the streaming softmax: output accumulator O^T (one query
// per lane), running reference max and this lane's share of the denominator.
template <int DB>
struct RowState {
  floatx16 o[DB];
  float m_run;
  // row sum of the weights: D <= 128 sums on the matrix core, and every
  // element of l_acc holds this lane's row sum; D = 256 (short of registers)
  // keeps the dot-product form, l_part summing this lane's half of the keys
  floatx4 l_acc;
  float l_part;
};

// S^T = K Q^T for the 64 keys of one LDS tile: sc[0] keys 0..31, sc[1] 32..63.
template <typename T, int D>
__device__ __forceinline__ void qk_tile(const u32x4* Ks, const u32x4* qf, int ln, int g,
                                        floatx16 (&sc)[2]) {
  using E = Elem<T>;
  constexpr int NC = D / 8;
  sc[0] = floatx16{};
  sc[1] = floatx16{};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const int c = 2 * s + g;
    sc[0] = E::mma32(Ks[ln * NC + (c ^ swz_k<D>(ln))], qf[s], sc[0]);
    sc[1] = E::mma32(Ks[(32 + ln) * NC + (c ^ swz_k<D>(32 + ln))], qf[s], sc[1]);
  }
}

// One K fragment (A operand of S^T = K Q^T): fragment f = 2 s + kb is key
// block kb (rows 32 kb .. + 31), contraction step s.
template <typename T, int D>
__device__ __forceinline__ u32x4 kfrag(const u32x4* Ks, int f, int ln, int g) {
  constexpr int NC = D / 8;
  const int row = 32 * (f & 1) + ln;
  const int c = 2 * (f >> 1) + g;
  return Ks[row * NC + (c ^ swz_k<D>(row))];
}
#ifndef ATTN_KPF
#define ATTN_KPF 8
#endif
// K fragments kept in flight ahead of their MFMA: the first kKPF are read
// before the softmax of the previous tile, so that their LDS latency hides
// behind it (8 is 32 VGPRs; it fits the two-waves-per-SIMD budget at D = 128)
constexpr int kKPF = ATTN_KPF;
template <typename T, int D, int KPF>
__device__ __forceinline__ void qk_tile_pf(const u32x4* Ks, const u32x4* qf, int ln, int g,
                                           u32x4 (&kf)[KPF], floatx16 (&sc)[2]) {
  using E = Elem<T>;
  constexpr int NF = 2 * (D / 16);
  sc[0] = floatx16{};
  sc[1] = floatx16{};
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const u32x4 a = kf[f % KPF];
    if (f + KPF < NF) kf[f % KPF] = kfrag<T, D>(Ks, f + KPF, ln, g);
    sc[f & 1] = E::mma32(a, qf[f >> 1], sc[f & 1]);
  }
}

// Transform + mask + online update of one tile's scores: the weights P,
// rounded and packed as the B operand of O^T += V^T P^T, and O rescaled when
// the reference max rises.
template <typename T, int D, int FLAGS>
__device__ __forceinline__ void softmax_p(floatx16 (&sc)[2], uint32_t (&pp)[16], RowState<D / 32>& st,
                                          const FwdArgs& a, int Sk, int n0, int ip, int ipa_w,
                                          int ipb_w, float slope_l2, int g) {
  using E = Elem<T>;
  constexpr bool MASK = (FLAGS & F_MASK) != 0;
  constexpr bool SOFTCAP = (FLAGS & F_SOFTCAP) != 0;
  constexpr bool ALIBI = (FLAGS & F_ALIBI) != 0;
  constexpr bool kRaw = !SOFTCAP && !ALIBI;  // max on raw scores, scale folded into exp
  constexpr int DB = D / 32;
  constexpr bool kMmaSum = D <= 128;         // row sums on the matrix core
  const int rb = n0 + 4 * g - ip;            // j - i' of element offset 0

  // With a softcap or ALiBi the scores are turned into log2-unit logits
  // relative to the current reference max m_ref (0 before any key): the
  // per-tile constant base = c_cap + slope * (j0 - i') - m_ref carries the
  // softcap offset, the ALiBi term of the tile's first key and m_ref, so each
  // score costs its softcap (or scale) and one fused multiply-add for ALiBi.
  if constexpr (!kRaw) {
    float base = (SOFTCAP ? a.c_cap : 0.f) - (st.m_run == kNegInf ? 0.f : st.m_run);
    if constexpr (ALIBI) base = __builtin_fmaf(slope_l2, (float)rb, base);
    const float m2cap = -2.f * a.c_cap;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sc[kb][r];
        if constexpr (SOFTCAP) {
          const float e = fast_exp2(x * a.c_score);
          x = __builtin_fmaf(m2cap, fast_rcp(1.f + e), base);
        } else {
          x = __builtin_fmaf(x, a.c_score, base);
        }
        // (the ALiBi term of key j0 + k added last: computed ahead of the
        // scores, the 32 terms would hold 32 registers)
        if constexpr (ALIBI) x = __builtin_fmaf(slope_l2, (float)key_of(kb, r), x);
        sc[kb][r] = x;
      }
  }
  if constexpr (MASK) {
    const bool full = n0 + kBN <= Sk && (!a.has_hi || n0 + kBN - 1 - ipa_w <= a.dmax) &&
                      (a.wl < 0 || ipb_w - n0 <= a.wl);
    if (!full) {
      // admissible iff lo <= j - i' <= hi, with 0 <= j < Sk folded in
      int hi = Sk - 1 - ip;
      if (a.has_hi) hi = min(hi, a.dmax);
      int lo = -ip;
      if (a.wl >= 0) lo = max(lo, -a.wl);
      int klo = max(lo - rb, 0), khi = min(hi - rb, kBN - 1);
      if (khi < klo) klo = khi = kBN;
      const uint32_t span = (uint32_t)(khi - klo);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((uint32_t)(key_of(kb, r) - klo) > span) sc[kb][r] = kNegInf;
    }
  }

  // row max: 32 values in-lane (a chain of three-input max), then the other
  // half of the keys
  float mx = __builtin_fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
  for (int q = 1; q < 16; ++q) {
    const int kb = q >> 3, r = 2 * (q & 7);
    mx = __builtin_fmaxf(__builtin_fmaxf(mx, sc[kb][r]), sc[kb][r + 1]);
  }
  // (with a softcap or ALiBi, mt is the tile max relative to m_ref)
  float mt = mx;
  if constexpr (kRaw) mt = mx == kNegInf ? kNegInf : mx * a.c_score;
  mt = halves_max(mt);

  // raise the reference max only when the tile exceeds it by > 2^8
  if constexpr (kRaw) {
    const bool need = mt > st.m_run + kRescaleGap;
    if (wave_any(need)) {
      const float alpha = need ? fast_exp2(st.m_run - mt) : 1.f;
      st.m_run = need ? mt : st.m_run;
      if constexpr (D <= 128) st.l_acc = st.l_acc * alpha;
      else st.l_part *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) st.o[db] *= alpha;
    }
  } else {
    // m_ref + mt > m_run + 8: above the gap, or the first admissible keys
    const bool need = st.m_run == kNegInf ? mt != kNegInf : mt > kRescaleGap;
    if (wave_any(need)) {
      const float m_new = (st.m_run == kNegInf ? 0.f : st.m_run) + mt;
      const float alpha = need ? fast_exp2(st.m_run - m_new) : 1.f;
      const float shift = need ? mt : 0.f;  // logits relative to the new reference
      st.m_run = need ? m_new : st.m_run;
      if constexpr (D <= 128) st.l_acc = st.l_acc * alpha;
      else st.l_part *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) st.o[db] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][r] -= shift;
    }
  }
  const float m_use = st.m_run == kNegInf ? 0.f : st.m_run;

  // weights, rounded to the input type, packed as the PV B operand
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p0, p1;
      if constexpr (kRaw) {
        p0 = fast_exp2(__builtin_fmaf(sc[kb][r], a.c_score, -m_use));
        p1 = fast_exp2(__builtin_fmaf(sc[kb][r + 1], a.c_score, -m_use));
      } else {
        p0 = fast_exp2(sc[kb][r]);
        p1 = fast_exp2(sc[kb][r + 1]);
      }
      pp[kb * 8 + r / 2] = E::pack2(p0, p1);
      if constexpr (!kMmaSum) st.l_part = E::dot2(pp[kb * 8 + r / 2], E::kOnePair, st.l_part);
    }
}

// O^T += V^T P^T for the 64 keys of one tile (weights pp from softmax_p).
template <typename T, int D>
__device__ __forceinline__ void pv_tile(const uint32_t (&pp)[16], const T* Vs, RowState<D / 32>& st,
                                        int lane, int g) {
  using E = Elem<T>;
  constexpr int DB = D / 32;
  constexpr bool kMmaSum = D <= 128;
  // O^T += V^T P^T, 16 keys per step; V^T through the LDS transpose read
  const int trow = 4 * g + ((lane & 15) >> 2);                // key row within a 16-key step
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);   // d within a 32-row block
  // Row sums of the rounded weights on the matrix core, from the same P^T
  // operand read as the B operand of the 16x16x32 instruction: lane l's 8
  // weights (all of query row l % 32) become column l % 16, k-block l / 16.
  // So column c holds row c in its k-blocks 0 and 2 and row c + 16 in 1 and 3.
  // The A operand is 0/1: output row m sums the k-blocks of parity (m / 4) & 1.
  // Lane l receives output rows 4 (l / 16) .. + 3 of column l % 16, which then
  // all hold the sum of row l % 32, its own row.  This costs no vector-ALU
  // work; the two-element dot product it replaces stalls behind other waves'
  // matrix instructions.
  const uint32_t one = ((lane >> 4) & 1) == ((lane >> 2) & 1) ? E::kOnePair : 0u;
  const u32x4 sel = {one, one, one, one};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4 pf = {pp[4 * ks], pp[4 * ks + 1], pp[4 * ks + 2], pp[4 * ks + 3]};
    if constexpr (kMmaSum) st.l_acc = E::mma16(sel, pf, st.l_acc);
    const int r0 = 16 * ks + trow;
    const int sw = swz_v<D>(r0);  // same for r0 + 8
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 32 * db + tcol;
      const int cidx = ((col >> 3) ^ sw) * 8 + (col & 7);
      const u32x2 lo = lds_read_tr16(Vs + r0 * D + cidx);
      const u32x2 hi = lds_read_tr16(Vs + (r0 + 8) * D + cidx);
      const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
      st.o[db] = E::mma32(va, pf, st.o[db]);
    }
  }
}

// One tile's softmax, then O += P V.
template <typename T, int D, int FLAGS>
__device__ __forceinline__ void softmax_pv(floatx16 (&sc)[2], const T* Vs, RowState<D / 32>& st,
                                           const FwdArgs& a, int Sk, int n0, int ip, int ipa_w,
                                           int ipb_w, float slope_l2, int lane, int g) {
  uint32_t pp[16];
  softmax_p<T, D, FLAGS>(sc, pp, st, a, Sk, n0, ip, ipa_w, ipb_w, slope_l2, g);
  pv_tile<T, D>(pp, Vs, st, lane, g);
}

// Key-split mode (F_SPLIT, for grids too small to fill the chip): the
// workgroup has two groups of kNW waves on the same 128 query rows; group 0
// takes the first half of the key tiles, group 1 the second, each with its own
// LDS buffers, and group 1 hands its (o, m, l) to group 0 at the end.
template <typename T, int D, int FLAGS>
__global__ __launch_bounds__((FLAGS & F_SPLIT) ? 2 * kThreads : kThreads)
__attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : 2, D > 128 ? 1 : 2)))
void fwd_mfma_kernel(FwdArgs a) {
  constexpr bool ALIBI = (FLAGS & F_ALIBI) != 0;
  constexpr bool PAGED = (FLAGS & F_PAGED) != 0;
  constexpr bool SPLIT = (FLAGS & F_SPLIT) != 0;
  constexpr int NG = SPLIT ? 2 : 1;      // key groups
  constexpr int NC = D / 8;              // 16-byte chunks per K/V row
  constexpr int TC = kBN * NC;           // chunks per K (or V) tile
  constexpr int CPT = TC / kThreads;     // chunks per thread per tile and tensor
  constexpr int KS = D / 16;             // contraction steps of K Q^T
  constexpr int DB = D / 32;             // 32-row blocks of O^T
  // K fragments read ahead in the plain step order (4 where the rotated order
  // also runs at head dim 128, so that both loops fit the registers)
  constexpr int KPF =
      ((FLAGS & F_SOFTCAP) != 0 && D == 128 && (FLAGS & (F_PAGED | F_SPLIT)) == 0) ? 4 : kKPF;
  static_assert(CPT * kThreads == TC, "tile must split evenly over the workgroup");

  // Four separate LDS objects so that the compiler can tell the buffer being
  // filled by the asynchronous copy from the buffers being read (one tile per
  // key group in each).
  __shared__ u32x4 kbuf0[NG * TC], kbuf1[NG * TC], vbuf0[NG * TC], vbuf1[NG * TC];

  const int tid_wg = threadIdx.x;
  const int wave_wg = __builtin_amdgcn_readfirstlane(tid_wg >> 6);  // wave-uniform
  const int grp = SPLIT ? wave_wg / kNW : 0;    // key group
  const int tid = tid_wg - grp * kThreads;      // thread within the group
  const int lane = tid & 63;
  const int wave = wave_wg - grp * kNW;         // wave within the group
  const int g = lane >> 5;               // lane half
  const int ln = lane & 31;

  // ---- work item: (query block, head, batch)
  const int id = blockIdx.x;
  const int round = id / a.nbh;
  const int u = id - round * a.nbh;
  const int bh = (a.nbh & 7) == 0 ? ((u & 7) * (a.nbh >> 3) + (u >> 3)) : u;
  const int qb = a.heavy_first ? (a.nqb - 1 - round) : round;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int kvh = h / a.group;
  const int m0 = qb * kBM;
  int Sq = a.Sq, Sk = a.Sk;
  int q_row = D, kv_row = D;  // elements between consecutive Q/O rows and K/V rows
  const T* Q;
  const T* K;
  const T* V;
  T* O;
  if constexpr (PAGED) {
    // this sequence's query rows [q0, q0 + Sq) and live keys [0, Sk), clamped
    // into the buffers (flagged when the prefix sum or a length was outside)
    const int c0 = __builtin_amdgcn_readfirstlane(a.cu_q[b]);
    const int c1 = __builtin_amdgcn_readfirstlane(a.cu_q[b + 1]);
    const int q0 = min(max(c0, 0), a.total_q), q1 = min(max(c1, q0), a.total_q);
    const int kl = __builtin_amdgcn_readfirstlane(a.kv_lens[b]);
    Sq = min(q1 - q0, a.max_sq);
    Sk = min(max(kl, 0), a.maxb * a.bs);
    if ((q0 != c0 || q1 != c1 || Sq != q1 - q0 || Sk != kl) && a.err && tid == 0) *a.err = 1;
    if (m0 >= Sq) return;  // no rows of this sequence in this block (whole workgroup)
    q_row = a.Hq * D;
    kv_row = a.Hkv * D;
    Q = reinterpret_cast<const T*>(a.q) + ((size_t)q0 * a.Hq + h) * D;
    O = reinterpret_cast<T*>(a.out) + ((size_t)q0 * a.Hq + h) * D;
    K = reinterpret_cast<const T*>(a.k) + (size_t)kvh * D;  // pool; tiles add their block
    V = reinterpret_cast<const T*>(a.v) + (size_t)kvh * D;
  } else {
    Q = reinterpret_cast<const T*>(a.q) + (size_t)bh * Sq * D;
    K = reinterpret_cast<const T*>(a.k) + (size_t)(b * a.Hkv + kvh) * a.kv_stride * D;
    V = reinterpret_cast<const T*>(a.v) + (size_t)(b * a.Hkv + kvh) * a.kv_stride * D;
    O = reinterpret_cast<T*>(a.out) + (size_t)bh * Sq * D;
  }
  const int off = Sk - Sq;

  // ---- admissible key ranges: [lo(i'_first), hi(i'_last))
  auto key_lo = [&](int ipa) { return a.wl >= 0 ? max(0, ipa - a.wl) : 0; };
  auto key_hi = [&](int ipb) { return a.has_hi ? min(Sk, max(0, ipb + a.dmax + 1)) : Sk; };
  const int wg_last = min(m0 + kBM, Sq) - 1;
  const int n_lo = key_lo(m0 + off);
  const int n_hi = key_hi(wg_last + off);
  const int t_first = n_lo / kBN;
  const int t_last = n_hi > n_lo ? (n_hi + kBN - 1) / kBN : t_first;   // one past
  // this group's tiles [t_begin, t_end); with one group that is all of them
  const int half = SPLIT ? (t_last - t_first + 1) / 2 : 0;
  const int t_begin = SPLIT && grp == 1 ? t_first + half : t_first;
  const int t_end = SPLIT && grp == 0 ? t_first + half : t_last;

  const int wq0 = m0 + wave * kQW;
  const bool wave_live = wq0 < Sq;
  const int wq_last = min(wq0 + kQW, Sq) - 1;
  const int ipa_w = wq0 + off, ipb_w = wq_last + off;
  const int w_lo = key_lo(ipa_w);
  const int w_hi = key_hi(ipb_w);
  auto live = [&](int t) { return wave_live && t < t_end && t * kBN < w_hi && (t + 1) * kBN > w_lo; };

  const int qi = wq0 + ln;  // this lane's query row
  const int ip = qi + off;  // its bottom-right aligned position

  // ---- this wave's Q rows as the B operand: lane -> (row ln, d = 16 s + 8 g .. +7)
  u32x4 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = qi < Sq ? load16(Q + (size_t)qi * q_row + 16 * s + 8 * g) : zero_u32x4();

  float slope_l2 = 0.f;
  if constexpr (ALIBI) slope_l2 = a.alibi[h] * kLog2e;

  RowState<DB> st;
#pragma unroll
  for (int db = 0; db < DB; ++db) st.o[db] = floatx16{};
  st.m_run = kNegInf;
  st.l_acc = floatx4{};
  st.l_part = 0.f;

  // ---- asynchronous tile copies global -> LDS.  Chunk c of a tile sits at
  // LDS slot c, i.e. row c / NC, swizzled chunk c % NC; keys past Sk read 0.
  // One head's K (or V) is < 2 GiB, and a paged tile spans < 2 GiB of the pool
  // (both checked by the host), so offsets within a tile fit int32.
  const int kv_bytes = Sk * D * (int)sizeof(T);
  // Paged: tile t is rows (t % m) * 64 .. + 63 of logical block t / m (m =
  // bs / 64).  Lane j of page_reg holds the physical block of logical block
  // pbase + j; the window moves forward when a copy needs a later block.
  const int m_tiles = PAGED ? a.bs / kBN : 1;
  int pbase = 0, page_reg = 0;
  auto load_pages = [&](int first) {
    pbase = first;
    const int j = first + lane;
    page_reg = j < a.maxb ? a.table[(size_t)b * a.maxb + j] : 0;
  };
  bool bad_page = false;  // a table entry outside the pool was used (wave-uniform)
  // Paged: a cursor (logical block lb, tile sub within it) per tensor for the
  // tile its next copy reads, advanced one tile per step instead of dividing.
  struct Cursor {
    int lb, sub;
  };
  auto advance = [&](Cursor& c) {
    if (++c.sub == m_tiles) {
      c.sub = 0;
      ++c.lb;
    }
  };
  // Buffer resource of tile t (at cursor c when paged); `ok` is false for a
  // tile whose block is outside the pool (its keys are masked, its copies read
  // nothing).  Every field is wave-uniform; the read-first-lane calls say so to
  // the compiler, which otherwise computes the clamped size on the vector unit
  // and wraps each copy in a loop over the distinct descriptors of the wave.
  auto tile_rsrc = [&](const T* base_t, int t, Cursor c, bool& ok) -> __amdgpu_buffer_rsrc_t {
    if constexpr (PAGED) {
      const int phys = __builtin_amdgcn_readlane(page_reg, c.lb - pbase);
      const int rows = __builtin_amdgcn_readfirstlane(min(max(Sk - t * kBN, 0), kBN));
      ok = rows == 0 || (unsigned)phys < (unsigned)a.num_blocks;
      bad_page |= !ok;
      const long long row0 = ok ? (long long)phys * a.bs + c.sub * kBN : 0;
      const int bytes = __builtin_amdgcn_readfirstlane(ok ? rows * kv_row * (int)sizeof(T) : 0);
      return make_rsrc32(base_t + row0 * kv_row, bytes);
    } else {
      ok = true;
      const int base = t * kBN * D * (int)sizeof(T);
      return make_rsrc32(reinterpret_cast<const char*>(base_t) + base, kv_bytes - base);
    }
  };
  auto dma_k = [&](u32x4* dst, __amdgpu_buffer_rsrc_t rs) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / NC, pc = c % NC;
      dma16(rs, dst + i * kThreads + wave * 64, (r * kv_row + (pc ^ swz_k<D>(r)) * 8) * (int)sizeof(T));
    }
  };
  auto dma_v = [&](u32x4* dst, __amdgpu_buffer_rsrc_t rs) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / NC, pc = c % NC;
      dma16(rs, dst + i * kThreads + wave * 64, (r * kv_row + (pc ^ swz_v<D>(r)) * 8) * (int)sizeof(T));
    }
  };

  // ---- software pipeline over the tiles t_begin + i:
  //   step i:  softmax(S(i)), O += P(i) V(i)
  //            S(i+1) = K(i+1) Q^T   (matrix cores, into the same registers)
  //   while K(i+2) and V(i+1) stream into the buffers freed by step i-1.
  // K(i) lives in kbuf[i % 2], V(i) in vbuf[i % 2].
  // Paged: kok0 / kok1 say whether the tile in kbuf0 / kbuf1 lies in the pool;
  // the softmax of a tile that does not sees a key bound at its first key, so
  // all of its keys are masked.
  const int n = t_end - t_begin;
  // Group 1 of a split workgroup runs the pipeline rotated by half a step:
  // step i does the matrix work first (O += P(i-1) V(i-1), then S(i)) and the
  // softmax of tile i after it, so that on each SIMD (one wave of each group)
  // one wave's vector phase meets the other's matrix phase between two
  // barriers.  The operations on O keep their order, so the result is the
  // same bit for bit.  Its copies run one tile later: K(i+1) and V(i) in step i.
  // (not over the paged pool, where the longer loop's scalar spills cost more
  // than the overlap gains: 61.3 vs 59.8 us on the chunked workload; the
  // rotated step reads its K fragments as it goes, without the prefetch of
  // the other order, which does not fit the registers at head dim 128)
  // Without the key split, every other workgroup runs rotated at head dim 64,
  // so that the two workgroups sharing a compute unit less often meet in the
  // same phase (B = 8 x 16 heads x 512 queries over 4096 keys, f16: 83.0 ->
  // 81.0 us; at head dim 128 the two loops together spill registers and the
  // 2048-token workload went from 73.8 to 81.1 us).
  // With a softcap (vector-bound: three transcendentals per score) the same
  // holds at head dim 128, given a shorter K prefetch so that both loops fit
  // (the long masked 8192-token workload: 555 -> 543 us); without one, the
  // rotated step's K reads without prefetch slow the matrix-bound loop.
  constexpr bool SOFTCAP = (FLAGS & F_SOFTCAP) != 0;
  const bool rot = !PAGED && (SPLIT ? D <= 128 && grp == 1
                                    : (D == 64 || (SOFTCAP && D <= 128)) && (blockIdx.x & 1) != 0);
  // steps every wave of the workgroup runs (barriers must match): group 0 of a
  // split workgroup has at least as many tiles as group 1, which needs one
  // step more than it has tiles
  const int n_steps = !SPLIT ? (rot && n > 0 ? n + 1 : n) : (D > 128 || PAGED) ? half
                      : (t_last > t_first ? max(half, t_last - t_first - half + 1) : 0);
  u32x4* const kb0 = kbuf0 + grp * TC;
  u32x4* const kb1 = kbuf1 + grp * TC;
  u32x4* const vb0 = vbuf0 + grp * TC;
  u32x4* const vb1 = vbuf1 + grp * TC;
  floatx16 sc[2];
  bool kok0 = true, kok1 = true;
  Cursor kc{0, 0}, vc{0, 0};  // paged: tiles of the next K and V copies
  if constexpr (PAGED) {
    kc.lb = t_begin / m_tiles;
    kc.sub = t_begin - kc.lb * m_tiles;
    vc = kc;
    load_pages(kc.lb);
  }
  bool ok_unused;
  if (n_steps > 0) {
    // K(0), V(0) and K(1); rotated: K(0) only.  Descriptors first, copies
    // after: the page ids may still be in flight, and a wait for them placed
    // between copies would wait for the copies too
    if constexpr (PAGED) {
      const __amdgpu_buffer_rsrc_t rk0 = n > 0 ? tile_rsrc(K, t_begin, kc, kok0) : make_rsrc32(K, 0);
      __amdgpu_buffer_rsrc_t rv0 = make_rsrc32(V, 0), rk1 = make_rsrc32(K, 0);
      advance(kc);
      if (!rot) {
        rv0 = n > 0 ? tile_rsrc(V, t_begin, vc, ok_unused) : make_rsrc32(V, 0);
        advance(vc);
        rk1 = n > 1 ? tile_rsrc(K, t_begin + 1, kc, kok1) : make_rsrc32(K, 0);
        advance(kc);
      }
      if (n > 0) {
        dma_k(kb0, rk0);
        if (!rot) dma_v(vb0, rv0);
      }
      if (!rot && n > 1) dma_k(kb1, rk1);
    } else {
      if (n > 0) {
        dma_k(kb0, tile_rsrc(K, t_begin, kc, kok0));
        if (!rot) dma_v(vb0, tile_rsrc(V, t_begin, vc, ok_unused));
      }
      if (!rot && n > 1) dma_k(kb1, tile_rsrc(K, t_begin + 1, kc, kok1));
    }
    wait_vmem();
    __syncthreads();
    if (!rot && n > 0 && live(t_begin)) qk_tile<T, D>(kb0, qf, ln, g, sc);
  }
  auto step = [&](int i, const u32x4* kread, const u32x4* vread, u32x4* kload, u32x4* vload,
                  bool& ok_load) {
    const int t = t_begin + i;
    const bool ok_t = ok_load;  // tile t, whose K buffer this step refills
    wait_vmem();
    __syncthreads();  // K(i+1), V(i) landed; everyone is done with step i-1's buffers
    if constexpr (PAGED) {
      // the copies below read tiles t + 2 (K, at kc) and t + 1 (V, at vc)
      if (i + 2 < n && kc.lb - pbase >= 64) load_pages(vc.lb);
      const __amdgpu_buffer_rsrc_t rk = i + 2 < n ? tile_rsrc(K, t + 2, kc, ok_load) : make_rsrc32(K, 0);
      const __amdgpu_buffer_rsrc_t rv = i + 1 < n ? tile_rsrc(V, t + 1, vc, ok_unused) : make_rsrc32(V, 0);
      advance(kc);
      advance(vc);
      if (i + 2 < n) dma_k(kload, rk);
      if (i + 1 < n) dma_v(vload, rv);
    } else {
      if (i + 2 < n) dma_k(kload, tile_rsrc(K, t + 2, kc, ok_load));
      if (i + 1 < n) dma_v(vload, tile_rsrc(V, t + 1, vc, ok_unused));
    }
    u32x4 kf[KPF];
#pragma unroll
    for (int p = 0; p < KPF; ++p) kf[p] = kfrag<T, D>(kread, p, ln, g);
    if (live(t))
      softmax_pv<T, D, FLAGS>(sc, reinterpret_cast<const T*>(vread), st, a,
                              PAGED && !ok_t ? t * kBN : Sk, t * kBN, ip, ipa_w, ipb_w, slope_l2,
                              lane, g);
    // S(i+1) overwrites S(i), already consumed: one score buffer per wave.
    // This matrix phase runs at raised wave priority so that, of the two waves
    // sharing a SIMD, the one with matrix work ready wins instruction issue
    // over the one in its softmax (vector) phase.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    if (i + 1 < n && live(t + 1)) qk_tile_pf<T, D, KPF>(kread, qf, ln, g, kf, sc);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  // the rotated step of group 1: K(i) is in kcur, V(i-1) in vprev; pp
  // carries tile i-1's weights from its softmax into this step
  uint32_t pp[16];
  auto step_rot = [&](int i, const u32x4* kcur, const u32x4* vprev, u32x4* kload, u32x4* vload,
                      bool& ok_cur, bool& ok_load) {
    const int t = t_begin + i;
    wait_vmem();
    __syncthreads();  // K(i), V(i-1) landed; everyone is done with step i-1's buffers
    if constexpr (PAGED) {
      // the copies below read tiles t + 1 (K, at kc) and t (V, at vc)
      if (i + 1 < n && kc.lb - pbase >= 64) load_pages(vc.lb);
      const __amdgpu_buffer_rsrc_t rk = i + 1 < n ? tile_rsrc(K, t + 1, kc, ok_load) : make_rsrc32(K, 0);
      const __amdgpu_buffer_rsrc_t rv = i < n ? tile_rsrc(V, t, vc, ok_unused) : make_rsrc32(V, 0);
      advance(kc);
      advance(vc);
      if (i + 1 < n) dma_k(kload, rk);
      if (i < n) dma_v(vload, rv);
    } else {
      if (i + 1 < n) dma_k(kload, tile_rsrc(K, t + 1, kc, ok_load));
      if (i < n) dma_v(vload, tile_rsrc(V, t, vc, ok_unused));
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    if (i >= 1 && live(t - 1)) pv_tile<T, D>(pp, reinterpret_cast<const T*>(vprev), st, lane, g);
    if (i < n && live(t)) qk_tile<T, D>(kcur, qf, ln, g, sc);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    if (i < n && live(t))
      softmax_p<T, D, FLAGS>(sc, pp, st, a, PAGED && !ok_cur ? t * kBN : Sk, t * kBN, ip, ipa_w, ipb_w,
                             slope_l2, g);
  };
  // (two loops, so that each carries only its own state across its steps)
  if (rot) {
    for (int i = 0; i < n_steps; i += 2) {
      step_rot(i, kb0, vb1, kb1, vb0, kok0, kok1);
      if (i + 1 < n_steps) step_rot(i + 1, kb1, vb0, kb0, vb1, kok1, kok0);
    }
  } else {
    for (int i = 0; i < n_steps; i += 2) {
      step(i, kb1, vb0, kb0, vb1, kok0);
      if (i + 1 < n_steps) step(i + 1, kb0, vb1, kb1, vb0, kok1);
    }
  }
  if (PAGED && bad_page && a.err && lane == 0) *a.err = 1;

  // ---- key groups: group 1 hands (o, m, l) to group 0 through LDS (the tile
  // buffers are free now), one 32-row block of O^T at a time; group 0 rebases
  // both to their common reference max.
  float l = D <= 128 ? st.l_acc[0] : halves_sum(st.l_part);
  if constexpr (SPLIT) {
    float* xo = reinterpret_cast<float*>(kbuf0);  // [64 lanes x 4 waves][16]
    float* xml = reinterpret_cast<float*>(vbuf0); // [64 x 4][2]
    const int slot = wave * 64 + lane;
    __syncthreads();  // every wave is done with the tile buffers
    if (grp == 1) {
      xml[2 * slot] = st.m_run;
      xml[2 * slot + 1] = l;
    }
    float a0 = 1.f, a1 = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if (grp == 1) {
#pragma unroll
        for (int r = 0; r < 16; r += 4)
          *reinterpret_cast<floatx4*>(xo + slot * 16 + r) =
              floatx4{st.o[db][r], st.o[db][r + 1], st.o[db][r + 2], st.o[db][r + 3]};
      }
      __syncthreads();
      if (grp == 0) {
        if (db == 0) {
          const float m1 = xml[2 * slot], l1 = xml[2 * slot + 1];
          const float m0 = st.m_run;
          const float M = __builtin_fmaxf(m0, m1);
          a0 = m0 == kNegInf ? 0.f : fast_exp2(m0 - M);
          a1 = m1 == kNegInf ? 0.f : fast_exp2(m1 - M);
          st.m_run = M;
          l = l * a0 + l1 * a1;
        }
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const floatx4 x = *reinterpret_cast<const floatx4*>(xo + slot * 16 + r);
#pragma unroll
          for (int c = 0; c < 4; ++c) st.o[db][r + c] = st.o[db][r + c] * a0 + x[c] * a1;
        }
      }
      __syncthreads();
    }
    if (grp == 1) return;
  }

  // ---- epilogue: O = o / l (0 when no key was admissible)
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (a.lse && qi < Sq && g == 0) {
    // lse = ln(sum_j e^{s_j}) = ln 2 * (m + log2 l) with the weights 2^(x - m)
    const float m_use = st.m_run == kNegInf ? 0.f : st.m_run;
    a.lse[(size_t)bh * Sq + qi] = l > 0.f ? (m_use + __log2f(l)) * kLn2 : kNegInf;
  }
  if constexpr (!PAGED) {
    if (a.stats) {
      // this lane holds d = 32 db + 8 j + 4 g .. + 3 of row qi; the other lane
      // half holds the rest
      const T* dorow = reinterpret_cast<const T*>(a.dout) + ((size_t)bh * Sq + min(qi, Sq - 1)) * D;
      float part = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(dorow + 32 * db + 8 * j + 4 * g);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t hw = (w[c >> 1] >> (16 * (c & 1))) & 0xffffu;
            part = __builtin_fmaf(st.o[db][4 * j + c], Elem<T>::to_float(hw), part);
          }
        }
      const float delta = halves_sum(part) * inv;
      if (qi < Sq && g == 0) {
        const float m_use = st.m_run == kNegInf ? 0.f : st.m_run;
        float2* srow = reinterpret_cast<float2*>(a.stats) + (size_t)bh * Sq + qi;
        *srow = float2{l > 0.f ? m_use + __log2f(l) : __builtin_inff(), delta};
      }
    }
  }
  // The output goes through a per-wave LDS block so that every store
  // instruction writes whole rows (64 lanes x 16 bytes = RPI full rows), and
  // the stores are non-temporal: the rows go out as full lines instead of
  // lingering as dirty cache lines that the next kernel would have to write
  // back (measured: the paged decode run right after the 2048-token prefill
  // takes 212 instead of 222 us, and the prefill itself is no slower).
  if constexpr (!SPLIT) __syncthreads();  // other waves may still read the last V tile
  if (a.out) {
    using E = Elem<T>;
    constexpr int NCH = D / 8;         // 16-byte chunks per row
    constexpr int RPI = 64 / NCH;      // rows per store instruction
    u32x4* stg = (wave < 2 ? kbuf0 : kbuf1) + (wave & 1) * (32 * NCH);
    u32x2* stg2 = reinterpret_cast<u32x2*>(stg);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w[0] = E::pack2(st.o[db][4 * j] * inv, st.o[db][4 * j + 1] * inv);
        w[1] = E::pack2(st.o[db][4 * j + 2] * inv, st.o[db][4 * j + 3] * inv);
        const int c = 4 * db + j;
        stg2[(ln * NCH + (c ^ (ln & (NCH - 1)))) * 2 + g] = w;
      }
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / NCH, c = lane % NCH;
      const u32x4 v = stg[r * NCH + (c ^ (r & (NCH - 1)))];
      if (wq0 + r < Sq) {
        u32x4* dst = reinterpret_cast<u32x4*>(O + (size_t)(wq0 + r) * q_row + 8 * c);
        __builtin_nontemporal_store(v, dst);
      }
    }
  }
}

template <int FLAGS>
hipError_t launch_flags(const FwdArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_mfma_kernel<ATTN_ELEM, ATTN_D, FLAGS>), dim3(grid),
                     dim3((FLAGS & F_SPLIT) ? 2 * kThreads : kThreads), 0, stream, a);
  return hipGetLastError();
}

// The key split needs two sets of tiles: at head dim 256 they do not fit.
constexpr bool kCanSplit = ATTN_D <= 128;

template <int FLAGS>
hipError_t launch_split(const FwdArgs& a, int grid, hipStream_t stream) {
  if constexpr (kCanSplit) return launch_flags<FLAGS | F_SPLIT>(a, grid, stream);
  else return launch_flags<FLAGS>(a, grid, stream);  // never taken
}

// Factor from a raw score (q . k) to the exponent of the weight: log2(e) *
// scale, or 2 log2(e) scale / cap for the softcap's exponential.  Without a
// softcap or ALiBi the kernel masks raw scores with -inf and folds this factor
// into the exponent, where a zero scale would turn a masked score into
// -inf * 0 = NaN; a zero scale therefore enters as the smallest normal float
// instead: every finite score times it is below 2^-100 in magnitude, so every
// admissible weight is still exactly 1 (uniform attention, as for scale 0)
// while a masked score keeps weight 0.
float score_factor(float scale, float softcap, bool alibi) {
  if (softcap > 0.f) return 2.f * kLog2e * scale / softcap;
  const float c = kLog2e * scale;
  return (c == 0.f && !alibi) ? __FLT_MIN__ : c;
}

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

}  // namespace

hipError_t ATTN_CAT(launch_fwd_mfma_, ATTN_TAG)(const FwdProblem& p, hipStream_t stream) {
  FwdArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.alibi = p.alibi;
  a.out = p.out;
  a.lse = p.lse;
  a.dout = p.dout;
  a.stats = p.stats;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.kv_stride = p.kv_stride > 0 ? p.kv_stride : p.Sk;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.group = p.Hq / p.Hkv;
  a.nbh = p.B * p.Hq;
  a.nqb = (p.Sq + kBM - 1) / kBM;
  a.heavy_first = p.causal;
  a.wl = p.wl;
  a.has_hi = p.causal || p.wr >= 0;
  a.dmax = p.causal ? (p.wr >= 0 ? min(p.wr, 0) : 0) : p.wr;
  const bool softcap = p.softcap > 0.f;
  a.c_score = score_factor(p.scale, p.softcap, p.alibi != nullptr);
  a.c_cap = kLog2e * p.softcap;
  const int grid = a.nqb * a.nbh;
  const bool mask = p.causal || p.wl >= 0 || p.wr >= 0 || (p.Sk % kBN) != 0;
  // Fewer workgroups than two per compute unit leave SIMDs with a single
  // wave: split the key range of each workgroup over two wave groups instead
  // (only worth it with enough key tiles to share).
  const bool split = kCanSplit && grid < 2 * device_cus() && p.Sk >= 8 * kBN;
  const int flags = (mask ? F_MASK : 0) | (softcap ? F_SOFTCAP : 0) | (p.alibi ? F_ALIBI : 0) |
                    (split ? F_SPLIT : 0);
  switch (flags) {
    case F_SPLIT | 0: return launch_split<0>(a, grid, stream);
    case F_SPLIT | 1: return launch_split<1>(a, grid, stream);
    case F_SPLIT | 2: return launch_split<2>(a, grid, stream);
    case F_SPLIT | 3: return launch_split<3>(a, grid, stream);
    case F_SPLIT | 4: return launch_split<4>(a, grid, stream);
    case F_SPLIT | 5: return launch_split<5>(a, grid, stream);
    case F_SPLIT | 6: return launch_split<6>(a, grid, stream);
    case F_SPLIT | 7: return launch_split<7>(a, grid, stream);
    case 0: return launch_flags<0>(a, grid, stream);
    case 1: return launch_flags<1>(a, grid, stream);
    case 2: return launch_flags<2>(a, grid, stream);
    case 3: return launch_flags<3>(a, grid, stream);
    case 4: return launch_flags<4>(a, grid, stream);
    case 5: return launch_flags<5>(a, grid, stream);
    case 6: return launch_flags<6>(a, grid, stream);
    default: return launch_flags<7>(a, grid, stream);
  }
}

hipError_t ATTN_CAT(launch_paged_prefill_, ATTN_TAG)(const PagedPrefillProblem& p, hipStream_t stream) {
  FwdArgs a = {};
  a.q = p.q;
  a.k = p.k_pool;
  a.v = p.v_pool;
  a.alibi = p.alibi;
  a.out = p.out;
  a.lse = nullptr;
  a.dout = nullptr;
  a.stats = nullptr;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.group = p.Hq / p.Hkv;
  a.nbh = p.B * p.Hq;
  a.nqb = (p.max_sq + kBM - 1) / kBM;
  a.heavy_first = p.causal;
  a.table = p.block_table;
  a.kv_lens = p.seq_lens;
  a.cu_q = p.cu_seqlens_q;
  a.err = p.error_flag;
  a.maxb = p.max_blocks;
  a.bs = p.block_size;
  a.num_blocks = p.num_blocks;
  a.total_q = p.total_q;
  a.max_sq = p.max_sq;
  a.wl = p.wl;
  a.has_hi = p.causal || p.wr >= 0;
  a.dmax = p.causal ? (p.wr >= 0 ? min(p.wr, 0) : 0) : p.wr;
  const bool softcap = p.softcap > 0.f;
  a.c_score = score_factor(p.scale, p.softcap, p.alibi != nullptr);
  a.c_cap = kLog2e * p.softcap;
  const int grid = a.nqb * a.nbh;
  // lengths vary per sequence: the masked variants always; the key split on
  // the same rule as the dense launch, with the longest possible key range
  const bool split = kCanSplit && grid < 2 * device_cus() &&
                     (long long)p.max_blocks * p.block_size >= 8 * kBN;
  constexpr int PM = F_PAGED | F_MASK;
  const int flags = (softcap ? F_SOFTCAP : 0) | (p.alibi ? F_ALIBI : 0) | (split ? F_SPLIT : 0);
  switch (flags) {
    case 0: return launch_flags<PM>(a, grid, stream);
    case F_SOFTCAP: return launch_flags<PM | F_SOFTCAP>(a, grid, stream);
    case F_ALIBI: return launch_flags<PM | F_ALIBI>(a, grid, stream);
    case F_SOFTCAP | F_ALIBI: return launch_flags<PM | F_SOFTCAP | F_ALIBI>(a, grid, stream);
    case F_SPLIT: return launch_split<PM>(a, grid, stream);
    case F_SPLIT | F_SOFTCAP: return launch_split<PM | F_SOFTCAP>(a, grid, stream);
    case F_SPLIT | F_ALIBI: return launch_split<PM | F_ALIBI>(a, grid, stream);
    default: return launch_split<PM | F_SOFTCAP | F_ALIBI>(a, grid, stream);
  }
}

}  // namespace attn
