// bwd_mfma.hip -- attention backward on the matrix cores (bf16 / f16, head
// dim 64, 128 or 256): dQ, dK, dV by recompute.
//
// Kernel-contract page, attention_flash_backward: with P the stable-softmax
// weights of the forward (recomputed from Q, K and the forward's per-row
// log-sum-exp), dV += P^T dO, dP = dO V^T, dS = (dP - rowsum(P dP)) P, times
// 1 - tanh^2(s_pre / c) under a softcap c, dQ = scale dS K, dK = scale dS^T Q,
// with dK / dV summed over each KV head's query group.  rowsum(P dP) equals
// dO . O (the derivation page's section 1: O is the P-weighted sum of V rows),
// which the forward pass computes per row from its float32 accumulator
// (`stats`, together with the log-sum-exp in log2 units).
//
// Two kernels, each owning what it writes, so no atomics and a fixed order:
//
//  * bwd_dkdv_kernel: a workgroup owns 128 keys of one (sequence, KV head),
//    each of its 8 waves 16 of them (two waves per SIMD: the state of a
//    16-key wave fits half the register file).  It walks every query head of
//    the group and every 32-query tile that can see those keys; the tiles of
//    Q, dO and the row statistics are copied global -> LDS asynchronously,
//    double buffered, shared by the 8 waves.  Per tile and wave, on the
//    16x16x32 instruction with the wave's keys in the accumulator columns
//    (lane l: key l % 16):
//      S  = Q K^T   (Q rows from LDS, K in registers)     8 MFMAs at D = 128
//      dP = dO V^T  (dO rows from LDS, V in registers)    8
//      dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T read through the
//      LDS transpose read and P, dS already in the B-operand layout   8 + 8
//    At D = 256 the two accumulators would not fit: there each key block gets
//    two workgroups, each accumulating the dK/dV columns of one half of the
//    head dimension (both still contract S and dP over all of it, so S and dP
//    are computed twice).
//  * bwd_dq_kernel: the forward kernel's shape -- 4 waves x 32 query rows, K
//    and V tiles of 64 keys through LDS -- with, per tile,
//      S^T = K Q^T and dP^T = V dO^T (Q and dO in registers)          16 + 16
//      dQ^T += K^T dS^T (K^T through the LDS transpose read)          16
//    Its launch has extra workgroups after the dQ ones: those sum the float32
//    partials of the dK/dV key blocks that were split into chunks (in chunk
//    order), filling the compute units that the dQ tail leaves idle.
#include <limits.h>

#include "device_common.h"
#include "launch.h"

#ifndef ATTN_ELEM
#error "build with -DATTN_ELEM=<__bf16|_Float16> -DATTN_D=<64|128|256> -DATTN_TAG=<name>"
#endif
#define ATTN_CAT2(a, b) a##b
#define ATTN_CAT(a, b) ATTN_CAT2(a, b)

namespace attn {
namespace {

constexpr int kNW = 4;         // dQ: waves per workgroup
constexpr int kThreads = kNW * 64;
constexpr int kBQ = 32;       // dK/dV: queries per tile
constexpr int kKW = 16;       // dK/dV: keys per wave
constexpr int kKvW = 8;       // dK/dV: waves per workgroup (two per SIMD)
constexpr int kKvThreads = kKvW * 64;
constexpr int kBK = kKvW * kKW;  // dK/dV: keys per workgroup
constexpr int kBN = 64;       // dQ: keys per tile
constexpr int kQW = 32;       // dQ: query rows per wave
constexpr int kBM = kNW * kQW;  // dQ: query rows per workgroup

enum : int { B_MASK = 1, B_SOFTCAP = 2, B_ALIBI = 4 };

// dK/dV workgroups per key block: one per half of the head dimension at D = 256
template <int D>
constexpr int kDHalves = D > 128 ? 2 : 1;

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* alibi;
  const float2* stats;  // [B * Hq * Sq]: (LSE in log2 units, +inf without keys; dO . O)
  void* dq;
  void* dk;
  void* dv;
  int Sq, Sk, Hq, Hkv, group;
  int wl;        // left window, -1 = unbounded
  int has_hi;    // is j - i' bounded above?
  int dmax;      // that bound
  float scale;   // softmax scale
  float c_score; // log2(e) * scale; with softcap 2 * log2(e) * scale / cap
  float c_cap;   // log2(e) * cap
  int nbh_kv;    // B * Hkv
  int nbh;       // B * Hq
  int nqb;       // dQ: 128-row query blocks per head
  int heavy_first;
  int nkb;       // 128-key blocks per KV head
  int chunk;     // dK/dV items per workgroup (see BwdProblem)
  int nchunk;    // chunk slots per key block
  float* part;   // [nbh_kv][nkb][nchunk][2][128][D] float32 partial dK, dV
};

// XOR swizzle of the 16-byte chunk index of tile row r: the matrix-operand
// row reads (32 rows, one chunk each) hit distinct banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D >= 128 ? (r & 15) : ((r >> 1) & 7);
}

// Transformed score in log2 units (softcap, then ALiBi) of the raw dot
// product x, and tanh(s_pre / cap) for the softcap derivative.
template <bool SOFTCAP, bool ALIBI>
__device__ __forceinline__ float transform(float x, const BwdArgs& a, float slope_l2, int rel,
                                           float& t) {
  float y;
  if constexpr (SOFTCAP) {
    const float e = fast_exp2(x * a.c_score);
    t = 1.f - 2.f * fast_rcp(1.f + e);
    y = a.c_cap * t;
  } else {
    t = 0.f;
    y = x * a.c_score;
  }
  if constexpr (ALIBI) y = __builtin_fmaf(slope_l2, (float)rel, y);
  return y;
}

// A = X^T (d rows x 16 tile rows per step) through the LDS transpose read, for
// the 32x32x16 instruction: step ks covers tile rows 16 ks .. 16 ks + 15 in
// the order the accumulator holds them (rows 4 g .. 4 g + 3, then 8 + 4 g ..),
// d block db.  Tile rows are D elements, chunks swizzled by swz.
template <typename T, int D>
__device__ __forceinline__ u32x4 tr_operand(const T* X, int ks, int db, int lane) {
  const int g = (lane >> 5) & 1;
  const int trow = 4 * g + ((lane & 15) >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int r0 = 16 * ks + trow;
  const int col = 32 * db + tcol;
  const int c_lo = ((col >> 3) ^ swz<D>(r0)) * 8 + (col & 7);
  const int c_hi = ((col >> 3) ^ swz<D>(r0 + 8)) * 8 + (col & 7);
  const u32x2 lo = lds_read_tr16(X + r0 * D + c_lo);
  const u32x2 hi = lds_read_tr16(X + (r0 + 8) * D + c_hi);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Asynchronous copy of rows [row0, row0 + ROWS) of a [*, D] tensor (rows past
// `rows_left` read zero) into a swizzled LDS tile, by all threads.
template <typename T, int D, int ROWS>
__device__ __forceinline__ void copy_tile(const T* base, int rows_left, u32x4* dst, int tid,
                                          int wave) {
  constexpr int NC = D / 8;
  constexpr int TC = ROWS * NC;
  constexpr int CPT = TC / kThreads;
  static_assert(CPT * kThreads == TC, "tile must split evenly over the workgroup");
  const __amdgpu_buffer_rsrc_t rs = make_rsrc32(base, rows_left * D * (int)sizeof(T));
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = i * kThreads + tid;
    const int r = c / NC, pc = c % NC;
    dma16(rs, dst + i * kThreads + wave * 64, (r * D + (pc ^ swz<D>(r)) * 8) * (int)sizeof(T));
  }
}

// ---------------------------------------------------------------- dK, dV

// A = X^T (16 d rows x the tile's 32 queries) for the 16x16x32 instruction,
// through the LDS transpose read: lane l (lane group G = l / 16) takes d row
// 16 db + l % 16, and its 8 k-slots are tile rows 4 G .. 4 G + 3, then
// 16 + 4 G .. + 3 -- the rows the same lane holds in the 16x16 accumulator
// layout of S and dP (rows 4 G .. + 3 of each 16-row block), so P and dS are
// the B operands as they stand.  Tile rows are D elements, chunks swizzled.
template <typename T, int D>
__device__ __forceinline__ u32x4 tr16_operand(const T* X, int db, int lane) {
  const int G = lane >> 4;
  const int r = (lane & 15) >> 2, p = lane & 3;  // row r, piece p of a 4 x 16 block
  const int row0 = 4 * G + r, row1 = 16 + 4 * G + r;
  const int col = 16 * db + 4 * p;
  const int c0 = ((col >> 3) ^ swz<D>(row0)) * 8 + (col & 7);
  const int c1 = ((col >> 3) ^ swz<D>(row1)) * 8 + (col & 7);
  const u32x2 lo = lds_read_tr16(X + row0 * D + c0);
  const u32x2 hi = lds_read_tr16(X + row1 * D + c1);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Asynchronous copy of the 32 rows of Q and of dO that start at q and dout
// (rows past `rows_left` read zero) into their swizzled LDS tiles, by all
// threads of a dK/dV workgroup; each wave copies 64 chunks of one tensor.
template <typename T, int D>
__device__ __forceinline__ void copy_q_do(const T* q, const T* dout, int rows_left, u32x4* qd, u32x4* od,
                                          int tid, int wave) {
  constexpr int NC = D / 8;
  constexpr int TC = kBQ * NC;                 // chunks per tensor
  constexpr int CPT = 2 * TC / kKvThreads;     // chunks per thread
  static_assert(CPT * kKvThreads == 2 * TC && TC % 64 == 0, "tiles must split evenly over the waves");
  const int bytes = rows_left * D * (int)sizeof(T);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc32(q, bytes);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc32(dout, bytes);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c0 = i * kKvThreads + wave * 64;   // this wave's first chunk (wave-uniform)
    const bool is_o = c0 >= TC;
    const int cc = (is_o ? c0 - TC : c0) + (tid & 63);
    const int r = cc / NC, pc = cc % NC;
    const int off = (r * D + (pc ^ swz<D>(r)) * 8) * (int)sizeof(T);
    dma16(is_o ? ro : rq, (is_o ? od : qd) + (is_o ? c0 - TC : c0), off);
  }
}

// dK/dV: transpose-read operands in flight ahead of their product (4 timed
// best of 2, 4, 6 and 8 on the causal 2K workload)
constexpr int kTrPF = 4;

template <typename T, int D, int FLAGS>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdArgs a) {
  using E = Elem<T>;
  constexpr bool MASK = (FLAGS & B_MASK) != 0;
  constexpr bool SOFTCAP = (FLAGS & B_SOFTCAP) != 0;
  constexpr bool ALIBI = (FLAGS & B_ALIBI) != 0;
  constexpr int NC = D / 8;
  constexpr int KS = D / 32;       // 16x16x32 steps of S and dP over d
  constexpr int TC = kBQ * NC;
  // D = 256: each workgroup accumulates the dK, dV columns of one half of the
  // head dimension (S and dP are still contracted over all of it), which keeps
  // the accumulators within two waves' share of the register file
  constexpr int NH = kDHalves<D>;
  constexpr int DB = D / 16 / NH;  // 16-column blocks of dK^T, dV^T per workgroup

  __shared__ u32x4 qbuf0[TC], qbuf1[TC], obuf0[TC], obuf1[TC];
  __shared__ float2 sbuf0[kBQ], sbuf1[kBQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4;  // lane group: accumulator rows 4 G .. 4 G + 3 of each 16-row block
  const int n = lane & 15;  // this lane's key within the wave's 16; also its A-operand row

  // ---- work item: chunk ch of key block kblk of (b, kvh); low key blocks
  // see the most queries under a causal mask, so they go first
  const int dh = NH > 1 ? (int)(blockIdx.x % NH) : 0;  // half of the head dimension
  const int db0 = dh * DB;                              // its first 16-column block
  const int id = blockIdx.x / NH;
  const int kc = id / a.nbh_kv;
  const int bkv = id - kc * a.nbh_kv;
  const int kblk = kc / a.nchunk;
  const int ch = kc - kblk * a.nchunk;
  const int b = bkv / a.Hkv;
  const int kvh = bkv - b * a.Hkv;
  const int Sq = a.Sq, Sk = a.Sk, off = Sk - Sq;
  const int k0 = kblk * kBK;
  const int j0 = k0 + wave * kKW;  // this wave's first key
  const int j = j0 + n;            // this lane's key
  const size_t kv_off = (size_t)(b * a.Hkv + kvh) * Sk * D;
  const T* K = reinterpret_cast<const T*>(a.k) + kv_off;
  const T* V = reinterpret_cast<const T*>(a.v) + kv_off;

  // K and V rows of this lane's key as B operands: step s is d = 32 s + 8 G .. + 7
  u32x4 kf[KS], vf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kf[s] = j < Sk ? load16(K + (size_t)j * D + 32 * s + 8 * G) : zero_u32x4();
    vf[s] = j < Sk ? load16(V + (size_t)j * D + 32 * s + 8 * G) : zero_u32x4();
  }

  // admissible iff lo <= j - i' <= hi
  const int lo = a.wl >= 0 ? -a.wl : INT_MIN / 2;
  const int hi = a.has_hi ? a.dmax : INT_MAX / 2;
  // query rows that can see a key of this workgroup: i' in [k0 - hi, k_last - lo]
  const int k_last = min(k0 + kBK, Sk) - 1;
  const int q_lo = a.has_hi ? max(0, k0 - hi - off) : 0;
  const int q_hi = a.wl >= 0 ? min(Sq, k_last - lo - off + 1) : Sq;  // one past
  const int t_lo = q_lo / kBQ;
  const int nt = q_hi > q_lo && k_last >= k0 ? (q_hi + kBQ - 1) / kBQ - t_lo : 0;
  const int n_all = nt * a.group;
  const int n_ch = n_all > 0 ? (n_all + a.chunk - 1) / a.chunk : 1;  // chunks of this block
  if (ch >= n_ch) return;  // the whole workgroup: an unused chunk slot
  const int it0 = ch * a.chunk;
  const int n_items = min(n_all, it0 + a.chunk) - it0;

  // per wave: keys [j0, jw_last]
  const int jw_last = min(j0 + kKW, Sk) - 1;
  auto live = [&](int q0) {
    if (jw_last < j0) return false;
    const int ql = min(q0 + kBQ, Sq) - 1;
    const int dlo = j0 - (ql + off), dhi = jw_last - (q0 + off);
    return dhi >= lo && dlo <= hi;
  };
  auto full = [&](int q0) {
    const int dlo = j0 - (q0 + kBQ - 1 + off), dhi = j0 + kKW - 1 - (q0 + off);
    return q0 + kBQ <= Sq && j0 + kKW <= Sk && dlo >= lo && dhi <= hi;
  };

  floatx4 dkt[DB], dvt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkt[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    dvt[db] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // The items of this chunk are the flattened indices it0 .. over (head,
  // tile).  A cursor (query head, first query row) walks them in order, one
  // for the copies and one for the computation a step behind, so that no item
  // divides by the tile count.
  struct Cursor {
    int h, q0;
  };
  const int q_end = (t_lo + nt) * kBQ;
  auto advance = [&](Cursor& c) {
    c.q0 += kBQ;
    if (c.q0 == q_end) {
      c.q0 = t_lo * kBQ;
      ++c.h;
    }
  };
  Cursor cur_copy = {kvh * a.group + it0 / nt, (t_lo + it0 % nt) * kBQ};
  Cursor cur_comp = cur_copy;
  auto copy_item = [&](u32x4* qd, u32x4* od, float2* sd) {
    const int h = cur_copy.h, q0 = cur_copy.q0;
    advance(cur_copy);
    const size_t row0 = (size_t)(b * a.Hq + h) * Sq + q0;
    copy_q_do<T, D>(reinterpret_cast<const T*>(a.q) + row0 * D, reinterpret_cast<const T*>(a.dout) + row0 * D,
                    Sq - q0, qd, od, tid, wave);
    if (wave == 0) {
      // 32 (LSE, dO.O) pairs: one dword per lane
      const __amdgpu_buffer_rsrc_t rs = make_rsrc32(a.stats + row0, (Sq - q0) * 8);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (ATTN_LDS void*)sd, 4, 4 * lane, 0, 0, 0);
    }
  };

  auto compute = [&](const u32x4* qs, const u32x4* os, const float2* ss) {
    const int h = cur_comp.h, q0 = cur_comp.q0;
    advance(cur_comp);
    if (!live(q0)) return;
    // S = Q K^T, dP = dO V^T in two 16-query blocks: block qb holds queries
    // 16 qb + 4 G .. + 3 (rows) x this wave's 16 keys (lane n)
    floatx4 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
      dp[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const int r = 16 * qb + n;  // A operand: query row 16 qb + l % 16, d = 32 st + 8 G .. + 7
        const int c = (4 * st + G) ^ swz<D>(r);
        s[qb] = E::mma16(qs[r * NC + c], kf[st], s[qb]);
        dp[qb] = E::mma16(os[r * NC + c], vf[st], dp[qb]);
      }
    }
    // The A operands of the dV and dK products (operand f: dO^T for even f,
    // Q^T for odd, 16-column block db0 + f / 2) do not depend on P: the first
    // kTrPF are read before the element-wise work, whose time hides their
    // latency, and each later one kTrPF products ahead of its use.
    const T* Os = reinterpret_cast<const T*>(os);
    const T* Qs = reinterpret_cast<const T*>(qs);
    // (Not at head dim 256, where the registers are short.)
    constexpr int NF = 2 * DB;
    constexpr int PF = D > 128 ? 0 : (kTrPF < NF ? kTrPF : NF);
    auto tr_op = [&](int f) { return tr16_operand<T, D>((f & 1) ? Qs : Os, db0 + (f >> 1), lane); };
    u32x4 trf[PF > 0 ? PF : 1];
#pragma unroll
    for (int f = 0; f < PF; ++f) trf[f] = tr_op(f);
    float slope_l2 = 0.f;
    if constexpr (ALIBI) slope_l2 = a.alibi[h] * kLog2e;
    // statistics of rows 16 qb + 4 G .. + 3: LSE (log2 units) and dO . O
    const float4* sp = reinterpret_cast<const float4*>(ss);
    float lse2[2][4], dlt[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float4 s01 = sp[8 * qb + 2 * G], s23 = sp[8 * qb + 2 * G + 1];
      lse2[qb][0] = s01.x, lse2[qb][1] = s01.z, lse2[qb][2] = s23.x, lse2[qb][3] = s23.z;
      dlt[qb][0] = s01.y, dlt[qb][1] = s01.w, dlt[qb][2] = s23.y, dlt[qb][3] = s23.w;
    }
    // exponents of P (transformed score minus the row's LSE), tanh(s / cap)
    // for the softcap derivative
    float e[2][4], th[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (!SOFTCAP && !ALIBI) {
          e[qb][c] = __builtin_fmaf(s[qb][c], a.c_score, -lse2[qb][c]);
        } else {
          const int rel = j - (q0 + 16 * qb + 4 * G + c + off);
          e[qb][c] = transform<SOFTCAP, ALIBI>(s[qb][c], a, slope_l2, rel, th[qb][c]) - lse2[qb][c];
        }
      }
    // the mask, on tiles that straddle a boundary only
    if (MASK && !full(q0)) {
      const uint32_t span = (uint32_t)(hi - lo);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int qrow = q0 + 16 * qb + 4 * G + c;
          const int rel = j - (qrow + off);
          const bool out = qrow >= Sq || j >= Sk || (uint32_t)(rel - lo) > span;
          e[qb][c] = out ? kNegInf : e[qb][c];
        }
    }
    // P and dS as the B operands of the dV and dK products: k-slots 8 G + 4 qb
    // + c are query rows 16 qb + 4 G + c
    u32x4 pf, df;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float pv[4], dsv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float p = fast_exp2(e[qb][c]);
        float d = p * (dp[qb][c] - dlt[qb][c]);
        if constexpr (SOFTCAP) d *= 1.f - th[qb][c] * th[qb][c];
        pv[c] = p;
        dsv[c] = d;
      }
      pf[2 * qb] = E::pack2(pv[0], pv[1]);
      pf[2 * qb + 1] = E::pack2(pv[2], pv[3]);
      df[2 * qb] = E::pack2(dsv[0], dsv[1]);
      df[2 * qb + 1] = E::pack2(dsv[2], dsv[3]);
    }
    // dV^T += dO^T P, dK^T += Q^T dS over the tile's 32 queries
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      u32x4 op;
      if constexpr (PF > 0) {
        op = trf[f % PF];
        if (f + PF < NF) trf[f % PF] = tr_op(f + PF);
      } else {
        op = tr_op(f);
      }
      if (f & 1) dkt[f >> 1] = E::mma16(op, df, dkt[f >> 1]);
      else dvt[f >> 1] = E::mma16(op, pf, dvt[f >> 1]);
    }
  };

  if (n_items > 0) copy_item(qbuf0, obuf0, sbuf0);
  wait_vmem();
  __syncthreads();
  for (int it = 0; it < n_items; it += 2) {
    if (it + 1 < n_items) copy_item(qbuf1, obuf1, sbuf1);
    compute(qbuf0, obuf0, sbuf0);
    wait_vmem();
    __syncthreads();
    if (it + 1 < n_items) {
      if (it + 2 < n_items) copy_item(qbuf0, obuf0, sbuf0);
      compute(qbuf1, obuf1, sbuf1);
      wait_vmem();
      __syncthreads();
    }
  }

  // ---- a block of several chunks: this chunk's float32 partials (summed by
  // the dQ launch's extra workgroups); this lane's key row, d = 16 db + 4 G .. + 3
  if (n_ch > 1) {
    float* pk = a.part + ((((size_t)bkv * a.nkb + kblk) * a.nchunk + ch) * 2) * kBK * D +
                (size_t)(j - k0) * D + 16 * db0;
    float* pv = pk + (size_t)kBK * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      *reinterpret_cast<floatx4*>(pk + 16 * db + 4 * G) = dkt[db];
      *reinterpret_cast<floatx4*>(pv + 16 * db + 4 * G) = dvt[db];
    }
    return;
  }
  // ---- store: this lane's key row, d = 16 db + 4 G .. + 3
  if (j < Sk) {
    T* dkr = reinterpret_cast<T*>(a.dk) + kv_off + (size_t)j * D + 16 * db0;
    T* dvr = reinterpret_cast<T*>(a.dv) + kv_off + (size_t)j * D + 16 * db0;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x2 wk = {E::pack2(dkt[db][0] * a.scale, dkt[db][1] * a.scale),
                        E::pack2(dkt[db][2] * a.scale, dkt[db][3] * a.scale)};
      const u32x2 wv = {E::pack2(dvt[db][0], dvt[db][1]), E::pack2(dvt[db][2], dvt[db][3])};
      *reinterpret_cast<u32x2*>(dkr + 16 * db + 4 * G) = wk;
      *reinterpret_cast<u32x2*>(dvr + 16 * db + 4 * G) = wv;
    }
  }
}

// Sum of the chunks' partials of every multi-chunk key block, in chunk
// order: one thread per 4 d of one key row.
template <typename T, int D>
__device__ __forceinline__ void reduce_rows(const BwdArgs& a, int wg) {
  using E = Elem<T>;
  constexpr int TPR = D / 4;              // threads per key row
  constexpr int RPW = 256 / TPR;          // key rows per workgroup
  const int blk = wg / (kBK / RPW);       // (bkv, key block)
  const int r = (wg % (kBK / RPW)) * RPW + threadIdx.x / TPR;
  const int d4 = (threadIdx.x % TPR) * 4;
  const int bkv = blk / a.nkb, kblk = blk - bkv * a.nkb;
  const int Sq = a.Sq, Sk = a.Sk, off = Sk - Sq;
  const int k0 = kblk * kBK;
  const int j = k0 + r;
  if (j >= Sk) return;
  // chunks of this block, as the dK/dV kernel counts them
  const int lo = a.wl >= 0 ? -a.wl : INT_MIN / 2;
  const int hi = a.has_hi ? a.dmax : INT_MAX / 2;
  const int k_last = min(k0 + kBK, Sk) - 1;
  const int q_lo = a.has_hi ? max(0, k0 - hi - off) : 0;
  const int q_hi = a.wl >= 0 ? min(Sq, k_last - lo - off + 1) : Sq;
  const int nt = q_hi > q_lo ? (q_hi + kBQ - 1) / kBQ - q_lo / kBQ : 0;
  const int n_all = nt * a.group;
  const int n_ch = n_all > 0 ? (n_all + a.chunk - 1) / a.chunk : 1;
  if (n_ch < 2) return;
  const float* base = a.part + (((size_t)bkv * a.nkb + kblk) * a.nchunk) * 2 * kBK * D +
                      (size_t)r * D + d4;
  floatx4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < n_ch; ++c) {
    const floatx4 xk = *reinterpret_cast<const floatx4*>(base + (size_t)c * 2 * kBK * D);
    const floatx4 xv = *reinterpret_cast<const floatx4*>(base + (size_t)c * 2 * kBK * D + kBK * D);
    sk += xk;
    sv += xv;
  }
  const int b = bkv / a.Hkv, kvh = bkv - b * a.Hkv;
  const size_t row = ((size_t)(b * a.Hkv + kvh) * Sk + j) * D + d4;
  const u32x2 wk = {E::pack2(sk[0] * a.scale, sk[1] * a.scale), E::pack2(sk[2] * a.scale, sk[3] * a.scale)};
  const u32x2 wv = {E::pack2(sv[0], sv[1]), E::pack2(sv[2], sv[3])};
  *reinterpret_cast<u32x2*>(reinterpret_cast<T*>(a.dk) + row) = wk;
  *reinterpret_cast<u32x2*>(reinterpret_cast<T*>(a.dv) + row) = wv;
}

// ---------------------------------------------------------------- dQ

template <typename T, int D, int FLAGS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : 2, D > 128 ? 1 : 2)))
void bwd_dq_kernel(BwdArgs a) {
  using E = Elem<T>;
  constexpr bool MASK = (FLAGS & B_MASK) != 0;
  constexpr bool SOFTCAP = (FLAGS & B_SOFTCAP) != 0;
  constexpr bool ALIBI = (FLAGS & B_ALIBI) != 0;
  constexpr int NC = D / 8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TC = kBN * NC;

  __shared__ u32x4 kbuf0[TC], kbuf1[TC], vbuf0[TC], vbuf1[TC];

  // workgroups past the dQ grid sum the dK/dV chunk partials (the last ones
  // dispatched: they fill the compute units the dQ tail leaves idle)
  if ((int)blockIdx.x >= a.nbh * a.nqb) {
    reduce_rows<T, D>(a, (int)blockIdx.x - a.nbh * a.nqb);
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int ln = lane & 31;

  // ---- work item: (query block, head, batch), heaviest first when causal;
  // contiguous runs of heads per dispatch round go to one XCD (shared K/V)
  const int id = blockIdx.x;
  const int round = id / a.nbh;
  const int u = id - round * a.nbh;
  const int bh = (a.nbh & 7) == 0 ? ((u & 7) * (a.nbh >> 3) + (u >> 3)) : u;
  const int qb = a.heavy_first ? (a.nqb - 1 - round) : round;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int kvh = h / a.group;
  const int m0 = qb * kBM;
  const int Sq = a.Sq, Sk = a.Sk, off = Sk - Sq;
  const size_t kv_off = (size_t)(b * a.Hkv + kvh) * Sk * D;
  const T* K = reinterpret_cast<const T*>(a.k) + kv_off;
  const T* V = reinterpret_cast<const T*>(a.v) + kv_off;

  const int lo = a.wl >= 0 ? -a.wl : INT_MIN / 2;
  const int hi = a.has_hi ? a.dmax : INT_MAX / 2;
  auto key_lo = [&](int ipa) { return a.wl >= 0 ? max(0, ipa - a.wl) : 0; };
  auto key_hi = [&](int ipb) { return a.has_hi ? min(Sk, max(0, ipb + a.dmax + 1)) : Sk; };
  const int wg_last = min(m0 + kBM, Sq) - 1;
  const int n_lo = key_lo(m0 + off);
  const int n_hi = key_hi(wg_last + off);
  const int t_begin = n_lo / kBN;
  const int t_end = n_hi > n_lo ? (n_hi + kBN - 1) / kBN : t_begin;
  const int n = t_end - t_begin;

  const int wq0 = m0 + wave * kQW;
  const bool wave_live = wq0 < Sq;
  const int wq_last = min(wq0 + kQW, Sq) - 1;
  const int w_lo = key_lo(wq0 + off);
  const int w_hi = key_hi(wq_last + off);
  auto live = [&](int t) { return wave_live && t * kBN < w_hi && (t + 1) * kBN > w_lo; };
  auto full = [&](int t) {
    const int n0 = t * kBN;
    return n0 + kBN <= Sk && wq0 + kQW <= Sq && (n0 + kBN - 1) - (wq0 + off) <= hi &&
           n0 - (wq0 + kQW - 1 + off) >= lo;
  };

  const int qi = wq0 + ln;
  const int ip = qi + off;
  const T* Qr = reinterpret_cast<const T*>(a.q) + ((size_t)bh * Sq + qi) * D;
  const T* dOr = reinterpret_cast<const T*>(a.dout) + ((size_t)bh * Sq + qi) * D;
  u32x4 qf[KS], of[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = qi < Sq ? load16(Qr + 16 * s + 8 * g) : zero_u32x4();
    of[s] = qi < Sq ? load16(dOr + 16 * s + 8 * g) : zero_u32x4();
  }
  const float2 stt = qi < Sq ? a.stats[(size_t)bh * Sq + qi] : float2{__builtin_inff(), 0.f};
  float slope_l2 = 0.f;
  if constexpr (ALIBI) slope_l2 = a.alibi[h] * kLog2e;

  floatx16 dqt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqt[db] = floatx16{};

  const int kv_rows = Sk;
  auto copy_kv = [&](int t, u32x4* kd, u32x4* vd) {
    const int n0 = t * kBN;
    copy_tile<T, D, kBN>(K + (size_t)n0 * D, kv_rows - n0, kd, tid, wave);
    copy_tile<T, D, kBN>(V + (size_t)n0 * D, kv_rows - n0, vd, tid, wave);
  };

  auto compute = [&](int t, const u32x4* ks_, const u32x4* vs_) {
    if (!live(t)) return;
    const int n0 = t * kBN;
    // S^T = K Q^T and dP^T = V dO^T: sc[kb] keys 32 kb .. + 31 (rows) x queries (lanes)
    floatx16 sc[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = floatx16{};
      dp[kb] = floatx16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int r = 32 * kb + ln;
        const int c = (2 * s + g) ^ swz<D>(r);
        sc[kb] = E::mma32(ks_[r * NC + c], qf[s], sc[kb]);
        dp[kb] = E::mma32(vs_[r * NC + c], of[s], dp[kb]);
      }
    }
    const bool need_mask = MASK && !full(t);
    uint32_t dsp[16];
    if constexpr (!SOFTCAP && !ALIBI) {
      // exponents of P in place of the scores (scaled score minus the row's
      // LSE, one FMA), the mask on tiles that straddle a boundary only
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][r] = __builtin_fmaf(sc[kb][r], a.c_score, -stt.x);
      if (need_mask) {
        const uint32_t span = (uint32_t)(hi - lo);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = n0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            const int rel = key - ip;
            const bool out = qi >= Sq || key >= Sk || (uint32_t)(rel - lo) > span;
            sc[kb][r] = out ? kNegInf : sc[kb][r];
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float d0 = fast_exp2(sc[kb][r]) * (dp[kb][r] - stt.y);
          const float d1 = fast_exp2(sc[kb][r + 1]) * (dp[kb][r + 1] - stt.y);
          dsp[kb * 8 + r / 2] = E::pack2(d0, d1);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float dv2[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int key = n0 + 32 * kb + 8 * ((r + c) >> 2) + 4 * g + ((r + c) & 3);
            const int rel = key - ip;
            float tt;
            float x = transform<SOFTCAP, ALIBI>(sc[kb][r + c], a, slope_l2, rel, tt);
            if (need_mask && (qi >= Sq || key >= Sk || rel < lo || rel > hi)) x = kNegInf;
            const float p = fast_exp2(x - stt.x);
            float d = p * (dp[kb][r + c] - stt.y);
            if constexpr (SOFTCAP) d *= 1.f - tt * tt;
            dv2[c] = d;
          }
          dsp[kb * 8 + r / 2] = E::pack2(dv2[0], dv2[1]);
        }
    }
    // dQ^T += K^T dS^T over the tile's 64 keys, 16 per step
    const T* Ks = reinterpret_cast<const T*>(ks_);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 df = {dsp[4 * ks], dsp[4 * ks + 1], dsp[4 * ks + 2], dsp[4 * ks + 3]};
#pragma unroll
      for (int db = 0; db < DB; ++db)
        dqt[db] = E::mma32(tr_operand<T, D>(Ks, ks, db, lane), df, dqt[db]);
    }
  };

  if (n > 0) copy_kv(t_begin, kbuf0, vbuf0);
  wait_vmem();
  __syncthreads();
  for (int i = 0; i < n; i += 2) {
    if (i + 1 < n) copy_kv(t_begin + i + 1, kbuf1, vbuf1);
    compute(t_begin + i, kbuf0, vbuf0);
    wait_vmem();
    __syncthreads();
    if (i + 1 < n) {
      if (i + 2 < n) copy_kv(t_begin + i + 2, kbuf0, vbuf0);
      compute(t_begin + i + 1, kbuf1, vbuf1);
      wait_vmem();
      __syncthreads();
    }
  }

  if (qi < Sq) {
    T* dqr = reinterpret_cast<T*>(a.dq) + ((size_t)bh * Sq + qi) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 w;
        w[0] = E::pack2(dqt[db][4 * jj] * a.scale, dqt[db][4 * jj + 1] * a.scale);
        w[1] = E::pack2(dqt[db][4 * jj + 2] * a.scale, dqt[db][4 * jj + 3] * a.scale);
        *reinterpret_cast<u32x2*>(dqr + 32 * db + 8 * jj + 4 * g) = w;
      }
  }
}

template <int FLAGS>
hipError_t launch_pair(const BwdArgs& a, int grid_kv, int grid_q, hipStream_t stream) {
  if (grid_kv > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<ATTN_ELEM, ATTN_D, FLAGS>), dim3(grid_kv), dim3(kKvThreads), 0,
                       stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RPW = 256 / (ATTN_D / 4);
  const int grid_red = grid_kv > 0 && a.nchunk > 1 ? a.nbh_kv * a.nkb * (kBK / RPW) : 0;
  if (grid_q + grid_red > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<ATTN_ELEM, ATTN_D, FLAGS>), dim3(grid_q + grid_red), dim3(kThreads), 0,
                       stream, a);
  return hipGetLastError();
}

// Row statistics of the backward from the forward's saved output and LSE:
// stats[row] = (lse in log2 units, or +inf for a row without keys; dO . O).
// D / 8 lanes per row, one 16-byte load of O and of dO each.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_rowstats_kernel(const T* out, const T* dout, const float* lse,
                                                           float2* stats, long long rows) {
  constexpr int LPR = D / 8;       // lanes per row
  constexpr int RPW = 64 / LPR;    // rows per wave
  const int lane = threadIdx.x & 63;
  const long long row = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int c = lane % LPR;
  float part = 0.f;
  if (row < rows) {
    const u32x4 o = load16(out + row * D + 8 * c);
    const u32x4 d = load16(dout + row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t ho = (o[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      const uint32_t hd = (d[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      part = __builtin_fmaf(Elem<T>::to_float(ho), Elem<T>::to_float(hd), part);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
  if (row < rows && c == 0) {
    const float l = lse[row];
    stats[row] = float2{l == kNegInf ? __builtin_inff() : l * kLog2e, part};
  }
}

}  // namespace

hipError_t ATTN_CAT(launch_bwd_rowstats_, ATTN_TAG)(const void* out, const void* dout, const float* lse,
                                                    float* stats, long long rows, hipStream_t stream) {
  constexpr int RPB = 4 * (64 / (ATTN_D / 8));  // rows per workgroup
  const long long grid = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((bwd_rowstats_kernel<ATTN_ELEM, ATTN_D>), dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const ATTN_ELEM*>(out), reinterpret_cast<const ATTN_ELEM*>(dout), lse,
                     reinterpret_cast<float2*>(stats), rows);
  return hipGetLastError();
}

hipError_t ATTN_CAT(launch_bwd_mfma_, ATTN_TAG)(const BwdProblem& p, hipStream_t stream) {
  BwdArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.dout = p.dout;
  a.alibi = p.alibi;
  a.stats = reinterpret_cast<const float2*>(p.stats);
  a.dq = p.dq;
  a.dk = p.dk;
  a.dv = p.dv;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.group = p.Hq / p.Hkv;
  a.wl = p.wl;
  a.has_hi = p.causal || p.wr >= 0;
  a.dmax = p.causal ? (p.wr >= 0 ? min(p.wr, 0) : 0) : p.wr;
  a.scale = p.scale;
  const bool softcap = p.softcap > 0.f;
  a.c_score = softcap ? 2.f * kLog2e * p.scale / p.softcap : kLog2e * p.scale;
  a.c_cap = kLog2e * p.softcap;
  a.nbh_kv = p.B * p.Hkv;
  a.nbh = p.B * p.Hq;
  a.nqb = (p.Sq + kBM - 1) / kBM;
  a.heavy_first = p.causal;
  a.nkb = (p.Sk + kBK - 1) / kBK;
  a.chunk = p.chunk_items;
  a.nchunk = p.max_chunks;
  a.part = p.partials;
  const int grid_kv = a.nbh_kv * a.nkb * a.nchunk * kDHalves<ATTN_D>;
  const int grid_q = a.nbh * a.nqb;
  const bool mask = p.causal || p.wl >= 0 || p.wr >= 0 || (p.Sk % kBK) != 0 || (p.Sq % kBM) != 0;
  const int flags = (mask ? B_MASK : 0) | (softcap ? B_SOFTCAP : 0) | (p.alibi ? B_ALIBI : 0);
  switch (flags) {
    case 0: return launch_pair<0>(a, grid_kv, grid_q, stream);
    case 1: return launch_pair<1>(a, grid_kv, grid_q, stream);
    case 2: return launch_pair<2>(a, grid_kv, grid_q, stream);
    case 3: return launch_pair<3>(a, grid_kv, grid_q, stream);
    case 4: return launch_pair<4>(a, grid_kv, grid_q, stream);
    case 5: return launch_pair<5>(a, grid_kv, grid_q, stream);
    case 6: return launch_pair<6>(a, grid_kv, grid_q, stream);
    default: return launch_pair<7>(a, grid_kv, grid_q, stream);
  }
}

}  // namespace attn
