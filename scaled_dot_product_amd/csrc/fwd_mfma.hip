// fwd_mfma.hip -- attention forward for bf16 / f16 on the gfx950 matrix cores.
//
// Computes what the kernel-contract page ("fuel-reference-backend -- attention
// kernel contracts", attention_naive / attention_flash) defines, with the
// streaming softmax of the derivation page ("gfx942 unified attention, from the
// math up", section 3) and its causal tile early exit (section 4).
//
// Compiled once per (element type, head dim): ATTN_ELEM is __bf16 or _Float16,
// ATTN_D is 64 or 128, ATTN_TAG names the exported launcher.
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

enum : int { F_MASK = 1, F_SOFTCAP = 2, F_ALIBI = 4 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alibi;
  void* out;
  float* lse;   // per-row log-sum-exp (natural log), or nullptr
  int Sq, Sk, Hq, Hkv, group, nbh, nqb;
  int heavy_first;
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
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
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

// Transform + mask + online update of one tile's scores, then O += P V.
template <typename T, int D, int FLAGS>
__device__ __forceinline__ void softmax_pv(floatx16 (&sc)[2], const T* Vs, RowState<D / 32>& st,
                                           const FwdArgs& a, int n0, int ip, int ipa_w, int ipb_w,
                                           float slope_l2, int lane, int g) {
  using E = Elem<T>;
  constexpr bool MASK = (FLAGS & F_MASK) != 0;
  constexpr bool SOFTCAP = (FLAGS & F_SOFTCAP) != 0;
  constexpr bool ALIBI = (FLAGS & F_ALIBI) != 0;
  constexpr bool kRaw = !SOFTCAP && !ALIBI;  // max on raw scores, scale folded into exp
  constexpr int DB = D / 32;
  const int Sk = a.Sk;
  const int rb = n0 + 4 * g - ip;            // j - i' of element offset 0

  if constexpr (!kRaw) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sc[kb][r];
        if constexpr (SOFTCAP) {
          const float e = fast_exp2(x * a.c_score);
          x = a.c_cap - 2.f * a.c_cap * fast_rcp(1.f + e);
        } else {
          x *= a.c_score;
        }
        if constexpr (ALIBI) x = __builtin_fmaf(slope_l2, (float)(rb + key_of(kb, r)), x);
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
  float mt = mx;
  if constexpr (kRaw) mt = mx == kNegInf ? kNegInf : mx * a.c_score;
  mt = halves_max(mt);

  // raise the reference max only when the tile exceeds it by > 2^8
  const bool need = mt > st.m_run + kRescaleGap;
  if (wave_any(need)) {
    const float alpha = need ? fast_exp2(st.m_run - mt) : 1.f;
    st.m_run = need ? mt : st.m_run;
    st.l_part *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) st.o[db] *= alpha;
  }
  const float m_use = st.m_run == kNegInf ? 0.f : st.m_run;

  // weights, rounded to the input type, packed as the PV B operand
  uint32_t pp[16];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p0, p1;
      if constexpr (kRaw) {
        p0 = fast_exp2(__builtin_fmaf(sc[kb][r], a.c_score, -m_use));
        p1 = fast_exp2(__builtin_fmaf(sc[kb][r + 1], a.c_score, -m_use));
      } else {
        p0 = fast_exp2(sc[kb][r] - m_use);
        p1 = fast_exp2(sc[kb][r + 1] - m_use);
      }
      const uint32_t pk = E::pack2(p0, p1);
      pp[kb * 8 + r / 2] = pk;
      st.l_part = E::dot2(pk, E::kOnePair, st.l_part);
    }

  // O^T += V^T P^T, 16 keys per step; V^T through the LDS transpose read
  const int trow = 4 * g + ((lane & 15) >> 2);                // key row within a 16-key step
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);   // d within a 32-row block
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4 pf = {pp[4 * ks], pp[4 * ks + 1], pp[4 * ks + 2], pp[4 * ks + 3]};
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

template <typename T, int D, int FLAGS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_mfma_kernel(FwdArgs a) {
  constexpr bool ALIBI = (FLAGS & F_ALIBI) != 0;
  constexpr int NC = D / 8;              // 16-byte chunks per K/V row
  constexpr int TC = kBN * NC;           // chunks per K (or V) tile
  constexpr int CPT = TC / kThreads;     // chunks per thread per tile and tensor
  constexpr int KS = D / 16;             // contraction steps of K Q^T
  constexpr int DB = D / 32;             // 32-row blocks of O^T
  static_assert(CPT * kThreads == TC, "tile must split evenly over the workgroup");

  // Four separate LDS objects so that the compiler can tell the buffer being
  // filled by the asynchronous copy from the buffers being read.
  __shared__ u32x4 kbuf0[TC], kbuf1[TC], vbuf0[TC], vbuf1[TC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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
  const int Sq = a.Sq, Sk = a.Sk, off = Sk - Sq;
  const int m0 = qb * kBM;

  const T* Q = reinterpret_cast<const T*>(a.q) + (size_t)bh * Sq * D;
  const T* K = reinterpret_cast<const T*>(a.k) + (size_t)(b * a.Hkv + kvh) * Sk * D;
  const T* V = reinterpret_cast<const T*>(a.v) + (size_t)(b * a.Hkv + kvh) * Sk * D;
  T* O = reinterpret_cast<T*>(a.out) + (size_t)bh * Sq * D;

  // ---- admissible key ranges: [lo(i'_first), hi(i'_last))
  auto key_lo = [&](int ipa) { return a.wl >= 0 ? max(0, ipa - a.wl) : 0; };
  auto key_hi = [&](int ipb) { return a.has_hi ? min(Sk, max(0, ipb + a.dmax + 1)) : Sk; };
  const int wg_last = min(m0 + kBM, Sq) - 1;
  const int n_lo = key_lo(m0 + off);
  const int n_hi = key_hi(wg_last + off);
  const int t_begin = n_lo / kBN;
  const int t_end = n_hi > n_lo ? (n_hi + kBN - 1) / kBN : t_begin;

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
    qf[s] = qi < Sq ? load16(Q + (size_t)qi * D + 16 * s + 8 * g) : zero_u32x4();

  float slope_l2 = 0.f;
  if constexpr (ALIBI) slope_l2 = a.alibi[h] * kLog2e;

  RowState<DB> st;
#pragma unroll
  for (int db = 0; db < DB; ++db) st.o[db] = floatx16{};
  st.m_run = kNegInf;
  st.l_part = 0.f;

  // ---- asynchronous tile copies global -> LDS.  Chunk c of a tile sits at
  // LDS slot c, i.e. row c / NC, swizzled chunk c % NC; keys past Sk read 0.
  // one head's K (or V) is < 2 GiB (checked by the host), so offsets fit int32
  const int kv_bytes = Sk * D * (int)sizeof(T);
  auto dma_k = [&](u32x4* dst, int t) {
    const int base = t * kBN * D * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc32(reinterpret_cast<const char*>(K) + base, kv_bytes - base);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / NC, pc = c % NC;
      dma16(rs, dst + i * kThreads + wave * 64, (r * D + (pc ^ swz_k<D>(r)) * 8) * (int)sizeof(T));
    }
  };
  auto dma_v = [&](u32x4* dst, int t) {
    const int base = t * kBN * D * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc32(reinterpret_cast<const char*>(V) + base, kv_bytes - base);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = i * kThreads + tid;
      const int r = c / NC, pc = c % NC;
      dma16(rs, dst + i * kThreads + wave * 64, (r * D + (pc ^ swz_v<D>(r)) * 8) * (int)sizeof(T));
    }
  };

  // ---- software pipeline over the tiles t_begin + i:
  //   step i:  softmax(S(i)), O += P(i) V(i)
  //            S(i+1) = K(i+1) Q^T   (matrix cores, into the same registers)
  //   while K(i+2) and V(i+1) stream into the buffers freed by step i-1.
  // K(i) lives in kbuf[i % 2], V(i) in vbuf[i % 2].
  const int n = t_end - t_begin;
  floatx16 sc[2];
  if (n > 0) {
    dma_k(kbuf0, t_begin);
    dma_v(vbuf0, t_begin);
    if (n > 1) dma_k(kbuf1, t_begin + 1);
    wait_vmem();
    __syncthreads();
    if (live(t_begin)) qk_tile<T, D>(kbuf0, qf, ln, g, sc);
  }
  auto step = [&](int i, const u32x4* kread, const u32x4* vread, u32x4* kload, u32x4* vload) {
    const int t = t_begin + i;
    wait_vmem();
    __syncthreads();  // K(i+1), V(i) landed; everyone is done with step i-1's buffers
    if (i + 2 < n) dma_k(kload, t + 2);
    if (i + 1 < n) dma_v(vload, t + 1);
    if (live(t))
      softmax_pv<T, D, FLAGS>(sc, reinterpret_cast<const T*>(vread), st, a, t * kBN, ip, ipa_w,
                              ipb_w, slope_l2, lane, g);
    // S(i+1) overwrites S(i), already consumed: one score buffer per wave.
    // This matrix phase runs at raised wave priority so that, of the two waves
    // sharing a SIMD, the one with matrix work ready wins instruction issue
    // over the one in its softmax (vector) phase.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    if (i + 1 < n && live(t + 1)) qk_tile<T, D>(kread, qf, ln, g, sc);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  for (int i = 0; i < n; i += 2) {
    step(i, kbuf1, vbuf0, kbuf0, vbuf1);
    if (i + 1 < n) step(i + 1, kbuf0, vbuf1, kbuf1, vbuf0);
  }

  // ---- epilogue: O = o / l (0 when no key was admissible)
  const float l = halves_sum(st.l_part);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (a.lse && qi < Sq && g == 0) {
    // lse = ln(sum_j e^{s_j}) = ln 2 * (m + log2 l) with the weights 2^(x - m)
    const float m_use = st.m_run == kNegInf ? 0.f : st.m_run;
    a.lse[(size_t)bh * Sq + qi] = l > 0.f ? (m_use + __log2f(l)) * kLn2 : kNegInf;
  }
  if (qi < Sq) {
    using E = Elem<T>;
    T* orow = O + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w[0] = E::pack2(st.o[db][4 * j] * inv, st.o[db][4 * j + 1] * inv);
        w[1] = E::pack2(st.o[db][4 * j + 2] * inv, st.o[db][4 * j + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * j + 4 * g) = w;
      }
  }
}

template <int FLAGS>
hipError_t launch_flags(const FwdArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_mfma_kernel<ATTN_ELEM, ATTN_D, FLAGS>), dim3(grid), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
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
  a.Sq = p.Sq;
  a.Sk = p.Sk;
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
  a.c_score = softcap ? 2.f * kLog2e * p.scale / p.softcap : kLog2e * p.scale;
  a.c_cap = kLog2e * p.softcap;
  const int grid = a.nqb * a.nbh;
  const bool mask = p.causal || p.wl >= 0 || p.wr >= 0 || (p.Sk % kBN) != 0;
  const int flags = (mask ? F_MASK : 0) | (softcap ? F_SOFTCAP : 0) | (p.alibi ? F_ALIBI : 0);
  switch (flags) {
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

}  // namespace attn
