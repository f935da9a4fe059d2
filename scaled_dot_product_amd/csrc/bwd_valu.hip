// bwd_valu.hip -- attention backward in float32 or float64 throughout (vector
// ALU): the gradients of the kernel-contract page's attention_flash_backward
// (recompute of the softmax from Q, K, V and dO; dK/dV summed over each KV
// head's query group) for F32 and F64 inputs.  Meant for correctness at the
// element type's tolerance, not for speed; deterministic (no atomics, fixed
// orders).
//
//   bwd_valu_rows_kernel: per query row, a first pass over the keys gives the
//     row's softmax (max, sum) and its output O; then Delta = dO . O (which is
//     sum_j P dP, derivation page section 1), and a second pass forms
//     dS = P (dP - Delta) (times 1 - tanh^2 of the pre-softcap score with a
//     softcap) and dQ = scale sum_j dS K_j.  It stores (LSE, Delta) per row.
//   bwd_valu_keys_kernel: per key row of a KV head, the walk over its group's
//     query heads and rows: P from the stored LSE, dP = dO . V_j, dS as above,
//     dV_j += P dO_i and dK_j += scale dS Q_i.
// LPR lanes share one row and each owns D / LPR of the head dim, as in the
// vector-ALU forward; K/V (rows kernel) and Q/dO (keys kernel) tiles are
// staged in LDS.
#include <limits.h>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThreads = 256;

template <typename T> struct BMath;
template <> struct BMath<float> {
  static __device__ float fma(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
  static __device__ float exp(float x) { return expf(x); }
  static __device__ float log(float x) { return logf(x); }
  static __device__ float tanh(float x) { return tanhf(x); }
  static __device__ float max(float a, float b) { return __builtin_fmaxf(a, b); }
};
template <> struct BMath<double> {
  static __device__ double fma(double a, double b, double c) { return __builtin_fma(a, b, c); }
  static __device__ double exp(double x) { return ::exp(x); }
  static __device__ double log(double x) { return ::log(x); }
  static __device__ double tanh(double x) { return ::tanh(x); }
  static __device__ double max(double a, double b) { return __builtin_fmax(a, b); }
};

struct BVArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* alibi;
  void* stats;  // [B, Hq, Sq] pairs of T: (natural-log LSE, -inf without keys; Delta)
  void* dq;
  void* dk;
  void* dv;
  int Sq, Sk, Hq, Hkv, group, nbh, nbkv, nqb, nkb;
  int wl, has_hi, dmax;
  float scale, softcap;
};

// Lanes per row and rows per LDS tile, as in the vector-ALU forward.
template <typename T, int D> struct BGeom {
  static constexpr int LPR = D / 32 > 4 ? D / 32 : 4;
  static constexpr int ROWS = kThreads / LPR;
  static constexpr int TILE = (int)(32768 / (D * sizeof(T))) < 32 ? (int)(32768 / (D * sizeof(T))) : 32;
};

// Score of one (query, key) pair from its dot product: scaled, softcapped,
// ALiBi-biased; `pre` is the scaled score before the softcap.
template <typename T>
__device__ __forceinline__ T score(T dot, const BVArgs& a, T slope, int rel, T& pre) {
  using M = BMath<T>;
  const T cap = (T)a.softcap;
  T x = dot * (T)a.scale;
  pre = x;
  if (a.softcap > 0.f) x = cap * M::tanh(x / cap);
  if (a.alibi) x = M::fma(slope, (T)rel, x);
  return x;
}

// Sum over the LPR lanes of one row.
template <typename T, int LPR>
__device__ __forceinline__ T row_sum(T x) {
#pragma unroll
  for (int w = 1; w < LPR; w <<= 1) x += __shfl_xor(x, w);
  return x;
}

// Copies rows [r0, r0 + TILE) of a [rows, D] matrix into an LDS tile (rows
// at or past `rows` read as zero).
template <typename T, int D, int TILE>
__device__ __forceinline__ void load_tile(T (*dst)[D], const T* src, int r0, int rows, int tid) {
  constexpr int EPC = 16 / (int)sizeof(T);
  for (int c = tid; c < TILE * D / EPC; c += kThreads) {
    const int r = c / (D / EPC), cc = c % (D / EPC);
    u32x4 x = zero_u32x4();
    if (r0 + r < rows) x = *reinterpret_cast<const u32x4*>(src + (size_t)(r0 + r) * D + EPC * cc);
    *reinterpret_cast<u32x4*>(&dst[r][EPC * cc]) = x;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_valu_rows_kernel(BVArgs a) {
  using M = BMath<T>;
  using G = BGeom<T, D>;
  constexpr int LPR = G::LPR, ROWS = G::ROWS, TILE = G::TILE;
  constexpr int SL = D / LPR;
  constexpr T kNInf = -__builtin_huge_val();
  __shared__ T ks[TILE][D];
  __shared__ T vs[TILE][D];

  const int tid = threadIdx.x;
  const int row = tid / LPR, qd = tid % LPR;
  const int bh = blockIdx.x % a.nbh, qb = blockIdx.x / a.nbh;
  const int b = bh / a.Hq, h = bh - b * a.Hq, kvh = h / a.group;
  const int Sq = a.Sq, Sk = a.Sk, off = Sk - Sq;
  const int qi = qb * ROWS + row, ip = qi + off;
  const T* Q = static_cast<const T*>(a.q) + (size_t)bh * Sq * D;
  const T* dO = static_cast<const T*>(a.dout) + (size_t)bh * Sq * D;
  const T* K = static_cast<const T*>(a.k) + (size_t)(b * a.Hkv + kvh) * Sk * D;
  const T* V = static_cast<const T*>(a.v) + (size_t)(b * a.Hkv + kvh) * Sk * D;

  T qv[SL], dov[SL], o[SL], dq[SL];
#pragma unroll
  for (int e = 0; e < SL; ++e) {
    qv[e] = qi < Sq ? Q[(size_t)qi * D + qd * SL + e] : T(0);
    dov[e] = qi < Sq ? dO[(size_t)qi * D + qd * SL + e] : T(0);
    o[e] = dq[e] = T(0);
  }
  const T slope = a.alibi ? (T)a.alibi[h] : T(0);
  int lo = -ip, hi = Sk - 1 - ip;  // admissible: lo <= j - i' <= hi
  if (a.wl >= 0) lo = max(lo, -a.wl);
  if (a.has_hi) hi = min(hi, a.dmax);

  // pass 1: the row's softmax and output
  T m = kNInf, l = T(0);
  for (int n0 = 0; n0 < Sk; n0 += TILE) {
    __syncthreads();
    load_tile<T, D, TILE>(ks, K, n0, Sk, tid);
    load_tile<T, D, TILE>(vs, V, n0, Sk, tid);
    __syncthreads();
    // one key at a time: the running max is raised when a key exceeds it
#pragma unroll 2
    for (int j = 0; j < TILE; ++j) {
      T part = T(0);
#pragma unroll
      for (int e = 0; e < SL; ++e) part = M::fma(qv[e], ks[j][qd * SL + e], part);
      const int rel = n0 + j - ip;
      T pre;
      T x = score(row_sum<T, LPR>(part), a, slope, rel, pre);
      if (rel < lo || rel > hi) continue;
      const T m_new = M::max(m, x);
      const T alpha = M::exp(m - m_new);  // 0 when m is -inf
      const T pj = M::exp(x - m_new);
      l = M::fma(l, alpha, pj);
#pragma unroll
      for (int e = 0; e < SL; ++e) o[e] = M::fma(pj, vs[j][qd * SL + e], o[e] * alpha);
      m = m_new;
    }
  }
  const T lse = l > T(0) ? m + M::log(l) : kNInf;
  T dpart = T(0);
#pragma unroll
  for (int e = 0; e < SL; ++e) dpart = M::fma(dov[e], l > T(0) ? o[e] / l : T(0), dpart);
  const T delta = row_sum<T, LPR>(dpart);

  // pass 2: dS and dQ
  for (int n0 = 0; n0 < Sk; n0 += TILE) {
    __syncthreads();
    load_tile<T, D, TILE>(ks, K, n0, Sk, tid);
    load_tile<T, D, TILE>(vs, V, n0, Sk, tid);
    __syncthreads();
    if (lse == kNInf) continue;
#pragma unroll 2
    for (int j = 0; j < TILE; ++j) {
      T part = T(0), dpp = T(0);
#pragma unroll
      for (int e = 0; e < SL; ++e) {
        part = M::fma(qv[e], ks[j][qd * SL + e], part);
        dpp = M::fma(dov[e], vs[j][qd * SL + e], dpp);
      }
      const int rel = n0 + j - ip;
      T pre;
      const T x = score(row_sum<T, LPR>(part), a, slope, rel, pre);
      const T dp = row_sum<T, LPR>(dpp);
      const bool adm = rel >= lo && rel <= hi;
      const T p = adm ? M::exp(x - lse) : T(0);
      T ds = p * (dp - delta);
      if (a.softcap > 0.f) {
        const T t = M::tanh(pre / (T)a.softcap);
        ds *= T(1) - t * t;
      }
#pragma unroll
      for (int e = 0; e < SL; ++e) dq[e] = M::fma(ds, ks[j][qd * SL + e], dq[e]);
    }
  }
  if (qi < Sq) {
    T* dqrow = static_cast<T*>(a.dq) + ((size_t)bh * Sq + qi) * D + qd * SL;
#pragma unroll
    for (int e = 0; e < SL; ++e) dqrow[e] = dq[e] * (T)a.scale;
    if (qd == 0) {
      T* st = static_cast<T*>(a.stats) + ((size_t)bh * Sq + qi) * 2;
      st[0] = lse;
      st[1] = delta;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_valu_keys_kernel(BVArgs a) {
  using M = BMath<T>;
  using G = BGeom<T, D>;
  constexpr int LPR = G::LPR, ROWS = G::ROWS, TILE = G::TILE;
  constexpr int SL = D / LPR;
  constexpr T kNInf = -__builtin_huge_val();
  __shared__ T qs[TILE][D];
  __shared__ T os[TILE][D];
  __shared__ T ss[TILE][2];

  const int tid = threadIdx.x;
  const int row = tid / LPR, qd = tid % LPR;
  const int bkv = blockIdx.x % a.nbkv, kb = blockIdx.x / a.nbkv;
  const int b = bkv / a.Hkv, kvh = bkv - b * a.Hkv;
  const int Sq = a.Sq, Sk = a.Sk, off = Sk - Sq;
  const int j = kb * ROWS + row;
  const T* K = static_cast<const T*>(a.k) + (size_t)bkv * Sk * D;
  const T* V = static_cast<const T*>(a.v) + (size_t)bkv * Sk * D;

  T kv[SL], vv[SL], dk[SL], dv[SL];
#pragma unroll
  for (int e = 0; e < SL; ++e) {
    kv[e] = j < Sk ? K[(size_t)j * D + qd * SL + e] : T(0);
    vv[e] = j < Sk ? V[(size_t)j * D + qd * SL + e] : T(0);
    dk[e] = dv[e] = T(0);
  }
  for (int hh = 0; hh < a.group; ++hh) {
    const int h = kvh * a.group + hh;
    const size_t bh = (size_t)b * a.Hq + h;
    const T* Q = static_cast<const T*>(a.q) + bh * Sq * D;
    const T* dO = static_cast<const T*>(a.dout) + bh * Sq * D;
    const T* St = static_cast<const T*>(a.stats) + bh * Sq * 2;
    const T slope = a.alibi ? (T)a.alibi[h] : T(0);
    for (int i0 = 0; i0 < Sq; i0 += TILE) {
      __syncthreads();
      load_tile<T, D, TILE>(qs, Q, i0, Sq, tid);
      load_tile<T, D, TILE>(os, dO, i0, Sq, tid);
      for (int r = tid; r < TILE * 2; r += kThreads)
        ss[r / 2][r % 2] = i0 + r / 2 < Sq ? St[(size_t)(i0 + r / 2) * 2 + r % 2] : kNInf;
      __syncthreads();
#pragma unroll 4
      for (int r = 0; r < TILE; ++r) {
        const int i = i0 + r;
        T part = T(0), dpp = T(0);
#pragma unroll
        for (int e = 0; e < SL; ++e) {
          part = M::fma(qs[r][qd * SL + e], kv[e], part);
          dpp = M::fma(os[r][qd * SL + e], vv[e], dpp);
        }
        const int rel = j - (i + off);
        bool adm = i < Sq && j < Sk && (a.wl < 0 || rel >= -a.wl) && (!a.has_hi || rel <= a.dmax);
        const T lse = ss[r][0];
        adm = adm && lse != kNInf;
        T pre;
        const T x = score(row_sum<T, LPR>(part), a, slope, rel, pre);
        const T dp = row_sum<T, LPR>(dpp);
        const T p = adm ? M::exp(x - lse) : T(0);
        T ds = adm ? p * (dp - ss[r][1]) : T(0);
        if (a.softcap > 0.f) {
          const T t = M::tanh(pre / (T)a.softcap);
          ds *= T(1) - t * t;
        }
#pragma unroll
        for (int e = 0; e < SL; ++e) {
          dv[e] = M::fma(p, os[r][qd * SL + e], dv[e]);
          dk[e] = M::fma(ds, qs[r][qd * SL + e], dk[e]);
        }
      }
    }
  }
  if (j < Sk) {
    T* dkrow = static_cast<T*>(a.dk) + ((size_t)bkv * Sk + j) * D + qd * SL;
    T* dvrow = static_cast<T*>(a.dv) + ((size_t)bkv * Sk + j) * D + qd * SL;
#pragma unroll
    for (int e = 0; e < SL; ++e) {
      dkrow[e] = dk[e] * (T)a.scale;
      dvrow[e] = dv[e];
    }
  }
}

template <typename T, int D>
hipError_t launch_bv(BVArgs a, hipStream_t stream) {
  constexpr int ROWS = BGeom<T, D>::ROWS;
  a.nqb = (a.Sq + ROWS - 1) / ROWS;
  a.nkb = (a.Sk + ROWS - 1) / ROWS;
  if (a.nbh > 0 && a.nqb > 0) {
    hipLaunchKernelGGL((bwd_valu_rows_kernel<T, D>), dim3(a.nqb * a.nbh), dim3(kThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.nbkv > 0 && a.nkb > 0)
    hipLaunchKernelGGL((bwd_valu_keys_kernel<T, D>), dim3(a.nkb * a.nbkv), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bv_d(const BVArgs& a, int D, hipStream_t stream) {
  switch (D) {
    case 32: return launch_bv<T, 32>(a, stream);
    case 64: return launch_bv<T, 64>(a, stream);
    case 128: return launch_bv<T, 128>(a, stream);
    default: return launch_bv<T, 256>(a, stream);
  }
}

}  // namespace

hipError_t launch_bwd_valu(const BwdProblem& p, bool f64, void* stats, hipStream_t stream) {
  BVArgs a = {};
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.dout = p.dout;
  a.alibi = p.alibi;
  a.stats = stats;
  a.dq = p.dq;
  a.dk = p.dk;
  a.dv = p.dv;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.group = p.Hq / p.Hkv;
  a.nbh = p.B * p.Hq;
  a.nbkv = p.B * p.Hkv;
  a.wl = p.wl;
  a.has_hi = p.causal || p.wr >= 0;
  a.dmax = p.causal ? (p.wr >= 0 ? min(p.wr, 0) : 0) : p.wr;
  a.scale = p.scale;
  a.softcap = p.softcap;
  return f64 ? launch_bv_d<double>(a, p.D, stream) : launch_bv_d<float>(a, p.D, stream);
}

}  // namespace attn
