// fwd_f32.hip -- attention forward in float32 or float64 throughout (vector
// ALU), dense or over the paged pool.
//
// Same definition as the matrix-core path (kernel-contract page,
// attention_naive and attention_paged_naive; derivation page sections 1-5),
// for F32 and F64 inputs:
// LPR lanes share one query row and each owns D / LPR of the head dim;
// key/value tiles are staged in LDS; the per-tile online update uses the exact
// tile max and the accurate exp of the element type.  Meant for correctness
// at the element type's tolerance, not for speed.  The paged form takes
// packed queries [total_q, Hq, D] (sequence b owning rows cu[b] .. cu[b+1]-1,
// or row b alone when there is no prefix sum: decode) and gathers each key
// row through the block table, with the same clamps and error flag as the
// matrix-core paged kernels.
#include <limits.h>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThreads = 256;

template <typename T> struct VMath;
template <> struct VMath<float> {
  static __device__ float fma(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
  static __device__ float exp(float x) { return expf(x); }
  static __device__ float log(float x) { return logf(x); }
  static __device__ float tanh(float x) { return tanhf(x); }
  static __device__ float max(float a, float b) { return __builtin_fmaxf(a, b); }
};
template <> struct VMath<double> {
  static __device__ double fma(double a, double b, double c) { return __builtin_fma(a, b, c); }
  static __device__ double exp(double x) { return ::exp(x); }
  static __device__ double log(double x) { return ::log(x); }
  static __device__ double tanh(double x) { return ::tanh(x); }
  static __device__ double max(double a, double b) { return __builtin_fmax(a, b); }
};

struct VArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alibi;
  void* out;
  float* lse;  // per-row log-sum-exp (natural log), or nullptr
  int Sq, Sk, Hq, Hkv, group, nbh, nqb;
  int kv_stride;  // dense: keys between consecutive (sequence, KV head) slices of k and v
  int wl, has_hi, dmax;
  float scale, softcap;
  // paged form
  const int32_t* table;  // [B, maxb]
  const int32_t* lens;   // [B] live keys
  const int32_t* cu;     // [B + 1] query row prefix sum, or nullptr: row b is sequence b's query
  int32_t* err;          // device error flag or nullptr
  int maxb, bs, num_blocks, total_q, max_sq;
};

// Lanes per query row and keys per LDS tile for element type T and head dim D:
// at most 32 elements of q and of o per lane, and K + V tiles within 64 KiB.
template <typename T, int D> struct VGeom {
  static constexpr int LPR = D / 32 > 4 ? D / 32 : 4;
  static constexpr int ROWS = kThreads / LPR;
  static constexpr int KEYS = (int)(32768 / (D * sizeof(T))) < 32 ? (int)(32768 / (D * sizeof(T))) : 32;
};

template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(kThreads) void fwd_valu_kernel(VArgs a) {
  using M = VMath<T>;
  using G = VGeom<T, D>;
  constexpr int LPR = G::LPR, ROWS = G::ROWS, KEYS = G::KEYS;
  constexpr int SL = D / LPR;              // head-dim slice per lane
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr T kNInf = -__builtin_huge_val();
  __shared__ T ks[KEYS][D];
  __shared__ T vs[KEYS][D];
  __shared__ int kvalid[KEYS];  // paged: the key's block lies in the pool

  const int tid = threadIdx.x;
  const int row = tid / LPR, qd = tid % LPR;
  const int bh = blockIdx.x % a.nbh;
  const int qb = blockIdx.x / a.nbh;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int kvh = h / a.group;
  int Sq = a.Sq, Sk = a.Sk;
  const int m0 = qb * ROWS;
  // query and output rows: Q + qi * q_row (dense [B, Hq, Sq, D]; packed
  // [total_q, Hq, D] when paged), keys through the block table when paged
  const T* Q = static_cast<const T*>(a.q) + (size_t)bh * Sq * D;
  T* O = static_cast<T*>(a.out) + (size_t)bh * Sq * D;
  size_t q_row = D;
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  if constexpr (PAGED) {
    const int c0 = a.cu ? a.cu[b] : b, c1 = a.cu ? a.cu[b + 1] : b + 1;
    const int q0 = min(max(c0, 0), a.total_q), q1 = min(max(c1, q0), a.total_q);
    const int kl = a.lens[b];
    Sq = min(q1 - q0, a.max_sq);
    Sk = min(max(kl, 0), a.maxb * a.bs);
    if ((q0 != c0 || q1 != c1 || Sq != q1 - q0 || Sk != kl) && a.err && tid == 0) *a.err = 1;
    if (m0 >= Sq) return;  // no rows of this sequence here (the whole workgroup)
    q_row = (size_t)a.Hq * D;
    Q = static_cast<const T*>(a.q) + ((size_t)q0 * a.Hq + h) * D;
    O = static_cast<T*>(a.out) + ((size_t)q0 * a.Hq + h) * D;
  } else {
    K += (size_t)(b * a.Hkv + kvh) * a.kv_stride * D;
    V += (size_t)(b * a.Hkv + kvh) * a.kv_stride * D;
  }
  const int off = Sk - Sq;
  const int qi = m0 + row;
  const int ip = qi + off;

  T qv[SL], o[SL];
#pragma unroll
  for (int e = 0; e < SL; ++e) {
    qv[e] = qi < Sq ? Q[(size_t)qi * q_row + qd * SL + e] : T(0);
    o[e] = T(0);
  }
  const T slope = a.alibi ? (T)a.alibi[h] : T(0);
  const T scale = (T)a.scale, cap = (T)a.softcap;

  const int last = min(m0 + ROWS, Sq) - 1;
  const int n_lo = a.wl >= 0 ? max(0, m0 + off - a.wl) : 0;
  const int n_hi = a.has_hi ? min(Sk, max(0, last + off + a.dmax + 1)) : Sk;
  int lo = -ip, hi = Sk - 1 - ip;  // admissible: lo <= j - i' <= hi
  if (a.wl >= 0) lo = max(lo, -a.wl);
  if (a.has_hi) hi = min(hi, a.dmax);

  T m = kNInf, l = T(0);
  for (int n0 = (n_lo / KEYS) * KEYS; n0 < n_hi; n0 += KEYS) {
    __syncthreads();
    for (int c = tid; c < KEYS * D / EPC; c += kThreads) {
      const int r = c / (D / EPC), cc = c % (D / EPC);
      u32x4 kk = zero_u32x4(), vv = zero_u32x4();
      if (n0 + r < Sk) {
        size_t krow = (size_t)(n0 + r);
        bool ok = true;
        if constexpr (PAGED) {
          const int key = n0 + r;
          const int phys = a.table[(size_t)b * a.maxb + key / a.bs];
          ok = (unsigned)phys < (unsigned)a.num_blocks;
          krow = ((size_t)phys * a.bs + key % a.bs) * a.Hkv + kvh;
        }
        if (ok) {
          kk = *reinterpret_cast<const u32x4*>(K + krow * D + EPC * cc);
          vv = *reinterpret_cast<const u32x4*>(V + krow * D + EPC * cc);
        }
      }
      *reinterpret_cast<u32x4*>(&ks[r][EPC * cc]) = kk;
      *reinterpret_cast<u32x4*>(&vs[r][EPC * cc]) = vv;
    }
    if constexpr (PAGED) {
      // a key whose table entry lies outside the pool is masked and flagged
      for (int r = tid; r < KEYS; r += kThreads) {
        const int key = n0 + r;
        int ok = 1;
        if (key < Sk) {
          const int phys = a.table[(size_t)b * a.maxb + key / a.bs];
          ok = (unsigned)phys < (unsigned)a.num_blocks;
          if (!ok && a.err) *a.err = 1;
        }
        kvalid[r] = ok;
      }
    }
    __syncthreads();

    T s[KEYS];
    T mt = kNInf;
#pragma unroll
    for (int j = 0; j < KEYS; ++j) {
      T part = T(0);
#pragma unroll
      for (int e = 0; e < SL; ++e) part = M::fma(qv[e], ks[j][qd * SL + e], part);
#pragma unroll
      for (int w = 1; w < LPR; w <<= 1) part += __shfl_xor(part, w);
      T x = part * scale;
      if (a.softcap > 0.f) x = cap * M::tanh(x / cap);
      const int rel = n0 + j - ip;
      if (a.alibi) x = M::fma(slope, (T)rel, x);
      if (rel < lo || rel > hi) x = kNInf;
      if (PAGED && !kvalid[j]) x = kNInf;
      s[j] = x;
      mt = M::max(mt, x);
    }
    const T m_new = M::max(m, mt);
    if (m_new == kNInf) continue;  // nothing admissible so far for this row
    const T alpha = M::exp(m - m_new);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < SL; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < KEYS; ++j) {
      const T pj = M::exp(s[j] - m_new);
      l += pj;
#pragma unroll
      for (int e = 0; e < SL; ++e) o[e] = M::fma(pj, vs[j][qd * SL + e], o[e]);
    }
    m = m_new;
  }

  if (qi < Sq) {
    T* orow = O + (size_t)qi * q_row + qd * SL;
#pragma unroll
    for (int e = 0; e < SL; ++e) orow[e] = l > T(0) ? o[e] / l : T(0);
    if (a.lse && qd == 0) a.lse[(size_t)bh * Sq + qi] = l > T(0) ? (float)(m + M::log(l)) : kNegInf;
  }
}

template <typename T, int D, bool PAGED>
hipError_t launch_valu(const VArgs& a0, int rows, hipStream_t stream) {
  VArgs a = a0;
  a.nqb = (rows + VGeom<T, D>::ROWS - 1) / VGeom<T, D>::ROWS;
  hipLaunchKernelGGL((fwd_valu_kernel<T, D, PAGED>), dim3(a.nqb * a.nbh), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, bool PAGED>
hipError_t launch_valu_d(const VArgs& a, int D, int rows, hipStream_t stream) {
  switch (D) {
    case 32: return launch_valu<T, 32, PAGED>(a, rows, stream);
    case 64: return launch_valu<T, 64, PAGED>(a, rows, stream);
    case 128: return launch_valu<T, 128, PAGED>(a, rows, stream);
    default: return launch_valu<T, 256, PAGED>(a, rows, stream);
  }
}

}  // namespace

hipError_t launch_fwd_valu(const FwdProblem& p, bool f64, hipStream_t stream) {
  VArgs a = {};
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.alibi = p.alibi;
  a.out = p.out;
  a.lse = p.lse;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.kv_stride = p.kv_stride > 0 ? p.kv_stride : p.Sk;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.group = p.Hq / p.Hkv;
  a.nbh = p.B * p.Hq;
  a.nqb = 0;
  a.wl = p.wl;
  a.has_hi = p.causal || p.wr >= 0;
  a.dmax = p.causal ? (p.wr >= 0 ? min(p.wr, 0) : 0) : p.wr;
  a.scale = p.scale;
  a.softcap = p.softcap;
  return f64 ? launch_valu_d<double, false>(a, p.D, p.Sq, stream)
             : launch_valu_d<float, false>(a, p.D, p.Sq, stream);
}

hipError_t launch_paged_valu(const PagedPrefillProblem& p, bool f64, hipStream_t stream) {
  VArgs a = {};
  a.q = p.q;
  a.k = p.k_pool;
  a.v = p.v_pool;
  a.alibi = p.alibi;
  a.out = p.out;
  a.lse = nullptr;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.group = p.Hq / p.Hkv;
  a.nbh = p.B * p.Hq;
  a.wl = p.wl;
  a.has_hi = p.causal || p.wr >= 0;
  a.dmax = p.causal ? (p.wr >= 0 ? min(p.wr, 0) : 0) : p.wr;
  a.scale = p.scale;
  a.softcap = p.softcap;
  a.table = p.block_table;
  a.lens = p.seq_lens;
  a.cu = p.cu_seqlens_q;
  a.err = p.error_flag;
  a.maxb = p.max_blocks;
  a.bs = p.block_size;
  a.num_blocks = p.num_blocks;
  a.total_q = p.total_q;
  a.max_sq = p.max_sq;
  return f64 ? launch_valu_d<double, true>(a, p.D, p.max_sq, stream)
             : launch_valu_d<float, true>(a, p.D, p.max_sq, stream);
}

}  // namespace attn
