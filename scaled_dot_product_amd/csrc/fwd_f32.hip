// fwd_f32.hip -- attention forward in float32 throughout (vector ALU).
//
// Same definition as the matrix-core path (kernel-contract page,
// attention_naive; derivation page sections 1-4), for F32 inputs: four lanes
// share one query row and each owns a quarter of the head dim; key/value
// tiles of 32 keys are staged in LDS; the per-tile online update uses the
// exact tile max and accurate expf.  Meant for correctness at f32 tolerance,
// not for speed.
#include <limits.h>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kRows = 64;     // query rows per workgroup (4 lanes each)
constexpr int kKeys = 32;     // keys per tile
constexpr int kThreads = 256;

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* alibi;
  float* out;
  float* lse;  // per-row log-sum-exp (natural log), or nullptr
  int Sq, Sk, Hq, Hkv, group, nbh, nqb;
  int wl, has_hi, dmax;
  float scale, softcap;
};

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(F32Args a) {
  constexpr int SL = D / 4;  // head-dim slice per lane
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];

  const int tid = threadIdx.x;
  const int quad = tid >> 2, qd = tid & 3;
  const int bh = blockIdx.x % a.nbh;
  const int qb = blockIdx.x / a.nbh;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int kvh = h / a.group;
  const int Sq = a.Sq, Sk = a.Sk, off = Sk - Sq;
  const int m0 = qb * kRows;
  const int qi = m0 + quad;
  const int ip = qi + off;

  const float* Q = a.q + (size_t)bh * Sq * D;
  const float* K = a.k + (size_t)(b * a.Hkv + kvh) * Sk * D;
  const float* V = a.v + (size_t)(b * a.Hkv + kvh) * Sk * D;

  float qv[SL], o[SL];
#pragma unroll
  for (int e = 0; e < SL; ++e) {
    qv[e] = qi < Sq ? Q[(size_t)qi * D + qd * SL + e] : 0.f;
    o[e] = 0.f;
  }
  const float slope = a.alibi ? a.alibi[h] : 0.f;

  const int last = min(m0 + kRows, Sq) - 1;
  const int n_lo = a.wl >= 0 ? max(0, m0 + off - a.wl) : 0;
  const int n_hi = a.has_hi ? min(Sk, max(0, last + off + a.dmax + 1)) : Sk;
  int lo = -ip, hi = Sk - 1 - ip;  // admissible: lo <= j - i' <= hi
  if (a.wl >= 0) lo = max(lo, -a.wl);
  if (a.has_hi) hi = min(hi, a.dmax);

  float m = kNegInf, l = 0.f;
  for (int n0 = (n_lo / kKeys) * kKeys; n0 < n_hi; n0 += kKeys) {
    __syncthreads();
    for (int c = tid; c < kKeys * D / 4; c += kThreads) {
      const int r = c / (D / 4), cc = c % (D / 4);
      floatx4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (n0 + r < Sk) {
        kk = *reinterpret_cast<const floatx4*>(K + (size_t)(n0 + r) * D + 4 * cc);
        vv = *reinterpret_cast<const floatx4*>(V + (size_t)(n0 + r) * D + 4 * cc);
      }
      *reinterpret_cast<floatx4*>(&ks[r][4 * cc]) = kk;
      *reinterpret_cast<floatx4*>(&vs[r][4 * cc]) = vv;
    }
    __syncthreads();

    float s[kKeys];
    float mt = kNegInf;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < SL; ++e) part = __builtin_fmaf(qv[e], ks[j][qd * SL + e], part);
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      float x = part * a.scale;
      if (a.softcap > 0.f) x = a.softcap * tanhf(x / a.softcap);
      const int rel = n0 + j - ip;
      if (a.alibi) x = __builtin_fmaf(slope, (float)rel, x);
      if (rel < lo || rel > hi) x = kNegInf;
      s[j] = x;
      mt = __builtin_fmaxf(mt, x);
    }
    const float m_new = __builtin_fmaxf(m, mt);
    if (m_new == kNegInf) continue;  // nothing admissible so far for this row
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < SL; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = expf(s[j] - m_new);
      l += p;
#pragma unroll
      for (int e = 0; e < SL; ++e) o[e] = __builtin_fmaf(p, vs[j][qd * SL + e], o[e]);
    }
    m = m_new;
  }

  if (qi < Sq) {
    float* orow = a.out + ((size_t)bh * Sq + qi) * D + qd * SL;
#pragma unroll
    for (int e = 0; e < SL; ++e) orow[e] = l > 0.f ? o[e] / l : 0.f;
    if (a.lse && qd == 0) a.lse[(size_t)bh * Sq + qi] = l > 0.f ? m + logf(l) : kNegInf;
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdProblem& p, hipStream_t stream) {
  F32Args a;
  a.q = static_cast<const float*>(p.q);
  a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v);
  a.alibi = p.alibi;
  a.out = static_cast<float*>(p.out);
  a.lse = p.lse;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.group = p.Hq / p.Hkv;
  a.nbh = p.B * p.Hq;
  a.nqb = (p.Sq + kRows - 1) / kRows;
  a.wl = p.wl;
  a.has_hi = p.causal || p.wr >= 0;
  a.dmax = p.causal ? (p.wr >= 0 ? min(p.wr, 0) : 0) : p.wr;
  a.scale = p.scale;
  a.softcap = p.softcap;
  const int grid = a.nqb * a.nbh;
  if (p.D == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
