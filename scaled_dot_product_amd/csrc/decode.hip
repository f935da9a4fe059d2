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
// Partial kernel: one workgroup per (split, KV head [x 16-head chunk], sequence).
//   * The split's tokens are cut into 16-token blocks dealt round-robin to the
//     4 waves; every wave keeps its own online-softmax state, so there is no
//     barrier until the final 4-way merge through LDS.
//   * Scores for all query heads of the KV head at once on the 16x16x32
//     matrix instruction: Q (up to 16 heads, padded) is the A operand, 16
//     gathered key rows the B operand, loaded straight from the pool (each
//     token row is 16 B per lane, 64 contiguous bytes per 4 lanes).
//   * P V on the vector ALU: each lane owns one 16-byte d-chunk of a few
//     tokens (V rows loaded whole and coalesced), the weights reach it through
//     a small per-wave LDS slab.
//   * Output per (sequence, head, split): normalised partial o[D] and its
//     natural-log LSE, into the caller's workspace.
// Merge kernel: one workgroup per (sequence, head), splits combined in fixed
// order, result cast to the input type.
#include <limits.h>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTB = 16;  // tokens per block
constexpr float kRescaleGap = 8.0f;
constexpr float kLn2 = 0.69314718055994531f;

struct DecArgs {
  const void* q;
  const void* kp;
  const void* vp;
  const int32_t* table;
  const int32_t* lens;
  const float* alibi;
  float* ws_o;
  float* ws_lse;
  int32_t* err;
  int Hq, Hkv, group, hchunks, num_blocks, bs, maxb, splits;
  int softcap;
  float c_score;  // log2(e) * scale; with softcap 2 * log2(e) * scale / cap
  float c_cap;    // log2(e) * cap
};

// All-reduce over each row of 16 lanes (rotations by 8, 4, 2, 1).
template <int N>
__device__ __forceinline__ float ror16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x120 + N, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float x) {
  x = __builtin_fmaxf(x, ror16<8>(x));
  x = __builtin_fmaxf(x, ror16<4>(x));
  x = __builtin_fmaxf(x, ror16<2>(x));
  return __builtin_fmaxf(x, ror16<1>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += ror16<8>(x);
  x += ror16<4>(x);
  x += ror16<2>(x);
  return x + ror16<1>(x);
}
// x[l] + x[l ^ 16] in every lane.
__device__ __forceinline__ float xor16_sum(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
// Completes this wave's LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <typename T, int D, int HT>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(DecArgs a) {
  using E = Elem<T>;
  constexpr int NCH = D / 8;      // 16-byte chunks per token row
  constexpr int TG = 64 / NCH;    // token groups of the PV layout
  constexpr int TPL = kTB / TG;   // V tokens per lane per block
  constexpr int KS = D / 32;      // steps of the 16x16x32 score product
  __shared__ floatx4 p_lds[kWaves][kTB][4];   // weights [token][head/4]
  __shared__ float al_lds[kWaves][16];         // rescale factors per head
  __shared__ float o_lds[kWaves][HT][D];
  __shared__ float m_lds[kWaves][16];
  __shared__ float l_lds[kWaves][16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, b = blockIdx.z;
  const int kvh = blockIdx.y / a.hchunks, hc = blockIdx.y - kvh * a.hchunks;
  const int h0 = kvh * a.group + hc * 16;
  const int nh = min(16, a.group - hc * 16);

  // live length, clamped into the table's capacity (flagged when outside)
  const int cap = a.maxb * a.bs;
  int ctx = a.lens[b];
  if (ctx < 0 || ctx > cap) {
    if (a.err && tid == 0) *a.err = 1;
    ctx = ctx < 0 ? 0 : cap;
  }
  const int per = (ctx + a.splits - 1) / a.splits;
  const int chunk = (per + kTB - 1) / kTB * kTB;
  const int t0 = min(ctx, split * chunk);
  const int t1 = min(ctx, t0 + chunk);
  const int nblk = (t1 - t0 + kTB - 1) / kTB;

  // Q as the A operand: lane -> head row (lane & 15), d = 32 ks + 8 (lane >> 4) .. +7
  const int hgrp = lane >> 4;
  const int tl = lane & 15;
  const T* Qb = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.Hq + h0) * D;
  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = tl < nh ? load16(Qb + tl * D + 32 * ks + 8 * hgrp) : zero_u32x4();

  // score layout: lane holds token tl of the block for heads 4*hgrp + r
  float slope_l2[4], m_run[4], l_part[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hh = 4 * hgrp + r;
    slope_l2[r] = (a.alibi && hh < nh) ? a.alibi[h0 + hh] * kLog2e : 0.f;
    m_run[r] = kNegInf;
    l_part[r] = 0.f;
  }

  // PV layout: lane owns chunk c of tokens tg + TG * i of each block
  const int c = lane % NCH, tg = lane / NCH;
  float o[HT][8];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;

  const size_t tok_stride = (size_t)a.Hkv * D;
  const T* Kp = reinterpret_cast<const T*>(a.kp) + (size_t)kvh * D;
  const T* Vp = reinterpret_cast<const T*>(a.vp) + (size_t)kvh * D;
  const int32_t* trow = a.table + (size_t)b * a.maxb;
  const float qpos = (float)(ctx - 1);

  // Physical row offset of logical token t, or -1 if its block id is invalid.
  auto row_of = [&](int t) -> long long {
    const int page = t / a.bs;
    const int phys = trow[page];
    if ((unsigned)phys >= (unsigned)a.num_blocks) {
      if (a.err) *a.err = 1;
      return -1;
    }
    return ((long long)phys * a.bs + (t - page * a.bs)) * (long long)tok_stride;
  };

  for (int bi = wave; bi < nblk; bi += kWaves) {
    const int tb = t0 + bi * kTB;
    // gather: 16 key rows (score layout), TPL value rows per lane (PV layout)
    const int tk = tb + tl;
    u32x4 kf[KS];
    bool kok = false;
    if (tk < t1) {
      const long long row = row_of(tk);
      if (row >= 0) {
        kok = true;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = load16(Kp + row + 32 * ks + 8 * hgrp);
      }
    }
    if (!kok) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = zero_u32x4();
    }
    u32x4 vf[TPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const int tv = tb + tg + TG * i;
      vf[i] = zero_u32x4();
      if (tv < t1) {
        const long long row = row_of(tv);
        if (row >= 0) vf[i] = load16(Vp + row + 8 * c);
      }
    }

    // scores: 16 heads x 16 tokens
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = E::mma16(qf[ks], kf[ks], s);

    float mx[4];
    bool need = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = s[r];
      if (a.softcap) {
        const float ex = fast_exp2(x * a.c_score);
        x = a.c_cap - 2.f * a.c_cap * fast_rcp(1.f + ex);
      } else {
        x *= a.c_score;
      }
      x = __builtin_fmaf(slope_l2[r], (float)tk - qpos, x);
      s[r] = kok ? x : kNegInf;
      mx[r] = row16_max(s[r]);
      need |= mx[r] > m_run[r] + kRescaleGap;
    }
    const bool rescale = wave_any(need);
    float alpha[4];
    floatx4 pw;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      alpha[r] = 1.f;
      if (rescale && mx[r] > m_run[r] + kRescaleGap) {
        alpha[r] = fast_exp2(m_run[r] - mx[r]);
        m_run[r] = mx[r];
      }
      l_part[r] *= alpha[r];
      const float m_use = m_run[r] == kNegInf ? 0.f : m_run[r];
      pw[r] = fast_exp2(s[r] - m_use);
      l_part[r] += pw[r];
    }
    p_lds[wave][tl][hgrp] = pw;
    if (rescale && tl == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) al_lds[wave][4 * hgrp + r] = alpha[r];
    }
    wave_lds_sync();

    if (rescale) {
#pragma unroll
      for (int hh = 0; hh < HT; ++hh) {
        const float al = al_lds[wave][hh];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] *= al;
      }
    }
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const int tt = tg + TG * i;
      float pv[HT];
#pragma unroll
      for (int q4 = 0; q4 < (HT + 3) / 4; ++q4) {
        const floatx4 w4 = p_lds[wave][tt][q4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * q4 + r < HT) pv[4 * q4 + r] = w4[r];
      }
      float vv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vv[2 * e] = E::lo(vf[i][e]);
        vv[2 * e + 1] = E::hi(vf[i][e]);
      }
#pragma unroll
      for (int hh = 0; hh < HT; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = __builtin_fmaf(pv[hh], vv[e], o[hh][e]);
    }
  }

  // ---- wave totals: l over the 16 token lanes, o over the token groups
#pragma unroll
  for (int r = 0; r < 4; ++r) l_part[r] = row16_sum(l_part[r]);
#pragma unroll
  for (int hh = 0; hh < HT; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = o[hh][e];
      if constexpr (D == 64) x += ror16<8>(x);
      x = xor16_sum(x);
      x = halves_sum(x);
      o[hh][e] = x;
    }
  if (tg == 0) {
#pragma unroll
    for (int hh = 0; hh < HT; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) o_lds[wave][hh][c * 8 + e] = o[hh][e];
  }
  if (tl == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m_lds[wave][4 * hgrp + r] = m_run[r];
      l_lds[wave][4 * hgrp + r] = l_part[r];
    }
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
        num = __builtin_fmaf(wt, o_lds[w][hh][d], num);
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

struct MergeArgs {
  const float* ws_o;
  const float* ws_lse;
  void* out;
  int splits;
};

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(MergeArgs a) {
  const size_t bh = blockIdx.x;
  const int d = threadIdx.x;
  const float* lse = a.ws_lse + bh * a.splits;
  float M = kNegInf;
  for (int s = 0; s < a.splits; ++s) M = __builtin_fmaxf(M, lse[s]);
  float r = 0.f;
  if (M != kNegInf) {
    float num = 0.f, den = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float w = expf(lse[s] - M);
      num = __builtin_fmaf(w, a.ws_o[(bh * a.splits + s) * D + d], num);
      den += w;
    }
    r = num / den;
  }
  reinterpret_cast<T*>(a.out)[bh * D + d] = (T)r;
}

template <typename T, int D, int HT>
hipError_t launch_partial(const DecArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_partial_kernel<T, D, HT>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_typed(const DecodeProblem& p, const DecArgs& a, int ht, hipStream_t stream) {
  const dim3 grid(p.splits, p.Hkv * a.hchunks, p.B);
  hipError_t e;
  switch (ht) {
    case 1: e = launch_partial<T, D, 1>(a, grid, stream); break;
    case 2: e = launch_partial<T, D, 2>(a, grid, stream); break;
    case 4: e = launch_partial<T, D, 4>(a, grid, stream); break;
    case 8: e = launch_partial<T, D, 8>(a, grid, stream); break;
    default: e = launch_partial<T, D, 16>(a, grid, stream); break;
  }
  if (e != hipSuccess) return e;
  MergeArgs m{p.ws_o, p.ws_lse, p.out, p.splits};
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(p.B * p.Hq), dim3(D), 0, stream, m);
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
  a.err = p.error_flag;
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
  const int g = a.group < 16 ? a.group : 16;
  const int ht = g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : g <= 8 ? 8 : 16;
  if (dtype == 2) {
    return p.D == 128 ? launch_typed<__bf16, 128>(p, a, ht, stream)
                      : launch_typed<__bf16, 64>(p, a, ht, stream);
  }
  return p.D == 128 ? launch_typed<_Float16, 128>(p, a, ht, stream)
                    : launch_typed<_Float16, 64>(p, a, ht, stream);
}

}  // namespace attn
