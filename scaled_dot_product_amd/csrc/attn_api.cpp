// attn_api.cpp -- the C ABI declared in include/attn.h.
//
// Argument validation is pure host code (no HIP call), so the *_check entry
// points work on machines without a GPU.  The compute entry points validate,
// narrow the sizes, pick the kernel for (dtype, head dim) and enqueue it on the
// caller's stream.  Nothing is allocated and no state is kept.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "attn.h"
#include "launch.h"

namespace attn {
hipError_t launch_fwd_mfma_bf16_d128(const FwdProblem& p, hipStream_t stream);
hipError_t launch_fwd_mfma_bf16_d64(const FwdProblem& p, hipStream_t stream);
hipError_t launch_fwd_mfma_f16_d128(const FwdProblem& p, hipStream_t stream);
hipError_t launch_fwd_mfma_f16_d64(const FwdProblem& p, hipStream_t stream);
hipError_t launch_fwd_mfma_bf16_d256(const FwdProblem& p, hipStream_t stream);
hipError_t launch_fwd_mfma_f16_d256(const FwdProblem& p, hipStream_t stream);

hipError_t launch_fwd_mfma(const FwdProblem& p, int dtype, hipStream_t stream) {
  if (dtype == ATTN_BF16)
    return p.D == 256 ? launch_fwd_mfma_bf16_d256(p, stream)
         : p.D == 128 ? launch_fwd_mfma_bf16_d128(p, stream) : launch_fwd_mfma_bf16_d64(p, stream);
  return p.D == 256 ? launch_fwd_mfma_f16_d256(p, stream)
       : p.D == 128 ? launch_fwd_mfma_f16_d128(p, stream) : launch_fwd_mfma_f16_d64(p, stream);
}

hipError_t launch_bwd_mfma_bf16_d128(const BwdProblem& p, hipStream_t stream);
hipError_t launch_bwd_mfma_bf16_d64(const BwdProblem& p, hipStream_t stream);
hipError_t launch_bwd_mfma_f16_d128(const BwdProblem& p, hipStream_t stream);
hipError_t launch_bwd_mfma_f16_d64(const BwdProblem& p, hipStream_t stream);
hipError_t launch_bwd_mfma_bf16_d256(const BwdProblem& p, hipStream_t stream);
hipError_t launch_bwd_mfma_f16_d256(const BwdProblem& p, hipStream_t stream);

hipError_t launch_bwd_mfma(const BwdProblem& p, int dtype, hipStream_t stream) {
  if (dtype == ATTN_BF16)
    return p.D == 256 ? launch_bwd_mfma_bf16_d256(p, stream)
         : p.D == 128 ? launch_bwd_mfma_bf16_d128(p, stream) : launch_bwd_mfma_bf16_d64(p, stream);
  return p.D == 256 ? launch_bwd_mfma_f16_d256(p, stream)
       : p.D == 128 ? launch_bwd_mfma_f16_d128(p, stream) : launch_bwd_mfma_f16_d64(p, stream);
}

hipError_t launch_bwd_rowstats_bf16_d128(const void*, const void*, const float*, float*, long long, hipStream_t);
hipError_t launch_bwd_rowstats_bf16_d64(const void*, const void*, const float*, float*, long long, hipStream_t);
hipError_t launch_bwd_rowstats_f16_d128(const void*, const void*, const float*, float*, long long, hipStream_t);
hipError_t launch_bwd_rowstats_f16_d64(const void*, const void*, const float*, float*, long long, hipStream_t);
hipError_t launch_bwd_rowstats_bf16_d256(const void*, const void*, const float*, float*, long long, hipStream_t);
hipError_t launch_bwd_rowstats_f16_d256(const void*, const void*, const float*, float*, long long, hipStream_t);

hipError_t launch_bwd_rowstats(const void* out, const void* dout, const float* lse, float* stats,
                               long long rows, int D, int dtype, hipStream_t stream) {
  if (dtype == ATTN_BF16)
    return D == 256 ? launch_bwd_rowstats_bf16_d256(out, dout, lse, stats, rows, stream)
         : D == 128 ? launch_bwd_rowstats_bf16_d128(out, dout, lse, stats, rows, stream)
                    : launch_bwd_rowstats_bf16_d64(out, dout, lse, stats, rows, stream);
  return D == 256 ? launch_bwd_rowstats_f16_d256(out, dout, lse, stats, rows, stream)
       : D == 128 ? launch_bwd_rowstats_f16_d128(out, dout, lse, stats, rows, stream)
                  : launch_bwd_rowstats_f16_d64(out, dout, lse, stats, rows, stream);
}

hipError_t launch_paged_prefill_bf16_d128(const PagedPrefillProblem& p, hipStream_t stream);
hipError_t launch_paged_prefill_bf16_d64(const PagedPrefillProblem& p, hipStream_t stream);
hipError_t launch_paged_prefill_f16_d128(const PagedPrefillProblem& p, hipStream_t stream);
hipError_t launch_paged_prefill_f16_d64(const PagedPrefillProblem& p, hipStream_t stream);
hipError_t launch_paged_prefill_bf16_d256(const PagedPrefillProblem& p, hipStream_t stream);
hipError_t launch_paged_prefill_f16_d256(const PagedPrefillProblem& p, hipStream_t stream);

hipError_t launch_paged_prefill(const PagedPrefillProblem& p, int dtype, hipStream_t stream) {
  if (dtype == ATTN_BF16)
    return p.D == 256 ? launch_paged_prefill_bf16_d256(p, stream)
         : p.D == 128 ? launch_paged_prefill_bf16_d128(p, stream) : launch_paged_prefill_bf16_d64(p, stream);
  return p.D == 256 ? launch_paged_prefill_f16_d256(p, stream)
       : p.D == 128 ? launch_paged_prefill_f16_d128(p, stream) : launch_paged_prefill_f16_d64(p, stream);
}
}  // namespace attn

namespace {

constexpr int64_t kMaxLen = int64_t(1) << 30;   // positions stay far inside int32
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

bool valid_dtype(int32_t d) { return d == ATTN_F32 || d == ATTN_F16 || d == ATTN_BF16 || d == ATTN_F64; }
int64_t elem_bytes(int32_t d) { return d == ATTN_F64 ? 8 : (d == ATTN_F32 ? 4 : 2); }
// Dense forward head dims: the matrix-core path (F16, BF16) takes 64, 128 and
// 256, the vector-ALU path (F32, F64) 32, 64, 128 and 256.
bool fwd_head_dim_ok(int32_t dtype, int64_t D) {
  if (dtype == ATTN_F32 || dtype == ATTN_F64) return D == 32 || D == 64 || D == 128 || D == 256;
  return D == 64 || D == 128 || D == 256;
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b * ... without overflow (all factors >= 0); false on overflow.
bool mul(int64_t a, int64_t b, int64_t* r) {
  if (a != 0 && b > std::numeric_limits<int64_t>::max() / a) return false;
  *r = a * b;
  return true;
}
bool mul4(int64_t a, int64_t b, int64_t c, int64_t d, int64_t* r) {
  int64_t x, y;
  return mul(a, b, &x) && mul(x, c, &y) && mul(y, d, r);
}

struct Span {
  const void* p;
  int64_t bytes;
};
bool overlaps(Span a, Span b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

bool bad_scale(float s) { return !std::isfinite(s) || s < 0.f; }
bool bad_softcap(float c) { return !std::isfinite(c) || c < 0.f; }

// Byte sizes of the dense operands; fills q/kv/out byte counts.
attn_status_t fwd_shape(const attn_fwd_params_t* p, int64_t* q_bytes, int64_t* kv_bytes) {
  if (p->B < 0 || p->Hq < 0 || p->Hkv < 0 || p->Sq < 0 || p->Sk < 0 || p->D < 0)
    return ATTN_ERR_SHAPE;
  if (p->Hkv == 0 || p->Hq % p->Hkv != 0) return ATTN_ERR_GQA;
  if (!fwd_head_dim_ok(p->dtype, p->D)) return ATTN_ERR_HEAD_DIM;
  if (p->Sq > kMaxLen || p->Sk > kMaxLen) return ATTN_ERR_SHAPE;
  int64_t bh;
  if (!mul(p->B, p->Hq, &bh) || bh > kMaxLen) return ATTN_ERR_SHAPE;
  const int64_t qblocks = (p->Sq + 31) / 32;  // the smallest row block of any forward kernel
  int64_t grid;
  if (!mul(bh, qblocks, &grid) || grid > kMaxGrid) return ATTN_ERR_SHAPE;
  const int64_t es = elem_bytes(p->dtype);
  if (!mul4(p->B, p->Hq, p->Sq, p->D * es, q_bytes)) return ATTN_ERR_SHAPE;
  if (!mul4(p->B, p->Hkv, p->Sk, p->D * es, kv_bytes)) return ATTN_ERR_SHAPE;
  if (p->Sk * p->D * es > INT32_MAX) return ATTN_ERR_SHAPE;  // one head's K (or V) < 2 GiB
  return ATTN_OK;
}

attn_status_t check_fwd(const void* q, const void* k, const void* v, const float* alibi,
                        const void* out, const attn_fwd_params_t* p) {
  if (!p) return ATTN_ERR_NULL;
  if (!valid_dtype(p->dtype)) return ATTN_ERR_DTYPE;
  int64_t qb, kvb;
  const attn_status_t st = fwd_shape(p, &qb, &kvb);
  if (st != ATTN_OK) return st;
  if (bad_scale(p->softmax_scale) || bad_softcap(p->softcap)) return ATTN_ERR_PARAM;
  if (p->window_left < -1 || p->window_right < -1) return ATTN_ERR_PARAM;
  if (p->has_k_len && (p->k_len < 0 || p->k_len > p->Sk)) return ATTN_ERR_PARAM;
  if (qb > 0 && (!q || !out)) return ATTN_ERR_NULL;
  if (qb > 0 && kvb > 0 && (!k || !v)) return ATTN_ERR_NULL;
  const void* ptrs[] = {q, k, v, alibi, out};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return ATTN_ERR_ALIGN;
  const Span o{out, qb};
  if (overlaps(o, Span{q, qb}) || overlaps(o, Span{k, kvb}) || overlaps(o, Span{v, kvb}) ||
      overlaps(o, Span{alibi, p->Hq * 4}))
    return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

// The split count of a paged decode: the caller's, or with num_splits = 0
// one chosen from the shape.  The split form runs persistent workers over
// (sequence, KV head, head chunk, split) items, two 4-wave workgroups per
// compute unit.  With fewer (sequence, KV head, head chunk) groups than
// compute units it streams at close to the HBM ceiling from about 1024 items
// (measured at B = 4 x 32768 tokens: 2.2 TB/s with 8 splits, 5.4 with 32, 5.2
// with 64; B = 16 x 8192: 8 splits best); with more groups, about 4096 items
// balance the workers better (B = 32 x 512..8192 tokens: 5.5 TB/s with 16
// splits; B = 256 x 512..4096: 6.4 TB/s with 2).  The automatic count asks
// for that many, keeps each split of the longest sequence the block table
// can hold at 256 tokens or more, and stays within 1..256.
constexpr int64_t kAutoSplitItems = 1024;
constexpr int64_t kAutoSplitItemsWide = 4096;
constexpr int64_t kAutoSplitWideGroups = 256;
constexpr int64_t kAutoSplitMinTokens = 256;
int64_t paged_splits(const attn_paged_params_t* p) {
  if (p->num_splits != 0) return p->num_splits;
  const int64_t hchunks = (p->Hq / p->Hkv + 15) / 16;
  const int64_t groups = p->B * p->Hkv * hchunks;
  const int64_t target = groups >= kAutoSplitWideGroups ? kAutoSplitItemsWide : kAutoSplitItems;
  int64_t s = groups > 0 ? (target + groups - 1) / groups : 1;
  const int64_t by_len = p->max_blocks_per_seq * p->block_size / kAutoSplitMinTokens;
  if (s > by_len) s = by_len;
  return s < 1 ? 1 : (s > 256 ? 256 : s);
}

int64_t paged_ws_lse_offset(const attn_paged_params_t* p) {
  const int64_t o_bytes = p->B * p->Hq * paged_splits(p) * p->D * 4;
  return (o_bytes + 255) / 256 * 256;
}

attn_status_t paged_shape(const attn_paged_params_t* p) {
  if (p->B < 0 || p->Hq < 0 || p->Hkv < 0 || p->D < 0 || p->num_blocks < 0 ||
      p->max_blocks_per_seq < 0)
    return ATTN_ERR_SHAPE;
  if (p->block_size < 1) return ATTN_ERR_SHAPE;
  if (p->Hkv == 0 || p->Hq % p->Hkv != 0) return ATTN_ERR_GQA;
  if (!fwd_head_dim_ok(p->dtype, p->D)) return ATTN_ERR_HEAD_DIM;
  if (p->num_splits < 0 || p->num_splits > 256) return ATTN_ERR_PARAM;
  if (p->B > 65535 || p->Hq > 65535) return ATTN_ERR_SHAPE;
  const int64_t hchunks = (p->Hq / p->Hkv + 15) / 16;
  if (p->Hkv * hchunks > 65535) return ATTN_ERR_SHAPE;
  int64_t cap, pool_tokens;
  if (!mul(p->max_blocks_per_seq, p->block_size, &cap) || cap > kMaxLen) return ATTN_ERR_SHAPE;
  if (!mul(p->num_blocks, p->block_size, &pool_tokens) || pool_tokens > (int64_t(1) << 40))
    return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

}  // namespace

// The LSE output of attn_fwd_lse: float32 [B, Hq, Sq], 4-byte aligned, and
// disjoint from every input and from out.
static attn_status_t check_lse(const void* q, const void* k, const void* v, const float* alibi,
                               const void* out, const float* lse, const attn_fwd_params_t* p) {
  const int64_t es = elem_bytes(p->dtype);
  const int64_t rows = p->B * p->Hq * p->Sq;
  if (rows > 0 && !lse) return ATTN_ERR_NULL;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3) != 0) return ATTN_ERR_ALIGN;
  const Span l{lse, rows * 4};
  const int64_t qb = rows * p->D * es, kvb = p->B * p->Hkv * p->Sk * p->D * es;
  if (overlaps(l, Span{q, qb}) || overlaps(l, Span{k, kvb}) || overlaps(l, Span{v, kvb}) ||
      overlaps(l, Span{alibi, p->Hq * 4}) || overlaps(l, Span{out, qb}))
    return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

static attn_status_t launch_fwd(const void* q, const void* k, const void* v, const float* alibi, void* out,
                         float* lse, const attn_fwd_params_t* p, void* stream) {
  if (p->B == 0 || p->Hq == 0 || p->Sq == 0) return ATTN_OK;
  attn::FwdProblem fp;
  fp.q = q;
  fp.k = k;
  fp.v = v;
  fp.alibi = alibi;
  fp.out = out;
  fp.lse = lse;
  fp.B = (int)p->B;
  fp.Hq = (int)p->Hq;
  fp.Hkv = (int)p->Hkv;
  fp.Sq = (int)p->Sq;
  // the live key prefix: masks, alignment and tile counts use its length,
  // the addressing of k and v their capacity Sk
  const int64_t live = p->has_k_len ? p->k_len : p->Sk;
  fp.Sk = (int)live;
  fp.kv_stride = (int)p->Sk;
  fp.D = (int)p->D;
  fp.causal = p->causal != 0;
  // Windows wider than every possible distance are the same as no window.
  fp.wl = (p->window_left < 0 || p->window_left >= live) ? -1 : (int)p->window_left;
  fp.wr = (p->window_right < 0 || p->window_right >= p->Sq) ? -1 : (int)p->window_right;
  fp.scale = p->softmax_scale;
  fp.softcap = p->softcap;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = (p->dtype == ATTN_F32 || p->dtype == ATTN_F64)
                            ? attn::launch_fwd_valu(fp, p->dtype == ATTN_F64, s)
                            : attn::launch_fwd_mfma(fp, p->dtype, s);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" {

attn_status_t attn_fwd_check(const void* q, const void* k, const void* v, const float* alibi,
                             const void* out, const attn_fwd_params_t* p) {
  return check_fwd(q, k, v, alibi, out, p);
}

attn_status_t attn_fwd(const void* q, const void* k, const void* v, const float* alibi, void* out,
                       const attn_fwd_params_t* p, void* stream) {
  const attn_status_t st = check_fwd(q, k, v, alibi, out, p);
  if (st != ATTN_OK) return st;
  return launch_fwd(q, k, v, alibi, out, nullptr, p, stream);
}

attn_status_t attn_fwd_lse_check(const void* q, const void* k, const void* v, const float* alibi,
                                 const void* out, const float* lse, const attn_fwd_params_t* p) {
  const attn_status_t st = check_fwd(q, k, v, alibi, out, p);
  return st != ATTN_OK ? st : check_lse(q, k, v, alibi, out, lse, p);
}

attn_status_t attn_fwd_lse(const void* q, const void* k, const void* v, const float* alibi,
                           void* out, float* lse, const attn_fwd_params_t* p, void* stream) {
  const attn_status_t st = attn_fwd_lse_check(q, k, v, alibi, out, lse, p);
  if (st != ATTN_OK) return st;
  return launch_fwd(q, k, v, alibi, out, lse, p, stream);
}

// Backward workspace: the forward's row statistics (8 bytes a row), then, at
// a 256-byte boundary, the float32 dK/dV partials of the key blocks split
// into several chunks.
struct BwdLayout {
  int wl, wr;               // windows clamped to the useful range
  int chunk_items, max_chunks;
  int64_t stats_bytes, part_offset, part_bytes, total;
};
static BwdLayout bwd_layout(const attn_fwd_params_t* p) {
  BwdLayout L;
  L.wl = (p->window_left < 0 || p->window_left >= p->Sk) ? -1 : (int)p->window_left;
  L.wr = (p->window_right < 0 || p->window_right >= p->Sq) ? -1 : (int)p->window_right;
  const bool valu = p->dtype == ATTN_F32 || p->dtype == ATTN_F64;
  if (valu) {
    L.chunk_items = 1;
    L.max_chunks = 1;
  } else {
    attn::bwd_chunking((int)p->B, (int)p->Hkv, (int)p->Hq, (int)p->Sq, (int)p->Sk, (int)p->D, p->causal != 0,
                       L.wl, L.wr, &L.chunk_items, &L.max_chunks);
  }
  // per query row: two floats (matrix cores) or two values of the element type
  L.stats_bytes = p->B * p->Hq * p->Sq * (valu ? 2 * elem_bytes(p->dtype) : 8);
  L.part_offset = (L.stats_bytes + 255) / 256 * 256;
  const int64_t nkb = (p->Sk + 127) / 128;
  L.part_bytes = L.max_chunks > 1 ? p->B * p->Hkv * nkb * L.max_chunks * 2 * 128 * p->D * 4 : 0;
  L.total = L.part_bytes > 0 ? L.part_offset + L.part_bytes : L.stats_bytes;
  return L;
}

size_t attn_bwd_workspace_size(const attn_fwd_params_t* p) {
  if (!p || !valid_dtype(p->dtype)) return 0;
  int64_t qb, kvb;
  if (fwd_shape(p, &qb, &kvb) != ATTN_OK) return 0;
  return (size_t)bwd_layout(p).total;
}

attn_status_t attn_bwd_check(const void* q, const void* k, const void* v, const void* dout,
                             const float* alibi, const void* dq, const void* dk, const void* dv,
                             const void* workspace, size_t workspace_bytes,
                             const attn_fwd_params_t* p) {
  if (!p) return ATTN_ERR_NULL;
  if (!valid_dtype(p->dtype)) return ATTN_ERR_DTYPE;
  // q, k, v, alibi and the parameters as for the forward, with dq in out's place
  attn_status_t st = check_fwd(q, k, v, alibi, dq, p);
  if (st != ATTN_OK) return st;
  if (p->has_k_len) return ATTN_ERR_PARAM;  // the backward takes every key live
  int64_t qb, kvb;
  fwd_shape(p, &qb, &kvb);
  if (qb > 0 && !dout) return ATTN_ERR_NULL;
  if (kvb > 0 && (!dk || !dv)) return ATTN_ERR_NULL;
  const int64_t ws_need = bwd_layout(p).total;
  if (ws_need > 0 && (!workspace || workspace_bytes < (size_t)ws_need)) return ATTN_ERR_WORKSPACE;
  const void* ptrs[] = {dout, dk, dv, workspace};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return ATTN_ERR_ALIGN;
  const Span in[] = {{q, qb}, {k, kvb}, {v, kvb}, {dout, qb}, {alibi, p->Hq * 4}};
  const Span outs[] = {{dq, qb}, {dk, kvb}, {dv, kvb}, {workspace, ws_need}};
  for (int i = 0; i < 4; ++i) {
    for (const Span& x : in)
      if (overlaps(outs[i], x)) return ATTN_ERR_ALIAS;
    for (int j2 = i + 1; j2 < 4; ++j2)
      if (overlaps(outs[i], outs[j2])) return ATTN_ERR_ALIAS;
  }
  return ATTN_OK;
}

// The backward after validation: the row statistics into the workspace
// (recomputed by the forward kernel, or from a saved forward's out and lse
// when those are given), then dK/dV and dQ.
static attn_status_t run_bwd(const void* q, const void* k, const void* v, const void* out,
                             const float* lse, const void* dout, const float* alibi, void* dq,
                             void* dk, void* dv, void* workspace, const attn_fwd_params_t* p,
                             void* stream) {
  if (p->B == 0 || p->Hkv == 0) return ATTN_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const BwdLayout lay = bwd_layout(p);
  const int wl = lay.wl, wr = lay.wr;
  if (p->dtype == ATTN_F32 || p->dtype == ATTN_F64) {
    // vector-ALU path: recomputes the row statistics itself (a saved out and
    // lse are not read)
    attn::BwdProblem bp = {};
    bp.q = q;
    bp.k = k;
    bp.v = v;
    bp.dout = dout;
    bp.alibi = alibi;
    bp.dq = dq;
    bp.dk = dk;
    bp.dv = dv;
    bp.B = (int)p->B;
    bp.Hq = (int)p->Hq;
    bp.Hkv = (int)p->Hkv;
    bp.Sq = (int)p->Sq;
    bp.Sk = (int)p->Sk;
    bp.D = (int)p->D;
    bp.causal = p->causal != 0;
    bp.wl = wl;
    bp.wr = wr;
    bp.scale = p->softmax_scale;
    bp.softcap = p->softcap;
    return attn::launch_bwd_valu(bp, p->dtype == ATTN_F64, workspace, s) == hipSuccess ? ATTN_OK
                                                                                     : ATTN_ERR_HIP;
  }
  // 1. the row statistics (LSE, dO . O) into the workspace
  if (p->Hq > 0 && p->Sq > 0 && out) {
    if (attn::launch_bwd_rowstats(out, dout, lse, static_cast<float*>(workspace), p->B * p->Hq * p->Sq,
                                  (int)p->D, p->dtype, s) != hipSuccess)
      return ATTN_ERR_HIP;
  } else if (p->Hq > 0 && p->Sq > 0) {
    attn::FwdProblem fp;
    fp.q = q;
    fp.k = k;
    fp.v = v;
    fp.alibi = alibi;
    fp.out = nullptr;
    fp.lse = nullptr;
    fp.dout = dout;
    fp.stats = static_cast<float*>(workspace);
    fp.B = (int)p->B;
    fp.Hq = (int)p->Hq;
    fp.Hkv = (int)p->Hkv;
    fp.Sq = (int)p->Sq;
    fp.Sk = (int)p->Sk;
    fp.D = (int)p->D;
    fp.causal = p->causal != 0;
    fp.wl = wl;
    fp.wr = wr;
    fp.scale = p->softmax_scale;
    fp.softcap = p->softcap;
    if (attn::launch_fwd_mfma(fp, p->dtype, s) != hipSuccess) return ATTN_ERR_HIP;
  }
  // 2. dK, dV (every key row, zero where no query sees it) and dQ
  attn::BwdProblem bp;
  bp.q = q;
  bp.k = k;
  bp.v = v;
  bp.dout = dout;
  bp.alibi = alibi;
  bp.stats = static_cast<const float*>(workspace);
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.B = (int)p->B;
  bp.Hq = (int)p->Hq;
  bp.Hkv = (int)p->Hkv;
  bp.Sq = (int)p->Sq;
  bp.Sk = (int)p->Sk;
  bp.D = (int)p->D;
  bp.causal = p->causal != 0;
  bp.wl = wl;
  bp.wr = wr;
  bp.scale = p->softmax_scale;
  bp.softcap = p->softcap;
  bp.chunk_items = lay.chunk_items;
  bp.max_chunks = lay.max_chunks;
  bp.partials = lay.part_bytes > 0
                    ? reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.part_offset)
                    : nullptr;
  return attn::launch_bwd_mfma(bp, p->dtype, s) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* dout,
                       const float* alibi, void* dq, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, const attn_fwd_params_t* p, void* stream) {
  const attn_status_t st =
      attn_bwd_check(q, k, v, dout, alibi, dq, dk, dv, workspace, workspace_bytes, p);
  if (st != ATTN_OK) return st;
  return run_bwd(q, k, v, nullptr, nullptr, dout, alibi, dq, dk, dv, workspace, p, stream);
}

attn_status_t attn_bwd_lse_check(const void* q, const void* k, const void* v, const void* out,
                                 const float* lse, const void* dout, const float* alibi,
                                 const void* dq, const void* dk, const void* dv,
                                 const void* workspace, size_t workspace_bytes,
                                 const attn_fwd_params_t* p) {
  attn_status_t st = attn_bwd_check(q, k, v, dout, alibi, dq, dk, dv, workspace, workspace_bytes, p);
  if (st != ATTN_OK) return st;
  const int64_t rows = p->B * p->Hq * p->Sq;
  const int64_t qb = rows * p->D * elem_bytes(p->dtype);
  if (rows > 0 && (!out || !lse)) return ATTN_ERR_NULL;
  if ((out && !aligned16(out)) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3) != 0)) return ATTN_ERR_ALIGN;
  // out and lse are read only: they may alias each other's inputs, never what is written
  const Span ins[] = {{out, qb}, {lse, rows * 4}};
  const int64_t kvb = p->B * p->Hkv * p->Sk * p->D * elem_bytes(p->dtype);
  const Span outs[] = {{dq, qb}, {dk, kvb}, {dv, kvb}, {workspace, bwd_layout(p).total}};
  for (const Span& x : ins)
    for (const Span& o : outs)
      if (overlaps(x, o)) return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

attn_status_t attn_bwd_lse(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, const void* dout, const float* alibi, void* dq,
                           void* dk, void* dv, void* workspace, size_t workspace_bytes,
                           const attn_fwd_params_t* p, void* stream) {
  const attn_status_t st = attn_bwd_lse_check(q, k, v, out, lse, dout, alibi, dq, dk, dv, workspace,
                                              workspace_bytes, p);
  if (st != ATTN_OK) return st;
  return run_bwd(q, k, v, p->B * p->Hq * p->Sq > 0 ? out : nullptr, lse, dout, alibi, dq, dk, dv,
                 workspace, p, stream);
}

size_t attn_paged_decode_workspace_size(const attn_paged_params_t* p) {
  if (!p || paged_shape(p) != ATTN_OK) return 0;
  const int64_t lse_bytes = p->B * p->Hq * paged_splits(p) * 4;
  return (size_t)(paged_ws_lse_offset(p) + lse_bytes);
}

attn_status_t attn_paged_decode_check(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      const float* alibi, const void* out, const void* workspace,
                                      size_t workspace_bytes, const int32_t* error_flag,
                                      const attn_paged_params_t* p) {
  if (!p) return ATTN_ERR_NULL;
  if (!valid_dtype(p->dtype)) return ATTN_ERR_DTYPE;
  const attn_status_t st = paged_shape(p);
  if (st != ATTN_OK) return st;
  if (bad_scale(p->softmax_scale) || bad_softcap(p->softcap)) return ATTN_ERR_PARAM;
  const int64_t es = elem_bytes(p->dtype);
  const int64_t q_bytes = p->B * p->Hq * p->D * es;
  int64_t pool_bytes;
  if (!mul4(p->num_blocks, p->block_size, p->Hkv, p->D * es, &pool_bytes)) return ATTN_ERR_SHAPE;
  const int64_t table_bytes = p->B * p->max_blocks_per_seq * 4;
  const int64_t lens_bytes = p->B * 4;
  if (q_bytes > 0) {
    if (!q || !out || !seq_lens) return ATTN_ERR_NULL;
    if (table_bytes > 0 && !block_table) return ATTN_ERR_NULL;
    if (pool_bytes > 0 && (!k_pool || !v_pool)) return ATTN_ERR_NULL;
  }
  const size_t need = attn_paged_decode_workspace_size(p);
  if (q_bytes > 0 && (!workspace || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  const void* ptrs[] = {q, k_pool, v_pool, block_table, seq_lens, alibi, out, workspace};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return ATTN_ERR_ALIGN;
  if (error_flag && (reinterpret_cast<uintptr_t>(error_flag) & 3u)) return ATTN_ERR_ALIGN;
  const Span o{out, q_bytes}, ws{workspace, (int64_t)need};
  const Span inputs[] = {{q, q_bytes},          {k_pool, pool_bytes},    {v_pool, pool_bytes},
                         {block_table, table_bytes}, {seq_lens, lens_bytes}, {alibi, p->Hq * 4},
                         {error_flag, 4}};
  for (const Span& in : inputs)
    if (overlaps(o, in) || overlaps(ws, in)) return ATTN_ERR_ALIAS;
  if (overlaps(o, ws)) return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

attn_status_t attn_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const float* alibi, void* out, void* workspace,
                                size_t workspace_bytes, int32_t* error_flag,
                                const attn_paged_params_t* p, void* stream) {
  const attn_status_t st = attn_paged_decode_check(q, k_pool, v_pool, block_table, seq_lens, alibi,
                                                   out, workspace, workspace_bytes, error_flag, p);
  if (st != ATTN_OK) return st;
  if (p->B == 0 || p->Hq == 0) return ATTN_OK;
  if (p->dtype == ATTN_F32 || p->dtype == ATTN_F64) {
    // vector-ALU path: the paged forward with one query per sequence at the
    // sequence's last position (bottom-right causal admits every live key)
    attn::PagedPrefillProblem pp;
    pp.q = q;
    pp.k_pool = k_pool;
    pp.v_pool = v_pool;
    pp.block_table = block_table;
    pp.seq_lens = seq_lens;
    pp.cu_seqlens_q = nullptr;
    pp.alibi = alibi;
    pp.out = out;
    pp.error_flag = error_flag;
    pp.B = (int)p->B;
    pp.Hq = (int)p->Hq;
    pp.Hkv = (int)p->Hkv;
    pp.D = (int)p->D;
    pp.total_q = (int)p->B;
    pp.max_sq = 1;
    pp.num_blocks = p->num_blocks > INT32_MAX ? INT32_MAX : (int)p->num_blocks;
    pp.block_size = (int)p->block_size;
    pp.max_blocks = (int)p->max_blocks_per_seq;
    pp.causal = 1;
    pp.wl = pp.wr = -1;
    pp.scale = p->softmax_scale;
    pp.softcap = p->softcap;
    const hipError_t e = attn::launch_paged_valu(pp, p->dtype == ATTN_F64, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
  }
  attn::DecodeProblem dp;
  dp.q = q;
  dp.k_pool = k_pool;
  dp.v_pool = v_pool;
  dp.block_table = block_table;
  dp.seq_lens = seq_lens;
  dp.alibi = alibi;
  dp.out = out;
  dp.ws_o = static_cast<float*>(workspace);
  dp.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + paged_ws_lse_offset(p));
  dp.error_flag = error_flag;
  dp.B = (int)p->B;
  dp.Hq = (int)p->Hq;
  dp.Hkv = (int)p->Hkv;
  dp.D = (int)p->D;
  dp.num_blocks = p->num_blocks > INT32_MAX ? INT32_MAX : (int)p->num_blocks;
  dp.block_size = (int)p->block_size;
  dp.max_blocks = (int)p->max_blocks_per_seq;
  dp.splits = (int)paged_splits(p);
  dp.scale = p->softmax_scale;
  dp.softcap = p->softcap;
  const hipError_t e = attn::launch_paged_decode(dp, p->dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status_t attn_paged_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        const float* alibi, void* out, int32_t* error_flag,
                                        const attn_paged_params_t* p, void* stream) {
  if (!p) return ATTN_ERR_NULL;
  // the size check comes first and makes no HIP call (sizes beyond the array
  // are rejected before the device is touched); invalid parameters are
  // reported by attn_paged_decode_check below
  if (attn_paged_decode_workspace_size(p) > (size_t)ATTN_DECODE_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
  const attn_status_t st = attn_paged_decode_check(q, k_pool, v_pool, block_table, seq_lens, alibi,
                                                   out, nullptr, 0, error_flag, p);
  // (the check reports a missing workspace when one is needed; here it is the scratch array)
  if (st != ATTN_OK && st != ATTN_ERR_WORKSPACE) return st;
  void* ws = attn::decode_scratch();
  if (!ws) return ATTN_ERR_HIP;
  return attn_paged_decode(q, k_pool, v_pool, block_table, seq_lens, alibi, out, ws,
                           (size_t)ATTN_DECODE_SCRATCH_BYTES, error_flag, p, stream);
}

attn_status_t attn_paged_prefill_check(const void* q, const void* k_pool, const void* v_pool,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       const int32_t* cu_seqlens_q, const float* alibi,
                                       const void* out, const int32_t* error_flag,
                                       const attn_varlen_params_t* p) {
  if (!p) return ATTN_ERR_NULL;
  if (!valid_dtype(p->dtype)) return ATTN_ERR_DTYPE;
  const bool valu = p->dtype == ATTN_F32 || p->dtype == ATTN_F64;
  if (p->B < 0 || p->Hq < 0 || p->Hkv < 0 || p->D < 0 || p->total_q < 0 || p->max_seqlen_q < 0 ||
      p->num_blocks < 0 || p->max_blocks_per_seq < 0 || p->block_size < 1)
    return ATTN_ERR_SHAPE;
  if (p->Hkv == 0 || p->Hq % p->Hkv != 0) return ATTN_ERR_GQA;
  if (!fwd_head_dim_ok(p->dtype, p->D)) return ATTN_ERR_HEAD_DIM;
  if (!valu && p->block_size % 64 != 0) return ATTN_ERR_UNSUPPORTED;  // matrix-core path
  if (bad_scale(p->softmax_scale) || bad_softcap(p->softcap)) return ATTN_ERR_PARAM;
  if (p->window_left < -1 || p->window_right < -1) return ATTN_ERR_PARAM;
  if (p->total_q > kMaxLen || p->max_seqlen_q > kMaxLen) return ATTN_ERR_SHAPE;
  const int64_t es = elem_bytes(p->dtype);
  int64_t cap, bh, grid, q_bytes, pool_bytes;
  if (!mul(p->max_blocks_per_seq, p->block_size, &cap) || cap > kMaxLen) return ATTN_ERR_SHAPE;
  if (!mul(p->B, p->Hq, &bh) || bh > kMaxLen) return ATTN_ERR_SHAPE;
  // query blocks of 128 rows (matrix cores) or at least 32 (vector ALU)
  if (!mul(bh, (p->max_seqlen_q + 31) / 32, &grid) || grid > kMaxGrid) return ATTN_ERR_SHAPE;
  if (!mul4(p->total_q, p->Hq, p->D, es, &q_bytes)) return ATTN_ERR_SHAPE;
  if (!mul4(p->num_blocks, p->block_size, p->Hkv, p->D * es, &pool_bytes)) return ATTN_ERR_SHAPE;
  // one 64-key tile spans 64 token rows of the pool: its offsets must fit int32
  if (64 * p->Hkv * p->D * es > INT32_MAX) return ATTN_ERR_SHAPE;
  const int64_t table_bytes = p->B * p->max_blocks_per_seq * 4;
  const int64_t lens_bytes = p->B * 4, cu_bytes = (p->B + 1) * 4;
  const bool work = q_bytes > 0 && p->B > 0;
  if (work) {
    if (!q || !out || !seq_lens || !cu_seqlens_q) return ATTN_ERR_NULL;
    if (table_bytes > 0 && !block_table) return ATTN_ERR_NULL;
    if (pool_bytes > 0 && (!k_pool || !v_pool)) return ATTN_ERR_NULL;
  }
  const void* ptrs16[] = {q, k_pool, v_pool, alibi, out};
  for (const void* ptr : ptrs16)
    if (ptr && !aligned16(ptr)) return ATTN_ERR_ALIGN;
  const void* ptrs4[] = {block_table, seq_lens, cu_seqlens_q, error_flag};
  for (const void* ptr : ptrs4)
    if (ptr && (reinterpret_cast<uintptr_t>(ptr) & 3u)) return ATTN_ERR_ALIGN;
  const Span o{out, q_bytes};
  const Span inputs[] = {{q, q_bytes},          {k_pool, pool_bytes},    {v_pool, pool_bytes},
                         {block_table, table_bytes}, {seq_lens, lens_bytes}, {cu_seqlens_q, cu_bytes},
                         {alibi, p->Hq * 4},    {error_flag, 4}};
  for (const Span& in : inputs)
    if (overlaps(o, in)) return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

attn_status_t attn_paged_prefill(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* cu_seqlens_q, const float* alibi, void* out,
                                 int32_t* error_flag, const attn_varlen_params_t* p,
                                 void* stream) {
  const attn_status_t st = attn_paged_prefill_check(q, k_pool, v_pool, block_table, seq_lens,
                                                    cu_seqlens_q, alibi, out, error_flag, p);
  if (st != ATTN_OK) return st;
  if (p->B == 0 || p->Hq == 0 || p->total_q == 0 || p->max_seqlen_q == 0) return ATTN_OK;
  attn::PagedPrefillProblem pp;
  pp.q = q;
  pp.k_pool = k_pool;
  pp.v_pool = v_pool;
  pp.block_table = block_table;
  pp.seq_lens = seq_lens;
  pp.cu_seqlens_q = cu_seqlens_q;
  pp.alibi = alibi;
  pp.out = out;
  pp.error_flag = error_flag;
  pp.B = (int)p->B;
  pp.Hq = (int)p->Hq;
  pp.Hkv = (int)p->Hkv;
  pp.D = (int)p->D;
  pp.total_q = (int)p->total_q;
  pp.max_sq = (int)p->max_seqlen_q;
  pp.num_blocks = p->num_blocks > INT32_MAX ? INT32_MAX : (int)p->num_blocks;
  pp.block_size = (int)p->block_size;
  pp.max_blocks = (int)p->max_blocks_per_seq;
  pp.causal = p->causal != 0;
  const int64_t cap = p->max_blocks_per_seq * p->block_size;
  // windows wider than every possible distance are the same as no window
  pp.wl = (p->window_left < 0 || p->window_left >= cap) ? -1 : (int)p->window_left;
  pp.wr = (p->window_right < 0 || p->window_right >= p->max_seqlen_q) ? -1 : (int)p->window_right;
  pp.scale = p->softmax_scale;
  pp.softcap = p->softcap;
  const hipError_t e =
      (p->dtype == ATTN_F32 || p->dtype == ATTN_F64)
          ? attn::launch_paged_valu(pp, p->dtype == ATTN_F64, static_cast<hipStream_t>(stream))
          : attn::launch_paged_prefill(pp, p->dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

const char* attn_status_str(attn_status_t status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "required pointer is NULL";
    case ATTN_ERR_DTYPE: return "invalid dtype";
    case ATTN_ERR_SHAPE: return "invalid or too large shape";
    case ATTN_ERR_GQA: return "Hq must be a positive multiple of Hkv";
    case ATTN_ERR_HEAD_DIM: return "head dim not built for this dtype";
    case ATTN_ERR_PARAM: return "parameter out of range";
    case ATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case ATTN_ERR_ALIAS: return "output overlaps an input";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_UNSUPPORTED: return "supported by the contract but not built";
    case ATTN_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

int32_t attn_version(void) { return 100; }

}  // extern "C"
