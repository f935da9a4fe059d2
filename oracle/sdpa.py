"""Plain CPU float64 reference for attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the package entry
file and the CPU-baseline leg of the benchmark use it.  It shares no code with
the HIP library (no helpers, no tables, no pre/post-processing) and it never
reads anything the HIP library produced.

Sources (cited by page title and section; no other authority is used):

* "fuel-reference-backend -- attention kernel contracts" (the kernel-contract
  page), sections ``attention_naive``, ``attention_flash``,
  ``attention_paged_naive`` and ``attention_flash_backward``: shapes
  ``[B, H, S, D]``, GQA broadcast, the order of the score transforms (scale,
  softcap, ALiBi), the mask rules, stable softmax, the zero output of a fully
  masked row, paged address translation with its implicit causal position,
  and the gradient closed form of the backward pass.
* "gfx942 unified attention, from the math up" (the derivation page): section 1
  (definition), section 2 (shift invariance of softmax), section 3 (the online
  recurrence), section 4 (bottom-right causal alignment when Sq != Sk),
  section 5 (paged pool layout and GQA as repeat-interleave) and section 8
  (split-KV decode combining partial results).

Readings taken where the pages are silent or disagree (each is repeated in the
design notes of the repository):

* Causal and window masks are bottom-right aligned: query row ``i`` sits at
  absolute position ``i' = i + Sk - Sq`` (derivation page section 4; the
  kernel-contract page's paged section uses the same shift).  For Sq == Sk this
  is exactly the kernel-contract page's literal rule.
* Window bounds are inclusive: key ``j`` is admissible iff
  ``i' - left <= j <= i' + right``; ``None`` means unbounded on that side.
* ALiBi adds ``slope[h] * (j - i')``; slopes are float32 ``[Hq]``.
* ``softcap=None`` (or 0) disables the softcap; a negative value is an error.
* KV head of query head ``h`` is ``h // (Hq // Hkv)`` (contiguous groups).
* ``k_len`` (the kernel-contract page's live-prefix parameter of
  ``attention_naive``; ``None`` = all ``Sk`` keys): the page says only that
  it selects a live prefix for decode.  Read here as: the first ``k_len``
  key/value rows are the whole key sequence and the rest of the ``Sk`` rows
  do not exist, so positions align to the live length,
  ``i' = i + k_len - Sq``, as the paged section aligns to the context length.

Every function computes in float64; inputs of any float dtype are upcast.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "kv_head_of",
    "query_positions",
    "admissible",
    "transform_scores",
    "sdpa_naive_f64",
    "sdpa_online_f64",
    "sdpa_lse_f64",
    "attention_partial_f64",
    "lse_merge_f64",
    "paged_gather",
    "paged_decode_f64",
    "paged_prefill_varlen_f64",
    "sdpa_backward_f64",
    "softmax_backward",
    "softcap_derivative",
    "score_input_grads",
    "admissible_pair_count",
]


def _check_common(q, k, v, alibi, softcap):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be rank 4 [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if v.shape != k.shape:
        raise ValueError("v must have the shape of k")
    if Bk != B or Dk != D:
        raise ValueError("batch and head dim of k must match q")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if alibi is not None and np.shape(alibi) != (Hq,):
        raise ValueError("ALiBi slopes must be [Hq]")
    if softcap is not None and softcap < 0:
        raise ValueError("softcap must be >= 0 (0 or None disables it)")
    return B, Hq, Hkv, Sq, Sk, D


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head serving query head ``h``: each KV head is shared by a contiguous
    group of ``Hq // Hkv`` query heads (kernel-contract page, intro; derivation
    page section 5, where K/V are repeat-interleaved to the query heads)."""
    return h // (Hq // Hkv)


def query_positions(Sq: int, Sk: int) -> np.ndarray:
    """Absolute position of each query row: ``i + Sk - Sq`` (bottom-right
    alignment, derivation page section 4)."""
    return np.arange(Sq, dtype=np.int64) + (Sk - Sq)


def admissible(Sq, Sk, causal, window_left=None, window_right=None, rows=None):
    """Boolean ``[rows, Sk]``: may query row i attend to key j?

    Kernel-contract page, ``attention_naive``: causal masks keys in the future
    of the query, a left window masks keys more than ``left`` before it, a
    right window masks keys more than ``right`` after it.  Positions are the
    bottom-right aligned ``i'`` of :func:`query_positions`.
    """
    ip = query_positions(Sq, Sk)
    if rows is not None:
        ip = ip[rows]
    ip = ip[:, None]
    j = np.arange(Sk, dtype=np.int64)[None, :]
    ok = np.ones((ip.shape[0], Sk), dtype=bool)
    if causal:
        ok &= j <= ip
    if window_left is not None:
        ok &= j >= ip - window_left
    if window_right is not None:
        ok &= j <= ip + window_right
    return ok


def live_keys(k, v, k_len):
    """The live key prefix of the kernel-contract page's ``k_len`` parameter
    of ``attention_naive`` (``None`` = all ``Sk`` keys): only the first
    ``k_len`` key/value rows of every head take part; the rows after them are
    not read.  Returns ``(k, v)`` cut to that prefix."""
    Sk = k.shape[2]
    if k_len is None:
        return k, v
    if not 0 <= k_len <= Sk:
        raise ValueError("k_len must lie in [0, Sk]")
    return k[:, :, :k_len], v[:, :, :k_len]


def transform_scores(s, softcap=None, slope=None, rel=None):
    """Score transforms in the order the kernel-contract page fixes for
    ``attention_naive``: the already scaled score first goes through the
    softcap ``c * tanh(s / c)``, then ALiBi adds ``slope * (j - i')``."""
    if softcap:
        s = softcap * np.tanh(s / softcap)
    if slope is not None:
        s = s + slope * rel
    return s


def _scores(qrows, kmat, scale, softcap, slope, rel, ok):
    s = (qrows @ kmat.T) * scale
    s = transform_scores(s, softcap, slope, rel)
    return np.where(ok, s, -np.inf)


def sdpa_naive_f64(q, k, v, *, scale, causal=False, window_left=None,
                   window_right=None, softcap=None, alibi=None, row_block=512, k_len=None):
    """Materialised-score attention, the definition itself.

    Derivation page section 1 (output row = softmax-weighted convex combination
    of V rows), section 2 (subtract the row max before exponentiating) and the
    kernel-contract page's ``attention_naive`` (mask, softcap, ALiBi, GQA, the
    ``k_len`` live key prefix, and a row with no admissible key gives an
    all-zero output row).  Score rows are computed ``row_block`` queries at a
    time only to bound memory.

    Returns float64 ``[B, Hq, Sq, D]``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Sq, Sk, D = _check_common(q, k, v, alibi, softcap)
    slopes = None if alibi is None else np.asarray(alibi, dtype=np.float64)
    out = np.zeros((B, Hq, Sq, D), dtype=np.float64)
    k, v = live_keys(k, v, k_len)
    Sk = k.shape[2]
    if Sq == 0 or Sk == 0:
        return out
    ip_all = query_positions(Sq, Sk)
    j = np.arange(Sk, dtype=np.int64)[None, :]
    ones = np.ones((Sk, 1), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            # V with a trailing column of ones: the same products give the
            # unnormalised output and its denominator, so the one division at
            # the end sees sums taken in the same order.
            v1 = np.concatenate([v[b, g], ones], axis=1)
            for r0 in range(0, Sq, row_block):
                rows = slice(r0, min(Sq, r0 + row_block))
                ok = admissible(Sq, Sk, causal, window_left, window_right, rows)
                rel = j - ip_all[rows][:, None]
                slope = None if slopes is None else slopes[h]
                s = _scores(q[b, h, rows], k[b, g], scale, softcap, slope, rel, ok)
                has_key = ok.any(axis=1)
                m = np.where(has_key, s.max(axis=1), 0.0)[:, None]
                p = np.exp(s - m)                      # exp(-inf) == 0
                acc = p @ v1
                den = acc[:, D:D + 1]
                o = np.divide(acc[:, :D], den, out=np.zeros_like(acc[:, :D]),
                              where=has_key[:, None])
                out[b, h, rows] = o
    return out


def sdpa_lse_f64(q, k, *, scale, causal=False, window_left=None, window_right=None,
                 softcap=None, alibi=None, row_block=512, k_len=None):
    """Natural-log log-sum-exp of each query row's transformed admissible
    scores, ``log(sum_j exp(s_j))``, with ``-inf`` for a row with no
    admissible key.

    This is the per-row state the derivation page's section 3 recurrence ends
    with (``m + log l``) and the quantity its section 8 combines across key
    splits; the kernel-contract page's ``attention_flash_backward`` consumes
    it from the forward pass.  Computed from the materialised scores exactly
    as ``sdpa_naive_f64`` forms them, stabilised by the row max (section 2).

    Returns float64 ``[B, Hq, Sq]``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, Hkv, Sq, Sk, D = _check_common(q, k, k, alibi, softcap)
    slopes = None if alibi is None else np.asarray(alibi, dtype=np.float64)
    lse = np.full((B, Hq, Sq), -np.inf)
    k, _ = live_keys(k, k, k_len)
    Sk = k.shape[2]
    if Sq == 0 or Sk == 0:
        return lse
    ip_all = query_positions(Sq, Sk)
    j = np.arange(Sk, dtype=np.int64)[None, :]
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            for r0 in range(0, Sq, row_block):
                rows = slice(r0, min(Sq, r0 + row_block))
                ok = admissible(Sq, Sk, causal, window_left, window_right, rows)
                rel = j - ip_all[rows][:, None]
                slope = None if slopes is None else slopes[h]
                s = _scores(q[b, h, rows], k[b, g], scale, softcap, slope, rel, ok)
                has_key = ok.any(axis=1)
                m = np.where(has_key, s.max(axis=1), 0.0)
                l = np.exp(s - m[:, None]).sum(axis=1)
                lse[b, h, rows] = np.where(has_key, m + np.log(np.where(has_key, l, 1.0)),
                                           -np.inf)
    return lse


def sdpa_online_f64(q, k, v, *, scale, tile=16, causal=False, window_left=None,
                    window_right=None, softcap=None, alibi=None, k_len=None):
    """Streaming (online) softmax over key tiles of width ``tile``.

    Derivation page section 3: running max ``m``, denominator ``l`` and
    unnormalised output ``o`` start at ``-inf, 0, 0``; each tile raises the max,
    rescales the old state by ``alpha = exp(m_old - m_new)`` and adds the tile's
    weights ``exp(s - m_new)``; the result is ``o / l``.  The kernel-contract
    page's ``attention_flash`` states the same recurrence and that a row whose
    ``l`` stays 0 outputs zero.  While no admissible key has been seen the max
    is still ``-inf``; then ``alpha`` is taken as 1 and the weights as 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Sq, Sk, D = _check_common(q, k, v, alibi, softcap)
    if tile < 1:
        raise ValueError("tile must be >= 1")
    slopes = None if alibi is None else np.asarray(alibi, dtype=np.float64)
    out = np.zeros((B, Hq, Sq, D), dtype=np.float64)
    k, v = live_keys(k, v, k_len)
    Sk = k.shape[2]
    if Sq == 0 or Sk == 0:
        return out
    ip = query_positions(Sq, Sk)[:, None]
    ok_all = admissible(Sq, Sk, causal, window_left, window_right)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            m = np.full((Sq,), -np.inf)
            l = np.zeros((Sq,))
            o = np.zeros((Sq, D))
            for t0 in range(0, Sk, tile):
                t1 = min(Sk, t0 + tile)
                jt = np.arange(t0, t1, dtype=np.int64)[None, :]
                slope = None if slopes is None else slopes[h]
                s = _scores(q[b, h], k[b, g, t0:t1], scale, softcap, slope,
                            jt - ip, ok_all[:, t0:t1])
                m_new = np.maximum(m, s.max(axis=1))
                live = np.isfinite(m_new)
                safe = np.where(live, m_new, 0.0)
                alpha = np.where(live, np.exp(m - safe), 1.0)
                p = np.where(live[:, None], np.exp(s - safe[:, None]), 0.0)
                l = alpha * l + p.sum(axis=1)
                o = alpha[:, None] * o + p @ v[b, g, t0:t1]
                m = m_new
            out[b, h] = np.divide(o, l[:, None], out=np.zeros_like(o),
                                  where=(l > 0)[:, None])
    return out


def attention_partial_f64(q_rows, k_rows, v_rows, *, scale, softcap=None,
                          slope=None, rel=None, ok=None):
    """One partial result over a subset of keys, for split-KV decode.

    Returns ``(o, lse)`` for a ``[R, D]`` block of queries against the given
    ``[N, D]`` keys: ``o`` is the softmax-normalised output over that subset
    and ``lse = m + log(l)`` its log-sum-exp (``-inf`` and a zero row when the
    subset holds no admissible key).  Together they carry exactly the state of
    the derivation page's section-3 recurrence, which is what section 8 needs
    to combine partial outputs of the split key dimension.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k_rows = np.asarray(k_rows, dtype=np.float64)
    v_rows = np.asarray(v_rows, dtype=np.float64)
    R, D = q_rows.shape
    N = k_rows.shape[0]
    if ok is None:
        ok = np.ones((R, N), dtype=bool)
    if rel is None:
        rel = np.zeros((R, N))
    if N == 0:
        return np.zeros((R, D)), np.full((R,), -np.inf)
    s = _scores(q_rows, k_rows, scale, softcap, slope, rel, ok)
    has_key = ok.any(axis=1)
    m = np.where(has_key, s.max(axis=1), 0.0)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = np.divide(p @ v_rows, l[:, None], out=np.zeros((R, D)),
                  where=has_key[:, None])
    lse = np.where(has_key, m + np.log(np.where(has_key, l, 1.0)), -np.inf)
    return o, lse


def lse_merge_f64(o_parts, lse_parts):
    """Combine partial results ``o_parts [P, R, D]`` / ``lse_parts [P, R]``.

    Re-basing each part to the common max ``M = max_s lse_s`` with weight
    ``exp(lse_s - M)`` is the section-3 rescale of the derivation page applied
    across parts instead of tiles; parts with ``lse = -inf`` weigh 0 and a row
    with no live part is zero.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    live = np.isfinite(M)
    w = np.where(live[None, :], np.exp(lse_parts - np.where(live, M, 0.0)[None, :]), 0.0)
    num = (w[:, :, None] * o_parts).sum(axis=0)
    den = w.sum(axis=0)
    return np.divide(num, den[:, None], out=np.zeros_like(num), where=live[:, None])


def paged_gather(pool, block_table, seq_len, b, block_size):
    """Dense ``[seq_len, Hkv, D]`` rows of sequence ``b`` from a paged pool.

    Kernel-contract page, ``attention_paged_naive``: logical key position ``t``
    lives in physical block ``block_table[b, t // block_size]`` at slot
    ``t % block_size`` of a ``[num_blocks, block_size, Hkv, D]`` pool.  Indices
    outside ``[0, num_blocks)`` are rejected (the page bounds-checks them).
    """
    pool = np.asarray(pool)
    t = np.arange(int(seq_len), dtype=np.int64)
    phys = np.asarray(block_table)[b, t // block_size].astype(np.int64)
    if phys.size and (phys.min() < 0 or phys.max() >= pool.shape[0]):
        raise IndexError("block_table entry outside the pool")
    return pool[phys, t % block_size]


def paged_decode_f64(q, k_pool, v_pool, block_table, seq_lens, *, scale,
                     softcap=None, alibi=None):
    """Paged-cache attention (kernel-contract page, ``attention_paged_naive``).

    For each sequence the live keys ``0 .. seq_lens[b]-1`` are gathered with
    :func:`paged_gather` and the dense definition is applied with the implicit
    causal mask: query slot ``i`` sits at ``seq_lens[b] - Sq + i``, which is the
    bottom-right alignment of :func:`query_positions` with ``Sk = seq_lens[b]``.
    At ``Sq = 1`` every live key is admissible (derivation page section 4:
    a single decode query sees all keys).  ``q`` is ``[B, Hq, Sq, D]``, pools are
    ``[num_blocks, block_size, Hkv, D]``; returns float64 ``[B, Hq, Sq, D]``.
    """
    q = np.asarray(q, dtype=np.float64)
    k_pool = np.asarray(k_pool)
    v_pool = np.asarray(v_pool)
    if k_pool.shape != v_pool.shape or k_pool.ndim != 4:
        raise ValueError("k_pool and v_pool must both be [num_blocks, block_size, Hkv, D]")
    B, Hq, Sq, D = q.shape
    block_size = k_pool.shape[1]
    out = np.zeros((B, Hq, Sq, D), dtype=np.float64)
    for b in range(B):
        ctx = int(seq_lens[b])
        kb = paged_gather(k_pool, block_table, ctx, b, block_size)
        vb = paged_gather(v_pool, block_table, ctx, b, block_size)
        kb = np.transpose(kb, (1, 0, 2))[None]          # [1, Hkv, ctx, D]
        vb = np.transpose(vb, (1, 0, 2))[None]
        out[b:b + 1] = sdpa_naive_f64(q[b:b + 1], kb, vb, scale=scale,
                                      causal=True, softcap=softcap, alibi=alibi)
    return out


def paged_prefill_varlen_f64(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, *, scale,
                             causal=True, window_left=None, window_right=None, softcap=None,
                             alibi=None):
    """Variable-length prefill over the paged pool (kernel-contract page,
    ``attention_paged_naive``, with the packed query layout of the derivation
    page's section 5: queries ``[total_q, Hq, D]`` with a ``cu_seqlens_q``
    prefix sum, and each sequence's key length in ``seq_lens``).

    Sequence ``b`` owns query rows ``cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1``;
    its live keys ``0 .. seq_lens[b]-1`` are gathered with :func:`paged_gather`
    and the dense definition is applied with query row ``i`` at position
    ``seq_lens[b] - Sq_b + i`` (the implicit bottom-right alignment) -- with
    the causal mask when ``causal``, windows as for the dense form.  Returns
    float64 ``[total_q, Hq, D]``; rows outside every sequence stay zero.
    """
    q = np.asarray(q, dtype=np.float64)
    k_pool = np.asarray(k_pool)
    v_pool = np.asarray(v_pool)
    if q.ndim != 3 or k_pool.shape != v_pool.shape or k_pool.ndim != 4:
        raise ValueError("q must be [total_q, Hq, D]; pools [num_blocks, block_size, Hkv, D]")
    cu = [int(c) for c in cu_seqlens_q]
    if any(b < a for a, b in zip(cu, cu[1:])) or (cu and (cu[0] < 0 or cu[-1] > q.shape[0])):
        raise ValueError("cu_seqlens_q must be a non-decreasing prefix sum within total_q")
    block_size = k_pool.shape[1]
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(len(cu) - 1):
        r0, r1 = cu[b], cu[b + 1]
        if r1 == r0:
            continue
        ctx = int(seq_lens[b])
        kb = np.transpose(paged_gather(k_pool, block_table, ctx, b, block_size), (1, 0, 2))[None]
        vb = np.transpose(paged_gather(v_pool, block_table, ctx, b, block_size), (1, 0, 2))[None]
        qb = np.transpose(q[r0:r1], (1, 0, 2))[None]            # [1, Hq, Sq_b, D]
        ob = sdpa_naive_f64(qb, kb, vb, scale=scale, causal=causal, window_left=window_left,
                            window_right=window_right, softcap=softcap, alibi=alibi)
        out[r0:r1] = np.transpose(ob[0], (1, 0, 2))
    return out


def softmax_backward(p, dp):
    """``dS = (dP - sum_j' P dP) P`` row by row (kernel-contract page,
    ``attention_flash_backward``: the softmax backward)."""
    return (dp - (p * dp).sum(axis=1, keepdims=True)) * p


def softcap_derivative(s_pre, softcap):
    """``d/ds_pre [c tanh(s_pre / c)] = 1 - tanh^2(s_pre / c)`` (kernel-contract
    page, ``attention_flash_backward``: the softcap-derivative factor)."""
    return 1.0 - np.tanh(s_pre / softcap) ** 2


def score_input_grads(ds, qrows, kmat, scale):
    """``(dQ rows, dK)`` of the scaled scores ``s_pre = scale Q K^T`` for the
    score gradient ``ds``: ``scale dS K`` and ``scale dS^T Q``."""
    return scale * (ds @ kmat), scale * (ds.T @ qrows)


def sdpa_backward_f64(q, k, v, do, *, scale, causal=False, window_left=None,
                      window_right=None, softcap=None, alibi=None, row_block=256):
    """Gradients ``(dq, dk, dv)`` of the attention forward with respect to
    ``q, k, v`` for the upstream gradient ``do`` of its output.

    Kernel-contract page, ``attention_flash_backward``: recompute each row's
    stable-softmax weights ``P`` (and its pre-softcap score), then

    * ``dV[j] += P[i, j] dO[i]``
    * ``dP[i, j] = dO[i] . V[j]``
    * ``dS[i, j] = (dP[i, j] - sum_j' P[i, j'] dP[i, j']) P[i, j]``, times
      ``1 - tanh^2(s_pre / c)`` when a softcap ``c`` is set (``s_pre`` = the
      scaled score before the softcap; ALiBi adds a constant, no factor)
    * ``dQ[i] += scale sum_j dS[i, j] K[j]`` and ``dK[j] += scale sum_i dS[i, j] Q[i]``.

    dK and dV are ``[B, Hkv, Sk, D]``, summed over the query heads of each KV
    head's group; dQ is ``[B, Hq, Sq, D]``.  A row with no admissible key
    contributes nothing (its weights are all zero).  Rows are processed
    ``row_block`` at a time only to bound memory.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Hkv, Sq, Sk, D = _check_common(q, k, v, alibi, softcap)
    if do.shape != q.shape:
        raise ValueError("do must have the shape of q")
    slopes = None if alibi is None else np.asarray(alibi, dtype=np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if Sq == 0 or Sk == 0:
        return dq, dk, dv
    ip_all = query_positions(Sq, Sk)
    j = np.arange(Sk, dtype=np.int64)[None, :]
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            for r0 in range(0, Sq, row_block):
                rows = slice(r0, min(Sq, r0 + row_block))
                ok = admissible(Sq, Sk, causal, window_left, window_right, rows)
                has_key = ok.any(axis=1)
                s_pre = (q[b, h, rows] @ k[b, g].T) * scale
                s = transform_scores(s_pre, softcap, None if slopes is None else slopes[h],
                                     j - ip_all[rows][:, None])
                s = np.where(ok, s, -np.inf)
                m = np.where(has_key, s.max(axis=1), 0.0)[:, None]
                e = np.exp(s - m)                                   # 0 where masked
                den = e.sum(axis=1, keepdims=True)
                p = np.divide(e, den, out=np.zeros_like(e), where=has_key[:, None])
                dov = do[b, h, rows]
                dv[b, g] += p.T @ dov
                dp = dov @ v[b, g].T
                ds = softmax_backward(p, dp)
                if softcap:
                    ds = ds * softcap_derivative(s_pre, softcap)
                dqr, dkr = score_input_grads(ds, q[b, h, rows], k[b, g], scale)
                dq[b, h, rows] += dqr
                dk[b, g] += dkr
    return dq, dk, dv


def admissible_pair_count(Sq, Sk, causal, window_left=None, window_right=None):
    """Number of admissible (query, key) pairs of one head, counted from the
    mask of :func:`admissible` row by row."""
    total = 0
    for r0 in range(0, Sq, 1024):
        rows = slice(r0, min(Sq, r0 + 1024))
        total += int(admissible(Sq, Sk, causal, window_left, window_right, rows).sum())
    return total
