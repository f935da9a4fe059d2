"""Brute-force attention in 50-digit decimal arithmetic, for tiny inputs.

TEST INFRASTRUCTURE ONLY (same rule as :mod:`oracle.sdpa`: only the tests,
the smoke check and the benchmark's CPU-baseline leg may use it).

This is a second, independent statement of the definition: pure Python loops
over ``(b, h, i, j)`` with :class:`decimal.Decimal`, no NumPy and no code
shared with :mod:`oracle.sdpa`.  It follows, term by term:

* the derivation page ("gfx942 unified attention, from the math up"),
  section 1: the output row is ``sum_j a_j V_j`` with
  ``a_j = exp(s_j) / sum_j' exp(s_j')`` over the admissible keys;
* the kernel-contract page ("fuel-reference-backend -- attention kernel
  contracts"), ``attention_naive``: ``s = scale * q.k``, then softcap
  ``c * tanh(s / c)``, then ALiBi ``+ slope * (j - i)``; inadmissible keys drop
  out; no admissible key gives a zero row.

Here no max is subtracted (the decimal exponent range makes it unnecessary),
so agreement with the NumPy oracle also checks that its max subtraction and
its online rescaling do not change the result (derivation page sections 2-3).
Positions use the bottom-right alignment ``i' = i + Sk - Sq``.
"""
from __future__ import annotations

from decimal import Decimal, getcontext, localcontext

PREC = 50


def _exp(x: Decimal) -> Decimal:
    return x.exp()


def _tanh(x: Decimal) -> Decimal:
    # tanh from its definition in terms of exp.
    e2 = (2 * x).exp()
    return (e2 - 1) / (e2 + 1)


def _admit(i_abs: int, j: int, causal: bool, left, right) -> bool:
    if causal and j > i_abs:
        return False
    if left is not None and j + left < i_abs:
        return False
    if right is not None and j > i_abs + right:
        return False
    return True


def sdpa_bruteforce(q, k, v, *, scale, causal=False, window_left=None,
                    window_right=None, softcap=None, alibi=None):
    """``q``: nested lists ``[B][Hq][Sq][D]`` of numbers (converted exactly to
    Decimal via their repr); ``k``, ``v``: ``[B][Hkv][Sk][D]``.  Returns nested
    lists of Decimal, ``[B][Hq][Sq][D]``."""
    with localcontext() as ctx:
        ctx.prec = PREC
        B = len(q)
        Hq = len(q[0]) if B else 0
        Hkv = len(k[0]) if B else 0
        out = []
        sc = Decimal(repr(float(scale)))
        cap = Decimal(repr(float(softcap))) if softcap else None
        for b in range(B):
            ob = []
            for h in range(Hq):
                g = h // (Hq // Hkv)
                Sq = len(q[b][h])
                Sk = len(k[b][g])
                oh = []
                for i in range(Sq):
                    i_abs = i + Sk - Sq
                    D = len(q[b][h][i])
                    weights = []
                    for j in range(Sk):
                        if not _admit(i_abs, j, causal, window_left, window_right):
                            continue
                        dot = sum((Decimal(repr(float(q[b][h][i][d])))
                                   * Decimal(repr(float(k[b][g][j][d]))) for d in range(D)),
                                  Decimal(0))
                        s = sc * dot
                        if cap is not None:
                            s = cap * _tanh(s / cap)
                        if alibi is not None:
                            s = s + Decimal(repr(float(alibi[h]))) * (j - i_abs)
                        weights.append((j, _exp(s)))
                    den = sum((w for _, w in weights), Decimal(0))
                    row = []
                    for d in range(D):
                        if not weights:
                            row.append(Decimal(0))
                            continue
                        num = sum((w * Decimal(repr(float(v[b][g][j][d]))) for j, w in weights),
                                  Decimal(0))
                        row.append(num / den)
                    oh.append(row)
                ob.append(oh)
            out.append(ob)
        return out


def lse_bruteforce(q, k, *, scale, causal=False, window_left=None, window_right=None,
                   softcap=None, alibi=None):
    """Log-sum-exp ``ln(sum_j exp(s_j))`` of each query row's admissible
    transformed scores, term by term in 50-digit decimal (no max subtracted);
    ``None`` for a row with no admissible key.  Same inputs as
    :func:`sdpa_bruteforce`; returns nested lists ``[B][Hq][Sq]``."""
    with localcontext() as ctx:
        ctx.prec = PREC
        sc = Decimal(repr(float(scale)))
        cap = Decimal(repr(float(softcap))) if softcap else None
        out = []
        for b in range(len(q)):
            Hq, Hkv = len(q[b]), len(k[b])
            ob = []
            for h in range(Hq):
                g = h // (Hq // Hkv)
                Sq, Sk = len(q[b][h]), len(k[b][g])
                oh = []
                for i in range(Sq):
                    i_abs = i + Sk - Sq
                    total = Decimal(0)
                    seen = False
                    for j in range(Sk):
                        if not _admit(i_abs, j, causal, window_left, window_right):
                            continue
                        dot = sum((Decimal(repr(float(q[b][h][i][d])))
                                   * Decimal(repr(float(k[b][g][j][d]))) for d in range(len(q[b][h][i]))),
                                  Decimal(0))
                        s_ = sc * dot
                        if cap is not None:
                            s_ = cap * _tanh(s_ / cap)
                        if alibi is not None:
                            s_ = s_ + Decimal(repr(float(alibi[h]))) * (j - i_abs)
                        total += _exp(s_)
                        seen = True
                    oh.append(total.ln() if seen else None)
                ob.append(oh)
            out.append(ob)
        return out


def paged_bruteforce(q, k_pool, v_pool, block_table, seq_lens, *, scale,
                     softcap=None, alibi=None):
    """Paged form of :func:`sdpa_bruteforce` (kernel-contract page,
    ``attention_paged_naive``): key ``t`` of sequence ``b`` is read from block
    ``block_table[b][t // bs]``, slot ``t % bs`` of ``[blocks][bs][Hkv][D]``
    nested lists, and the query sits at ``seq_lens[b] - Sq + i``."""
    bs = len(k_pool[0])
    Hkv = len(k_pool[0][0])
    out = []
    for b in range(len(q)):
        ctx = int(seq_lens[b])
        kb = [[k_pool[block_table[b][t // bs]][t % bs][g] for t in range(ctx)] for g in range(Hkv)]
        vb = [[v_pool[block_table[b][t // bs]][t % bs][g] for t in range(ctx)] for g in range(Hkv)]
        out.append(sdpa_bruteforce([q[b]], [kb], [vb], scale=scale, causal=True,
                                   softcap=softcap, alibi=alibi)[0])
    return out
