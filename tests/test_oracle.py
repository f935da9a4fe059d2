"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check uses a value from a
50-digit brute force of the definition (golden fixtures), a closed form, an
invariance the pages state, or a special case whose answer is known exactly.
``test_oracle_mutants.py`` plants plausible mistakes in the oracle and shows
that these checks catch each of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import sdpa as osd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_cases.json")


def _load_golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _rand(rng, *shape, amp=1.0):
    return rng.standard_normal(shape) * amp


# --------------------------------------------------------------------------
# Reusable checks (also driven by the mutant tests)
# --------------------------------------------------------------------------

def check_golden_dense(fn):
    """50-digit brute force of the definition (golden fixtures)."""
    for c in _load_golden():
        if c["kind"] != "dense":
            continue
        got = fn(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]), scale=c["scale"],
                 causal=c["causal"], window_left=c["window_left"],
                 window_right=c["window_right"], softcap=c["softcap"],
                 alibi=None if c["alibi"] is None else np.array(c["alibi"]))
        exp = np.array(c["expected"], dtype=np.float64)
        np.testing.assert_allclose(got, exp, rtol=0, atol=1e-13, err_msg=c["name"])


def check_golden_paged(fn):
    for c in _load_golden():
        if c["kind"] != "paged":
            continue
        got = fn(np.array(c["q"]), np.array(c["k_pool"]), np.array(c["v_pool"]),
                 np.array(c["block_table"]), np.array(c["seq_lens"]), scale=c["scale"],
                 softcap=c["softcap"])
        exp = np.array(c["expected"], dtype=np.float64)
        np.testing.assert_allclose(got, exp, rtol=0, atol=1e-13, err_msg=c["name"])


def check_zero_query_causal_means(fn):
    """Q = 0 makes every admissible score equal, so each output row is the
    plain mean of its admissible V rows.  The causal mask is built as the
    derivation page (section 4) states it: ``triu(ones, diagonal=Sk-Sq+1)``
    marks the masked entries.  Rows with no admissible key must be zero."""
    rng = np.random.default_rng(0)
    for Sq, Sk in ((7, 7), (3, 9), (9, 4)):
        v = _rand(rng, 1, 1, Sk, 5)
        q = np.zeros((1, 1, Sq, 5))
        k = _rand(rng, 1, 1, Sk, 5)
        masked = np.triu(np.ones((Sq, Sk), dtype=bool), k=Sk - Sq + 1)
        want = np.zeros((Sq, 5))
        for i in range(Sq):
            keep = ~masked[i]
            if keep.any():
                want[i] = v[0, 0][keep].mean(axis=0)
        got = fn(q, k, v, scale=0.3, causal=True)[0, 0]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def check_zero_query_window_means(fn):
    """Q = 0 with a sliding window: row i averages V over
    ``[i'-left, i'+right]`` clipped to the keys (inclusive bounds); checked
    through prefix sums of V."""
    rng = np.random.default_rng(1)
    Sq, Sk, D = 6, 10, 3
    v = _rand(rng, 1, 1, Sk, D)
    k = _rand(rng, 1, 1, Sk, D)
    csum = np.concatenate([np.zeros((1, D)), np.cumsum(v[0, 0], axis=0)])
    for left, right in ((2, 1), (0, 3), (4, 0)):
        got = fn(np.zeros((1, 1, Sq, D)), k, v, scale=1.0, window_left=left,
                 window_right=right)[0, 0]
        for i in range(Sq):
            ip = i + Sk - Sq
            lo, hi = max(0, ip - left), min(Sk - 1, ip + right)
            want = (csum[hi + 1] - csum[lo]) / (hi - lo + 1)
            np.testing.assert_allclose(got[i], want, rtol=0, atol=1e-14)


def check_alibi_geometric(fn, softcap=None):
    """Q = 0 with ALiBi slope ``a``: the weight of key j is proportional to
    ``r^j`` with ``r = e^a`` over the admissible keys ``0..n`` (causal, so
    ``n = i'``).  With ``V_j = j`` the output is the mean of a truncated
    geometric law, ``r/(1-r) - (n+1) r^(n+1) / (1 - r^(n+1))``.  Softcap of a
    zero score is zero, so a softcap applied before ALiBi (the kernel-contract
    page's order) leaves this unchanged."""
    Sq = Sk = 9
    slopes = np.array([0.5, 0.125])
    v = np.broadcast_to(np.arange(Sk, dtype=np.float64)[None, None, :, None], (1, 1, Sk, 2)).copy()
    q = np.zeros((1, 2, Sq, 2))
    k = np.ones((1, 1, Sk, 2))
    got = fn(q, k, v, scale=1.0, causal=True, softcap=softcap, alibi=slopes)
    for h, a in enumerate(slopes):
        r = math.exp(a)
        for i in range(Sq):
            n = i
            want = 0.0 if n == 0 else r / (1 - r) - (n + 1) * r ** (n + 1) / (1 - r ** (n + 1))
            np.testing.assert_allclose(got[0, h, i], [want, want], rtol=1e-12, atol=1e-12)


def check_two_key_ratio(fn):
    """Two keys whose scaled scores differ by exactly ln 3 get weights 3/4 and
    1/4 (derivation page section 1: weights are normalised exponentials)."""
    d = math.log(3.0)
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[[d, 5.0], [0.0, -2.0]]]])
    v = np.array([[[[4.0, 1.0], [8.0, -3.0]]]])
    got = fn(q, k, v, scale=1.0)[0, 0, 0]
    np.testing.assert_allclose(got, [0.75 * 4 + 0.25 * 8, 0.75 * 1 + 0.25 * -3], rtol=1e-14, atol=1e-14)


def check_single_key_exact(fn):
    """Window (0, 0) admits only key ``i'``: the weight is exactly 1, so the
    output row is that V row bit for bit; causal row 0 likewise."""
    rng = np.random.default_rng(2)
    q, k, v = (_rand(rng, 1, 2, 8, 4) for _ in range(3))
    got = fn(q, k, v, scale=0.7, window_left=0, window_right=0)
    assert np.array_equal(got, v)
    got = fn(q, k, v, scale=0.7, causal=True)
    assert np.array_equal(got[:, :, 0], v[:, :, 0])


def check_constant_v_exact(fn):
    """Constant V rows equal to a power of two give that constant exactly in
    every row with an admissible key (a convex combination, one division)."""
    rng = np.random.default_rng(3)
    q, k = _rand(rng, 1, 2, 12, 4, amp=3), _rand(rng, 1, 2, 12, 4, amp=3)
    for c in (0.0, 0.25, -8.0):
        v = np.full((1, 2, 12, 4), c)
        got = fn(q, k, v, scale=0.5, causal=True, window_left=3, softcap=2.0,
                 alibi=np.array([0.3, 0.1]))
        assert np.array_equal(got, v), c


def check_shift_invariance(fn):
    """Adding the same vector w to every key shifts each score row by the
    constant ``scale * q_i . w``; softmax ignores it (derivation page
    section 2), including shifts of +-1e3 that overflow a naive exp."""
    rng = np.random.default_rng(4)
    q, k, v = (_rand(rng, 1, 2, 10, 3) for _ in range(3))
    base = fn(q, k, v, scale=1.0, causal=True, alibi=np.array([0.2, 0.05]))
    for w in (np.array([1000.0, 0.0, 0.0]), np.array([-700.0, 300.0, 0.0]), rng.standard_normal(3)):
        qn = np.where(np.abs(q) < 1e-3, 1e-3, q)
        k2 = k + w[None, None, None, :]
        got = fn(qn, k2, v, scale=1.0, causal=True, alibi=np.array([0.2, 0.05]))
        ref = fn(qn, k, v, scale=1.0, causal=True, alibi=np.array([0.2, 0.05]))
        assert np.all(np.isfinite(got))
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-9)
    assert np.all(np.isfinite(base))


def check_gqa_is_repeat_interleave(fn):
    """GQA equals MHA on K/V repeated to the query heads in contiguous groups
    (derivation page section 5)."""
    rng = np.random.default_rng(5)
    q = _rand(rng, 2, 8, 5, 3)
    k, v = _rand(rng, 2, 2, 7, 3), _rand(rng, 2, 2, 7, 3)
    got = fn(q, k, v, scale=0.5, causal=True)
    ref = fn(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), scale=0.5, causal=True)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-15)
    # And the group of query head h really is h // 4: head 5 uses KV head 1.
    single = fn(q[:, 5:6], k[:, 1:2], v[:, 1:2], scale=0.5, causal=True)
    np.testing.assert_allclose(got[:, 5:6], single, rtol=0, atol=1e-15)


def check_softcap_limits(fn):
    """A huge cap reproduces the uncapped result; a tiny cap with huge scores
    saturates every score to the cap, so each row is the plain mean of V."""
    rng = np.random.default_rng(6)
    q, k, v = (_rand(rng, 1, 1, 6, 4) for _ in range(3))
    np.testing.assert_allclose(fn(q, k, v, scale=0.5, softcap=1e9), fn(q, k, v, scale=0.5),
                               rtol=1e-12, atol=1e-14)
    qpos = np.abs(q) + 1.0
    kpos = np.abs(k) + 1.0
    got = fn(qpos, kpos, v, scale=1e6, softcap=1.0)
    np.testing.assert_allclose(got[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (6, 4)),
                               rtol=0, atol=1e-14)


_LIVE_KWS = (dict(scale=0.7, causal=True),
             dict(scale=0.6, window_left=2, window_right=1),
             dict(scale=0.8, causal=True, softcap=0.5, alibi=[0.25, 0.75]))
_LIVE_LENS = (0, 1, 3, 5, 8)


def _live_prefix_case():
    """Keys of capacity 8 whose rows past the live prefix hold NaN: a key
    read past ``k_len`` poisons its row."""
    rng = np.random.default_rng(91)
    q8 = lambda *s: np.round(rng.standard_normal(s) * 8) / 8
    q, k, v = q8(1, 2, 5, 3), q8(1, 1, 8, 3), q8(1, 1, 8, 3)
    return q, k, v


_LIVE_EXPECTED = {}


def _live_expected(kl, ki):
    """50-digit brute force over the key tensors cut to their first ``kl``
    rows (the live prefix taken as the whole key sequence), output and lse."""
    if (kl, ki) not in _LIVE_EXPECTED:
        from oracle.bruteforce import lse_bruteforce, sdpa_bruteforce
        q, k, v = _live_prefix_case()
        kw = _LIVE_KWS[ki]
        kt, vt = k[:, :, :kl].tolist(), v[:, :, :kl].tolist()
        out = np.array(sdpa_bruteforce(q.tolist(), kt, vt, **kw), dtype=np.float64)
        lse = lse_bruteforce(q.tolist(), kt, **kw)
        lse = np.array([[[-np.inf if x is None else float(x) for x in row] for row in h] for h in lse])
        _LIVE_EXPECTED[(kl, ki)] = (out, lse)
    return _LIVE_EXPECTED[(kl, ki)]


def check_live_prefix(fn):
    """Kernel-contract page, ``k_len`` of ``attention_naive``: only the first
    ``k_len`` key rows exist, the query positions align to that live length,
    and the rows after it are never read (they hold NaN here)."""
    q, k, v = _live_prefix_case()
    for kl in _LIVE_LENS:
        kd, vd = k.copy(), v.copy()
        kd[:, :, kl:] = np.nan
        vd[:, :, kl:] = np.nan
        for ki, kw in enumerate(_LIVE_KWS):
            exp, _ = _live_expected(kl, ki)
            got = fn(q, kd, vd, k_len=kl, **kw)
            np.testing.assert_allclose(got, exp, rtol=0, atol=1e-13, err_msg=f"k_len={kl} {kw}")


# --------------------------------------------------------------------------
# Tests
# --------------------------------------------------------------------------

DENSE_FNS = {
    "naive": osd.sdpa_naive_f64,
    "online_t1": lambda *a, **kw: osd.sdpa_online_f64(*a, tile=1, **kw),
    "online_t3": lambda *a, **kw: osd.sdpa_online_f64(*a, tile=3, **kw),
    "online_t16": lambda *a, **kw: osd.sdpa_online_f64(*a, tile=16, **kw),
}

CHECKS = [check_golden_dense, check_zero_query_causal_means, check_zero_query_window_means,
          check_alibi_geometric, check_two_key_ratio, check_single_key_exact,
          check_shift_invariance, check_gqa_is_repeat_interleave, check_softcap_limits,
          check_live_prefix]


@pytest.mark.parametrize("fn_name", list(DENSE_FNS))
@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_dense_pins(fn_name, check):
    check(DENSE_FNS[fn_name])


def test_alibi_geometric_with_softcap_first():
    check_alibi_geometric(osd.sdpa_naive_f64, softcap=0.3)


def test_constant_v_exact_naive():
    check_constant_v_exact(osd.sdpa_naive_f64)


def test_golden_paged():
    check_golden_paged(osd.paged_decode_f64)


def test_bruteforce_closed_forms():
    """The decimal brute force itself meets the closed forms."""
    from oracle.bruteforce import sdpa_bruteforce

    def bf(q, k, v, **kw):
        kw = {a: (b.tolist() if isinstance(b, np.ndarray) else b) for a, b in kw.items()}
        return np.array(sdpa_bruteforce(q.tolist(), k.tolist(), v.tolist(), **kw), dtype=np.float64)
    check_zero_query_causal_means(bf)
    check_two_key_ratio(bf)
    check_alibi_geometric(bf, softcap=0.3)


@pytest.mark.parametrize("tile", [1, 3, 16, 64])
def test_online_equals_naive(tile):
    """Derivation page section 3: the streaming recurrence is exact; only the
    order of additions differs from the materialised form."""
    rng = np.random.default_rng(10 + tile)
    q = _rand(rng, 1, 4, 37, 8, amp=2)
    k, v = _rand(rng, 1, 2, 53, 8, amp=2), _rand(rng, 1, 2, 53, 8)
    for kw in (dict(causal=True), dict(causal=True, window_left=5, window_right=0),
               dict(window_left=3, window_right=7, softcap=4.0, alibi=np.linspace(0.1, 0.6, 4)),
               dict(causal=True, softcap=1.0)):
        a = osd.sdpa_naive_f64(q, k, v, scale=0.4, **kw)
        b = osd.sdpa_online_f64(q, k, v, scale=0.4, tile=tile, **kw)
        np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-13)


def test_fully_masked_rows_zero():
    """Kernel-contract page: a row with no admissible key is all zero --
    Sq > Sk under bottom-right causal, and the 64-row block of the
    window-512 variant of the 2048-query workload (Sk = 1984)."""
    rng = np.random.default_rng(7)
    q = _rand(rng, 1, 2, 6, 3)
    k, v = _rand(rng, 1, 2, 4, 3), _rand(rng, 1, 2, 4, 3)
    for fn in DENSE_FNS.values():
        out = fn(q, k, v, scale=1.0, causal=True)
        assert np.all(out[:, :, :2] == 0.0)
        assert np.all(out[:, :, 2:] != 0.0)
    ok = osd.admissible(2048, 1984, True, 512, 0)
    has = ok.any(axis=1)
    assert not has[:64].any() and has[64:].all()


def test_empty_extents():
    q = np.zeros((1, 1, 0, 4))
    k = np.ones((1, 1, 5, 4))
    assert osd.sdpa_naive_f64(q, k, k, scale=1.0).shape == (1, 1, 0, 4)
    q = np.ones((1, 1, 3, 4))
    k = np.ones((1, 1, 0, 4))
    assert np.all(osd.sdpa_naive_f64(q, k, k, scale=1.0) == 0)


def test_split_merge_equals_single_pass():
    """Combining partial results over any partition of the keys gives the
    single-pass result (derivation page sections 3 and 8), including empty
    parts and a row whose only keys fall in one part."""
    rng = np.random.default_rng(8)
    q = _rand(rng, 3, 6, amp=2)
    k, v = _rand(rng, 50, 6, amp=2), _rand(rng, 50, 6)
    ref = osd.sdpa_naive_f64(q[None, None], k[None, None], v[None, None], scale=0.5,
                             softcap=3.0)[0, 0]
    for cuts in ([0, 50], [0, 7, 7, 30, 50], [0, 1, 2, 3, 49, 50], [0, 25, 50, 50]):
        os_, ls = [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            o, lse = osd.attention_partial_f64(q, k[a:b], v[a:b], scale=0.5, softcap=3.0)
            os_.append(o)
            ls.append(lse)
        np.testing.assert_allclose(osd.lse_merge_f64(os_, ls), ref, rtol=1e-12, atol=1e-13)
    o, lse = osd.lse_merge_f64([np.zeros((3, 6))], [np.full(3, -np.inf)]), None
    assert np.all(o == 0)


def test_partial_lse_value():
    """``lse`` of a partial is log(sum exp(s)): for Q = 0 over n keys it is
    exactly log(n)."""
    o, lse = osd.attention_partial_f64(np.zeros((2, 3)), np.ones((5, 3)), np.ones((5, 3)), scale=1.0)
    np.testing.assert_allclose(lse, [math.log(5)] * 2, rtol=1e-15)


def test_paged_equals_dense_and_decode_noncausal():
    """Paged decode equals dense attention over the gathered K/V, and at
    Sq = 1 the implicit causal mask admits every live key (derivation page
    section 4), so it equals the non-causal result."""
    rng = np.random.default_rng(9)
    bs, Hkv, Hq, D = 4, 2, 4, 5
    lens = np.array([5, 8, 1, 11], dtype=np.int32)
    nblk = (lens + bs - 1) // bs
    perm = rng.permutation(int(nblk.sum()))
    table = np.full((4, 3), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    kp, vp = _rand(rng, int(nblk.sum()), bs, Hkv, D), _rand(rng, int(nblk.sum()), bs, Hkv, D)
    q = _rand(rng, 4, Hq, 1, D)
    got = osd.paged_decode_f64(q, kp, vp, table, lens, scale=0.6, alibi=np.linspace(0.1, 0.4, 4))
    for b in range(4):
        kb = np.stack([kp[table[b, t // bs], t % bs] for t in range(lens[b])], axis=1)[None]
        vb = np.stack([vp[table[b, t // bs], t % bs] for t in range(lens[b])], axis=1)[None]
        for causal in (True, False):
            ref = osd.sdpa_naive_f64(q[b:b + 1], kb, vb, scale=0.6, causal=causal,
                                     alibi=np.linspace(0.1, 0.4, 4))
            np.testing.assert_allclose(got[b:b + 1], ref, rtol=0, atol=1e-14)


def test_paged_gather_rejects_out_of_pool():
    pool = np.zeros((3, 2, 1, 1))
    with pytest.raises(IndexError):
        osd.paged_gather(pool, np.array([[0, 3]]), 4, 0, 2)
    with pytest.raises(IndexError):
        osd.paged_gather(pool, np.array([[-1, 0]]), 1, 0, 2)


def test_pair_count_closed_forms():
    """Admissible pairs: causal square = S(S+1)/2; bottom-right Sq < Sk adds
    ``Sq*(Sk-Sq)``; causal window L gives sum_i min(i, L) + 1."""
    assert osd.admissible_pair_count(2048, 2048, True) == 2048 * 2049 // 2
    assert osd.admissible_pair_count(512, 4096, True) == 512 * 513 // 2 + 512 * (4096 - 512)
    S, L = 8192, 4096
    assert osd.admissible_pair_count(S, S, True, L, 0) == sum(min(i, L) + 1 for i in range(S))
    assert osd.admissible_pair_count(5, 5, False) == 25


def test_argument_errors():
    q = np.zeros((1, 3, 2, 4))
    k = np.zeros((1, 2, 2, 4))
    with pytest.raises(ValueError):
        osd.sdpa_naive_f64(q, k, k, scale=1.0)
    with pytest.raises(ValueError):
        osd.sdpa_naive_f64(q[:, :2], k, k, scale=1.0, softcap=-1.0)
    with pytest.raises(ValueError):
        osd.sdpa_naive_f64(q[:, :2], k, k, scale=1.0, alibi=np.zeros(3))


# --------------------------------------------------------------------------
# Per-row log-sum-exp (the forward state the backward pass consumes)
# --------------------------------------------------------------------------

def _lse_cases():
    rng = np.random.default_rng(77)
    q8 = lambda *s: np.round(rng.standard_normal(s) * 8) / 8  # multiples of 1/8: exact in decimal
    base = dict(q=q8(1, 2, 4, 3), k=q8(1, 1, 5, 3))
    return [
        (base, dict(scale=0.7)),
        (base, dict(scale=0.7, causal=True)),
        (base, dict(scale=0.7, window_left=1, window_right=0)),
        (base, dict(scale=0.7, causal=True, softcap=0.5, alibi=[0.25, 0.75])),
        (dict(q=q8(1, 2, 6, 3), k=q8(1, 1, 4, 3)), dict(scale=0.9, causal=True)),   # Sq > Sk: empty rows
        (dict(q=q8(2, 4, 3, 2), k=q8(2, 2, 3, 2)), dict(scale=1.1, window_left=0, window_right=1)),
    ]


@pytest.mark.parametrize("case", range(6))
def test_lse_matches_decimal_bruteforce(case):
    """sdpa_lse_f64 against the log of the 50-digit sum of exponentials (no
    max subtracted), every mask/softcap/ALiBi combination; empty rows -inf."""
    from oracle.bruteforce import lse_bruteforce
    t, kw = _lse_cases()[case]
    got = osd.sdpa_lse_f64(t["q"], t["k"], **kw)
    ref = lse_bruteforce(t["q"].tolist(), t["k"].tolist(), **kw)
    for idx in np.ndindex(got.shape):
        r = ref[idx[0]][idx[1]][idx[2]]
        if r is None:
            assert got[idx] == -np.inf
        else:
            assert abs(got[idx] - float(r)) <= 1e-12 * max(1.0, abs(float(r)))
    if case == 4:
        assert np.all(got[..., :2] == -np.inf) and np.all(np.isfinite(got[..., 2:]))


def test_lse_live_prefix_matches_decimal_bruteforce():
    """sdpa_lse_f64 with ``k_len``: the 50-digit lse over the cut tensors,
    with NaN in the rows past the live prefix."""
    q, k, v = _live_prefix_case()
    for kl in _LIVE_LENS:
        kd = k.copy()
        kd[:, :, kl:] = np.nan
        for ki, kw in enumerate(_LIVE_KWS):
            _, exp = _live_expected(kl, ki)
            got = osd.sdpa_lse_f64(q, kd, k_len=kl, **kw)
            fin = np.isfinite(exp)
            assert np.array_equal(np.isfinite(got), fin), (kl, kw)
            np.testing.assert_allclose(got[fin], exp[fin], rtol=1e-12, atol=1e-12)
            assert np.all(got[~fin] == -np.inf)


def test_live_prefix_full_and_errors():
    """``k_len = Sk`` is the call without it; ``k_len`` outside [0, Sk] is an
    error."""
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 2, 4, 3), _rand(rng, 1, 1, 6, 3), _rand(rng, 1, 1, 6, 3)
    for fn in DENSE_FNS.values():
        np.testing.assert_array_equal(fn(q, k, v, scale=0.5, causal=True, k_len=6),
                                      fn(q, k, v, scale=0.5, causal=True))
        for bad in (-1, 7):
            with pytest.raises(ValueError):
                fn(q, k, v, scale=0.5, k_len=bad)


def test_lse_closed_forms():
    """Q = 0: every admissible score is 0, so lse = log(number of admissible
    keys); with ALiBi the causal row sums a geometric series."""
    Sq = Sk = 9
    q = np.zeros((1, 1, Sq, 4))
    k = np.ones((1, 1, Sk, 4))
    got = osd.sdpa_lse_f64(q, k, scale=0.3, causal=True)[0, 0]
    np.testing.assert_allclose(got, [math.log(i + 1) for i in range(Sq)], rtol=0, atol=1e-15)
    got = osd.sdpa_lse_f64(q, k, scale=0.3, window_left=2, window_right=3)[0, 0]
    want = [math.log(min(Sk - 1, i + 3) - max(0, i - 2) + 1) for i in range(Sq)]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)
    slope = 0.4
    got = osd.sdpa_lse_f64(q, k, scale=0.3, causal=True, alibi=np.array([slope]))[0, 0]
    r = math.exp(-slope)
    want = [math.log((1 - r ** (i + 1)) / (1 - r)) for i in range(Sq)]
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)


def test_lse_shift_is_additive():
    """Adding one vector w to every key adds scale * (q . w) to each row's
    scores, so the lse moves by exactly that amount -- including shifts of
    +-1e3 that overflow an unstabilised exp (derivation page section 2)."""
    rng = np.random.default_rng(5)
    q = _rand(rng, 1, 2, 7, 4)
    k = _rand(rng, 1, 1, 11, 4)
    base = osd.sdpa_lse_f64(q, k, scale=0.5, causal=True)
    for amp in (1e3, -1e3):
        w = np.full(4, amp / 4)
        sh = osd.sdpa_lse_f64(q, k + w, scale=0.5, causal=True)
        delta = 0.5 * (q[0] @ w)                    # [Hq, Sq]
        np.testing.assert_allclose(sh[0] - base[0], delta, rtol=1e-10, atol=1e-9)


# --------------------------------------------------------------------------
# Variable-length prefill over the paged pool
# --------------------------------------------------------------------------

def _varlen_case(rng, Hq=2, Hkv=1, D=3, bs=4, sq=(3, 0, 5), sk=(6, 2, 3)):
    q8 = lambda *s: np.round(rng.standard_normal(s) * 8) / 8
    nblk = [(c + bs - 1) // bs for c in sk]
    nb = sum(nblk)
    perm = rng.permutation(nb)
    table = np.full((len(sk), max(nblk)), -1, dtype=np.int64)
    pos = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    cu = np.concatenate([[0], np.cumsum(sq)]).astype(np.int64)
    return dict(q=q8(int(cu[-1]), Hq, D), kp=q8(nb, bs, Hkv, D), vp=q8(nb, bs, Hkv, D),
                table=table, lens=np.array(sk), cu=cu)


@pytest.mark.parametrize("kw", [dict(causal=True), dict(causal=True, softcap=0.7, alibi=[0.3, 0.6]),
                                dict(causal=False, window_left=1, window_right=1)])
def test_varlen_matches_decimal_bruteforce(kw):
    """Each sequence's rows against the 50-digit definition on its own keys,
    gathered here by plain indexing of the pool (block table, slot)."""
    from oracle.bruteforce import sdpa_bruteforce
    c = _varlen_case(np.random.default_rng(3))
    kw = dict(kw)
    got = osd.paged_prefill_varlen_f64(c["q"], c["kp"], c["vp"], c["table"], c["lens"], c["cu"],
                                       scale=0.8, **kw)
    bs = c["kp"].shape[1]
    for b in range(len(c["lens"])):
        r0, r1 = int(c["cu"][b]), int(c["cu"][b + 1])
        ctx = int(c["lens"][b])
        if r1 == r0:
            continue
        krows = [[c["kp"][c["table"][b][t // bs]][t % bs][g].tolist() for t in range(ctx)]
                 for g in range(c["kp"].shape[2])]
        vrows = [[c["vp"][c["table"][b][t // bs]][t % bs][g].tolist() for t in range(ctx)]
                 for g in range(c["vp"].shape[2])]
        qrows = [[c["q"][r][h].tolist() for r in range(r0, r1)] for h in range(c["q"].shape[1])]
        ref = np.array(sdpa_bruteforce([qrows], [krows], [vrows], scale=0.8, **kw), dtype=np.float64)
        np.testing.assert_allclose(np.transpose(got[r0:r1], (1, 0, 2)), ref[0], rtol=1e-12, atol=1e-12)
    # sequence 2 has 5 queries but 3 keys: causal rows 0 and 1 sit before every key
    if kw.get("causal"):
        r0 = int(c["cu"][2])
        assert np.all(got[r0:r0 + 2] == 0) and np.all(np.abs(got[r0 + 2:r0 + 5]).sum(-1) > 0)


def test_varlen_equal_lengths_is_the_paged_form():
    """With every sequence of the same query length, packing the rows is only
    a relayout of the [B, Hq, Sq, D] paged form."""
    rng = np.random.default_rng(8)
    c = _varlen_case(rng, Hq=4, Hkv=2, D=5, bs=3, sq=(4, 4, 4), sk=(7, 4, 9))
    got = osd.paged_prefill_varlen_f64(c["q"], c["kp"], c["vp"], c["table"], c["lens"], c["cu"],
                                       scale=0.5, causal=True, alibi=[0.1, 0.2, 0.3, 0.4])
    q4 = np.transpose(c["q"].reshape(3, 4, 4, 5), (0, 2, 1, 3))   # [B, Hq, Sq, D]
    ref = osd.paged_decode_f64(q4, c["kp"], c["vp"], c["table"], c["lens"], scale=0.5,
                               alibi=[0.1, 0.2, 0.3, 0.4])
    np.testing.assert_allclose(got.reshape(3, 4, 4, 5), np.transpose(ref, (0, 2, 1, 3)),
                               rtol=1e-13, atol=1e-14)
    with pytest.raises(ValueError):
        osd.paged_prefill_varlen_f64(c["q"], c["kp"], c["vp"], c["table"], c["lens"],
                                     [0, 5, 3, 12], scale=0.5)


# --------------------------------------------------------------------------
# Backward pass (kernel-contract page, attention_flash_backward)
# --------------------------------------------------------------------------

BWD_KW = [
    dict(),
    dict(causal=True),
    dict(causal=True, window_left=2, window_right=0),
    dict(window_left=1, window_right=2),
    dict(softcap=1.5),
    dict(alibi=[0.5, -0.3]),
    dict(causal=True, softcap=2.0, alibi=[0.25, 0.75]),
]


def _bwd_case(rng, B=1, Hq=2, Hkv=1, Sq=4, Sk=5, D=3, amp=1.0):
    return (_rand(rng, B, Hq, Sq, D, amp=amp), _rand(rng, B, Hkv, Sk, D, amp=amp),
            _rand(rng, B, Hkv, Sk, D), _rand(rng, B, Hq, Sq, D))


def check_bwd_finite_differences(bwd):
    """Each gradient is the derivative of L = sum(dO * O) through the (pinned)
    forward definition: central differences, step 1e-5, on every element of
    q, k and v; the truncation error is O(h^2) ~ 1e-10 and the rounding error
    ~ 1e-16 / h, both far under the 1e-7 bar."""
    rng = np.random.default_rng(41)
    h = 1e-5
    for kw in BWD_KW:
        for Sq, Sk in ((4, 5), (6, 4)):           # (6, 4) causal: rows 0, 1 have no key
            q, k, v, do = _bwd_case(rng, Sq=Sq, Sk=Sk, amp=1.3)
            got = bwd(q, k, v, do, scale=0.7, **kw)

            def loss(q_, k_, v_):
                return float(np.sum(do * osd.sdpa_naive_f64(q_, k_, v_, scale=0.7, **kw)))
            for which, x in enumerate((q, k, v)):
                num = np.zeros_like(x)
                for idx in np.ndindex(x.shape):
                    xp, xm = x.copy(), x.copy()
                    xp[idx] += h
                    xm[idx] -= h
                    args_p = [q, k, v]
                    args_m = [q, k, v]
                    args_p[which], args_m[which] = xp, xm
                    num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
                err = np.abs(got[which] - num).max()
                assert err < 1e-7, (kw, Sq, Sk, "qkv"[which], err)


def check_bwd_constant_v(bwd):
    """V rows all equal to one vector c make O = c for every row with a key,
    independent of q and k: dQ = dK = 0, and dV[j] = sum_i P[i, j] dO[i], so
    the dV rows of a head sum to the sum of its dO rows with a key."""
    rng = np.random.default_rng(42)
    q, k, _, do = _bwd_case(rng, Hq=4, Hkv=2, Sq=7, Sk=5, D=4)
    c = rng.standard_normal(4)
    v = np.broadcast_to(c, (1, 2, 5, 4)).copy()
    for kw in (dict(), dict(causal=True), dict(causal=True, softcap=1.0, alibi=[0.1, 0.2, 0.3, 0.4])):
        dq, dk, dv = bwd(q, k, v, do, scale=0.9, **kw)
        assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13, kw
        has_key = osd.admissible(7, 5, kw.get("causal", False)).any(axis=1)
        for g in range(2):
            want = do[0, 2 * g:2 * g + 2][:, has_key].sum(axis=(0, 1))
            np.testing.assert_allclose(dv[0, g].sum(axis=0), want, rtol=1e-12, atol=1e-12)


def check_bwd_dk_rows_sum_to_zero(bwd):
    """Adding one vector w to every key shifts each row's scores by the
    per-row constant scale q_i . w, which softmax ignores (derivation page,
    section 2): without a softcap the dK rows of each KV head sum to zero,
    masks and ALiBi included."""
    rng = np.random.default_rng(43)
    q, k, v, do = _bwd_case(rng, B=2, Hq=4, Hkv=2, Sq=6, Sk=8, D=5)
    for kw in (dict(), dict(causal=True), dict(window_left=2, window_right=1, alibi=[0.3, -0.2, 0.5, 0.1])):
        _, dk, _ = bwd(q, k, v, do, scale=0.6, **kw)
        assert np.abs(dk.sum(axis=2)).max() < 1e-12, kw


def check_bwd_gqa_is_summed_mha(bwd):
    """GQA = MHA on repeat-interleaved K/V (derivation page, section 5), so
    the GQA dK/dV of a KV head is the sum of the MHA dK/dV of its group."""
    rng = np.random.default_rng(44)
    q, k, v, do = _bwd_case(rng, Hq=6, Hkv=2, Sq=5, Sk=6, D=3)
    kw = dict(causal=True, softcap=2.5, alibi=[0.1, 0.2, 0.3, 0.4, 0.5, 0.6])
    dq, dk, dv = bwd(q, k, v, do, scale=0.8, **kw)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    dq2, dk2, dv2 = bwd(q, kr, vr, do, scale=0.8, **kw)
    np.testing.assert_allclose(dq, dq2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(1, 2, 3, 6, 3).sum(axis=2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(1, 2, 3, 6, 3).sum(axis=2), rtol=1e-12, atol=1e-13)


def check_bwd_empty_rows_and_linearity(bwd):
    """Rows with no admissible key contribute nothing: their dQ rows are 0 and
    their dO is ignored; the gradients are linear in dO."""
    rng = np.random.default_rng(45)
    q, k, v, do = _bwd_case(rng, Sq=7, Sk=4, D=3)      # causal: rows 0..2 have no key
    kw = dict(causal=True, alibi=[0.2, 0.4])
    dq, dk, dv = bwd(q, k, v, do, scale=1.1, **kw)
    assert np.all(dq[:, :, :3] == 0)
    do2 = do.copy()
    do2[:, :, :3] = rng.standard_normal(do2[:, :, :3].shape) * 100
    _, dk2, dv2 = bwd(q, k, v, do2, scale=1.1, **kw)
    np.testing.assert_allclose(dk2, dk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv2, dv, rtol=1e-12, atol=1e-12)
    e = rng.standard_normal(do.shape)
    sums = bwd(q, k, v, do + 2 * e, scale=1.1, **kw)
    parts = [a + 2 * b for a, b in zip(bwd(q, k, v, do, scale=1.1, **kw), bwd(q, k, v, e, scale=1.1, **kw))]
    for x, y in zip(sums, parts):
        np.testing.assert_allclose(x, y, rtol=1e-11, atol=1e-12)


BWD_CHECKS = [check_bwd_finite_differences, check_bwd_constant_v, check_bwd_dk_rows_sum_to_zero,
              check_bwd_gqa_is_summed_mha, check_bwd_empty_rows_and_linearity]


@pytest.mark.parametrize("check", BWD_CHECKS, ids=lambda c: c.__name__)
def test_backward_pins(check):
    check(osd.sdpa_backward_f64)


def test_backward_zero_extents_and_errors():
    q = np.zeros((1, 2, 0, 4))
    k = np.zeros((1, 1, 3, 4))
    dq, dk, dv = osd.sdpa_backward_f64(q, k, k, q, scale=1.0)
    assert dq.shape == (1, 2, 0, 4) and np.all(dk == 0) and np.all(dv == 0)
    with pytest.raises(ValueError):
        osd.sdpa_backward_f64(np.zeros((1, 2, 3, 4)), k, k, np.zeros((1, 2, 2, 4)), scale=1.0)
