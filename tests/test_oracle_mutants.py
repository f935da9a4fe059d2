"""Plant plausible mistakes in the oracle and show the pins catch each one.

Every mutant replaces one helper of :mod:`oracle.sdpa` (on the CPU, through
``monkeypatch``) with a wrong variant -- a dropped term, a flipped sign, a
shifted index, a swapped operand or order.  The test passes only if at least
one of the pin checks of ``test_oracle.py`` fails under that mutant, so a pin
suite that could not tell the mutant from the real oracle is itself a failure.
"""
import numpy as np
import pytest

from oracle import sdpa as osd
import test_oracle as pins

_real_admissible = osd.admissible
_real_transform = osd.transform_scores
_real_gather = osd.paged_gather
_real_live = osd.live_keys


def _adm_exclusive(Sq, Sk, causal, window_left=None, window_right=None, rows=None):
    ok = _real_admissible(Sq, Sk, causal, None, None, rows)
    ip = osd.query_positions(Sq, Sk)
    ip = (ip if rows is None else ip[rows])[:, None]
    j = np.arange(Sk)[None, :]
    if window_left is not None:
        ok &= j > ip - window_left
    if window_right is not None:
        ok &= j < ip + window_right
    return ok


def _adm_swapped_window(Sq, Sk, causal, window_left=None, window_right=None, rows=None):
    return _real_admissible(Sq, Sk, causal, window_right, window_left, rows)


def _adm_strict_causal(Sq, Sk, causal, window_left=None, window_right=None, rows=None):
    ok = _real_admissible(Sq, Sk, False, window_left, window_right, rows)
    if causal:
        ip = osd.query_positions(Sq, Sk)
        ip = (ip if rows is None else ip[rows])[:, None]
        ok &= np.arange(Sk)[None, :] < ip
    return ok


def _live_ignored(k, v, k_len):
    _real_live(k, v, k_len)            # keeps the argument checks
    return k, v


def _live_one_short(k, v, k_len):
    if k_len is None:
        return k, v
    return _real_live(k, v, max(0, k_len - 1))


def _tf_alibi_sign(s, softcap=None, slope=None, rel=None):
    return _real_transform(s, softcap, None if slope is None else -slope, rel)


def _tf_order_swapped(s, softcap=None, slope=None, rel=None):
    if slope is not None:
        s = s + slope * rel
    if softcap:
        s = softcap * np.tanh(s / softcap)
    return s


def _tf_cap_factor_dropped(s, softcap=None, slope=None, rel=None):
    if softcap:
        s = np.tanh(s / softcap)
    if slope is not None:
        s = s + slope * rel
    return s


def _tf_alibi_abs(s, softcap=None, slope=None, rel=None):
    # Distance without its sign: |j - i'| instead of (j - i').
    return _real_transform(s, softcap, slope, None if rel is None else np.abs(rel))


def _scores_unscaled(qrows, kmat, scale, softcap, slope, rel, ok):
    s = qrows @ kmat.T
    s = osd.transform_scores(s, softcap, slope, rel)
    return np.where(ok, s, -np.inf)


def _scores_kq_swapped(qrows, kmat, scale, softcap, slope, rel, ok):
    # Keys scored against the wrong query row order (a transposed index).
    s = (qrows[::-1] @ kmat.T) * scale
    s = osd.transform_scores(s, softcap, slope, rel)
    return np.where(ok, s, -np.inf)


def _gather_slot_wrong(pool, block_table, seq_len, b, block_size):
    t = np.arange(int(seq_len))
    phys = np.asarray(block_table)[b, t // block_size]
    return np.asarray(pool)[phys, (t + 1) % block_size]


def _gather_row_wrong(pool, block_table, seq_len, b, block_size):
    # Every sequence reads the block table row of sequence 0.
    t = np.arange(int(seq_len))
    phys = np.asarray(block_table)[0, t // block_size].clip(0)
    return np.asarray(pool)[phys, t % block_size]


def _sm_bwd_row_term_dropped(p, dp):
    return dp * p


def _cap_deriv_dropped(s_pre, softcap):
    return np.ones_like(s_pre)


def _cap_deriv_unsquared(s_pre, softcap):
    return 1.0 - np.tanh(s_pre / softcap)


def _grads_dk_unscaled(ds, qrows, kmat, scale):
    return scale * (ds @ kmat), ds.T @ qrows


def _grads_dk_rows_permuted(ds, qrows, kmat, scale):
    # dK taken against the query rows in reverse order (a transposed index)
    return scale * (ds @ kmat), scale * (ds.T @ qrows[::-1])


MUTANTS = {
    "causal_top_left": ("query_positions", lambda Sq, Sk: np.arange(Sq)),
    "causal_strict": ("admissible", _adm_strict_causal),
    "window_exclusive": ("admissible", _adm_exclusive),
    "window_sides_swapped": ("admissible", _adm_swapped_window),
    "live_prefix_ignored": ("live_keys", _live_ignored),
    "live_prefix_one_short": ("live_keys", _live_one_short),
    "kv_head_modulo": ("kv_head_of", lambda h, Hq, Hkv: h % Hkv),
    "alibi_sign": ("transform_scores", _tf_alibi_sign),
    "alibi_abs_distance": ("transform_scores", _tf_alibi_abs),
    "softcap_after_alibi": ("transform_scores", _tf_order_swapped),
    "softcap_factor_dropped": ("transform_scores", _tf_cap_factor_dropped),
    "scale_dropped": ("_scores", _scores_unscaled),
    "query_rows_permuted": ("_scores", _scores_kq_swapped),
    "paged_slot_off_by_one": ("paged_gather", _gather_slot_wrong),
    "paged_wrong_sequence_row": ("paged_gather", _gather_row_wrong),
    "bwd_softmax_row_term_dropped": ("softmax_backward", _sm_bwd_row_term_dropped),
    "bwd_softcap_derivative_dropped": ("softcap_derivative", _cap_deriv_dropped),
    "bwd_softcap_derivative_unsquared": ("softcap_derivative", _cap_deriv_unsquared),
    "bwd_dk_unscaled": ("score_input_grads", _grads_dk_unscaled),
    "bwd_dk_query_rows_permuted": ("score_input_grads", _grads_dk_rows_permuted),
}


def _run_all_checks():
    failures = []
    checks = list(pins.CHECKS) + [pins.check_constant_v_exact]
    for check in checks:
        try:
            check(osd.sdpa_naive_f64)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failures.append(check.__name__)
    try:
        pins.check_golden_paged(osd.paged_decode_f64)
    except (AssertionError, ValueError, IndexError):
        failures.append("check_golden_paged")
    try:
        pins.test_paged_equals_dense_and_decode_noncausal()
    except (AssertionError, ValueError, IndexError):
        failures.append("paged_equals_dense")
    for check in pins.BWD_CHECKS:
        try:
            check(osd.sdpa_backward_f64)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failures.append(check.__name__)
    return failures


def test_unmutated_oracle_passes_every_check():
    assert _run_all_checks() == []


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(monkeypatch, name):
    attr, fake = MUTANTS[name]
    monkeypatch.setattr(osd, attr, fake)
    with np.errstate(all="ignore"):
        caught = _run_all_checks()
    assert caught, f"mutant {name} passed every pin"
