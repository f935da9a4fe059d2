"""The seeded synthetic inputs: determinism, shapes, and a valid paged layout."""
import numpy as np
import torch

import workloads as W


def test_dense_deterministic_and_shaped():
    w = W.TINY_F32
    a = W.dense_inputs(w)
    b = W.dense_inputs(w)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    q, k, v, alibi = a
    assert q.shape == (1, 4, 128, 64) and q.dtype == torch.float32
    assert k.shape == v.shape == (1, 4, 128, 64)
    assert alibi is None
    c = W.dense_inputs(w, seed=7)
    assert not torch.equal(c[0], q)


def test_masked_rows_variant_reuses_draws():
    w2 = W.GQA_CAUSAL_2K
    small = W.Dense("t2", "bf16", 1, 2, 1, 16, 16, 8, causal=True, seed=3)
    q, k, v, _ = W.dense_inputs(small)
    assert q.dtype == torch.bfloat16 and k.shape == (1, 1, 16, 8)
    assert W.GQA_MASKED_ROWS.seed == w2.seed and W.GQA_MASKED_ROWS.Sk == 1984


def test_bf16_cast_is_round_to_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8], dtype=np.float32)
    y = W.cast(x, "bf16").float().numpy()
    assert list(y) == [1.0, 1.0 + 2 ** -6, -1.0]


def test_paged_layout_is_a_permutation():
    rng = np.random.default_rng(0)
    lens = np.array([1, 64, 65, 0, 200], dtype=np.int32)
    table, nb = W.paged_layout(lens, 64, 4, rng)
    assert nb == 1 + 1 + 2 + 0 + 4
    used = []
    for b, c in enumerate(lens):
        n = (c + 63) // 64
        assert np.all(table[b, n:] == -1)
        used.extend(table[b, :n].tolist())
    assert sorted(used) == list(range(nb))


def test_paged_inputs_small():
    w = W.Paged("p", "bf16", 3, 4, 2, 16, 8, 5, 20, 2, 3, seed=11)
    q, kp, vp, table, lens, alibi = W.paged_inputs(w)
    assert q.shape == (3, 4, 1, 16)
    assert kp.shape == vp.shape and kp.shape[1:] == (8, 2, 16)
    assert lens.dtype == torch.int32 and table.dtype == torch.int32
    assert int(((lens + 7) // 8).sum()) == kp.shape[0]
    assert (lens >= 5).all() and (lens <= 20).all()


def test_alibi_slopes():
    s = W.alibi_slopes(32)
    assert s.dtype == np.float32
    assert s[0] == np.float32(2 ** -0.25) and s[31] == np.float32(2 ** -8)
