"""Parity of attn_fwd (HIP, through the C ABI) with the float64 oracle.

Small cases span several 128-row / 64-key tiles with ragged tails and every
mask combination; the full-size workloads are checked on their whole output,
in the launch configuration the benchmark times.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, compare

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64}


def gpu_fwd(sdpa, q, k, v, alibi, **kw):
    dev = torch.device("cuda:0")
    out = sdpa.attn_fwd(q.to(dev), k.to(dev), v.to(dev),
                        None if alibi is None else alibi.to(dev), **kw)
    torch.cuda.synchronize()
    return out


def oracle_heads(q, k, v, alibi, heads, **kw):
    """Oracle output for the sampled (b, h) pairs, stacked [n, Sq, D]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    res = []
    for b, h in heads:
        g = oracle.kv_head_of(h, Hq, Hkv)
        sl = None if alibi is None else W.to_f64(alibi)[h:h + 1]
        res.append(oracle.sdpa_naive_f64(W.to_f64(q[b:b + 1, h:h + 1]), W.to_f64(k[b:b + 1, g:g + 1]),
                                         W.to_f64(v[b:b + 1, g:g + 1]), alibi=sl, **kw)[0, 0])
    return np.stack(res)


def run_case(sdpa, dtype, B, Hq, Hkv, Sq, Sk, D, *, causal=False, wl=None, wr=None,
             softcap=None, alibi=False, amp=1.0, seed=0, heads=None, scale=None,
             window_left=None, window_right=None):
    wl = window_left if window_left is not None else wl
    wr = window_right if window_right is not None else wr
    name = (f"attn_fwd {dtype} B{B} H{Hq}/{Hkv} Sq{Sq} Sk{Sk} D{D} causal={causal} "
            f"win=({wl},{wr}) cap={softcap} alibi={alibi} seed={seed}")
    q, k, v = W.random_dense(dtype, B, Hq, Hkv, Sq, Sk, D, seed, amp)
    sl = torch.from_numpy(W.alibi_slopes(Hq)) if alibi else None
    # the ABI takes the scale as float32: both sides get that value
    kw = dict(scale=float(np.float32(1.0 / math.sqrt(D) if scale is None else scale)), causal=causal,
              window_left=wl, window_right=wr, softcap=softcap)
    announce(name)
    out = gpu_fwd(sdpa, q, k, v, sl, softmax_scale=kw["scale"], causal=causal,
                  window_left=wl, window_right=wr, softcap=softcap)
    if heads is None:
        ref = oracle.sdpa_naive_f64(W.to_f64(q), W.to_f64(k), W.to_f64(v),
                                    alibi=None if sl is None else W.to_f64(sl), **kw)
        compare(out, ref, DT[dtype], name)
    else:
        ref = oracle_heads(q, k, v, sl, heads, **kw)
        got = torch.stack([out[b, h] for b, h in heads])
        compare(got, ref, DT[dtype], name)
    return out


SMALL = [
    # (B, Hq, Hkv, Sq, Sk, kwargs)
    (1, 2, 2, 256, 256, dict()),
    (2, 2, 1, 300, 333, dict()),
    (1, 4, 2, 300, 300, dict(causal=True)),
    (2, 4, 1, 200, 517, dict(causal=True)),
    (1, 2, 2, 517, 200, dict(causal=True)),
    (1, 4, 4, 333, 333, dict(causal=True, wl=37, wr=0)),
    (1, 2, 1, 270, 290, dict(wl=50, wr=20)),
    (1, 2, 2, 190, 190, dict(softcap=5.0, amp=3.0)),
    (1, 4, 2, 300, 300, dict(causal=True, alibi=True)),
    (2, 8, 2, 257, 385, dict(causal=True, wl=100, wr=0, softcap=20.0, alibi=True, amp=1.5)),
    (1, 16, 2, 129, 129, dict(causal=True)),
    (1, 2, 2, 64, 1000, dict(wl=10, wr=3, alibi=True)),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_parity(gpu_lib, dtype, D, case):
    B, Hq, Hkv, Sq, Sk, kw = SMALL[case]
    run_case(gpu_lib, dtype, B, Hq, Hkv, Sq, Sk, D, seed=100 + case, **kw)


# Small grids with long key ranges: the launch splits each workgroup's key
# tiles over two wave groups and merges them; odd and even tile counts, rows
# with no admissible key, and every mask kind.
KEY_SPLIT = [
    (1, 2, 1, 128, 512, dict()),
    (1, 2, 2, 100, 577, dict()),
    (1, 4, 2, 700, 600, dict(causal=True)),                  # rows 0..99 empty
    (2, 2, 1, 333, 1111, dict(causal=True)),
    (1, 2, 2, 256, 900, dict(causal=True, wl=200, wr=0)),
    (1, 2, 1, 200, 640, dict(wl=300, wr=50, softcap=10.0, amp=2.0)),
    (1, 4, 4, 64, 2000, dict(alibi=True)),
    (1, 2, 2, 300, 1500, dict(causal=True, softcap=20.0, alibi=True, amp=1.5)),
]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64), ("bf16", 64), ("f16", 128)])
@pytest.mark.parametrize("case", range(len(KEY_SPLIT)))
def test_key_split_parity(gpu_lib, dtype, D, case):
    B, Hq, Hkv, Sq, Sk, kw = KEY_SPLIT[case]
    out = run_case(gpu_lib, dtype, B, Hq, Hkv, Sq, Sk, D, seed=300 + case, **kw)
    if kw.get("causal") and Sq > Sk:
        assert torch.count_nonzero(out[:, :, :Sq - Sk]).item() == 0


# Head dim 256 on the matrix cores (one wave per SIMD, no key split).
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", [0, 3, 5, 7, 9, 11])
def test_d256_parity(gpu_lib, dtype, case):
    B, Hq, Hkv, Sq, Sk, kw = SMALL[case]
    run_case(gpu_lib, dtype, B, Hq, Hkv, Sq, Sk, 256, seed=1000 + case, **kw)


@pytest.mark.parametrize("case", [
    (1, 4, 4, 128, 128, 64, dict()),
    (1, 4, 2, 200, 250, 128, dict(causal=True)),
    (2, 2, 1, 150, 150, 64, dict(causal=True, wl=30, wr=0, softcap=8.0, alibi=True)),
    (1, 2, 2, 100, 70, 128, dict(wl=5, wr=9)),
])
def test_f32_parity(gpu_lib, case):
    B, Hq, Hkv, Sq, Sk, D, kw = case
    run_case(gpu_lib, "f32", B, Hq, Hkv, Sq, Sk, D, seed=7, **kw)


# The vector-ALU path in float64, and both vector-ALU precisions at the head
# dims only it builds (32 and 256): every mask kind, ragged tiles, GQA.
VALU_CASES = [
    (1, 2, 2, 77, 77, dict()),
    (2, 4, 2, 130, 100, dict(causal=True)),                       # Sq > Sk: rows 0..29 empty
    (1, 4, 1, 100, 161, dict(causal=True, wl=40, wr=0, softcap=6.0, alibi=True, amp=2.0)),
    (1, 2, 2, 90, 70, dict(wl=9, wr=4)),
]


@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("case", range(len(VALU_CASES)))
def test_f64_parity(gpu_lib, D, case):
    B, Hq, Hkv, Sq, Sk, kw = VALU_CASES[case]
    run_case(gpu_lib, "f64", B, Hq, Hkv, Sq, Sk, D, seed=500 + case, **kw)


@pytest.mark.parametrize("D", [32, 256])
@pytest.mark.parametrize("case", range(len(VALU_CASES)))
def test_f32_new_head_dims(gpu_lib, D, case):
    B, Hq, Hkv, Sq, Sk, kw = VALU_CASES[case]
    run_case(gpu_lib, "f32", B, Hq, Hkv, Sq, Sk, D, seed=600 + case, **kw)


def test_tiny_f32_workload(gpu_lib):
    w = W.TINY_F32
    q, k, v, _ = W.dense_inputs(w)
    announce(w.name)
    out = gpu_fwd(gpu_lib, q, k, v, None, softmax_scale=w.scale)
    ref = oracle.sdpa_naive_f64(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale=w.scale)
    compare(out, ref, torch.float32, w.name)


def _workload_full(sdpa, w):
    """The whole output of a full-size workload, in the launch configuration
    the benchmark times, against the oracle's whole output."""
    q, k, v, sl = W.dense_inputs(w)
    announce(w.name)
    out = gpu_fwd(sdpa, q, k, v, sl, softmax_scale=w.scale, causal=w.causal,
                  window_left=w.window_left, window_right=w.window_right, softcap=w.softcap)
    ref = oracle.sdpa_naive_f64(W.to_f64(q), W.to_f64(k), W.to_f64(v),
                                alibi=None if sl is None else W.to_f64(sl), scale=w.scale,
                                causal=w.causal, window_left=w.window_left,
                                window_right=w.window_right, softcap=w.softcap)
    compare(out, ref, DT[w.dtype], w.name)
    return out


def test_gqa_causal_2k_workload(gpu_lib):
    _workload_full(gpu_lib, W.GQA_CAUSAL_2K)


def test_masked_rows_workload(gpu_lib):
    w = W.GQA_MASKED_ROWS
    out = _workload_full(gpu_lib, w)
    # Rows 0..63 have no admissible key in every head: exactly zero.
    assert torch.count_nonzero(out[:, :, :64]).item() == 0
    assert torch.count_nonzero(out[:, :, 64:].float().abs().sum(-1) == 0).item() == 0


def test_long_masked_8k_workload(gpu_lib):
    _workload_full(gpu_lib, W.LONG_MASKED_8K)


def test_chunked_prefill_workload(gpu_lib):
    _workload_full(gpu_lib, W.CHUNKED_PREFILL)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("mask", ["causal", "window", "ragged"])
def test_zero_scale_is_uniform_attention(gpu_lib, dtype, mask):
    """softmax_scale = 0 makes every admissible weight 1: each row is the mean
    of its admissible V rows, also where masked keys share a tile with
    admissible ones (causal diagonal, window edge, a ragged key tail)."""
    Sk = 200 if mask == "ragged" else 256
    kw = {"causal": dict(causal=True), "window": dict(window_left=40, window_right=3),
          "ragged": dict()}[mask]
    run_case(gpu_lib, dtype, 1, 4, 2, 256, Sk, 128, seed=31, scale=0.0, **kw)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_single_admissible_key_is_exact(gpu_lib, dtype):
    """Window (0, 0): weight exactly 1 on key i', so out == V row bit for bit."""
    q, k, v = W.random_dense(dtype, 1, 4, 2, 200, 200, 128, 11)
    announce(f"single key {dtype}")
    out = gpu_fwd(gpu_lib, q, k, v, None, window_left=0, window_right=0)
    ref = torch.repeat_interleave(v, 2, dim=1)
    assert torch.equal(out.cpu(), ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_constant_v_is_exact(gpu_lib, dtype):
    q, k, _ = W.random_dense(dtype, 1, 4, 2, 300, 300, 64, 12, amp=2.0)
    v = torch.full((1, 2, 300, 64), 0.25, dtype=DT[dtype])
    sl = torch.from_numpy(W.alibi_slopes(4))
    announce(f"constant v {dtype}")
    out = gpu_fwd(gpu_lib, q, k, v, sl, causal=True, window_left=40, softcap=10.0)
    assert torch.all(out.cpu() == 0.25)


def test_empty_extents(gpu_lib):
    q, k, v = W.random_dense("bf16", 1, 2, 2, 70, 0, 128, 13)
    announce("Sk = 0")
    out = gpu_fwd(gpu_lib, q, k, v, None, causal=True)
    assert torch.count_nonzero(out).item() == 0
    q, k, v = W.random_dense("bf16", 1, 2, 2, 0, 50, 128, 13)
    announce("Sq = 0")
    out = gpu_fwd(gpu_lib, q, k, v, None)
    assert out.shape == (1, 2, 0, 128)


def test_gqa_equals_repeated_mha_bitwise(gpu_lib):
    q, k, v = W.random_dense("bf16", 1, 8, 2, 260, 260, 128, 14)
    announce("gqa vs mha")
    a = gpu_fwd(gpu_lib, q, k, v, None, causal=True)
    b = gpu_fwd(gpu_lib, q, torch.repeat_interleave(k, 4, 1), torch.repeat_interleave(v, 4, 1),
                None, causal=True)
    assert torch.equal(a, b)


def test_rerun_is_bitwise_identical(gpu_lib):
    w = W.GQA_CAUSAL_2K
    q, k, v, _ = W.dense_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    announce("rerun determinism")
    a = gpu_lib.attn_fwd(q, k, v, causal=True)
    b = gpu_lib.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_binding_rejects_bad_arguments(gpu_lib):
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 4, 8, 128, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 3, 8, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(gpu_lib.AttnError) as e:
        gpu_lib.attn_fwd(q, k, k)
    assert e.value.status == 4
    with pytest.raises(ValueError):
        gpu_lib.attn_fwd(q, q.half(), q)
    with pytest.raises(ValueError):
        gpu_lib.attn_fwd(q, q.transpose(2, 3).contiguous().transpose(2, 3), q)
    with pytest.raises(gpu_lib.AttnError) as e:
        gpu_lib.attn_fwd(q[..., :96].contiguous(), q[..., :96].contiguous(), q[..., :96].contiguous())
    assert e.value.status == 5


# ----------------------------------------------------------------- LSE output

# Largest |lse_gpu - lse_oracle| allowed.  The kernels sum the weights as they
# enter the second matmul, i.e. rounded to the input dtype: round to nearest
# even has unit roundoff 2^-8 for bf16 (7 stored mantissa bits) and 2^-11 for
# f16 (10 bits), so if every weight of a row rounds the same way, ln(l) moves by
# up to that much.  The float32 path sums exact float32 weights.  A
# float32-accumulated score adds a relative 1e-5 of |lse|.
# f64: the LSE is stored in float32 for every dtype, so its rounding (half an
# ulp of |lse| <= 20, < 1e-6) is the bar
LSE_TOL = {"bf16": 2.0 ** -8 + 1e-4, "f16": 2.0 ** -11 + 1e-4, "f32": 2e-6, "f64": 1e-6}


def check_lse(got, ref, dtype, what):
    g = got.detach().to("cpu", torch.float64).numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    empty = ~np.isfinite(ref)
    assert np.all(np.isneginf(g[empty])), f"{what}: rows without keys must give -inf"
    assert np.all(np.isfinite(g[~empty])), f"{what}: non-finite lse on a row with keys"
    err = np.abs(g[~empty] - ref[~empty])
    bound = LSE_TOL[dtype] + 1e-5 * np.abs(ref[~empty])
    assert np.all(err <= bound), f"{what}: lse err {err.max(initial=0):.3g} (bound {LSE_TOL[dtype]:.3g})"


def run_lse_case(sdpa, dtype, B, Hq, Hkv, Sq, Sk, D, *, causal=False, wl=None, wr=None,
                 softcap=None, alibi=False, amp=1.0, seed=0):
    name = (f"attn_fwd_lse {dtype} B{B} H{Hq}/{Hkv} Sq{Sq} Sk{Sk} D{D} causal={causal} "
            f"win=({wl},{wr}) cap={softcap} alibi={alibi} seed={seed}")
    q, k, v = W.random_dense(dtype, B, Hq, Hkv, Sq, Sk, D, seed, amp)
    sl = torch.from_numpy(W.alibi_slopes(Hq)) if alibi else None
    dev = torch.device("cuda:0")
    args = (q.to(dev), k.to(dev), v.to(dev), None if sl is None else sl.to(dev))
    kw = dict(softmax_scale=float(np.float32(1.0 / math.sqrt(D))), causal=causal, window_left=wl, window_right=wr,
              softcap=softcap)
    announce(name)
    out, lse = sdpa.attn_fwd_lse(*args, **kw)
    plain = sdpa.attn_fwd(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, plain), f"{name}: out differs from attn_fwd"
    ref = oracle.sdpa_lse_f64(W.to_f64(q), W.to_f64(k), scale=kw["softmax_scale"], causal=causal,
                              window_left=wl, window_right=wr, softcap=softcap,
                              alibi=None if sl is None else W.to_f64(sl))
    check_lse(lse, ref, dtype, name)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64)])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_lse_parity(gpu_lib, dtype, D, case):
    B, Hq, Hkv, Sq, Sk, kw = SMALL[case]
    run_lse_case(gpu_lib, dtype, B, Hq, Hkv, Sq, Sk, D, seed=300 + case, **kw)


def test_lse_parity_d256(gpu_lib):
    B, Hq, Hkv, Sq, Sk, kw = KEY_SPLIT[7]
    run_lse_case(gpu_lib, "bf16", B, Hq, Hkv, Sq, Sk, 256, seed=1100, **kw)


@pytest.mark.parametrize("case", [2, 4, 7])
def test_lse_key_split_parity(gpu_lib, case):
    B, Hq, Hkv, Sq, Sk, kw = KEY_SPLIT[case]
    run_lse_case(gpu_lib, "bf16", B, Hq, Hkv, Sq, Sk, 128, seed=400 + case, **kw)


@pytest.mark.parametrize("case", [
    (1, 4, 2, 200, 250, 128, dict(causal=True)),
    (2, 2, 1, 150, 150, 64, dict(causal=True, wl=30, wr=0, softcap=8.0, alibi=True)),
    (1, 2, 2, 100, 70, 128, dict(causal=True)),          # Sq > Sk: rows 0..29 have no key
])
def test_lse_parity_f32(gpu_lib, case):
    B, Hq, Hkv, Sq, Sk, D, kw = case
    run_lse_case(gpu_lib, "f32", B, Hq, Hkv, Sq, Sk, D, seed=9, **kw)


@pytest.mark.parametrize("D", [32, 256])
def test_lse_parity_f64(gpu_lib, D):
    B, Hq, Hkv, Sq, Sk, kw = VALU_CASES[2]
    run_lse_case(gpu_lib, "f64", B, Hq, Hkv, Sq, Sk, D, seed=11, **kw)


# ------------------------------------------- a reference max raised every tile

RISING = [
    # (S, D, kwargs): S = Sq = Sk; 700 keys take the key split (two wave groups)
    (700, 128, dict(causal=True, softcap=1000.0, alibi=True)),
    (700, 128, dict(causal=True, alibi=True)),
    (700, 128, dict(softcap=1000.0)),
    (400, 128, dict(causal=True, softcap=1000.0, alibi=True)),
    (400, 64, dict(causal=True, alibi=True)),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(RISING)))
def test_rising_scores_rescale_every_tile(gpu_lib, dtype, case):
    """Scores that grow by about 32 log2 units per 64-key tile (q and k_j
    aligned along d = 0 with k_j[0] = j), so every tile raises the running
    max far past the rescale gap: the logits of every tile are re-based to the
    new reference inside the rescale branch (softcap / ALiBi), or the raw-score
    rescale runs every tile (neither).  Output and LSE against the oracle."""
    S, D, kw = RISING[case]
    kw = dict(kw)
    alibi = kw.pop("alibi", False)
    rng = np.random.default_rng(1500 + case)
    q = 0.1 * rng.standard_normal((1, 2, S, D), dtype=np.float32)
    k = 0.1 * rng.standard_normal((1, 1, S, D), dtype=np.float32)
    v = rng.standard_normal((1, 1, S, D), dtype=np.float32)
    q[..., 0] = 4.0
    k[0, 0, :, 0] = np.arange(S, dtype=np.float32)
    q, k, v = W.cast(q, dtype), W.cast(k, dtype), W.cast(v, dtype)
    sl = torch.from_numpy(W.alibi_slopes(2)) if alibi else None
    scale = float(np.float32(1.0 / math.sqrt(D)))
    name = f"rising scores {dtype} S{S} D{D} {kw} alibi={alibi}"
    announce(name)
    dev = torch.device("cuda:0")
    out, lse = gpu_lib.attn_fwd_lse(q.to(dev), k.to(dev), v.to(dev), None if sl is None else sl.to(dev),
                                    softmax_scale=scale, **kw)
    torch.cuda.synchronize()
    ref = oracle.sdpa_naive_f64(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale=scale,
                                alibi=None if sl is None else W.to_f64(sl), **kw)
    compare(out, ref, DT[dtype], name)
    ref_lse = oracle.sdpa_lse_f64(W.to_f64(q), W.to_f64(k), scale=scale,
                                  alibi=None if sl is None else W.to_f64(sl), **kw)
    check_lse(lse, ref_lse, dtype, name)
