"""Seeded random configurations of the forward entry points against the
float64 oracle: dtype, head dim, GQA ratio, ragged lengths (Sq above, below
and equal to Sk), causal, windows, softcap, ALiBi and the live prefix are
drawn per case, so that combinations the hand-written cases miss are covered.
Each case prints its configuration before its GPU step.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, compare
from test_fwd_gpu import DT, check_lse
from test_paged_prefill_gpu import gpu_run, make_case, oracle_run

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

HEAD_DIMS = {"bf16": (64, 128, 256), "f16": (64, 128, 256), "f32": (32, 64, 128, 256)}


def _opt(rng, p, draw):
    return draw() if rng.random() < p else None


def dense_config(seed):
    rng = np.random.default_rng(9000 + seed)
    dtype = ["bf16", "f16", "f32"][rng.integers(3)]
    D = int(rng.choice(HEAD_DIMS[dtype]))
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 3))
    Sk = int(rng.integers(1, 420))
    Sq = int(rng.choice([1, int(rng.integers(1, 300)), Sk]))
    causal = bool(rng.random() < 0.6)
    wl = _opt(rng, 0.35, lambda: int(rng.integers(0, 200)))
    wr = _opt(rng, 0.25, lambda: int(rng.integers(0, 60)))
    softcap = _opt(rng, 0.3, lambda: float(rng.choice([5.0, 20.0, 50.0])))
    alibi = bool(rng.random() < 0.3)
    k_len = _opt(rng, 0.3, lambda: int(rng.integers(0, Sk + 1)))
    amp = float(rng.choice([0.5, 1.0, 2.0]))
    return dict(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, causal=causal, wl=wl, wr=wr,
                softcap=softcap, alibi=alibi, k_len=k_len, amp=amp)


@pytest.mark.parametrize("seed", range(64))
def test_random_dense_forward(gpu_lib, seed):
    c = dense_config(seed)
    announce(f"random dense forward seed {seed}: {c}")
    q, k, v = W.random_dense(c["dtype"], c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Sk"], c["D"], 500 + seed,
                             c["amp"])
    sl = torch.from_numpy(W.alibi_slopes(c["Hq"])) if c["alibi"] else None
    scale = float(np.float32(1.0 / math.sqrt(c["D"])))
    kw = dict(softmax_scale=scale, causal=c["causal"], window_left=c["wl"], window_right=c["wr"],
              softcap=c["softcap"], k_len=c["k_len"])
    out, lse = gpu_lib.attn_fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV), None if sl is None else sl.to(DEV), **kw)
    torch.cuda.synchronize()
    okw = dict(scale=scale, causal=c["causal"], window_left=c["wl"], window_right=c["wr"],
               softcap=c["softcap"], k_len=c["k_len"], alibi=None if sl is None else W.to_f64(sl))
    ref = oracle.sdpa_naive_f64(W.to_f64(q), W.to_f64(k), W.to_f64(v), **okw)
    compare(out, ref, DT[c["dtype"]], f"seed {seed}", amp=c["amp"])
    ref_lse = oracle.sdpa_lse_f64(W.to_f64(q), W.to_f64(k), **okw)
    check_lse(lse, ref_lse, c["dtype"], f"seed {seed}")


@pytest.mark.parametrize("seed", range(32))
def test_random_paged_decode(gpu_lib, seed):
    rng = np.random.default_rng(9500 + seed)
    dtype = ["bf16", "f16"][rng.integers(2)]
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
    # batch and longest context together (B = 300: lengths ordered by a bitonic sort)
    B, hi = [(1, 1500), (3, 1500), (17, 300), (70, 300), (300, 40)][rng.integers(5)]
    bs = int(rng.choice([1, 5, 16, 32, 64, 128]))
    lens = rng.integers(0, hi + 1, size=B).astype(np.int32)
    max_blocks = max(1, (int(lens.max()) + bs - 1) // bs)
    splits = int(rng.integers(1, 17))
    softcap = _opt(rng, 0.3, lambda: float(rng.choice([10.0, 30.0])))
    alibi = bool(rng.random() < 0.3)
    w = W.Paged("random_decode", dtype, B, Hq, Hkv, D, bs, 0, hi, splits, max_blocks, softcap=softcap,
                alibi=alibi, seed=600 + seed)
    announce(f"random paged decode seed {seed}: {dtype} B{B} H{Hq}/{Hkv} D{D} bs{bs} max_len{hi} "
             f"splits{splits} cap={softcap} alibi={alibi}")
    q, kp, vp, table, sl, al = W.paged_inputs(w, seq_lens=lens)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    out = gpu_lib.attn_paged_decode(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), sl.to(DEV),
                                    None if al is None else al.to(DEV), softmax_scale=scale,
                                    softcap=softcap, num_splits=splits)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_f64(W.to_f64(q), W.to_f64(kp), W.to_f64(vp), table.numpy(), sl.numpy(),
                                  scale=scale, softcap=softcap, alibi=None if al is None else W.to_f64(al))
    compare(out, ref, DT[dtype], f"seed {seed}")


@pytest.mark.parametrize("seed", range(24))
def test_random_varlen_prefill(gpu_lib, seed):
    rng = np.random.default_rng(9800 + seed)
    dtype = ["bf16", "f16"][rng.integers(2)]
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    bs = int(rng.choice([64, 128, 192]))
    nseq = int(rng.integers(1, 5))
    sk = [int(x) for x in rng.integers(0, 700, size=nseq)]
    sq = [int(min(x, rng.integers(0, 300))) if rng.random() < 0.7 else int(rng.integers(0, 300)) for x in sk]
    kw = dict(causal=bool(rng.random() < 0.8),
              wl=_opt(rng, 0.3, lambda: int(rng.integers(0, 150))),
              wr=_opt(rng, 0.2, lambda: int(rng.integers(0, 40))),
              softcap=_opt(rng, 0.3, lambda: float(rng.choice([10.0, 30.0]))))
    if rng.random() < 0.3:
        kw["alibi"] = torch.from_numpy(W.alibi_slopes(Hq))
    kw["scale"] = float(np.float32(1.0 / math.sqrt(D)))
    announce(f"random varlen prefill seed {seed}: {dtype} H{Hq}/{Hkv} D{D} bs{bs} sq{sq} sk{sk} "
             f"{ {k: v for k, v in kw.items() if k != 'alibi'} } alibi={'alibi' in kw}")
    c = make_case(dtype, sq, sk, Hq, Hkv, D, bs, 700 + seed)
    out = gpu_run(gpu_lib, c, **kw)
    ref = oracle_run(c, **kw)
    compare(out, ref, DT[dtype], f"seed {seed}")


@pytest.mark.parametrize("seed", range(24))
def test_random_backward(gpu_lib, seed):
    """attn_bwd (or attn_bwd_lse from a saved forward) on random shapes and
    options: bf16/f16 on the matrix cores at the relative bars of the backward
    tests, f32/f64 on the vector ALU at theirs."""
    from test_bwd_gpu import compare_grad, compare_grad_valu
    c = dense_config(10_000 + seed)
    rng = np.random.default_rng(9900 + seed)
    c["dtype"] = ["bf16", "f16", "f32", "f64"][rng.integers(4)]
    c["D"] = int(rng.choice({"bf16": (64, 128, 256), "f16": (64, 128, 256), "f32": (32, 64, 128, 256),
                            "f64": (32, 64, 128)}[c["dtype"]]))
    c["amp"] = min(c["amp"], 1.0)
    c["Sq"], c["Sk"] = min(c["Sq"], 300), min(c["Sk"], 300)
    c["k_len"] = None
    saved = bool(rng.random() < 0.5)
    announce(f"random backward seed {seed} (saved forward: {saved}): {c}")
    q, k, v = W.random_dense(c["dtype"], c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Sk"], c["D"], 800 + seed,
                             c["amp"])
    do = W.random_dense(c["dtype"], c["B"], c["Hq"], c["Hkv"], c["Sq"], 1, c["D"], 850 + seed, 1.0)[0]
    sl = torch.from_numpy(W.alibi_slopes(c["Hq"])) if c["alibi"] else None
    scale = float(np.float32(1.0 / math.sqrt(c["D"])))
    kw = dict(softmax_scale=scale, causal=c["causal"], window_left=c["wl"], window_right=c["wr"],
              softcap=c["softcap"])
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    sld = None if sl is None else sl.to(DEV)
    if saved:
        out, lse = gpu_lib.attn_fwd_lse(qd, kd, vd, sld, **kw)
        grads = gpu_lib.attn_bwd_lse(qd, kd, vd, out, lse, dod, sld, **kw)
    else:
        grads = gpu_lib.attn_bwd(qd, kd, vd, dod, sld, **kw)
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward_f64(W.to_f64(q), W.to_f64(k), W.to_f64(v), W.to_f64(do), scale=scale,
                                   causal=c["causal"], window_left=c["wl"], window_right=c["wr"],
                                   softcap=c["softcap"], alibi=None if sl is None else W.to_f64(sl))
    for nm, got, r in zip(("dq", "dk", "dv"), grads, ref):
        if c["dtype"] in ("bf16", "f16"):
            compare_grad(got, r, c["dtype"], f"seed {seed} {nm}")
        else:
            compare_grad_valu(got, r, c["dtype"], f"seed {seed} {nm}")
