"""Parity of the dense forward's live key prefix (``k_len``) with the oracle.

The key and value tensors have a capacity of ``Sk`` rows per head; only the
first ``k_len`` are live.  The rows after the prefix hold NaN, so a kernel that
read one would poison its output.  Each case checks the output (and the
log-sum-exp) against the float64 oracle, and that the call equals, bit for
bit, the same call on K and V cut to the prefix.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, compare
from test_fwd_gpu import DT, check_lse

pytestmark = pytest.mark.gpu

CASES = [
    # (dtype, B, Hq, Hkv, Sq, Sk capacity, k_len, D, kwargs)
    ("bf16", 1, 4, 2, 1, 300, 0, 128, dict(causal=True)),          # no live key: zero rows
    ("bf16", 1, 4, 2, 1, 300, 1, 128, dict(causal=True)),
    ("bf16", 2, 4, 2, 1, 512, 300, 128, dict(causal=True)),        # decode step over a cache
    ("bf16", 1, 4, 1, 64, 300, 63, 128, dict(causal=True)),        # Sq > k_len: empty rows
    ("bf16", 1, 4, 1, 100, 300, 64, 64, dict(causal=True)),
    ("bf16", 2, 4, 2, 100, 333, 200, 128,
     dict(causal=True, wl=50, wr=0, softcap=20.0, alibi=True, amp=1.5)),
    ("bf16", 1, 2, 2, 130, 260, 260, 128, dict()),                 # k_len = Sk
    ("bf16", 1, 8, 2, 200, 1100, 1024, 128, dict(causal=True)),    # key-split path
    ("bf16", 1, 2, 1, 70, 400, 333, 256, dict(causal=True, wl=100)),
    ("f16", 1, 4, 2, 90, 300, 150, 128, dict(causal=True, alibi=True)),
    ("f16", 1, 2, 2, 1, 700, 640, 64, dict()),
    ("f32", 1, 4, 2, 50, 200, 120, 64, dict(causal=True, softcap=5.0, amp=2.0)),
    ("f32", 1, 2, 1, 40, 100, 0, 128, dict()),
    ("f64", 1, 2, 1, 33, 80, 45, 32, dict(causal=True, wl=9)),
    ("f64", 1, 2, 2, 20, 90, 90, 128, dict(alibi=True)),
]


def _case_inputs(dtype, B, Hq, Hkv, Sq, Sk, k_len, D, kw, seed):
    q, k, v = W.random_dense(dtype, B, Hq, Hkv, Sq, Sk, D, seed, kw.get("amp", 1.0))
    k[:, :, k_len:] = float("nan")
    v[:, :, k_len:] = float("nan")
    sl = torch.from_numpy(W.alibi_slopes(Hq)) if kw.get("alibi") else None
    return q, k, v, sl


@pytest.mark.parametrize("case", range(len(CASES)))
def test_live_prefix_matches_oracle(gpu_lib, case):
    dtype, B, Hq, Hkv, Sq, Sk, k_len, D, kw = CASES[case]
    name = f"attn_fwd k_len={k_len} {dtype} B{B} H{Hq}/{Hkv} Sq{Sq} Sk{Sk} D{D} {kw}"
    q, k, v, sl = _case_inputs(dtype, B, Hq, Hkv, Sq, Sk, k_len, D, kw, seed=100 + case)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    args = dict(softmax_scale=scale, causal=kw.get("causal", False), window_left=kw.get("wl"),
                window_right=kw.get("wr"), softcap=kw.get("softcap"))
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    sld = None if sl is None else sl.to(dev)
    announce(name)
    out, lse = gpu_lib.attn_fwd_lse(qd, kd, vd, sld, k_len=k_len, **args)
    plain = gpu_lib.attn_fwd(qd, kd, vd, sld, k_len=k_len, **args)
    cut = gpu_lib.attn_fwd(qd, kd[:, :, :k_len].contiguous(), vd[:, :, :k_len].contiguous(), sld, **args)
    torch.cuda.synchronize()
    okw = dict(scale=scale, causal=args["causal"], window_left=args["window_left"],
               window_right=args["window_right"], softcap=args["softcap"], k_len=k_len)
    al = None if sl is None else W.to_f64(sl)
    ref = oracle.sdpa_naive_f64(W.to_f64(q), W.to_f64(k), W.to_f64(v), alibi=al, **okw)
    compare(out, ref, DT[dtype], name)
    assert torch.equal(out, plain), f"{name}: attn_fwd_lse and attn_fwd outputs differ"
    assert torch.equal(out, cut), f"{name}: differs from the call on the cut tensors"
    ref_lse = oracle.sdpa_lse_f64(W.to_f64(q), W.to_f64(k), alibi=al, **okw)
    check_lse(lse, ref_lse, dtype, name)


def test_live_prefix_rejected_out_of_range(gpu_lib):
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.random_dense("bf16", 1, 2, 2, 4, 10, 128, 1))
    for bad in (-1, 11):
        with pytest.raises(gpu_lib.AttnError) as e:
            gpu_lib.attn_fwd(q, k, v, k_len=bad)
        assert e.value.status == 6  # ATTN_ERR_PARAM
