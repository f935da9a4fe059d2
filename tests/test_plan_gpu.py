"""The plan objects of the binding (arguments checked and marshalled once, one
C call per run) against the plain entry points and the oracle, including
runs after the tensors' contents changed in place."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, compare

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _decode_inputs(seed, lens, B=4, Hq=16, Hkv=4, D=128, bs=16, max_blocks=40):
    w = W.Paged("plan_decode", "bf16", B, Hq, Hkv, D, bs, 1, 1, 4, max_blocks, seed=seed)
    q, kp, vp, table, sl, _ = W.paged_inputs(w, seq_lens=lens)
    return w, q, kp, vp, table, sl


def test_paged_decode_plan_matches_entry_point_and_oracle(gpu_lib):
    lens = [300, 17, 640, 1]
    w, q, kp, vp, table, sl = _decode_inputs(31, lens)
    qd, kd, vd, td, ld = q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), sl.to(DEV)
    announce("PagedDecodePlan")
    plan = gpu_lib.PagedDecodePlan(qd, kd, vd, td, ld, num_splits=4)
    got = plan.run().clone()
    ref = gpu_lib.attn_paged_decode(qd, kd, vd, td, ld, num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    scale = float(np.float32(1.0 / math.sqrt(w.D)))
    exp = oracle.paged_decode_f64(W.to_f64(q), W.to_f64(kp), W.to_f64(vp), table.numpy(), sl.numpy(),
                                  scale=scale)
    compare(got, exp, torch.bfloat16, "PagedDecodePlan vs oracle")
    # the next step: a new query and shorter contexts, written in place
    q2 = W.random_dense("bf16", w.B, w.Hq, w.Hkv, 1, 1, w.D, 77)[0]
    qd.copy_(q2.to(DEV))
    sl2 = torch.tensor([299, 0, 513, 1], dtype=torch.int32)
    ld.copy_(sl2.to(DEV))
    got2 = plan.run()
    ref2 = gpu_lib.attn_paged_decode(qd, kd, vd, td, ld, num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(got2, ref2)
    exp2 = oracle.paged_decode_f64(W.to_f64(q2), W.to_f64(kp), W.to_f64(vp), table.numpy(), sl2.numpy(),
                                   scale=scale)
    compare(got2, exp2, torch.bfloat16, "PagedDecodePlan after in-place update vs oracle")
    assert plan.out is got2


def test_paged_decode_plan_fused_form(gpu_lib):
    # 512 (sequence, KV head) groups, one split each: the fused form
    lens = list(np.random.default_rng(5).integers(64, 600, size=64))
    w, q, kp, vp, table, sl = _decode_inputs(32, lens, B=64, Hq=32, Hkv=8, bs=64, max_blocks=10)
    args = [t.to(DEV) for t in (q, kp, vp, table, sl)]
    announce("PagedDecodePlan fused form")
    plan = gpu_lib.PagedDecodePlan(*args, num_splits=1)
    for _ in range(3):
        got = plan.run()
    ref = gpu_lib.attn_paged_decode(*args, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_fwd_plan_matches_entry_point(gpu_lib):
    q, k, v = (t.to(DEV) for t in W.random_dense("bf16", 1, 8, 2, 300, 500, 128, 41))
    announce("AttnFwdPlan")
    plan = gpu_lib.AttnFwdPlan(q, k, v, causal=True, window_left=100)
    got = plan.run().clone()
    ref = gpu_lib.attn_fwd(q, k, v, causal=True, window_left=100)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    q.mul_(-0.5)
    got2 = plan.run()
    ref2 = gpu_lib.attn_fwd(q, k, v, causal=True, window_left=100)
    torch.cuda.synchronize()
    assert torch.equal(got2, ref2)
    assert not torch.equal(got, got2)


def test_plans_reject_bad_arguments_when_built(gpu_lib):
    q, k, v = (t.to(DEV) for t in W.random_dense("bf16", 1, 4, 3, 8, 8, 128, 1))
    with pytest.raises(gpu_lib.AttnError):
        gpu_lib.AttnFwdPlan(q, k, v)  # Hq % Hkv != 0
    w, qp, kp, vp, table, sl = _decode_inputs(33, [5, 6, 7, 8])
    with pytest.raises(gpu_lib.AttnError):
        gpu_lib.PagedDecodePlan(qp.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), sl.to(DEV), num_splits=-1)
