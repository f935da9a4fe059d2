"""Parity of attn_bwd (HIP, through the C ABI) with the float64 oracle's
backward (kernel-contract page, attention_flash_backward).

Small cases span several 32/64/128-row tiles with ragged tails, rows without
keys, every mask kind, softcap and ALiBi, GQA; the full-size causal workload
is checked on sampled heads.  Inputs are rounded to the dtype first and the
oracle sees the rounded values.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}
DEV = torch.device("cuda:0")

# Bar for the gradients (the pages fix none): every gradient element is a sum
# of products one of whose factors -- P or dS -- enters the matrix cores
# rounded to the input dtype (unit roundoff u = 2^-8 for bf16, 2^-11 for f16),
# and the result is rounded once more to the dtype, so the tensor relative L2
# error is of the order of u.  Element-wise, cancellation in
# dS = P (dP - rowsum(P dP)) can make a small element's relative error large,
# so the element bar is taken relative to the largest element of the tensor.
# Measured over every gradient tensor of this file (bf16 and f16, head dims
# 64, 128 and 256, both entry points): relative L2 at most 0.80u, element
# error at most 1.53u of the largest element.  The bars, 1.25u and 2.5u, keep
# about 1.6x of margin over that, so a regression of 2x fails.
U = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
REL_BAR, EL_BAR = 1.25, 2.5


def compare_grad(got, ref, dtype, what):
    g = got.detach().to("cpu", torch.float64).numpy()
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    err = np.abs(g - ref)
    scale = np.abs(ref).max(initial=0.0)
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(g - ref) / nref if nref > 0 else np.linalg.norm(g)
    announce(f"{what}: rel L2 {rel:.3g}, max err {err.max(initial=0):.3g} of max |ref| {scale:.3g}")
    assert rel <= REL_BAR * U[dtype], f"{what}: relative L2 {rel:.3g} > {REL_BAR * U[dtype]:.3g}"
    assert err.max(initial=0.0) <= EL_BAR * U[dtype] * scale + 1e-6, \
        f"{what}: max err {err.max():.3g} > {EL_BAR * U[dtype]:.3g} * {scale:.3g}"


def run_bwd(sdpa, dtype, B, Hq, Hkv, Sq, Sk, D, *, causal=False, wl=None, wr=None, softcap=None,
            alibi=False, amp=1.0, seed=0, scale=None):
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    name = (f"attn_bwd {dtype} B{B} H{Hq}/{Hkv} Sq{Sq} Sk{Sk} D{D} causal={causal} "
            f"win=({wl},{wr}) cap={softcap} alibi={alibi} scale={scale} seed={seed}")
    q, k, v = W.random_dense(dtype, B, Hq, Hkv, Sq, Sk, D, seed, amp)
    do = W.random_dense(dtype, B, Hq, Hkv, Sq, 1, D, seed + 7919, 1.0)[0]
    sl = torch.from_numpy(W.alibi_slopes(Hq)) if alibi else None
    announce(name)
    dq, dk, dv = sdpa.attn_bwd(q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV),
                               None if sl is None else sl.to(DEV), softmax_scale=scale,
                               causal=causal, window_left=wl, window_right=wr, softcap=softcap)
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward_f64(W.to_f64(q), W.to_f64(k), W.to_f64(v), W.to_f64(do),
                                   scale=scale, causal=causal, window_left=wl, window_right=wr,
                                   softcap=softcap, alibi=None if sl is None else W.to_f64(sl))
    for nm, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        compare_grad(got, r, dtype, f"{name} {nm}")
    return (q, k, v, do, sl, scale), (dq, dk, dv)


CASES = [
    # (B, Hq, Hkv, Sq, Sk, kwargs)
    (1, 2, 2, 128, 128, dict()),                                   # aligned: no mask code
    (1, 4, 2, 200, 333, dict(causal=True)),
    (2, 4, 1, 300, 250, dict(causal=True)),                        # Sq > Sk: rows 0..49 empty
    (1, 2, 2, 190, 190, dict(softcap=5.0, amp=2.0)),
    (1, 4, 4, 257, 300, dict(causal=True, wl=64, wr=0, alibi=True)),
    (1, 8, 2, 130, 400, dict(wl=30, wr=20, softcap=20.0, alibi=True, amp=1.5)),
    (1, 2, 1, 64, 1000, dict()),
    (1, 2, 2, 700, 64, dict(causal=True)),
]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64)])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_bwd_parity(gpu_lib, dtype, D, case):
    B, Hq, Hkv, Sq, Sk, kw = CASES[case]
    run_bwd(gpu_lib, dtype, B, Hq, Hkv, Sq, Sk, D, seed=700 + case, **kw)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f16", 128)])
@pytest.mark.parametrize("case", [1, 4, 5])
def test_bwd_parity_other_dims(gpu_lib, dtype, D, case):
    B, Hq, Hkv, Sq, Sk, kw = CASES[case]
    run_bwd(gpu_lib, dtype, B, Hq, Hkv, Sq, Sk, D, seed=800 + case, **kw)


# Head dim 256: every dK/dV key block is covered by two workgroups, one per
# half of the head dimension; the last case has enough query tiles per key
# block to split them into chunks (float32 partials + their reduction).
D256_CASES = [0, 1, 2, 4, 5]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", D256_CASES)
def test_bwd_parity_d256(gpu_lib, dtype, case):
    B, Hq, Hkv, Sq, Sk, kw = CASES[case]
    run_bwd(gpu_lib, dtype, B, Hq, Hkv, Sq, Sk, 256, seed=850 + case, **kw)


def test_bwd_d256_chunked_key_blocks(gpu_lib):
    run_bwd(gpu_lib, "bf16", 1, 8, 2, 600, 300, 256, causal=True, seed=860)


def test_bwd_scale_zero_under_masks(gpu_lib):
    """softmax_scale = 0: uniform weights over each row's admissible keys, so
    dV averages dO and dQ = dK = 0; the masks must still apply (the exponent
    is formed before the mask)."""
    run_bwd(gpu_lib, "bf16", 1, 4, 2, 70, 90, 128, causal=True, wl=20, scale=0.0, seed=870)
    run_bwd(gpu_lib, "f16", 1, 2, 1, 33, 50, 64, causal=True, scale=0.0, seed=871)


@pytest.mark.parametrize("Sk", [2, 5, 16, 17, 37])
def test_bwd_key_counts_around_a_wave(gpu_lib, Sk):
    """Key counts below, at and just past the 16 keys a dK/dV wave owns (the
    other waves of the workgroup have no keys).  (Not a single key: there
    dS = P (dP - dO . O) is exactly 0 for every row, and the gradients' float32
    rounding residue has no nonzero reference to be measured against.)"""
    run_bwd(gpu_lib, "bf16", 1, 4, 2, 40, Sk, 128, causal=True, seed=880 + Sk)
    run_bwd(gpu_lib, "f16", 2, 2, 2, 24, Sk, 64, seed=890 + Sk)


def test_bwd_deterministic(gpu_lib):
    (q, k, v, do, sl, scale), first = run_bwd(gpu_lib, "bf16", 1, 4, 2, 200, 333, 128,
                                              causal=True, seed=900)
    again = gpu_lib.attn_bwd(q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), None,
                             softmax_scale=scale, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(first, again):
        assert torch.equal(a, b)


def test_bwd_no_queries_or_keys(gpu_lib):
    """Sq = 0: dk = dv = 0.  Sk = 0: dq = 0."""
    q, k, v = W.random_dense("bf16", 1, 2, 2, 0, 70, 64, 3, 1.0)
    do = torch.empty_like(q)
    announce("attn_bwd Sq=0")
    dk0 = torch.full_like(k, 7.0).to(DEV)
    dv0 = torch.full_like(v, 7.0).to(DEV)
    _, dk, dv = gpu_lib.attn_bwd(q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), None,
                                 dk=dk0, dv=dv0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0
    q, k, v = W.random_dense("bf16", 1, 2, 2, 90, 0, 64, 4, 1.0)
    do = torch.ones_like(q)
    announce("attn_bwd Sk=0")
    dq0 = torch.full_like(q, 7.0).to(DEV)
    dq, _, _ = gpu_lib.attn_bwd(q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), None, dq=dq0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dq).item() == 0


def test_bwd_gqa_causal_2k_workload(gpu_lib):
    """The 2048-token causal GQA workload (2 x 32 query heads over 8 KV heads,
    D = 128): dQ of two query heads and dK/dV of one KV head (its whole group
    of 4 query heads) against the oracle."""
    w = W.GQA_CAUSAL_2K
    q, k, v, _ = W.dense_inputs(w)
    do = W.random_dense(w.dtype, w.B, w.Hq, w.Hkv, w.Sq, 1, w.D, 4242, 1.0)[0]
    announce(f"attn_bwd {w.name}")
    dq, dk, dv = gpu_lib.attn_bwd(q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), None,
                                  softmax_scale=w.scale, causal=True)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    for b, g in ((1, 5),):
        hs = slice(g * G, (g + 1) * G)
        ref = oracle.sdpa_backward_f64(W.to_f64(q[b:b + 1, hs]), W.to_f64(k[b:b + 1, g:g + 1]),
                                       W.to_f64(v[b:b + 1, g:g + 1]), W.to_f64(do[b:b + 1, hs]),
                                       scale=w.scale, causal=True)
        compare_grad(dq[b:b + 1, hs], ref[0], w.dtype, f"{w.name} dq b{b} heads {hs}")
        compare_grad(dk[b:b + 1, g:g + 1], ref[1], w.dtype, f"{w.name} dk b{b} kv {g}")
        compare_grad(dv[b:b + 1, g:g + 1], ref[2], w.dtype, f"{w.name} dv b{b} kv {g}")


def run_bwd_lse(sdpa, dtype, B, Hq, Hkv, Sq, Sk, D, *, causal=False, wl=None, wr=None, softcap=None,
                alibi=False, amp=1.0, seed=0):
    """attn_bwd_lse from attn_fwd_lse's saved output and LSE, against the oracle."""
    name = (f"attn_bwd_lse {dtype} B{B} H{Hq}/{Hkv} Sq{Sq} Sk{Sk} D{D} causal={causal} "
            f"win=({wl},{wr}) cap={softcap} alibi={alibi} seed={seed}")
    q, k, v = W.random_dense(dtype, B, Hq, Hkv, Sq, Sk, D, seed, amp)
    do = W.random_dense(dtype, B, Hq, Hkv, Sq, 1, D, seed + 7919, 1.0)[0]
    sl = torch.from_numpy(W.alibi_slopes(Hq)) if alibi else None
    scale = float(np.float32(1.0 / math.sqrt(D)))
    announce(name)
    kw = dict(softmax_scale=scale, causal=causal, window_left=wl, window_right=wr, softcap=softcap)
    dsl = None if sl is None else sl.to(DEV)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    out, lse = gpu_fwd_lse(sdpa, qd, kd, vd, dsl, kw)
    dq, dk, dv = sdpa.attn_bwd_lse(qd, kd, vd, out, lse, dod, dsl, **kw)
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward_f64(W.to_f64(q), W.to_f64(k), W.to_f64(v), W.to_f64(do),
                                   scale=scale, causal=causal, window_left=wl, window_right=wr,
                                   softcap=softcap, alibi=None if sl is None else W.to_f64(sl))
    for nm, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        compare_grad(got, r, dtype, f"{name} {nm}")
    return (qd, kd, vd, out, lse, dod, dsl, kw), (dq, dk, dv)


def gpu_fwd_lse(sdpa, q, k, v, alibi, kw):
    return sdpa.attn_fwd_lse(q, k, v, alibi, **kw)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64)])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_bwd_lse_parity(gpu_lib, dtype, D, case):
    B, Hq, Hkv, Sq, Sk, kw = CASES[case]
    run_bwd_lse(gpu_lib, dtype, B, Hq, Hkv, Sq, Sk, D, seed=1700 + case, **kw)


@pytest.mark.parametrize("dtype,case", [("bf16", 1), ("f16", 5), ("bf16", 2)])
def test_bwd_lse_parity_d256(gpu_lib, dtype, case):
    B, Hq, Hkv, Sq, Sk, kw = CASES[case]
    run_bwd_lse(gpu_lib, dtype, B, Hq, Hkv, Sq, Sk, 256, seed=1750 + case, **kw)


def test_bwd_lse_deterministic_and_close_to_recompute(gpu_lib):
    """Reruns are bitwise equal; the gradients from the saved forward agree
    with attn_bwd's (recomputed statistics) to a few units of rounding."""
    args, first = run_bwd_lse(gpu_lib, "bf16", 1, 4, 2, 200, 333, 128, causal=True, seed=1900)
    qd, kd, vd, out, lse, dod, dsl, kw = args
    again = gpu_lib.attn_bwd_lse(qd, kd, vd, out, lse, dod, dsl, **kw)
    rec = gpu_lib.attn_bwd(qd, kd, vd, dod, dsl, **kw)
    torch.cuda.synchronize()
    for a, b, r in zip(first, again, rec):
        assert torch.equal(a, b)
        rf = r.double().cpu().numpy()
        compare_grad(a, rf, "bf16", "attn_bwd_lse vs attn_bwd")


def test_bwd_lse_no_queries_or_keys(gpu_lib):
    """Sq = 0: dk = dv = 0 (out and lse may be empty).  Sk = 0: dq = 0, every
    row's LSE is -inf."""
    q, k, v = W.random_dense("bf16", 1, 2, 2, 0, 70, 64, 3, 1.0)
    announce("attn_bwd_lse Sq=0")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = gpu_lib.attn_fwd_lse(qd, kd, vd, None)
    dk0 = torch.full_like(kd, 7.0)
    dv0 = torch.full_like(vd, 7.0)
    _, dk, dv = gpu_lib.attn_bwd_lse(qd, kd, vd, out, lse, torch.empty_like(qd), None, dk=dk0, dv=dv0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0
    q, k, v = W.random_dense("bf16", 1, 2, 2, 90, 0, 64, 4, 1.0)
    announce("attn_bwd_lse Sk=0")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = gpu_lib.attn_fwd_lse(qd, kd, vd, None)
    torch.cuda.synchronize()
    assert torch.isinf(lse).all() and (lse < 0).all()
    dq0 = torch.full_like(qd, 7.0)
    dq, _, _ = gpu_lib.attn_bwd_lse(qd, kd, vd, out, lse, torch.ones_like(qd), None, dq=dq0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dq).item() == 0


def test_bwd_lse_gqa_causal_2k_workload(gpu_lib):
    """The 2048-token causal GQA workload from its saved forward: dQ of one
    group of query heads and dK/dV of their KV head against the oracle."""
    w = W.GQA_CAUSAL_2K
    q, k, v, _ = W.dense_inputs(w)
    do = W.random_dense(w.dtype, w.B, w.Hq, w.Hkv, w.Sq, 1, w.D, 4243, 1.0)[0]
    announce(f"attn_bwd_lse {w.name}")
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    out, lse = gpu_lib.attn_fwd_lse(qd, kd, vd, None, softmax_scale=w.scale, causal=True)
    dq, dk, dv = gpu_lib.attn_bwd_lse(qd, kd, vd, out, lse, dod, None, softmax_scale=w.scale,
                                      causal=True)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    b, g = 0, 3
    hs = slice(g * G, (g + 1) * G)
    ref = oracle.sdpa_backward_f64(W.to_f64(q[b:b + 1, hs]), W.to_f64(k[b:b + 1, g:g + 1]),
                                   W.to_f64(v[b:b + 1, g:g + 1]), W.to_f64(do[b:b + 1, hs]),
                                   scale=w.scale, causal=True)
    compare_grad(dq[b:b + 1, hs], ref[0], w.dtype, f"{w.name} dq b{b} heads {hs}")
    compare_grad(dk[b:b + 1, g:g + 1], ref[1], w.dtype, f"{w.name} dk b{b} kv {g}")
    compare_grad(dv[b:b + 1, g:g + 1], ref[2], w.dtype, f"{w.name} dv b{b} kv {g}")


# F32 / F64: the vector-ALU backward, computing in the element type throughout.
# Bar: each gradient element is a sum of up to Sk (or group * Sq) products
# formed and accumulated in the element type, so its error is a modest multiple
# of that type's unit roundoff times the magnitudes involved: tensor rel-L2 at
# most 1e-5 (f32) / 1e-12 (f64), and every element within 1e-4 / 1e-10 of the
# tensor's largest element.
VALU_BAR = {"f32": (1e-5, 1e-4), "f64": (1e-12, 1e-10)}


def compare_grad_valu(got, ref, dtype, what):
    g = got.detach().to("cpu", torch.float64).numpy()
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    rel_bar, el_bar = VALU_BAR[dtype]
    err = np.abs(g - ref)
    scale = np.abs(ref).max(initial=0.0)
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(g - ref) / nref if nref > 0 else np.linalg.norm(g)
    announce(f"{what}: rel L2 {rel:.3g}, max err {err.max(initial=0):.3g} of max |ref| {scale:.3g}")
    assert rel <= rel_bar, f"{what}: relative L2 {rel:.3g} > {rel_bar}"
    assert err.max(initial=0.0) <= el_bar * scale + 1e-300, f"{what}: max err {err.max():.3g}"


@pytest.mark.parametrize("dtype,D", [("f32", 128), ("f64", 64), ("f32", 32), ("f64", 256)])
@pytest.mark.parametrize("case", [0, 1, 2, 3, 4, 5])
def test_bwd_valu_parity(gpu_lib, dtype, D, case):
    B, Hq, Hkv, Sq, Sk, kw = CASES[case]
    kw = dict(kw)
    q, k, v = W.random_dense(dtype, B, Hq, Hkv, Sq, Sk, D, 2700 + case, kw.pop("amp", 1.0))
    do = W.random_dense(dtype, B, Hq, Hkv, Sq, 1, D, 2800 + case, 1.0)[0]
    sl = torch.from_numpy(W.alibi_slopes(Hq)) if kw.pop("alibi", False) else None
    scale = float(np.float32(1.0 / math.sqrt(D)))
    opts = dict(causal=kw.get("causal", False), window_left=kw.get("wl"),
                window_right=kw.get("wr"), softcap=kw.get("softcap"))
    name = f"attn_bwd {dtype} D{D} case {case} {CASES[case]}"
    announce(name)
    dq, dk, dv = gpu_lib.attn_bwd(q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV),
                                  None if sl is None else sl.to(DEV), softmax_scale=scale, **opts)
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward_f64(W.to_f64(q), W.to_f64(k), W.to_f64(v), W.to_f64(do), scale=scale,
                                   causal=opts["causal"], window_left=opts["window_left"],
                                   window_right=opts["window_right"], softcap=opts["softcap"],
                                   alibi=None if sl is None else W.to_f64(sl))
    for nm, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        compare_grad_valu(got, r, dtype, f"{name} {nm}")


def test_bwd_valu_deterministic_and_saved_forward(gpu_lib):
    """F64: reruns are bitwise equal, and attn_bwd_lse (whose saved output and
    LSE the vector-ALU path does not need) gives the same gradients."""
    q, k, v = W.random_dense("f64", 1, 4, 2, 90, 130, 64, 2900, 1.0)
    do = W.random_dense("f64", 1, 4, 2, 90, 1, 64, 2901, 1.0)[0]
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    announce("attn_bwd f64 determinism")
    a = gpu_lib.attn_bwd(qd, kd, vd, dod, None, causal=True)
    b = gpu_lib.attn_bwd(qd, kd, vd, dod, None, causal=True)
    out, lse = gpu_lib.attn_fwd_lse(qd, kd, vd, None, causal=True)
    c = gpu_lib.attn_bwd_lse(qd, kd, vd, out, lse, dod, None, causal=True)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)
