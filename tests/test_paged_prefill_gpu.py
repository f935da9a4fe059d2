"""Parity of attn_paged_prefill (HIP, through the C ABI) with the float64
oracle's paged_prefill_varlen_f64: packed queries with a cu_seqlens_q prefix
sum, per-sequence key lengths, K/V gathered from a randomly permuted pool."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, compare

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32, "f64": torch.float64}


def cast(x, dtype):
    """float32 draws in the test dtype (float64: the exact float32 values)."""
    return W.cast(x, "f32").double() if dtype == "f64" else W.cast(x, dtype)
DEV = torch.device("cuda:0")


def make_case(dtype, sq, sk, Hq, Hkv, D, bs, seed, amp=1.0):
    """Packed q, pools and tables for query lengths `sq` and key lengths `sk`."""
    rng = np.random.default_rng(seed)
    nblk = [(c + bs - 1) // bs for c in sk]
    nb = max(sum(nblk), 1)
    perm = rng.permutation(nb)
    maxb = max(max(nblk), 1)
    table = np.full((len(sk), maxb), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    cu = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    tq = int(cu[-1])
    q = cast(rng.standard_normal((tq, Hq, D), dtype=np.float32) * np.float32(amp), dtype)
    kp = cast(rng.standard_normal((nb, bs, Hkv, D), dtype=np.float32) * np.float32(amp), dtype)
    vp = cast(rng.standard_normal((nb, bs, Hkv, D), dtype=np.float32), dtype)
    return dict(q=q, kp=kp, vp=vp, table=torch.from_numpy(table),
                lens=torch.from_numpy(np.asarray(sk, dtype=np.int32)), cu=torch.from_numpy(cu))


def gpu_run(sdpa, c, out=None, err=None, **kw):
    o = sdpa.attn_paged_prefill(c["q"].to(DEV), c["kp"].to(DEV), c["vp"].to(DEV), c["table"].to(DEV),
                                c["lens"].to(DEV), c["cu"].to(DEV),
                                None if kw.get("alibi") is None else kw["alibi"].to(DEV), out,
                                max_seqlen_q=kw.get("max_sq"), softmax_scale=kw["scale"],
                                causal=kw.get("causal", True), window_left=kw.get("wl"),
                                window_right=kw.get("wr"), softcap=kw.get("softcap"),
                                error_flag=err)
    torch.cuda.synchronize()
    return o


def oracle_run(c, **kw):
    return oracle.paged_prefill_varlen_f64(
        W.to_f64(c["q"]), W.to_f64(c["kp"]), W.to_f64(c["vp"]), c["table"].numpy(), c["lens"].numpy(),
        c["cu"].numpy(), scale=kw["scale"], causal=kw.get("causal", True), window_left=kw.get("wl"),
        window_right=kw.get("wr"), softcap=kw.get("softcap"),
        alibi=None if kw.get("alibi") is None else W.to_f64(kw["alibi"]))


CASES = [
    # (sq per sequence, sk per sequence, Hq, Hkv, bs, kwargs)
    ((300, 1, 129, 0, 64), (300, 700, 1000, 50, 64), 8, 2, 64, dict()),
    ((200, 77), (1500, 77), 4, 1, 128, dict()),
    ((128, 300), (100, 90), 4, 4, 64, dict()),                                 # Sk < Sq: early rows empty
    ((250, 40, 400), (900, 41, 401), 8, 2, 64, dict(wl=100, wr=0)),
    ((180, 33), (600, 200), 4, 2, 192, dict(softcap=30.0, alibi=True, amp=1.5)),
    ((64, 190), (64, 700), 2, 1, 64, dict(causal=False, wl=20, wr=5)),
]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64), ("bf16", 256)])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_paged_prefill_parity(gpu_lib, dtype, D, case):
    sq, sk, Hq, Hkv, bs, kw = CASES[case]
    kw = dict(kw)
    amp = kw.pop("amp", 1.0)
    c = make_case(dtype, sq, sk, Hq, Hkv, D, bs, 500 + case, amp)
    kw["scale"] = 1.0 / math.sqrt(D)
    if kw.pop("alibi", False):
        kw["alibi"] = torch.from_numpy(W.alibi_slopes(Hq))
    name = f"attn_paged_prefill {dtype} D{D} sq={sq} sk={sk} H{Hq}/{Hkv} bs{bs} {sorted(kw)}"
    announce(name)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = gpu_run(gpu_lib, c, err=err, **kw)
    assert err.item() == 0, f"{name}: error flag set"
    compare(got, oracle_run(c, **kw), DT[dtype], name)


def test_rows_outside_sequences_untouched(gpu_lib):
    c = make_case("bf16", (100, 50), (300, 60), 4, 2, 128, 64, 11)
    total = c["q"].shape[0]
    cu = c["cu"].clone()
    cu[2] = 120                                  # rows 120..149 belong to no sequence
    c["cu"] = cu
    out = torch.full((total, 4, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    announce("attn_paged_prefill: rows outside every sequence")
    gpu_run(gpu_lib, c, out=out, scale=0.088, max_sq=100)
    assert torch.all(out[120:] == 3.0)
    ref = oracle_run(c, scale=0.088)
    compare(out[:120], ref[:120], torch.bfloat16, "rows inside the sequences")


def test_equals_dense_prefill_bitwise(gpu_lib):
    """Same data as a dense [B, H, S, D] problem, laid out in a permuted pool:
    the paged kernel runs the same tiles in the same order, so it must return
    exactly what attn_fwd returns."""
    B, Hq, Hkv, Sq, Sk, D, bs = 2, 8, 2, 300, 512, 128, 64
    q, k, v = W.random_dense("bf16", B, Hq, Hkv, Sq, Sk, D, 21, 1.0)
    rng = np.random.default_rng(22)
    per = Sk // bs
    perm = rng.permutation(B * per)
    table = torch.from_numpy(perm.reshape(B, per).astype(np.int32))
    kp = torch.empty(B * per, bs, Hkv, D, dtype=q.dtype)
    vp = torch.empty_like(kp)
    for b in range(B):
        for n in range(per):
            kp[perm[b * per + n]] = k[b, :, n * bs:(n + 1) * bs].permute(1, 0, 2)
            vp[perm[b * per + n]] = v[b, :, n * bs:(n + 1) * bs].permute(1, 0, 2)
    qp = q.permute(0, 2, 1, 3).reshape(B * Sq, Hq, D).contiguous()
    c = dict(q=qp, kp=kp, vp=vp, table=table, lens=torch.full((B,), Sk, dtype=torch.int32),
             cu=torch.tensor([0, Sq, 2 * Sq], dtype=torch.int32))
    announce("attn_paged_prefill vs attn_fwd, bitwise")
    for kw in (dict(causal=True), dict(causal=True, wl=77, wr=0, softcap=20.0, alibi=True)):
        al = torch.from_numpy(W.alibi_slopes(Hq)) if kw.pop("alibi", False) else None
        got = gpu_run(gpu_lib, c, scale=0.088, alibi=al, **kw)
        dense = gpu_lib.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), None if al is None else al.to(DEV),
                                 softmax_scale=0.088, causal=True, window_left=kw.get("wl"),
                                 window_right=kw.get("wr"), softcap=kw.get("softcap"))
        torch.cuda.synchronize()
        assert torch.equal(got.reshape(B, Sq, Hq, D).permute(0, 2, 1, 3), dense), kw


def test_one_hot_paging_bit_exact(gpu_lib):
    """q = 1024 e0 in every row; k = 8 e0 only at logical token t*: its score
    (~724) makes every other weight underflow to exactly 0, so each row that
    may see t* returns V[t*] bit for bit -- whatever page t* sits in."""
    Hq, Hkv, D, bs = 4, 2, 128, 64
    sk = (700, 300)
    sq = (200, 100)
    c = make_case("bf16", sq, sk, Hq, Hkv, D, bs, 31)
    c["q"] = torch.zeros_like(c["q"])
    c["q"][..., 0] = 1024.0
    rng = np.random.default_rng(32)
    for ts in (0, 63, 64, 450, 699):
        kp = torch.zeros_like(c["kp"])
        tb = c["table"].numpy()
        kp[tb[0, ts // bs], ts % bs, :, 0] = 8.0
        for t2 in rng.integers(0, sk[1], size=1):   # sequence 1 gets its own t*
            kp[tb[1, t2 // bs], t2 % bs, :, 0] = 8.0
        cc = dict(c, kp=kp)
        announce(f"one-hot paging t*={ts}")
        got = gpu_run(gpu_lib, cc, scale=0.088).cpu()
        vrow = c["vp"][tb[0, ts // bs], ts % bs]           # [Hkv, D]
        ip0 = sk[0] - sq[0]
        for i in range(sq[0]):
            if ip0 + i >= ts:
                for h in range(Hq):
                    assert torch.equal(got[i, h], vrow[h // (Hq // Hkv)]), (ts, i, h)


def test_error_flag_and_masking(gpu_lib):
    c = make_case("bf16", (100, 100), (300, 300), 4, 2, 128, 64, 41)
    good = oracle_run(c, scale=0.088)
    # a table entry outside the pool in sequence 0: flagged, finite output,
    # sequence 1 unaffected
    t2 = c["table"].clone()
    t2[0, 1] = 10 ** 6
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    announce("attn_paged_prefill: bad block id")
    got = gpu_run(gpu_lib, dict(c, table=t2), err=err, scale=0.088)
    assert err.item() == 1
    assert torch.all(torch.isfinite(got.float()))
    compare(got[100:], good[100:], torch.bfloat16, "sequence without the bad block")
    # a key length beyond the table: clamped and flagged
    l2 = c["lens"].clone()
    l2[1] = 10 ** 6
    err.zero_()
    got = gpu_run(gpu_lib, dict(c, lens=l2), err=err, scale=0.088)
    assert err.item() == 1 and torch.all(torch.isfinite(got.float()))
    # a query length above max_seqlen_q: clamped and flagged
    err.zero_()
    gpu_run(gpu_lib, c, err=err, scale=0.088, max_sq=50)
    assert err.item() == 1


# F32 / F64: the vector-ALU paged kernel (any block size, head dims 32 to 256)
VALU_CASES = [
    # (sq per sequence, sk per sequence, Hq, Hkv, bs, kwargs)
    ((70, 1, 33, 0), (70, 200, 120, 30), 4, 2, 16, dict()),
    ((50, 20), (300, 20), 4, 1, 7, dict(wl=40, wr=0)),
    ((40, 61), (20, 90), 2, 2, 64, dict(softcap=30.0, alibi=True, amp=1.5)),   # Sk < Sq: early rows empty
    ((33, 45), (33, 100), 2, 1, 5, dict(causal=False, wl=10, wr=3)),
]


@pytest.mark.parametrize("dtype,D", [("f32", 128), ("f64", 64), ("f32", 32), ("f64", 256)])
@pytest.mark.parametrize("case", range(len(VALU_CASES)))
def test_paged_prefill_valu_parity(gpu_lib, dtype, D, case):
    sq, sk, Hq, Hkv, bs, kw = VALU_CASES[case]
    kw = dict(kw)
    amp = kw.pop("amp", 1.0)
    c = make_case(dtype, sq, sk, Hq, Hkv, D, bs, 540 + case, amp)
    kw["scale"] = float(np.float32(1.0 / math.sqrt(D)))
    if kw.pop("alibi", False):
        kw["alibi"] = torch.from_numpy(W.alibi_slopes(Hq))
    name = f"attn_paged_prefill {dtype} D{D} sq={sq} sk={sk} H{Hq}/{Hkv} bs{bs} {sorted(kw)}"
    announce(name)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = gpu_run(gpu_lib, c, err=err, **kw)
    assert err.item() == 0, f"{name}: error flag set"
    compare(got, oracle_run(c, **kw), DT[dtype], name)


def test_paged_prefill_valu_error_flag(gpu_lib):
    """Vector-ALU path: a block id outside the pool masks its keys and sets the
    flag; the other sequence is unaffected."""
    c = make_case("f32", (40, 30), (100, 60), 4, 2, 64, 16, 77)
    kw = dict(scale=0.125)
    ref = oracle_run(c, **kw)
    bad = c["table"].clone()
    bad[0, 2] = 10 ** 6                          # keys 32..47 of sequence 0
    c2 = dict(c, table=bad)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    announce("attn_paged_prefill f32: block id out of range")
    got = gpu_run(gpu_lib, c2, err=err, **kw)
    assert err.item() == 1
    assert torch.isfinite(got).all()
    compare(got[40:], ref[40:], torch.float32, "f32 paged prefill, unaffected sequence")
