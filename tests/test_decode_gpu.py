"""Parity of attn_paged_decode (HIP, through the C ABI) with the paged oracle.

Includes a bit-exact check of the integer paging (one-hot scores make the
output the V row of a single logical token, which encodes its (sequence,
position) in bf16-exact integers), the device-side error flag, and bitwise
rerun determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, compare

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}
DEV = torch.device("cuda:0")


def gpu_decode(sdpa, q, kp, vp, table, lens, alibi=None, **kw):
    out = sdpa.attn_paged_decode(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), lens.to(DEV),
                                 None if alibi is None else alibi.to(DEV), **kw)
    torch.cuda.synchronize()
    return out


def oracle_decode(q, kp, vp, table, lens, alibi=None, **kw):
    return oracle.paged_decode_f64(W.to_f64(q), W.to_f64(kp), W.to_f64(vp), table.numpy(),
                                   lens.numpy(), alibi=None if alibi is None else W.to_f64(alibi),
                                   **kw)


CASES = [
    # dtype, B, Hq, Hkv, D, block_size, lens, splits, softcap, alibi
    ("bf16", 5, 8, 2, 128, 16, [0, 1, 17, 64, 300], 3, None, False),
    ("bf16", 3, 32, 8, 128, 64, [512, 1000, 77], 8, None, False),
    ("f16", 4, 4, 4, 64, 7, [5, 50, 123, 13], 2, None, False),
    ("bf16", 2, 16, 1, 64, 1, [9, 40], 1, None, False),
    ("f16", 3, 6, 2, 128, 32, [200, 31, 97], 5, 10.0, True),
    ("bf16", 2, 32, 1, 128, 16, [333, 129], 4, None, True),
    ("bf16", 2, 24, 8, 64, 64, [700, 64], 8, 30.0, False),
    ("bf16", 3, 10, 5, 128, 48, [1, 480, 481], 16, None, False),
    # head dim 256
    ("bf16", 3, 8, 2, 256, 64, [700, 1, 129], 8, None, False),
    ("f16", 2, 16, 4, 256, 16, [333, 64], 4, 20.0, True),
    ("bf16", 2, 4, 4, 256, 5, [50, 17], 2, None, False),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_paged_parity(gpu_lib, case):
    dtype, B, Hq, Hkv, D, bs, lens, splits, cap, use_alibi = CASES[case]
    maxb = max((max(lens) + bs - 1) // bs, 1) + 1
    w = W.Paged("t", dtype, B, Hq, Hkv, D, bs, 0, 0, splits, maxb, seed=200 + case)
    q, kp, vp, table, sl, _ = W.paged_inputs(w, seq_lens=lens)
    alibi = torch.from_numpy(W.alibi_slopes(Hq)) if use_alibi else None
    scale = D ** -0.5
    announce(f"paged decode case {case}: {CASES[case]}")
    out = gpu_decode(gpu_lib, q, kp, vp, table, sl, alibi, softmax_scale=scale, softcap=cap,
                     num_splits=splits)
    ref = oracle_decode(q, kp, vp, table, sl, alibi, scale=scale, softcap=cap)
    compare(out, ref, DT[dtype], f"paged case {case}")
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.count_nonzero(out[b]).item() == 0


AUTO_SPLIT_CASES = [
    # dtype, B, Hq, Hkv, D, block_size, lens  (num_splits = 0: chosen by the library)
    ("bf16", 1, 32, 8, 128, 64, [20000]),            # 8 groups: many splits
    ("bf16", 2, 32, 8, 128, 16, [6000, 1]),
    ("f16", 3, 8, 2, 64, 32, [3000, 0, 700]),
    ("bf16", 1, 16, 4, 256, 64, [5000]),
    ("bf16", 2, 4, 4, 128, 16, [100, 255]),          # short capacity: few splits
    # 40 x 8 = 320 groups: about 4096 items (13 splits), the split form
    ("bf16", 40, 32, 8, 128, 64, [int(x) for x in np.random.default_rng(3).integers(300, 2000, 40)]),
]


@pytest.mark.parametrize("case", range(len(AUTO_SPLIT_CASES)))
def test_paged_parity_automatic_splits(gpu_lib, case):
    dtype, B, Hq, Hkv, D, bs, lens = AUTO_SPLIT_CASES[case]
    maxb = max((max(lens) + bs - 1) // bs, 1)
    w = W.Paged("t", dtype, B, Hq, Hkv, D, bs, 0, 0, 0, maxb, seed=260 + case)
    q, kp, vp, table, sl, _ = W.paged_inputs(w, seq_lens=lens)
    scale = D ** -0.5
    announce(f"paged decode with automatic splits, case {case}: {AUTO_SPLIT_CASES[case]}")
    out = gpu_decode(gpu_lib, q, kp, vp, table, sl, None, softmax_scale=scale, num_splits=0)
    ref = oracle_decode(q, kp, vp, table, sl, None, scale=scale)
    compare(out, ref, DT[dtype], f"automatic splits case {case}")
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.count_nonzero(out[b]).item() == 0


def wide_lens(B, hi, seed):
    """Lengths for the wide batches: empty, single-token, block-edge and long
    sequences mixed, the rest uniform on [0, hi]."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, hi + 1, size=B)
    edge = [0, 1, 15, 16, 17, 127, 128, 129, hi]
    lens[:len(edge)] = edge
    return rng.permutation(lens).astype(np.int32).tolist()


# Batches of at least 256 (sequence, KV head, 16-head chunk) groups, one per
# compute unit of a 256-CU chip or more.  With fewer than 1024 (group, split)
# items (4 per compute unit), and always at head dim 256, every group is a
# whole workgroup's item and the workgroup merges its chunks itself (the fused
# form); otherwise per-wave workers stream the items and the merge kernel
# combines them (the split form).
WIDE_CASES = [
    # dtype, B, Hq, Hkv, D, block_size, max len, splits, softcap, alibi
    ("bf16", 64, 8, 4, 128, 16, 700, 2, None, False),      # fused: 256 groups x 2 splits
    ("f16", 128, 4, 2, 64, 32, 300, 3, 15.0, True),        # fused
    ("bf16", 64, 40, 2, 128, 64, 400, 1, None, True),      # fused; 20 heads per KV head: 2 chunks
    ("bf16", 64, 16, 4, 256, 16, 500, 2, None, False),     # fused
    ("f16", 256, 2, 1, 128, 48, 200, 2, 30.0, False),      # fused
    ("bf16", 64, 8, 4, 128, 16, 700, 8, None, False),      # split form: 2048 items
    ("f16", 128, 4, 2, 64, 32, 300, 4, 15.0, True),        # split form
    ("bf16", 64, 16, 4, 256, 16, 500, 8, None, True),      # fused: head dim 256 keeps it with many items
]


@pytest.mark.parametrize("case", range(len(WIDE_CASES)))
def test_paged_parity_wide_batch(gpu_lib, case):
    dtype, B, Hq, Hkv, D, bs, hi, splits, cap, use_alibi = WIDE_CASES[case]
    lens = wide_lens(B, hi, 300 + case)
    maxb = (max(lens) + bs - 1) // bs + 1
    w = W.Paged("t", dtype, B, Hq, Hkv, D, bs, 0, 0, splits, maxb, seed=310 + case)
    q, kp, vp, table, sl, _ = W.paged_inputs(w, seq_lens=lens)
    alibi = torch.from_numpy(W.alibi_slopes(Hq)) if use_alibi else None
    scale = D ** -0.5
    announce(f"paged decode wide case {case}: {WIDE_CASES[case]}")
    out = gpu_decode(gpu_lib, q, kp, vp, table, sl, alibi, softmax_scale=scale, softcap=cap,
                     num_splits=splits)
    ref = oracle_decode(q, kp, vp, table, sl, alibi, scale=scale, softcap=cap)
    compare(out, ref, DT[dtype], f"paged wide case {case}")
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.count_nonzero(out[b]).item() == 0


# Batches above 256 sequences with block sizes that are multiples of 16: the
# lengths ordered by a bitonic sort in LDS; the split form up to 2048
# sequences, the fused form below 4 items per compute unit and, up to 4096
# sequences, for block tables of more than 1024 tokens.
LARGE_BATCH_CASES = [
    # dtype, B, Hq, Hkv, D, block_size, max len, splits, softcap, alibi
    ("bf16", 300, 8, 4, 128, 16, 300, 3, None, False),     # split form
    ("bf16", 512, 8, 8, 128, 64, 260, 8, None, False),     # split form
    ("f16", 300, 4, 2, 64, 64, 400, 1, 20.0, True),        # fused: 600 items
    ("bf16", 320, 16, 4, 256, 16, 150, 8, 30.0, True),     # fused at head dim 256 (1280 groups)
    ("f16", 512, 8, 2, 128, 16, 250, 8, None, True),       # split form
    ("bf16", 400, 32, 8, 128, 32, 200, 5, None, False),    # split form
    ("f16", 1100, 4, 2, 64, 32, 70, 3, 25.0, True),        # split form
    ("bf16", 2048, 2, 1, 128, 16, 40, 2, None, False),     # split form, its largest batch
    ("bf16", 700, 4, 1, 128, 32, 300, 1, None, True),      # fused: 700 items
    ("bf16", 2500, 2, 1, 128, 16, 1100, 1, None, False),   # fused: capacity 1120 tokens
    ("f16", 4096, 2, 1, 64, 32, 1100, 2, 15.0, False),     # fused, its largest batch
    ("bf16", 2049, 8, 2, 128, 64, 1100, 4, None, True),    # fused: one past the split form's limit
    ("bf16", 2300, 4, 1, 256, 16, 1050, 1, 30.0, False),   # fused at head dim 256
]


@pytest.mark.parametrize("case", range(len(LARGE_BATCH_CASES)))
def test_paged_parity_large_batch(gpu_lib, case):
    run_batch_case(gpu_lib, LARGE_BATCH_CASES[case], 400 + case, f"paged decode large-batch case {case}")


# Above 2048 sequences with block tables of at most 1024 tokens, and above
# 4096 sequences: the partial kernel over uniform 16-token blocks (one 2-wave
# workgroup per split and group) plus the merge kernel.  The workgroups rank
# the lengths in LDS up to 2048 sequences at head dim 128 (1024 at 64) and
# take them in index order beyond that.
PARTIAL_CASES = [
    # dtype, B, Hq, Hkv, D, block_size, max len, splits, softcap, alibi
    ("bf16", 4097, 2, 1, 128, 16, 20, 2, None, False),
    ("f16", 4500, 4, 2, 64, 32, 24, 3, 25.0, True),
    ("bf16", 4200, 8, 2, 256, 16, 17, 1, None, True),
    ("bf16", 2100, 2, 1, 128, 16, 40, 2, None, False),
    ("f16", 3000, 4, 1, 128, 64, 200, 1, None, True),
]


def run_batch_case(gpu_lib, case, seed, name):
    dtype, B, Hq, Hkv, D, bs, hi, splits, cap, use_alibi = case
    lens = wide_lens(B, hi, seed)
    maxb = (max(lens) + bs - 1) // bs + 1
    w = W.Paged("t", dtype, B, Hq, Hkv, D, bs, 0, 0, splits, maxb, seed=seed + 10)
    q, kp, vp, table, sl, _ = W.paged_inputs(w, seq_lens=lens)
    alibi = torch.from_numpy(W.alibi_slopes(Hq)) if use_alibi else None
    scale = D ** -0.5
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    announce(f"{name}: {case}")
    out = gpu_decode(gpu_lib, q, kp, vp, table, sl, alibi, softmax_scale=scale, softcap=cap,
                     num_splits=splits, error_flag=flag)
    assert flag.item() == 0
    ref = oracle_decode(q, kp, vp, table, sl, alibi, scale=scale, softcap=cap)
    compare(out, ref, DT[dtype], name)
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.count_nonzero(out[b]).item() == 0


@pytest.mark.parametrize("case", range(len(PARTIAL_CASES)))
def test_paged_parity_partial_kernel(gpu_lib, case):
    run_batch_case(gpu_lib, PARTIAL_CASES[case], 450 + case, f"paged decode partial-kernel case {case}")


@pytest.mark.parametrize("B,splits", [(300, 4), (300, 1), (4200, 4)])
def test_large_batch_error_flag_and_determinism(gpu_lib, B, splits):
    """16-token blocks at B = 300 (over sorted lengths: the split form with 4
    splits, the fused form with 1) and B = 4200 (the partial kernel): a block
    id outside the pool masks its keys and sets the flag, a length beyond the
    table's capacity is clamped and sets it, the other sequences are
    unaffected, and reruns are bitwise equal."""
    Hq, Hkv, D, bs, maxb = 8, 2, 128, 16, 20
    w = W.Paged("ep", "bf16", B, Hq, Hkv, D, bs, 0, 0, 4, maxb, seed=91)
    lens = wide_lens(B, 300, 92)
    q, kp, vp, table, sl, _ = W.paged_inputs(w, seq_lens=lens)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    announce(f"B={B}: valid call, rerun")
    a = gpu_decode(gpu_lib, q, kp, vp, table, sl, error_flag=flag, num_splits=splits)
    b = gpu_decode(gpu_lib, q, kp, vp, table, sl, error_flag=flag, num_splits=splits)
    assert flag.item() == 0
    assert torch.equal(a, b)
    ref = oracle_decode(q, kp, vp, table, sl, scale=D ** -0.5)
    compare(a, ref, torch.bfloat16, f"B={B}")
    victim = int(np.argmax(np.array(lens) > 2 * bs))
    bad = table.clone()
    bad[victim, 1] = 10 ** 6                                # keys 16..31 of that sequence are masked
    announce(f"B={B}: block id out of range")
    out = gpu_decode(gpu_lib, q, kp, vp, bad, sl, error_flag=flag, num_splits=splits)
    assert flag.item() == 1
    assert torch.isfinite(out.float()).all()
    others = [i for i in range(B) if i != victim]
    compare(out[others], ref[others], torch.bfloat16, f"B={B}, unaffected sequences")
    n = lens[victim]
    keep = [t for t in range(n) if not bs <= t < 2 * bs]
    kb = oracle.paged_gather(W.to_f64(kp), table.numpy(), n, victim, bs)[keep]
    vb = oracle.paged_gather(W.to_f64(vp), table.numpy(), n, victim, bs)[keep]
    r1 = oracle.sdpa_naive_f64(W.to_f64(q[victim:victim + 1]), kb.transpose(1, 0, 2)[None],
                               vb.transpose(1, 0, 2)[None], scale=D ** -0.5)
    compare(out[victim:victim + 1], r1, torch.bfloat16, f"B={B}, masked keys")
    flag.zero_()
    long = sl.clone()
    long[3] = maxb * bs + 5
    announce(f"B={B}: seq_len beyond capacity")
    gpu_decode(gpu_lib, q, kp, vp, table, long, error_flag=flag, num_splits=splits)
    assert flag.item() == 1


def test_paged_decode_workload(gpu_lib):
    w = W.PAGED_DECODE
    q, kp, vp, table, lens, _ = W.paged_inputs(w)
    announce(w.name)
    out = gpu_decode(gpu_lib, q, kp, vp, table, lens, softmax_scale=w.scale,
                     num_splits=w.num_splits)
    ref = oracle_decode(q, kp, vp, table, lens, scale=w.scale)
    compare(out, ref, torch.bfloat16, w.name)


@pytest.mark.parametrize("bs,splits,B,Hkv", [(64, 8, 4, 2), (16, 3, 4, 2), (5, 1, 4, 2),
                                             (16, 8, 64, 4), (32, 2, 128, 2),
                                             (16, 3, 300, 2), (64, 8, 300, 1), (16, 1, 300, 2),
                                             (16, 3, 4200, 1)])
def test_paging_is_bit_exact(gpu_lib, bs, splits, B, Hkv):
    """One-hot scores: q = 1024 e0 in every head and a single key row equal to
    8 e0 give that key a score of 1024 * 8 / sqrt(128) ~ 724 and every other
    key 0, so exp underflows to exactly 0 elsewhere and the output is exactly
    the V row of that logical token.  V rows hold (sequence % 128, position
    % 128, position // 128, kv head, sequence // 128) as bf16-exact integers;
    slots no table entry points at hold a finite sentinel so that a stray
    read is visible.  B = 4 runs the split form (and the partial kernel at
    block size 5); B = 128 with 2 splits and B = 300 with 1 the fused form
    (at least 256 groups, fewer than 1024 items); B = 64 with 8 splits and
    B = 300 with 3 or 8 the split form; B = 4200 the partial kernel over
    16-token blocks."""
    Hq, D = 8, 128
    lens = [130, 64, 7, 200] if B == 4 else np.random.default_rng(6).integers(1, 260, size=B).tolist()
    rng = np.random.default_rng(5)
    maxb = (max(lens) + bs - 1) // bs + 1
    table_np, nb = W.paged_layout(np.array(lens), bs, maxb, rng)
    nb_pool = nb + 3                        # three blocks nobody references
    kp = torch.zeros(nb_pool, bs, Hkv, D, dtype=torch.bfloat16)
    vp_np = np.full((nb_pool, bs, Hkv, D), 1e4, dtype=np.float32)
    for b, n in enumerate(lens):
        t = np.arange(n)
        blk, slot = table_np[b, t // bs], t % bs
        row = np.zeros((n, Hkv, D), dtype=np.float32)
        row[:, :, 0] = b % 128
        row[:, :, 1] = (t % 128)[:, None]
        row[:, :, 2] = (t // 128)[:, None]
        row[:, :, 3] = np.arange(Hkv)[None, :]
        row[:, :, 4] = b // 128
        vp_np[blk, slot] = row
    vp = torch.from_numpy(vp_np).to(torch.bfloat16)
    q = torch.zeros(B, Hq, 1, D, dtype=torch.bfloat16)
    q[..., 0] = 1024.0
    table = torch.from_numpy(table_np)
    sl = torch.tensor(lens, dtype=torch.int32)
    dq, dt, dsl = q.to(DEV), table.to(DEV), sl.to(DEV)
    dvp = vp.to(DEV)
    for frac in (0.0, 0.3, 0.5, 0.99, 1.0):
        kp.zero_()
        targets = []
        for b, n in enumerate(lens):
            t = min(n - 1, int(frac * n))
            targets.append(t)
            kp[table_np[b, t // bs], t % bs, :, 0] = 8.0
        announce(f"one-hot paging bs={bs} splits={splits} frac={frac}")
        out = gpu_lib.attn_paged_decode(dq, kp.to(DEV), dvp, dt, dsl, num_splits=splits)
        torch.cuda.synchronize()
        out = out.cpu()
        want = torch.zeros(B, Hq, 1, D, dtype=torch.bfloat16)
        tt = torch.tensor(targets, dtype=torch.float32)
        want[:, :, 0, 0] = (torch.arange(B) % 128).float()[:, None]
        want[:, :, 0, 4] = torch.div(torch.arange(B), 128, rounding_mode="floor").float()[:, None]
        want[:, :, 0, 1] = (tt % 128)[:, None]
        want[:, :, 0, 2] = torch.div(tt, 128, rounding_mode="floor")[:, None]
        want[:, :, 0, 3] = (torch.arange(Hq) // (Hq // Hkv)).float()[None, :]
        if not torch.equal(out, want):
            b, h = (out != want).any(dim=-1)[..., 0].nonzero()[0].tolist()
            raise AssertionError(f"sequence {b} head {h} target {targets[b]}: {out[b, h, 0, :5]}")


def test_error_flag_and_masking(gpu_lib):
    w = W.Paged("e", "bf16", 3, 8, 2, 128, 16, 0, 0, 4, 8, seed=9)
    lens = [40, 100, 33]
    q, kp, vp, table, sl, _ = W.paged_inputs(w, seq_lens=lens)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    announce("error flag: valid call")
    gpu_decode(gpu_lib, q, kp, vp, table, sl, error_flag=flag, num_splits=4)
    assert flag.item() == 0
    bad = table.clone()
    bad[1, 2] = 10 ** 6                      # keys 32..47 of sequence 1 are masked
    announce("error flag: block id out of range")
    out = gpu_decode(gpu_lib, q, kp, vp, bad, sl, error_flag=flag, num_splits=4)
    assert flag.item() == 1
    assert torch.isfinite(out.float()).all()
    # The other sequences are unaffected; sequence 1 equals attention without keys 32..47.
    ref = oracle_decode(q, kp, vp, table, sl, scale=128 ** -0.5)
    compare(out[[0, 2]], ref[[0, 2]], torch.bfloat16, "unaffected sequences")
    keep = [t for t in range(100) if not 32 <= t < 48]
    kb = oracle.paged_gather(W.to_f64(kp), table.numpy(), 100, 1, 16)[keep]
    vb = oracle.paged_gather(W.to_f64(vp), table.numpy(), 100, 1, 16)[keep]
    r1 = oracle.sdpa_naive_f64(W.to_f64(q[1:2]), kb.transpose(1, 0, 2)[None],
                               vb.transpose(1, 0, 2)[None], scale=128 ** -0.5)
    compare(out[1:2], r1, torch.bfloat16, "masked keys")
    flag.zero_()
    long = sl.clone()
    long[2] = 8 * 16 + 5                     # beyond the table's capacity: clamped
    announce("error flag: seq_len beyond capacity")
    gpu_decode(gpu_lib, q, kp, vp, table, long, error_flag=flag, num_splits=4)
    assert flag.item() == 1


def test_decode_rerun_is_bitwise_identical(gpu_lib):
    w = W.Paged("d", "bf16", 8, 32, 8, 128, 64, 100, 3000, 8, 48, seed=10)
    q, kp, vp, table, lens, _ = W.paged_inputs(w)
    q, kp, vp, table, lens = (x.to(DEV) for x in (q, kp, vp, table, lens))
    announce("decode determinism")
    a = gpu_lib.attn_paged_decode(q, kp, vp, table, lens)
    b = gpu_lib.attn_paged_decode(q, kp, vp, table, lens)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decode_equals_dense_prefill_path(gpu_lib):
    """A contiguous, identity-paged cache decodes to what attn_fwd gives for
    the same single query (both HIP paths, checked against the oracle)."""
    B, Hq, Hkv, D, S, bs = 2, 8, 2, 128, 256, 64
    q, k, v = W.random_dense("bf16", B, Hq, Hkv, 1, S, D, 21)
    kp = k.permute(0, 2, 1, 3).reshape(B * S // bs, bs, Hkv, D).contiguous()
    vp = v.permute(0, 2, 1, 3).reshape(B * S // bs, bs, Hkv, D).contiguous()
    table = torch.arange(B * S // bs, dtype=torch.int32).reshape(B, S // bs)
    lens = torch.full((B,), S, dtype=torch.int32)
    announce("decode vs dense")
    dec = gpu_decode(gpu_lib, q, kp, vp, table, lens)
    dense = gpu_lib.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    ref = oracle.sdpa_naive_f64(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale=D ** -0.5)
    compare(dec, ref, torch.bfloat16, "decode")
    compare(dense, ref, torch.bfloat16, "dense")


def test_wide_batch_error_flag_and_determinism(gpu_lib):
    """The fused form (256 groups): a block id outside the pool masks its keys
    and sets the flag, a length beyond the table's capacity is clamped and
    sets it, the other sequences are unaffected, and reruns are bitwise equal."""
    B, Hq, Hkv, D, bs, maxb = 64, 8, 4, 128, 16, 20
    w = W.Paged("ew", "bf16", B, Hq, Hkv, D, bs, 0, 0, 4, maxb, seed=77)
    lens = wide_lens(B, 300, 78)
    q, kp, vp, table, sl, _ = W.paged_inputs(w, seq_lens=lens)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    announce("wide batch: valid call, rerun")
    a = gpu_decode(gpu_lib, q, kp, vp, table, sl, error_flag=flag)
    b = gpu_decode(gpu_lib, q, kp, vp, table, sl, error_flag=flag)
    assert flag.item() == 0
    assert torch.equal(a, b)
    ref = oracle_decode(q, kp, vp, table, sl, scale=D ** -0.5)
    compare(a, ref, torch.bfloat16, "wide batch")
    victim = int(np.argmax(np.array(lens) > 2 * bs))       # a sequence with at least 3 blocks
    bad = table.clone()
    bad[victim, 1] = 10 ** 6                                # keys 16..31 of that sequence are masked
    announce("wide batch: block id out of range")
    out = gpu_decode(gpu_lib, q, kp, vp, bad, sl, error_flag=flag)
    assert flag.item() == 1
    assert torch.isfinite(out.float()).all()
    others = [i for i in range(B) if i != victim]
    compare(out[others], ref[others], torch.bfloat16, "wide batch, unaffected sequences")
    n = lens[victim]
    keep = [t for t in range(n) if not bs <= t < 2 * bs]
    kb = oracle.paged_gather(W.to_f64(kp), table.numpy(), n, victim, bs)[keep]
    vb = oracle.paged_gather(W.to_f64(vp), table.numpy(), n, victim, bs)[keep]
    r1 = oracle.sdpa_naive_f64(W.to_f64(q[victim:victim + 1]), kb.transpose(1, 0, 2)[None],
                               vb.transpose(1, 0, 2)[None], scale=D ** -0.5)
    compare(out[victim:victim + 1], r1, torch.bfloat16, "wide batch, masked keys")
    flag.zero_()
    long = sl.clone()
    long[3] = maxb * bs + 5
    announce("wide batch: seq_len beyond capacity")
    gpu_decode(gpu_lib, q, kp, vp, table, long, error_flag=flag)
    assert flag.item() == 1


# F32 / F64: the vector-ALU paged kernel with one query per sequence
VALU_DECODE = [
    # dtype, B, Hq, Hkv, D, block_size, lens, softcap, alibi
    ("f32", 4, 8, 2, 128, 16, [0, 1, 77, 300], None, False),
    ("f64", 3, 4, 4, 64, 7, [50, 123, 13], 15.0, True),
    ("f32", 2, 16, 1, 32, 64, [9, 400], None, True),
    ("f64", 2, 6, 2, 256, 5, [40, 2], None, False),
]


@pytest.mark.parametrize("case", range(len(VALU_DECODE)))
def test_paged_decode_valu_parity(gpu_lib, case):
    dtype, B, Hq, Hkv, D, bs, lens, cap, use_alibi = VALU_DECODE[case]
    maxb = max((max(lens) + bs - 1) // bs, 1) + 1
    w = W.Paged("v", "f32", B, Hq, Hkv, D, bs, 0, 0, 4, maxb, seed=260 + case)
    q, kp, vp, table, sl, _ = W.paged_inputs(w, seq_lens=lens)
    if dtype == "f64":
        q, kp, vp = q.double(), kp.double(), vp.double()
    alibi = torch.from_numpy(W.alibi_slopes(Hq)) if use_alibi else None
    scale = float(np.float32(D ** -0.5))
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    announce(f"paged decode vector-ALU case {case}: {VALU_DECODE[case]}")
    out = gpu_decode(gpu_lib, q, kp, vp, table, sl, alibi, softmax_scale=scale, softcap=cap,
                     error_flag=flag)
    assert flag.item() == 0
    ref = oracle_decode(q, kp, vp, table, sl, alibi, scale=scale, softcap=cap)
    compare(out, ref, {"f32": torch.float32, "f64": torch.float64}[dtype], f"valu decode {case}")
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.count_nonzero(out[b]).item() == 0


def test_paged_decode_valu_error_flag(gpu_lib):
    w = W.Paged("ve", "f32", 3, 8, 2, 64, 16, 0, 0, 4, 8, seed=9)
    lens = [40, 100, 33]
    q, kp, vp, table, sl, _ = W.paged_inputs(w, seq_lens=lens)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    bad = table.clone()
    bad[1, 2] = 10 ** 6                      # keys 32..47 of sequence 1 are masked
    announce("paged decode vector-ALU: block id out of range")
    out = gpu_decode(gpu_lib, q, kp, vp, bad, sl, error_flag=flag, softmax_scale=0.125)
    assert flag.item() == 1
    ref = oracle_decode(q, kp, vp, table, sl, scale=0.125)
    compare(out[[0, 2]], ref[[0, 2]], torch.float32, "valu decode, unaffected sequences")
    keep = [t for t in range(100) if not 32 <= t < 48]
    kb = oracle.paged_gather(W.to_f64(kp), table.numpy(), 100, 1, 16)[keep]
    vb = oracle.paged_gather(W.to_f64(vp), table.numpy(), 100, 1, 16)[keep]
    r1 = oracle.sdpa_naive_f64(W.to_f64(q[1:2]), kb.transpose(1, 0, 2)[None],
                               vb.transpose(1, 0, 2)[None], scale=0.125)
    compare(out[1:2], r1, torch.float32, "valu decode, masked keys")
    flag.zero_()
    long = sl.clone()
    long[2] = 8 * 16 + 5                     # beyond the table's capacity: clamped
    gpu_decode(gpu_lib, q, kp, vp, table, long, error_flag=flag)
    assert flag.item() == 1
