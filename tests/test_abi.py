"""The C ABI without a GPU: library load, exported symbols, host-only checks.

Only the ``*_check`` validators, the workspace-size query and the status
strings are called here; they make no HIP call.  Pointers are fake aligned
addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import scaled_dot_product_amd as sdpa
from scaled_dot_product_amd import attn_fwd_params_t, attn_paged_params_t

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK = 0
NULL, DTYPE, SHAPE, GQA, HEAD_DIM, PARAM, ALIGN, ALIAS, WORKSPACE, UNSUPPORTED = range(1, 11)

# Fake, 16-byte aligned, well separated device addresses.
Q, K, V, AL, OUT, KP, VP, TAB, LEN, WS, ERR = (0x100000000 * (i + 1) for i in range(11))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = sdpa.library()
    names = declared_functions()
    assert {"attn_fwd", "attn_fwd_check", "attn_paged_decode", "attn_paged_decode_check",
            "attn_paged_decode_workspace_size", "attn_status_str", "attn_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libattn.so does not export {n}"
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_binding_names_match_the_header():
    for n in declared_functions():
        assert callable(getattr(sdpa, n)), n


def test_status_strings_and_version():
    assert sdpa.attn_status_str(0) == "ok"
    for code in range(1, 12):
        assert sdpa.attn_status_str(code) not in ("ok", "unknown status")
    assert sdpa.attn_status_str(99) == "unknown status"
    assert sdpa.attn_version() >= 100


def fwd(**kw):
    base = dict(B=2, Hq=8, Hkv=2, Sq=100, Sk=130, D=128, dtype=sdpa.ATTN_BF16, causal=1,
                window_left=-1, window_right=-1, softmax_scale=0.125, softcap=0.0)
    base.update(kw)
    return attn_fwd_params_t(**base)


def check_fwd(p, q=Q, k=K, v=V, al=None, out=OUT):
    return sdpa.attn_fwd_check(q, k, v, al, out, p)


def test_fwd_check_accepts_valid_calls():
    assert check_fwd(fwd()) == OK
    assert check_fwd(fwd(D=64, dtype=sdpa.ATTN_F16, causal=0, window_left=5, window_right=0,
                         softcap=30.0), al=AL) == OK
    assert check_fwd(fwd(dtype=sdpa.ATTN_F32)) == OK
    assert check_fwd(fwd(Hkv=8)) == OK
    # the matrix-core path takes 64, 128, 256; the vector-ALU path (F32, F64) 32 .. 256
    for dt in (sdpa.ATTN_BF16, sdpa.ATTN_F16):
        assert check_fwd(fwd(dtype=dt, D=256)) == OK, dt
    for dt in (sdpa.ATTN_F32, sdpa.ATTN_F64):
        for d in (32, 64, 128, 256):
            assert check_fwd(fwd(dtype=dt, D=d)) == OK, (dt, d)


@pytest.mark.parametrize("dt,d", [(sdpa.ATTN_BF16, 32), (sdpa.ATTN_F16, 512), (sdpa.ATTN_F32, 96),
                                  (sdpa.ATTN_F64, 80), (sdpa.ATTN_F64, 512)])
def test_fwd_check_head_dim_per_dtype(dt, d):
    assert check_fwd(fwd(dtype=dt, D=d)) == HEAD_DIM


def test_fwd_check_f64_sizes_and_alias():
    # F64 operands are 8 bytes an element: out overlapping the end of q aliases
    p = fwd(dtype=sdpa.ATTN_F64, B=1, Hq=2, Hkv=2, Sq=4, Sk=4, D=32)
    q_bytes = 1 * 2 * 4 * 32 * 8
    assert check_fwd(p, out=Q + q_bytes) == OK
    assert check_fwd(p, out=Q + q_bytes - 16) == ALIAS
    # one head's K must stay under 2 GiB: Sk * D * 8 bytes
    assert check_fwd(fwd(dtype=sdpa.ATTN_F64, D=256, Sk=(1 << 20))) == SHAPE
    assert check_fwd(fwd(dtype=sdpa.ATTN_F64, D=256, Sk=(1 << 20) - 1)) == OK


def test_fwd_check_empty_tensors_may_be_null():
    assert check_fwd(fwd(Sq=0), q=None, out=None) == OK
    assert check_fwd(fwd(Sk=0), k=None, v=None) == OK
    assert check_fwd(fwd(B=0), q=None, k=None, v=None, out=None) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), DTYPE),
    (dict(B=-1), SHAPE), (dict(Sq=-2), SHAPE), (dict(Sk=-1), SHAPE),
    (dict(Sq=(1 << 30) + 1), SHAPE),
    (dict(Hkv=3), GQA), (dict(Hkv=0), GQA),
    (dict(D=96), HEAD_DIM), (dict(D=512), HEAD_DIM), (dict(D=32), HEAD_DIM),
    (dict(softmax_scale=float("nan")), PARAM), (dict(softmax_scale=-1.0), PARAM),
    (dict(softcap=-0.5), PARAM), (dict(softcap=float("inf")), PARAM),
    (dict(window_left=-2), PARAM), (dict(window_right=-5), PARAM),
    (dict(has_k_len=1, k_len=-1), PARAM), (dict(has_k_len=1, k_len=131), PARAM),
])
def test_fwd_check_rejects(kw, code):
    assert check_fwd(fwd(**kw)) == code


def test_fwd_check_live_prefix():
    # k_len is read only with has_k_len; with it, 0 .. Sk (= 130 here)
    assert check_fwd(fwd(k_len=-7)) == OK
    for kl in (0, 1, 129, 130):
        assert check_fwd(fwd(has_k_len=1, k_len=kl)) == OK, kl
        assert check_fwd(fwd(has_k_len=1, k_len=kl, dtype=sdpa.ATTN_F64, D=64)) == OK, kl
    p = sdpa.attn_fwd_params((2, 8, 100, 128), (2, 2, 130, 128), sdpa.ATTN_BF16, k_len=5)
    assert (p.has_k_len, p.k_len) == (1, 5)
    p = sdpa.attn_fwd_params((2, 8, 100, 128), (2, 2, 130, 128), sdpa.ATTN_BF16)
    assert p.has_k_len == 0


def test_fwd_check_pointers():
    assert check_fwd(fwd(), q=None) == NULL
    assert check_fwd(fwd(), out=None) == NULL
    assert check_fwd(fwd(), v=None) == NULL
    assert sdpa.attn_fwd_check(Q, K, V, None, OUT, None) == NULL
    assert check_fwd(fwd(), k=K + 8) == ALIGN
    assert check_fwd(fwd(), al=AL + 4) == ALIGN
    assert check_fwd(fwd(), out=Q) == ALIAS                # out == q
    assert check_fwd(fwd(), out=K + 4096) == ALIAS         # out inside k
    assert check_fwd(fwd(), al=OUT + 16) == ALIAS          # slopes inside out


LSE = 0x100000000 * 12


def test_fwd_lse_check():
    """attn_fwd_lse_check: everything attn_fwd_check rejects, plus the lse
    buffer (float32 [B, Hq, Sq]): required, 4-byte aligned, disjoint."""
    lse_check = lambda p, lse=LSE, **kw: sdpa.attn_fwd_lse_check(
        kw.get("q", Q), kw.get("k", K), kw.get("v", V), kw.get("al"), kw.get("out", OUT), lse, p)
    assert lse_check(fwd()) == OK
    assert lse_check(fwd(), lse=None) == NULL
    assert lse_check(fwd(Sq=0), lse=None) == OK            # no rows: may be NULL
    assert lse_check(fwd(), lse=LSE + 2) == ALIGN
    assert lse_check(fwd(), lse=LSE + 4) == OK             # float alignment suffices
    assert lse_check(fwd(), lse=OUT) == ALIAS               # lse == out
    assert lse_check(fwd(), lse=Q + 64) == ALIAS            # lse inside q
    assert lse_check(fwd(), lse=OUT - 4) == ALIAS           # last float overlaps out
    assert lse_check(fwd(), lse=OUT - 2 * 8 * 100 * 4) == OK  # ends exactly where out starts
    assert lse_check(fwd(D=80)) == HEAD_DIM                 # attn_fwd_check's rules first
    lib = sdpa.library()
    p = fwd()
    assert lib.attn_fwd_lse(Q, K, V, None, OUT, None, ctypes.byref(p), None) == NULL


def test_fwd_invalid_call_returns_before_any_launch():
    # attn_fwd validates first; on this GPU-less host nothing must be launched.
    lib = sdpa.library()
    p = fwd(D=80)
    assert lib.attn_fwd(Q, K, V, None, OUT, ctypes.byref(p), None) == HEAD_DIM
    p = fwd(Sq=0)
    assert lib.attn_fwd(None, K, V, None, None, ctypes.byref(p), None) == OK  # nothing to do


def paged(**kw):
    base = dict(B=4, Hq=32, Hkv=8, D=128, num_blocks=40, block_size=64, max_blocks_per_seq=10,
                dtype=sdpa.ATTN_BF16, num_splits=8, softmax_scale=0.088, softcap=0.0)
    base.update(kw)
    return attn_paged_params_t(**base)


def check_paged(p, ws_bytes=None, **ptrs):
    args = dict(q=Q, k=KP, v=VP, tab=TAB, lens=LEN, al=None, out=OUT, ws=WS, err=None)
    args.update(ptrs)
    if ws_bytes is None:
        ws_bytes = sdpa.attn_paged_decode_workspace_size(p)
    return sdpa.attn_paged_decode_check(args["q"], args["k"], args["v"], args["tab"],
                                        args["lens"], args["al"], args["out"], args["ws"],
                                        ws_bytes, args["err"], p)


def test_workspace_size():
    p = paged()
    o_bytes = 4 * 32 * 8 * 128 * 4
    lse_off = (o_bytes + 255) // 256 * 256
    assert sdpa.attn_paged_decode_workspace_size(p) == lse_off + 4 * 32 * 8 * 4
    assert sdpa.attn_paged_decode_workspace_size(paged(num_splits=-1)) == 0
    assert sdpa.attn_paged_decode_workspace_size(paged(D=100)) == 0


def test_automatic_split_count():
    """num_splits = 0: about 1024 (sequence, KV head, head chunk, split) items
    (4096 from 256 groups up), at least 256 tokens of block-table capacity
    per split, within 1..256; the workspace is that of the explicit count it
    picks."""
    ws = sdpa.attn_paged_decode_workspace_size
    # 4 sequences x 8 KV heads = 32 groups -> 32 splits (capacity 512 x 64 tokens)
    assert ws(paged(num_splits=0, max_blocks_per_seq=512)) == ws(paged(num_splits=32, max_blocks_per_seq=512))
    # one sequence: 8 groups -> 128 splits
    assert ws(paged(B=1, num_splits=0, max_blocks_per_seq=2048)) == \
        ws(paged(B=1, num_splits=128, max_blocks_per_seq=2048))
    # short capacity: 10 x 64 tokens -> 2 splits of at least 256 tokens
    assert ws(paged(num_splits=0)) == ws(paged(num_splits=2))
    # 256 groups and more: about 4096 items; 32 x 8 = 256 groups -> 16 splits
    assert ws(paged(B=32, num_splits=0, max_blocks_per_seq=512)) == \
        ws(paged(B=32, num_splits=16, max_blocks_per_seq=512))
    # 2048 groups -> 2 splits (capacity 10 x 64 tokens allows 2)
    assert ws(paged(B=256, num_splits=0, num_blocks=5000)) == ws(paged(B=256, num_splits=2, num_blocks=5000))
    # 8192 groups -> one split
    assert ws(paged(B=1024, num_splits=0, num_blocks=20000)) == \
        ws(paged(B=1024, num_splits=1, num_blocks=20000))
    # capacity below 256 tokens: one split
    assert ws(paged(num_splits=0, max_blocks_per_seq=3)) == ws(paged(num_splits=1, max_blocks_per_seq=3))


def test_paged_check_accepts_valid_calls():
    assert check_paged(paged()) == OK
    assert check_paged(paged(D=64, dtype=sdpa.ATTN_F16, block_size=16, num_splits=1,
                             softcap=20.0), al=AL, err=ERR) == OK
    assert check_paged(paged(Hkv=32, num_splits=256)) == OK
    assert check_paged(paged(num_splits=0)) == OK  # chosen by the library
    assert check_paged(paged(B=0), q=None, out=None, tab=None, lens=None, ws=None) == OK
    # F32 / F64 (vector-ALU path): any block size, head dims 32 to 256
    assert check_paged(paged(dtype=sdpa.ATTN_F32)) == OK
    assert check_paged(paged(dtype=sdpa.ATTN_F64, D=32, block_size=7)) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), DTYPE), (dict(dtype=sdpa.ATTN_F64, D=80), HEAD_DIM),
    (dict(B=-1), SHAPE), (dict(block_size=0), SHAPE), (dict(B=70000), SHAPE),
    (dict(max_blocks_per_seq=1 << 30), SHAPE),
    (dict(Hkv=5), GQA), (dict(D=32), HEAD_DIM),
    (dict(num_splits=-1), PARAM), (dict(num_splits=257), PARAM),
    (dict(softmax_scale=float("inf")), PARAM), (dict(softcap=-1.0), PARAM),
])
def test_paged_check_rejects(kw, code):
    assert check_paged(paged(**kw)) == code


def test_paged_check_pointers_and_workspace():
    p = paged()
    need = sdpa.attn_paged_decode_workspace_size(p)
    assert check_paged(p, q=None) == NULL
    assert check_paged(p, tab=None) == NULL
    assert check_paged(p, lens=None) == NULL
    assert check_paged(p, k=None) == NULL
    assert check_paged(p, ws=None) == WORKSPACE
    assert check_paged(p, ws_bytes=need - 1) == WORKSPACE
    assert check_paged(p, tab=TAB + 4) == ALIGN
    assert check_paged(p, err=ERR + 2) == ALIGN
    assert check_paged(p, out=KP + 256) == ALIAS
    assert check_paged(p, ws=LEN) == ALIAS
    assert check_paged(p, err=WS + 64) == ALIAS
    assert check_paged(p, out=WS + 1024) == ALIAS


def varlen(**kw):
    base = dict(B=3, Hq=8, Hkv=2, D=128, total_q=500, max_seqlen_q=300, num_blocks=40,
                block_size=64, max_blocks_per_seq=12, dtype=sdpa.ATTN_BF16, causal=1,
                window_left=-1, window_right=-1, softmax_scale=0.088, softcap=0.0)
    base.update(kw)
    return sdpa.attn_varlen_params_t(**base)


CU = 0x100000000 * 13


def check_varlen(p, **kw):
    a = dict(q=Q, kp=KP, vp=VP, tab=TAB, lens=LEN, cu=CU, al=None, out=OUT, err=None)
    a.update(kw)
    return sdpa.attn_paged_prefill_check(a["q"], a["kp"], a["vp"], a["tab"], a["lens"], a["cu"],
                                         a["al"], a["out"], a["err"], p)


def test_paged_prefill_check():
    assert check_varlen(varlen()) == OK
    assert check_varlen(varlen(block_size=128)) == OK
    assert check_varlen(varlen(dtype=sdpa.ATTN_F32)) == OK
    assert check_varlen(varlen(dtype=sdpa.ATTN_F64, block_size=16, D=32)) == OK  # vector-ALU path
    assert check_varlen(varlen(dtype=sdpa.ATTN_F32, D=80)) == HEAD_DIM
    assert check_varlen(varlen(block_size=16)) == UNSUPPORTED    # matrix cores: multiples of 64
    assert check_varlen(varlen(D=80)) == HEAD_DIM
    assert check_varlen(varlen(D=256)) == OK
    assert check_paged(paged(D=256)) == OK
    assert check_paged(paged(D=96)) == HEAD_DIM
    assert check_varlen(varlen(Hq=6, Hkv=4)) == GQA
    assert check_varlen(varlen(window_left=-2)) == PARAM
    assert check_varlen(varlen(softcap=-1.0)) == PARAM
    assert check_varlen(varlen(total_q=-1)) == SHAPE
    assert check_varlen(varlen(), cu=None) == NULL
    assert check_varlen(varlen(), lens=None) == NULL
    assert check_varlen(varlen(total_q=0), q=None, out=None, cu=None, lens=None) == OK
    assert check_varlen(varlen(), cu=CU + 2) == ALIGN
    assert check_varlen(varlen(), q=Q + 8) == ALIGN
    assert check_varlen(varlen(), out=Q) == ALIAS
    assert check_varlen(varlen(), cu=OUT + 64) == ALIAS
    assert check_varlen(None) == NULL
    lib = sdpa.library()
    p = varlen(D=80)
    assert lib.attn_paged_prefill(Q, KP, VP, TAB, LEN, CU, None, OUT, None, ctypes.byref(p), None) == HEAD_DIM


# ------------------------------------------------------------------ backward

DQ, DK, DV, DO, BWS = (0x100000000 * (i + 20) for i in range(5))


def check_bwd(p, q=Q, k=K, v=V, do=DO, al=None, dq=DQ, dk=DK, dv=DV, ws=BWS, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = sdpa.attn_bwd_workspace_size(p)
    return sdpa.attn_bwd_check(q, k, v, do, al, dq, dk, dv, ws, ws_bytes, p)


def test_bwd_check_accepts_valid_calls():
    assert check_bwd(fwd()) == OK
    assert check_bwd(fwd(D=64, dtype=sdpa.ATTN_F16, causal=0, window_left=5, window_right=0,
                         softcap=30.0), al=AL) == OK
    assert check_bwd(fwd(Sq=0), q=None, do=None, dq=None, ws=None, ws_bytes=0) == OK
    # F32 / F64 (vector-ALU backward): head dims 32 to 256
    assert check_bwd(fwd(dtype=sdpa.ATTN_F32)) == OK
    assert check_bwd(fwd(dtype=sdpa.ATTN_F64, D=256)) == OK
    # F16/BF16 (matrix cores): 64, 128 and 256
    for dt in (sdpa.ATTN_BF16, sdpa.ATTN_F16):
        assert check_bwd(fwd(dtype=dt, D=256)) == OK, dt
    assert check_bwd(fwd(dtype=sdpa.ATTN_F64, D=32)) == OK


def test_bwd_workspace_size():
    p = fwd(B=2, Hq=8, Hkv=2, Sq=100, Sk=130)
    # the forward's row statistics: 8 bytes per query row, at least
    assert sdpa.attn_bwd_workspace_size(p) >= 2 * 8 * 100 * 8
    assert sdpa.attn_bwd_workspace_size(fwd(D=80)) == 0
    # F64: two float64 values per query row, no partials
    assert sdpa.attn_bwd_workspace_size(fwd(B=2, Hq=8, Hkv=2, Sq=100, Sk=130, dtype=sdpa.ATTN_F64)) == 2 * 8 * 100 * 16
    assert sdpa.attn_bwd_workspace_size(None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=sdpa.ATTN_F64, D=80), HEAD_DIM),
    (dict(dtype=9), DTYPE), (dict(D=512), HEAD_DIM), (dict(D=32), HEAD_DIM), (dict(Hkv=3), GQA),
    (dict(softcap=-1.0), PARAM), (dict(has_k_len=1, k_len=130), PARAM),
])
def test_bwd_check_rejects(kw, code):
    assert check_bwd(fwd(**kw)) == code


def test_bwd_check_pointers_and_aliasing():
    p = fwd()
    need = sdpa.attn_bwd_workspace_size(p)
    assert check_bwd(p, do=None) == NULL
    assert check_bwd(p, dk=None) == NULL
    assert check_bwd(p, dq=None) == NULL
    assert check_bwd(p, ws=None) == WORKSPACE
    assert check_bwd(p, ws_bytes=need - 1) == WORKSPACE
    assert check_bwd(p, do=DO + 8) == ALIGN
    assert check_bwd(p, ws=BWS + 4) == ALIGN
    assert check_bwd(p, dq=Q + 256) == ALIAS        # an output over an input
    assert check_bwd(p, dk=DO) == ALIAS
    assert check_bwd(p, dv=DK + 64) == ALIAS        # two outputs overlapping
    assert check_bwd(p, ws=DQ + 16) == ALIAS        # workspace over an output
    assert sdpa.attn_bwd_check(Q, K, V, DO, None, DQ, DK, DV, BWS, need, None) == NULL


BO, BL = (0x100000000 * (i + 30) for i in range(2))   # saved forward output and LSE


def check_bwd_lse(p, out=BO, lse=BL, ws_bytes=None, **kw):
    if ws_bytes is None:
        ws_bytes = sdpa.attn_bwd_workspace_size(p)
    a = dict(q=Q, k=K, v=V, do=DO, al=None, dq=DQ, dk=DK, dv=DV, ws=BWS)
    a.update(kw)
    return sdpa.attn_bwd_lse_check(a["q"], a["k"], a["v"], out, lse, a["do"], a["al"], a["dq"],
                                   a["dk"], a["dv"], a["ws"], ws_bytes, p)


def test_bwd_lse_check():
    p = fwd()
    assert check_bwd_lse(p) == OK
    assert check_bwd_lse(p, out=None) == NULL
    assert check_bwd_lse(p, lse=None) == NULL
    assert check_bwd_lse(fwd(Sq=0), out=None, lse=None, q=None, do=None, dq=None, ws=None,
                         ws_bytes=0) == OK
    assert check_bwd_lse(p, out=BO + 8) == ALIGN
    assert check_bwd_lse(p, lse=BL + 2) == ALIGN
    assert check_bwd_lse(p, out=DQ) == ALIAS         # the saved output under a gradient
    assert check_bwd_lse(p, lse=BWS + 16) == ALIAS   # the LSE inside the workspace
    assert check_bwd_lse(p, out=Q) == OK             # read-only inputs may share memory
    # attn_bwd_check's rules come first
    assert check_bwd_lse(fwd(dtype=sdpa.ATTN_F32)) == OK
    assert check_bwd_lse(p, do=None) == NULL
    assert check_bwd_lse(p, ws_bytes=1) == WORKSPACE
    assert sdpa.attn_bwd_lse_check(Q, K, V, BO, BL, DO, None, DQ, DK, DV, BWS, 1 << 30, None) == NULL


def test_noalloc_decode_rejects_sizes_beyond_its_scratch_array():
    """attn_paged_decode_noalloc refuses, before touching the device, a call
    whose split partials would not fit the library's scratch array; the
    pointers here are never dereferenced."""
    lib = sdpa.library()
    fake = ctypes.c_void_p(1 << 20)
    # 512 sequences x 64 heads x 16 splits x (128 + 1) floats = 270 MB > 32 MiB
    p = sdpa.attn_paged_params((512, 64, 1, 128), (9000, 16, 8, 128), 600, sdpa.ATTN_BF16,
                               num_splits=16)
    assert sdpa.attn_paged_decode_workspace_size(p) > sdpa.DECODE_SCRATCH_BYTES
    st = lib.attn_paged_decode_noalloc(fake, fake, fake, fake, fake, None, fake, None,
                                       ctypes.byref(p), None)
    assert st == 9  # ATTN_ERR_WORKSPACE
    assert lib.attn_paged_decode_noalloc(fake, fake, fake, fake, fake, None, fake, None, None,
                                         None) == 1  # ATTN_ERR_NULL: no params
