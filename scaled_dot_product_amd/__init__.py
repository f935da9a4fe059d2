"""Attention forward on AMD Instinct MI355X (gfx950): Python binding of libattn.

The entry points mirror the C ABI of ``include/attn.h`` one to one and only
marshal arguments: tensor pointers, sizes and the caller's stream go to the
HIP library, where every step of the computation runs.  PyTorch supplies the
device memory (and allocates ``out`` / the decode workspace when the caller
does not pass them).  There is no fallback: if ``libattn.so`` is missing or
fails to load, every call raises.

    attn_fwd(q, k, v, alibi=None, out=None, *, softmax_scale=None, causal=False,
             window_left=None, window_right=None, softcap=None, k_len=None, stream=None)
    attn_fwd_lse(q, k, v, alibi=None, out=None, lse=None, *, ...)  -> (out, lse)
    attn_paged_prefill(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q,
                       alibi=None, out=None, *, max_seqlen_q=None, softmax_scale=None,
                       causal=True, window_left=None, window_right=None,
                       softcap=None, error_flag=None, stream=None)
    attn_paged_decode(q, k_pool, v_pool, block_table, seq_lens, alibi=None,
                      out=None, *, softmax_scale=None, softcap=None,
                      num_splits=0, workspace=None, error_flag=None, stream=None)
    attn_paged_decode_noalloc(q, k_pool, v_pool, block_table, seq_lens, alibi=None,
                              out=None, *, softmax_scale=None, softcap=None,
                              num_splits=0, error_flag=None, stream=None)

``num_splits=0`` (the default) lets the library choose the decode's split
count from the shape; a positive value (1..256) is used as given.

For calls repeated on the same tensors (a serving loop that rewrites q,
seq_lens and block_table in place each step), ``PagedDecodePlan`` and
``AttnFwdPlan`` do the checks and the marshalling once; their ``run()`` is one
call into the library.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "AttnError", "library", "LIB_PATH", "PagedDecodePlan", "AttnFwdPlan",
    "attn_fwd", "attn_fwd_check", "attn_fwd_params", "attn_fwd_lse", "attn_fwd_lse_check",
    "attn_paged_decode", "attn_paged_decode_check", "attn_paged_decode_workspace_size",
    "attn_paged_decode_noalloc", "DECODE_SCRATCH_BYTES",
    "attn_paged_params", "attn_status_str", "attn_version",
    "attn_paged_prefill", "attn_paged_prefill_check", "attn_varlen_params",
    "attn_bwd", "attn_bwd_check", "attn_bwd_workspace_size", "attn_bwd_lse", "attn_bwd_lse_check",
    "ATTN_F32", "ATTN_F16", "ATTN_BF16", "ATTN_F64",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_F32, ATTN_F16, ATTN_BF16, ATTN_F64 = 0, 1, 2, 3
_DTYPE_CODE = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16,
               torch.float64: ATTN_F64}

STATUS_NAMES = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_DTYPE", 3: "ATTN_ERR_SHAPE",
    4: "ATTN_ERR_GQA", 5: "ATTN_ERR_HEAD_DIM", 6: "ATTN_ERR_PARAM", 7: "ATTN_ERR_ALIGN",
    8: "ATTN_ERR_ALIAS", 9: "ATTN_ERR_WORKSPACE", 10: "ATTN_ERR_UNSUPPORTED", 11: "ATTN_ERR_HIP",
}


class AttnError(RuntimeError):
    """A non-OK status from libattn (``status`` holds the code)."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({attn_status_str(status)})")


class attn_fwd_params_t(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
                ("Sq", ctypes.c_int64), ("Sk", ctypes.c_int64), ("D", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("window_left", ctypes.c_int64), ("window_right", ctypes.c_int64),
                ("softmax_scale", ctypes.c_float), ("softcap", ctypes.c_float),
                ("k_len", ctypes.c_int64),
                ("has_k_len", ctypes.c_int32)]


class attn_paged_params_t(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
                ("D", ctypes.c_int64), ("num_blocks", ctypes.c_int64),
                ("block_size", ctypes.c_int64), ("max_blocks_per_seq", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("softcap", ctypes.c_float)]


class attn_varlen_params_t(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
                ("D", ctypes.c_int64), ("total_q", ctypes.c_int64), ("max_seqlen_q", ctypes.c_int64),
                ("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int64),
                ("max_blocks_per_seq", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("window_left", ctypes.c_int64),
                ("window_right", ctypes.c_int64), ("softmax_scale", ctypes.c_float),
                ("softcap", ctypes.c_float)]


_lib = None
_VP = ctypes.c_void_p


def library():
    """Load ``libattn.so`` (raises ImportError when it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m scaled_dot_product_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    fwd_p = ctypes.POINTER(attn_fwd_params_t)
    pag_p = ctypes.POINTER(attn_paged_params_t)
    lib.attn_fwd_check.argtypes = [_VP, _VP, _VP, _VP, _VP, fwd_p]
    lib.attn_fwd_check.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [_VP, _VP, _VP, _VP, _VP, fwd_p, _VP]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_lse_check.argtypes = [_VP, _VP, _VP, _VP, _VP, _VP, fwd_p]
    lib.attn_fwd_lse_check.restype = ctypes.c_int
    lib.attn_fwd_lse.argtypes = [_VP, _VP, _VP, _VP, _VP, _VP, fwd_p, _VP]
    lib.attn_fwd_lse.restype = ctypes.c_int
    lib.attn_paged_decode_workspace_size.argtypes = [pag_p]
    lib.attn_paged_decode_workspace_size.restype = ctypes.c_size_t
    lib.attn_paged_decode_check.argtypes = [_VP] * 8 + [ctypes.c_size_t, _VP, pag_p]
    lib.attn_paged_decode_check.restype = ctypes.c_int
    lib.attn_paged_decode.argtypes = [_VP] * 8 + [ctypes.c_size_t, _VP, pag_p, _VP]
    lib.attn_paged_decode.restype = ctypes.c_int
    lib.attn_paged_decode_noalloc.argtypes = [_VP] * 8 + [pag_p, _VP]
    lib.attn_paged_decode_noalloc.restype = ctypes.c_int
    var_p = ctypes.POINTER(attn_varlen_params_t)
    lib.attn_paged_prefill_check.argtypes = [_VP] * 9 + [var_p]
    lib.attn_paged_prefill_check.restype = ctypes.c_int
    lib.attn_paged_prefill.argtypes = [_VP] * 9 + [var_p, _VP]
    lib.attn_paged_prefill.restype = ctypes.c_int
    lib.attn_bwd_workspace_size.argtypes = [fwd_p]
    lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attn_bwd_check.argtypes = [_VP] * 9 + [ctypes.c_size_t, fwd_p]
    lib.attn_bwd_check.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [_VP] * 9 + [ctypes.c_size_t, fwd_p, _VP]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_lse_check.argtypes = [_VP] * 11 + [ctypes.c_size_t, fwd_p]
    lib.attn_bwd_lse_check.restype = ctypes.c_int
    lib.attn_bwd_lse.argtypes = [_VP] * 11 + [ctypes.c_size_t, fwd_p, _VP]
    lib.attn_bwd_lse.restype = ctypes.c_int
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def attn_status_str(status: int) -> str:
    return library().attn_status_str(int(status)).decode()


def attn_version() -> int:
    return int(library().attn_version())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else (t.data_ptr() or None)


def _need_device(name, t, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (materialise the view first)")


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def attn_fwd_params(q_shape, k_shape, dtype, *, softmax_scale=None, causal=False,
                    window_left=None, window_right=None, softcap=None,
                    k_len=None) -> attn_fwd_params_t:
    B, Hq, Sq, D = q_shape
    _, Hkv, Sk, _ = k_shape
    return attn_fwd_params_t(
        B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D,
        dtype=_DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype),
        causal=1 if causal else 0,
        window_left=-1 if window_left is None else int(window_left),
        window_right=-1 if window_right is None else int(window_right),
        softmax_scale=(1.0 / math.sqrt(D)) if softmax_scale is None else float(softmax_scale),
        softcap=0.0 if not softcap else float(softcap),
        k_len=0 if k_len is None else int(k_len),
        has_k_len=0 if k_len is None else 1)


def attn_fwd_check(q_ptr, k_ptr, v_ptr, alibi_ptr, out_ptr, params: attn_fwd_params_t) -> int:
    """Host-only argument check (no HIP call): returns the status code."""
    return int(library().attn_fwd_check(q_ptr, k_ptr, v_ptr, alibi_ptr, out_ptr,
                                        None if params is None else ctypes.byref(params)))


def attn_fwd_lse_check(q_ptr, k_ptr, v_ptr, alibi_ptr, out_ptr, lse_ptr,
                       params: attn_fwd_params_t) -> int:
    """Host-only argument check of attn_fwd_lse (no HIP call): the status code."""
    return int(library().attn_fwd_lse_check(q_ptr, k_ptr, v_ptr, alibi_ptr, out_ptr, lse_ptr,
                                            None if params is None else ctypes.byref(params)))


def _fwd_args(q, k, v, alibi, out, softmax_scale, causal, window_left, window_right, softcap,
              k_len=None):
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("alibi", alibi), ("out", out)):
        _need_device(name, t, dev)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, Hq, Sq, D]; k and v the same [B, Hkv, Sk, D]")
    if k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("batch and head dim of k/v must match q")
    if k.dtype != q.dtype or v.dtype != q.dtype or q.dtype not in _DTYPE_CODE:
        raise ValueError("q, k, v must share one dtype of float32 / float64 / float16 / bfloat16")
    if alibi is not None and (alibi.dtype != torch.float32 or alibi.shape != (q.shape[1],)):
        raise ValueError("alibi slopes must be float32 [Hq]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    p = attn_fwd_params(tuple(q.shape), tuple(k.shape), q.dtype, softmax_scale=softmax_scale,
                        causal=causal, window_left=window_left, window_right=window_right,
                        softcap=softcap, k_len=k_len)
    return dev, out, p


def attn_fwd(q, k, v, alibi=None, out=None, *, softmax_scale=None, causal=False,
             window_left=None, window_right=None, softcap=None, k_len=None, stream=None):
    """Attention forward over ``[B, H, S, D]`` device tensors (see attn.h);
    ``k_len`` (optional) is the live key prefix: only keys ``j < k_len`` exist."""
    lib = library()
    dev, out, p = _fwd_args(q, k, v, alibi, out, softmax_scale, causal, window_left,
                            window_right, softcap, k_len)
    st = lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alibi), _ptr(out), ctypes.byref(p),
                      _stream_handle(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_fwd")
    return out


def attn_fwd_lse(q, k, v, alibi=None, out=None, lse=None, *, softmax_scale=None, causal=False,
                 window_left=None, window_right=None, softcap=None, k_len=None, stream=None):
    """As :func:`attn_fwd`, and also the float32 ``[B, Hq, Sq]`` natural-log
    log-sum-exp of every row (``-inf`` for rows with no admissible key).
    Returns ``(out, lse)``."""
    lib = library()
    dev, out, p = _fwd_args(q, k, v, alibi, out, softmax_scale, causal, window_left,
                            window_right, softcap, k_len)
    _need_device("lse", lse, dev)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    elif lse.shape != q.shape[:3] or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hq, Sq]")
    st = lib.attn_fwd_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(alibi), _ptr(out), _ptr(lse),
                          ctypes.byref(p), _stream_handle(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_fwd_lse")
    return out, lse


def attn_bwd_workspace_size(params: attn_fwd_params_t) -> int:
    return int(library().attn_bwd_workspace_size(None if params is None else ctypes.byref(params)))


def attn_bwd_check(q_ptr, k_ptr, v_ptr, do_ptr, alibi_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr,
                   ws_bytes, params: attn_fwd_params_t) -> int:
    """Host-only argument check of attn_bwd (no HIP call): the status code."""
    return int(library().attn_bwd_check(q_ptr, k_ptr, v_ptr, do_ptr, alibi_ptr, dq_ptr, dk_ptr,
                                        dv_ptr, ws_ptr, ws_bytes,
                                        None if params is None else ctypes.byref(params)))


def attn_bwd(q, k, v, dout, alibi=None, *, softmax_scale=None, causal=False, window_left=None,
             window_right=None, softcap=None, dq=None, dk=None, dv=None, workspace=None,
             stream=None):
    """Gradients ``(dq, dk, dv)`` of :func:`attn_fwd` for the upstream gradient
    ``dout`` (see attn.h); dk/dv are summed over each KV head's query group."""
    lib = library()
    # (q stands in for the forward's output: only its shape and dtype are checked)
    dev, _, p = _fwd_args(q, k, v, alibi, q, softmax_scale, causal, window_left,
                          window_right, softcap)
    for name, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv), ("workspace", workspace)):
        _need_device(name, t, dev)
    if dout.shape != q.shape or dout.dtype != q.dtype:
        raise ValueError("dout must match q in shape and dtype")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{name} must match the shape and dtype of its input")
    need = attn_bwd_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(alibi), _ptr(dq), _ptr(dk),
                      _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(),
                      ctypes.byref(p), _stream_handle(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv


def attn_bwd_lse_check(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, do_ptr, alibi_ptr, dq_ptr, dk_ptr,
                       dv_ptr, ws_ptr, ws_bytes, params) -> int:
    """Host-only validation of an attn_bwd_lse call on raw pointers (see attn.h)."""
    return int(library().attn_bwd_lse_check(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, do_ptr, alibi_ptr,
                                            dq_ptr, dk_ptr, dv_ptr, ws_ptr, ws_bytes,
                                            None if params is None else ctypes.byref(params)))


def attn_bwd_lse(q, k, v, out, lse, dout, alibi=None, *, softmax_scale=None, causal=False,
                 window_left=None, window_right=None, softcap=None, dq=None, dk=None, dv=None,
                 workspace=None, stream=None):
    """Gradients ``(dq, dk, dv)`` from a saved forward: ``out`` and ``lse`` are what
    :func:`attn_fwd_lse` returned for the same inputs and options (see attn.h)."""
    lib = library()
    dev, _, p = _fwd_args(q, k, v, alibi, q, softmax_scale, causal, window_left,
                          window_right, softcap)
    for name, t in (("out", out), ("lse", lse), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv),
                    ("workspace", workspace)):
        _need_device(name, t, dev)
    for name, t in (("out", out), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:3]) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, Hq, Sq] tensor")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{name} must match the shape and dtype of its input")
    need = attn_bwd_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = lib.attn_bwd_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(alibi),
                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), ctypes.byref(p),
                          _stream_handle(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_bwd_lse")
    return dq, dk, dv


def attn_paged_params(q_shape, pool_shape, max_blocks_per_seq, dtype, *, softmax_scale=None,
                      softcap=None, num_splits=0) -> attn_paged_params_t:
    B, Hq, _, D = q_shape
    num_blocks, block_size, Hkv, _ = pool_shape
    return attn_paged_params_t(
        B=B, Hq=Hq, Hkv=Hkv, D=D, num_blocks=num_blocks, block_size=block_size,
        max_blocks_per_seq=max_blocks_per_seq,
        dtype=_DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype),
        num_splits=int(num_splits),
        softmax_scale=(1.0 / math.sqrt(D)) if softmax_scale is None else float(softmax_scale),
        softcap=0.0 if not softcap else float(softcap))


def attn_paged_decode_workspace_size(params: attn_paged_params_t) -> int:
    return int(library().attn_paged_decode_workspace_size(ctypes.byref(params)))


def attn_paged_decode_check(q_ptr, k_ptr, v_ptr, table_ptr, lens_ptr, alibi_ptr, out_ptr,
                            ws_ptr, ws_bytes, err_ptr, params: attn_paged_params_t) -> int:
    """Host-only argument check (no HIP call): returns the status code."""
    return int(library().attn_paged_decode_check(q_ptr, k_ptr, v_ptr, table_ptr, lens_ptr,
                                                 alibi_ptr, out_ptr, ws_ptr, ws_bytes, err_ptr,
                                                 None if params is None else ctypes.byref(params)))


def _paged_decode_args(q, k_pool, v_pool, block_table, seq_lens, alibi, out, workspace, error_flag,
                       softmax_scale, softcap, num_splits):
    """Shared marshalling of the two decode entry points: device, dtype and
    shape agreement of the tensors, the params struct, and `out`."""
    dev = q.device
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool),
                    ("block_table", block_table), ("seq_lens", seq_lens), ("alibi", alibi),
                    ("out", out), ("workspace", workspace), ("error_flag", error_flag)):
        _need_device(name, t, dev)
    if q.dim() != 4 or q.shape[2] != 1:
        raise ValueError("q must be [B, Hq, 1, D]")
    if k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("pools must both be [num_blocks, block_size, Hkv, D]")
    if k_pool.shape[3] != q.shape[3]:
        raise ValueError("pool head dim must match q")
    if k_pool.dtype != q.dtype or v_pool.dtype != q.dtype or q.dtype not in _DTYPE_CODE:
        raise ValueError("q and the pools must share one dtype")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != q.shape[0]:
        raise ValueError("block_table must be int32 [B, max_blocks_per_seq]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q.shape[0],):
        raise ValueError("seq_lens must be int32 [B]")
    if alibi is not None and (alibi.dtype != torch.float32 or alibi.shape != (q.shape[1],)):
        raise ValueError("alibi slopes must be float32 [Hq]")
    if error_flag is not None and (error_flag.dtype != torch.int32 or error_flag.numel() != 1):
        raise ValueError("error_flag must be one int32")
    p = attn_paged_params(tuple(q.shape), tuple(k_pool.shape), block_table.shape[1], q.dtype,
                          softmax_scale=softmax_scale, softcap=softcap, num_splits=num_splits)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    return p, out


def attn_paged_decode(q, k_pool, v_pool, block_table, seq_lens, alibi=None, out=None, *,
                      softmax_scale=None, softcap=None, num_splits=0, workspace=None,
                      error_flag=None, stream=None):
    """Paged split-KV decode, one query per sequence (see attn.h)."""
    lib = library()
    dev = q.device
    p, out = _paged_decode_args(q, k_pool, v_pool, block_table, seq_lens, alibi, out, workspace,
                                error_flag, softmax_scale, softcap, num_splits)
    need = attn_paged_decode_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.attn_paged_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                               _ptr(seq_lens), _ptr(alibi), _ptr(out), _ptr(workspace), ws_bytes,
                               _ptr(error_flag), ctypes.byref(p), _stream_handle(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_paged_decode")
    return out


class PagedDecodePlan:
    """``attn_paged_decode`` with its arguments checked and marshalled once.

    Takes the arguments of :func:`attn_paged_decode` and keeps references to
    its tensors (``out`` and the workspace are allocated here when not given).
    Between runs the caller may change the tensors' contents in place -- the
    next token's ``q``, longer ``seq_lens``, new ``block_table`` entries --
    but never their shapes, dtypes or storage.  ``run()`` makes the one C call
    (which still validates the arguments host-side) on the stream given here
    and returns ``out``.  The host cost per step is then that call alone, not
    the per-call Python checks.
    """

    def __init__(self, q, k_pool, v_pool, block_table, seq_lens, alibi=None, out=None, *,
                 softmax_scale=None, softcap=None, num_splits=0, workspace=None,
                 error_flag=None, stream=None):
        lib = library()
        dev = q.device
        p, out = _paged_decode_args(q, k_pool, v_pool, block_table, seq_lens, alibi, out,
                                    workspace, error_flag, softmax_scale, softcap, num_splits)
        need = attn_paged_decode_workspace_size(p)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
        ptrs = (_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
                _ptr(alibi), _ptr(out), _ptr(workspace))
        st = lib.attn_paged_decode_check(*ptrs, ws_bytes, _ptr(error_flag), ctypes.byref(p))
        if st != 0:
            raise AttnError(st, "attn_paged_decode")
        self.out = out
        self._keep = (q, k_pool, v_pool, block_table, seq_lens, alibi, workspace, error_flag, p)
        self._fn = lib.attn_paged_decode
        self._args = (*ptrs, ws_bytes, _ptr(error_flag), ctypes.byref(p), _stream_handle(stream, dev))

    def run(self):
        st = self._fn(*self._args)
        if st != 0:
            raise AttnError(st, "attn_paged_decode")
        return self.out


class AttnFwdPlan:
    """``attn_fwd`` with its arguments checked and marshalled once (the same
    contract as :class:`PagedDecodePlan`: tensors keep their shapes and
    storage between runs; ``run()`` is one C call on the stream given here and
    returns ``out``)."""

    def __init__(self, q, k, v, alibi=None, out=None, *, softmax_scale=None, causal=False,
                 window_left=None, window_right=None, softcap=None, k_len=None, stream=None):
        lib = library()
        dev, out, p = _fwd_args(q, k, v, alibi, out, softmax_scale, causal, window_left,
                                window_right, softcap, k_len)
        ptrs = (_ptr(q), _ptr(k), _ptr(v), _ptr(alibi), _ptr(out))
        st = lib.attn_fwd_check(*ptrs, ctypes.byref(p))
        if st != 0:
            raise AttnError(st, "attn_fwd")
        self.out = out
        self._keep = (q, k, v, alibi, p)
        self._fn = lib.attn_fwd
        self._args = (*ptrs, ctypes.byref(p), _stream_handle(stream, dev))

    def run(self):
        st = self._fn(*self._args)
        if st != 0:
            raise AttnError(st, "attn_fwd")
        return self.out


DECODE_SCRATCH_BYTES = 32 << 20  # ATTN_DECODE_SCRATCH_BYTES in attn.h


def attn_paged_decode_noalloc(q, k_pool, v_pool, block_table, seq_lens, alibi=None, out=None, *,
                              softmax_scale=None, softcap=None, num_splits=0, error_flag=None,
                              stream=None):
    """attn_paged_decode without a workspace argument: the library's
    device-resident scratch array (DECODE_SCRATCH_BYTES per GPU) serves as it,
    so the call allocates nothing when `out` is given (see attn.h; calls that
    overlap in time on one GPU race on that array)."""
    lib = library()
    dev = q.device
    p, out = _paged_decode_args(q, k_pool, v_pool, block_table, seq_lens, alibi, out, None,
                                error_flag, softmax_scale, softcap, num_splits)
    st = lib.attn_paged_decode_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                       _ptr(seq_lens), _ptr(alibi), _ptr(out), _ptr(error_flag),
                                       ctypes.byref(p), _stream_handle(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_paged_decode_noalloc")
    return out


def attn_varlen_params(q_shape, pool_shape, B, max_blocks_per_seq, max_seqlen_q, dtype, *,
                       softmax_scale=None, causal=True, window_left=None, window_right=None,
                       softcap=None) -> attn_varlen_params_t:
    total_q, Hq, D = q_shape
    num_blocks, block_size, Hkv, _ = pool_shape
    return attn_varlen_params_t(
        B=B, Hq=Hq, Hkv=Hkv, D=D, total_q=total_q, max_seqlen_q=int(max_seqlen_q),
        num_blocks=num_blocks, block_size=block_size, max_blocks_per_seq=max_blocks_per_seq,
        dtype=_DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype),
        causal=1 if causal else 0,
        window_left=-1 if window_left is None else int(window_left),
        window_right=-1 if window_right is None else int(window_right),
        softmax_scale=(1.0 / math.sqrt(D)) if softmax_scale is None else float(softmax_scale),
        softcap=0.0 if not softcap else float(softcap))


def attn_paged_prefill_check(q_ptr, kp_ptr, vp_ptr, table_ptr, lens_ptr, cu_ptr, alibi_ptr,
                             out_ptr, err_ptr, params: attn_varlen_params_t) -> int:
    """Host-only argument check of attn_paged_prefill (no HIP call)."""
    return int(library().attn_paged_prefill_check(
        q_ptr, kp_ptr, vp_ptr, table_ptr, lens_ptr, cu_ptr, alibi_ptr, out_ptr, err_ptr,
        None if params is None else ctypes.byref(params)))


def attn_paged_prefill(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, alibi=None,
                       out=None, *, max_seqlen_q=None, softmax_scale=None, causal=True,
                       window_left=None, window_right=None, softcap=None, error_flag=None,
                       stream=None):
    """Variable-length prefill over the paged pool (see attn.h).  ``q`` and
    ``out`` are packed ``[total_q, Hq, D]``; pass ``max_seqlen_q`` to avoid
    reading ``cu_seqlens_q`` back to the host."""
    lib = library()
    dev = q.device
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool),
                    ("block_table", block_table), ("seq_lens", seq_lens),
                    ("cu_seqlens_q", cu_seqlens_q), ("alibi", alibi), ("out", out),
                    ("error_flag", error_flag)):
        _need_device(name, t, dev)
    if q.dim() != 3:
        raise ValueError("q must be packed [total_q, Hq, D]")
    if k_pool.dim() != 4 or v_pool.shape != k_pool.shape or k_pool.shape[3] != q.shape[2]:
        raise ValueError("pools must both be [num_blocks, block_size, Hkv, D] with q's D")
    if k_pool.dtype != q.dtype or v_pool.dtype != q.dtype or q.dtype not in _DTYPE_CODE:
        raise ValueError("q and the pools must share one dtype")
    B = seq_lens.shape[0] if seq_lens.dim() == 1 else -1
    if seq_lens.dtype != torch.int32 or B < 0:
        raise ValueError("seq_lens must be int32 [B]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_blocks_per_seq]")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_q.shape != (B + 1,):
        raise ValueError("cu_seqlens_q must be int32 [B + 1]")
    if alibi is not None and (alibi.dtype != torch.float32 or alibi.shape != (q.shape[1],)):
        raise ValueError("alibi slopes must be float32 [Hq]")
    if error_flag is not None and (error_flag.dtype != torch.int32 or error_flag.numel() != 1):
        raise ValueError("error_flag must be one int32")
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if B > 0 else 0
    p = attn_varlen_params(tuple(q.shape), tuple(k_pool.shape), B, block_table.shape[1],
                           max_seqlen_q, q.dtype, softmax_scale=softmax_scale, causal=causal,
                           window_left=window_left, window_right=window_right, softcap=softcap)
    if out is None:
        out = torch.zeros_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    st = lib.attn_paged_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                _ptr(seq_lens), _ptr(cu_seqlens_q), _ptr(alibi), _ptr(out),
                                _ptr(error_flag), ctypes.byref(p), _stream_handle(stream, dev))
    if st != 0:
        raise AttnError(st, "attn_paged_prefill")
    return out
