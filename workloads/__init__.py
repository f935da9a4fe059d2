"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, and both the oracle side and the HIP side of the tests
(and the benchmark) take their inputs from here.

Recipe (stated once, used everywhere):

* ``numpy.random.default_rng(seed)``; the default seed of a workload is
  ``1000 + id`` (workload 2b reuses workload 2's draws).
* Dense workloads: float32 ``standard_normal`` drawn in the order Q, K, V,
  each ``[B, H, S, D]`` row-major, multiplied by the workload's ``amp``, then
  rounded to the working dtype with round-to-nearest-even (``torch`` cast).
* Paged workloads: ``seq_lens`` drawn uniform on ``[ctx_lo, ctx_hi]``
  (inclusive), then a random permutation of the ``sum ceil(ctx/bs)`` physical
  blocks, then Q ``[B, Hq, 1, D]`` and the K and V pools
  ``[num_blocks, bs, Hkv, D]`` (every slot, including the unused tail of each
  sequence's last block), all ``standard_normal``.  ``block_table`` is int32
  ``[B, max_blocks]`` holding the permuted block ids in logical order and -1
  past each sequence's last block.
* ALiBi slopes, when a workload uses them, are float32
  ``2 ** (-8 (h + 1) / Hq)``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

_TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Dense:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    D: int
    causal: bool
    window_left: Optional[int] = None
    window_right: Optional[int] = None
    softcap: Optional[float] = None
    alibi: bool = False
    amp: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


@dataclasses.dataclass(frozen=True)
class Paged:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    ctx_lo: int
    ctx_hi: int
    num_splits: int
    max_blocks: int
    softcap: Optional[float] = None
    alibi: bool = False
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


# The five workloads, plus 2b (the fully-masked-rows variant of 2).
TINY_F32 = Dense("tiny_f32_mha_s128_d64", "f32", 1, 4, 4, 128, 128, 64, causal=False, seed=1001)
GQA_CAUSAL_2K = Dense("gqa_causal_bf16_b2_h32x8_s2048_d128", "bf16", 2, 32, 8, 2048, 2048, 128,
                      causal=True, seed=1002)
GQA_MASKED_ROWS = Dense("gqa_causal_window512_bf16_b2_h32x8_sq2048_sk1984_d128", "bf16", 2, 32, 8,
                        2048, 1984, 128, causal=True, window_left=512, window_right=0, seed=1002)
LONG_MASKED_8K = Dense("long_causal_win4096_softcap50_alibi_bf16_b1_h32x8_s8192_d128", "bf16", 1,
                       32, 8, 8192, 8192, 128, causal=True, window_left=4096, window_right=0,
                       softcap=50.0, alibi=True, amp=1.5, seed=1003)
PAGED_DECODE = Paged("paged_decode_bf16_b64_h32x8_d128_ctx512-8192_bs64_split8", "bf16", 64, 32, 8,
                     128, 64, 512, 8192, 8, 128, seed=1004)
CHUNKED_PREFILL = Dense("chunked_prefill_f16_b4_h16_sq512_sk4096_d64", "f16", 4, 16, 16, 512, 4096,
                        64, causal=True, seed=1005)

WORKLOADS = {w.name: w for w in (TINY_F32, GQA_CAUSAL_2K, GQA_MASKED_ROWS, LONG_MASKED_8K,
                                 PAGED_DECODE, CHUNKED_PREFILL)}


def alibi_slopes(Hq: int) -> np.ndarray:
    return np.asarray([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=np.float32)


def cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 NumPy -> torch CPU tensor of ``dtype`` (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(_TORCH_DTYPE[dtype])


def dense_inputs(w: Dense, seed: Optional[int] = None):
    """``(q, k, v, alibi)`` torch CPU tensors for a dense workload.  Workload 2b
    draws workload 2's full-length K/V and keeps the first ``Sk`` keys."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    sk_draw = w.Sk
    if w is GQA_MASKED_ROWS:
        sk_draw = GQA_CAUSAL_2K.Sk
    q = rng.standard_normal((w.B, w.Hq, w.Sq, w.D), dtype=np.float32) * np.float32(w.amp)
    k = rng.standard_normal((w.B, w.Hkv, sk_draw, w.D), dtype=np.float32) * np.float32(w.amp)
    v = rng.standard_normal((w.B, w.Hkv, sk_draw, w.D), dtype=np.float32) * np.float32(w.amp)
    k, v = k[:, :, :w.Sk], v[:, :, :w.Sk]
    alibi = torch.from_numpy(alibi_slopes(w.Hq)) if w.alibi else None
    return cast(q, w.dtype), cast(k, w.dtype), cast(v, w.dtype), alibi


def random_dense(dtype, B, Hq, Hkv, Sq, Sk, D, seed, amp=1.0):
    """Ad-hoc dense case with the same recipe (tests of edge shapes)."""
    rng = np.random.default_rng(seed)
    if dtype == "f64":  # drawn in float64 directly: full 53-bit inputs
        q = rng.standard_normal((B, Hq, Sq, D)) * amp
        k = rng.standard_normal((B, Hkv, Sk, D)) * amp
        v = rng.standard_normal((B, Hkv, Sk, D)) * amp
        return torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)
    q = rng.standard_normal((B, Hq, Sq, D), dtype=np.float32) * np.float32(amp)
    k = rng.standard_normal((B, Hkv, Sk, D), dtype=np.float32) * np.float32(amp)
    v = rng.standard_normal((B, Hkv, Sk, D), dtype=np.float32) * np.float32(amp)
    return cast(q, dtype), cast(k, dtype), cast(v, dtype)


def paged_layout(seq_lens: np.ndarray, block_size: int, max_blocks: int, rng):
    """``(block_table int32 [B, max_blocks], num_blocks)`` with the blocks of
    all sequences randomly permuted over one shared pool."""
    nblk = [(int(c) + block_size - 1) // block_size for c in seq_lens]
    if max(nblk, default=0) > max_blocks:
        raise ValueError("a sequence needs more blocks than max_blocks")
    num_blocks = int(sum(nblk))
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((len(seq_lens), max_blocks), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, num_blocks


def paged_inputs(w: Paged, seed: Optional[int] = None, seq_lens=None):
    """``(q, k_pool, v_pool, block_table, seq_lens, alibi)`` torch CPU tensors
    for a paged decode workload (``seq_lens`` may be given to override the
    drawn lengths; the rest of the recipe is unchanged)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    if seq_lens is None:
        seq_lens = rng.integers(w.ctx_lo, w.ctx_hi + 1, size=w.B).astype(np.int32)
    else:
        seq_lens = np.asarray(seq_lens, dtype=np.int32)
    table, num_blocks = paged_layout(seq_lens, w.block_size, w.max_blocks, rng)
    q = rng.standard_normal((w.B, w.Hq, 1, w.D), dtype=np.float32)
    kp = rng.standard_normal((max(num_blocks, 1), w.block_size, w.Hkv, w.D), dtype=np.float32)
    vp = rng.standard_normal((max(num_blocks, 1), w.block_size, w.Hkv, w.D), dtype=np.float32)
    alibi = torch.from_numpy(alibi_slopes(w.Hq)) if w.alibi else None
    return (cast(q, w.dtype), cast(kp, w.dtype), cast(vp, w.dtype),
            torch.from_numpy(table), torch.from_numpy(seq_lens), alibi)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a (CPU or device) tensor to a float64 NumPy array."""
    return t.detach().to("cpu", torch.float64).numpy()
