"""Write ``tiny_cases.json``: tiny attention problems with 50-digit expected
outputs from :mod:`oracle.bruteforce` (the only code this script calls).

Inputs are multiples of 1/8 in [-2, 2], exactly representable in float64,
float32, bfloat16 and float16, so every side of a comparison sees the same
operands.  Each case names the passage of the pages it exercises:
"kernel contracts" is the fuel-reference-backend attention kernel-contract
page; "derivation" is "gfx942 unified attention, from the math up".

Run from the repository root:  python tests/golden/make_golden.py
"""
from __future__ import annotations

import json
import os
import random
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.bruteforce import paged_bruteforce, sdpa_bruteforce  # noqa: E402


def _t(rng, *shape):
    if len(shape) == 1:
        return [rng.randint(-16, 16) / 8 for _ in range(shape[0])]
    return [_t(rng, *shape[1:]) for _ in range(shape[0])]


DENSE = [
    # name, citation, B, Hq, Hkv, Sq, Sk, D, scale, causal, left, right, softcap, alibi
    ("mha_noncausal", "kernel contracts, attention_naive: softmax over all keys",
     1, 2, 2, 5, 5, 3, 0.5, False, None, None, None, False),
    ("gqa_causal_square", "kernel contracts, attention_naive: causal mask, GQA broadcast",
     1, 4, 2, 6, 6, 4, 0.5, True, None, None, None, False),
    ("causal_bottom_right_sq_lt_sk", "derivation section 4: bottom-right causal when Sq != Sk",
     2, 2, 1, 3, 6, 2, 0.75, True, None, None, None, False),
    ("causal_sq_gt_sk_masked_rows", "derivation section 4 + kernel contracts: rows with no key are zero",
     1, 2, 2, 6, 4, 2, 0.5, True, None, None, None, False),
    ("window_left2_right1", "kernel contracts, attention_naive: sliding window",
     1, 2, 2, 6, 6, 3, 0.5, False, 2, 1, None, False),
    ("causal_window_softcap_alibi", "kernel contracts, attention_naive: softcap then ALiBi, windowed causal",
     1, 2, 1, 6, 6, 3, 1.0, True, 1, 0, 0.7, True),
    ("softcap_large_scale", "kernel contracts, attention_naive: softcap c*tanh(s/c)",
     1, 1, 1, 4, 5, 3, 4.0, False, None, None, 1.5, False),
    ("alibi_sq_ne_sk", "kernel contracts: ALiBi slope*(j - i) at the bottom-right aligned position",
     1, 2, 2, 3, 5, 2, 0.5, False, None, None, None, True),
]


def main():
    rng = random.Random(20261202)
    cases = []
    for (name, cite, B, Hq, Hkv, Sq, Sk, D, scale, causal, left, right, cap, use_alibi) in DENSE:
        q = _t(rng, B, Hq, Sq, D)
        k = _t(rng, B, Hkv, Sk, D)
        v = _t(rng, B, Hkv, Sk, D)
        alibi = [2.0 ** (-(h + 1)) for h in range(Hq)] if use_alibi else None
        out = sdpa_bruteforce(q, k, v, scale=scale, causal=causal, window_left=left,
                              window_right=right, softcap=cap, alibi=alibi)
        cases.append(dict(kind="dense", name=name, cite=cite, scale=scale, causal=causal,
                          window_left=left, window_right=right, softcap=cap, alibi=alibi,
                          q=q, k=k, v=v, expected=json.loads(json.dumps(out, default=str))))
    # Paged: two sequences over a shuffled pool of 2-slot blocks, one of them empty.
    bs, Hq, Hkv, D = 2, 2, 1, 3
    seq_lens = [3, 4, 0]
    nblk = [(c + bs - 1) // bs for c in seq_lens]
    perm = list(range(sum(nblk)))
    rng.shuffle(perm)
    table, pos = [], 0
    for n in nblk:
        table.append(perm[pos:pos + n] + [-1] * (2 - n))
        pos += n
    kp = _t(rng, sum(nblk), bs, Hkv, D)
    vp = _t(rng, sum(nblk), bs, Hkv, D)
    q = _t(rng, len(seq_lens), Hq, 1, D)
    for cap, name in ((None, "paged_decode"), (0.9, "paged_decode_softcap")):
        out = paged_bruteforce(q, kp, vp, table, seq_lens, scale=0.5, softcap=cap)
        cases.append(dict(kind="paged", name=name,
                          cite="kernel contracts, attention_paged_naive: block-table gather, "
                               "implicit causal at seq_len - Sq + i; empty sequence gives zero",
                          scale=0.5, softcap=cap, q=q, k_pool=kp, v_pool=vp, block_table=table,
                          seq_lens=seq_lens, expected=json.loads(json.dumps(out, default=str))))
    with open(os.path.join(HERE, "tiny_cases.json"), "w") as f:
        json.dump({"generator": "tests/golden/make_golden.py (oracle.bruteforce, 50 digits)",
                   "cases": cases}, f, indent=1)
    print(f"wrote {len(cases)} cases")


if __name__ == "__main__":
    main()
