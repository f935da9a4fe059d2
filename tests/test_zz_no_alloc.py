"""attn_paged_decode_noalloc: the allocation-free decode entry point (its
workspace is the library's device-resident scratch array) against
attn_paged_decode with a caller-allocated workspace, through the C ABI.

Both run the same kernels on the same inputs, so the outputs must be
bitwise equal; they are also checked against the float64 oracle.  Two calls
in a row, the second with a smaller input, for each decode form that uses a
workspace: the split persistent kernel (fewer (sequence, KV head) groups than
compute units) and the partial kernel (B > 4096)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, compare

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

# dtype, B, Hq, Hkv, D, block_size, max len, splits, softcap, alibi
FORMS = {
    "split persistent": [("bf16", 8, 32, 8, 128, 64, 900, 8, None, False),
                         ("bf16", 3, 16, 4, 128, 16, 300, 4, 20.0, True)],
    "partial kernel": [("f16", 4200, 4, 2, 128, 16, 40, 2, None, True),
                       ("f16", 4100, 2, 2, 64, 32, 30, 3, None, False)],
}


def lens_for(B, hi, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, hi + 1, size=B)
    lens[:3] = [0, 1, hi]
    return lens.astype(np.int32).tolist()


@pytest.mark.parametrize("form", list(FORMS))
def test_noalloc_decode_matches_allocating_entry_point(gpu_lib, form):
    sdpa = gpu_lib
    for call, (dtype, B, Hq, Hkv, D, bs, hi, splits, cap, use_alibi) in enumerate(FORMS[form]):
        lens = lens_for(B, hi, 700 + call)
        maxb = (max(lens) + bs - 1) // bs + 1
        w = W.Paged("n", dtype, B, Hq, Hkv, D, bs, 0, 0, splits, maxb, seed=710 + call)
        q, kp, vp, table, sl, _ = W.paged_inputs(w, seq_lens=lens)
        alibi = torch.from_numpy(W.alibi_slopes(Hq)) if use_alibi else None
        args = [t.to(DEV) for t in (q, kp, vp, table, sl)]
        al = None if alibi is None else alibi.to(DEV)
        kw = dict(softmax_scale=D ** -0.5, softcap=cap, num_splits=splits)
        announce(f"noalloc decode, {form}, call {call}: {FORMS[form][call]}")
        flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        out_n = torch.full_like(args[0], float("nan"))
        sdpa.attn_paged_decode_noalloc(*args, al, out_n, error_flag=flag, **kw)
        out_a = sdpa.attn_paged_decode(*args, al, **kw)
        torch.cuda.synchronize()
        assert flag.item() == 0
        assert torch.equal(out_n, out_a), f"{form} call {call}: differs from attn_paged_decode"
        ref = oracle.paged_decode_f64(W.to_f64(q), W.to_f64(kp), W.to_f64(vp), table.numpy(),
                                      sl.numpy(), alibi=None if alibi is None else W.to_f64(alibi),
                                      scale=D ** -0.5, softcap=cap)
        compare(out_n, ref, {"bf16": torch.bfloat16, "f16": torch.float16}[dtype],
                f"noalloc {form} call {call}")
