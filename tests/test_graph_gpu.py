"""The library's launches under HIP graph capture (torch.cuda.CUDAGraph).

Host launch overhead dominates short decode and prefill calls (derivation
page, the section on host overhead and graph replay), so callers capture them.
Every buffer is allocated before capture and the library issues no memset or
allocation of its own; each replay is checked bitwise against the eager
result, with eager work and synchronisation between replays, and the first
replay's outputs are checked against the float64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import announce, compare

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager(gpu_lib):
    sdpa = gpu_lib
    dev = torch.device("cuda:0")
    announce("graph capture: attn_fwd + attn_fwd_lse + attn_paged_decode (split and fused forms)")
    q, k, v = W.random_dense("bf16", 1, 8, 2, 200, 300, 128, 41, 1.0)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(q)
    out2 = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, kp, vp, table, lens, _ = W.paged_inputs(W.PAGED_DECODE, seed=42, seq_lens=[700, 1500, 64, 3000])
    dq, kp, vp = dq[:4].to(dev), kp.to(dev), vp.to(dev)
    table, lens = table[:4].to(dev), lens.to(dev)
    dout = torch.empty_like(dq)
    p = sdpa.attn_paged_params(tuple(dq.shape), tuple(kp.shape), table.shape[1], dq.dtype, num_splits=8)
    ws = torch.zeros(sdpa.attn_paged_decode_workspace_size(p), dtype=torch.uint8, device=dev)
    # a batch of 64 sequences x 4 KV heads = 256 groups: the fused persistent decode
    ww = W.Paged("g", "bf16", 64, 8, 4, 128, 16, 1, 500, 8, 40, seed=43)
    wq, wkp, wvp, wtab, wlens, _ = W.paged_inputs(ww)
    wq, wkp, wvp, wtab, wlens = (t.to(dev) for t in (wq, wkp, wvp, wtab, wlens))
    wout = torch.empty_like(wq)
    scale = 1.0 / np.sqrt(128)

    def work():
        sdpa.attn_fwd(q, k, v, None, out, softmax_scale=scale, causal=True)
        sdpa.attn_fwd_lse(q, k, v, None, out2, lse, softmax_scale=scale, causal=True, window_left=64)
        sdpa.attn_paged_decode(dq, kp, vp, table, lens, None, dout, softmax_scale=scale,
                               num_splits=8, workspace=ws)
        sdpa.attn_paged_decode(wq, wkp, wvp, wtab, wlens, None, wout, softmax_scale=scale)

    work()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, out2, lse, dout, wout)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm up on the capture stream
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (out, out2, lse, dout, wout):
            t.fill_(7.0)                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("out", "out_lse", "lse", "decode", "decode_wide"),
                                   (out, out2, lse, dout, wout), eager):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from eager"
        if rep == 0:
            check_against_oracle(q, k, v, out, out2, lse, scale, (dq, kp, vp, table, lens, dout),
                                 (wq, wkp, wvp, wtab, wlens, wout))


def check_against_oracle(q, k, v, out, out2, lse, scale, dec, wide):
    """The replayed outputs against the float64 oracle, at the parity bars of
    the eager tests (bf16 outputs; LSE within 2^-8 + 1e-4)."""
    f = float(np.float32(scale))
    q64, k64, v64 = W.to_f64(q), W.to_f64(k), W.to_f64(v)
    compare(out, oracle.sdpa_naive_f64(q64, k64, v64, scale=f, causal=True), torch.bfloat16,
            "graph replay: attn_fwd")
    compare(out2, oracle.sdpa_naive_f64(q64, k64, v64, scale=f, causal=True, window_left=64),
            torch.bfloat16, "graph replay: attn_fwd_lse output")
    want = oracle.sdpa_lse_f64(q64, k64, scale=f, causal=True, window_left=64)
    err = np.abs(W.to_f64(lse) - want)
    assert np.all(err <= 2.0 ** -8 + 1e-4 + 1e-5 * np.abs(want)), \
        f"graph replay: lse max abs err {err.max():.3g}"
    for what, (dq, kp, vp, table, lens, dout) in (("split", dec), ("fused", wide)):
        ref = oracle.paged_decode_f64(W.to_f64(dq), W.to_f64(kp), W.to_f64(vp), table.cpu().numpy(),
                                      lens.cpu().numpy(), scale=f)
        compare(dout, ref, torch.bfloat16, f"graph replay: paged decode ({what} form)")
