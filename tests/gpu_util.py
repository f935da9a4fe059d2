"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""
import sys

import numpy as np
import torch


def announce(msg: str) -> None:
    """Name the case on the real stderr before a GPU step (survives a crash)."""
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def ulp_of(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Unit in the last place of |x| in the output dtype (normal range)."""
    mant, emin = {torch.bfloat16: (7, -126), torch.float16: (10, -14),
                  torch.float32: (23, -126)}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** emin)))
    return 2.0 ** (e - mant)


# float64 bar: both sides compute in float64; a score is a D-term dot product
# (D <= 256) and an output a convex combination, so each side is within a few
# hundred units of 2^-53 of the exact value for |O| of a few units (< 1e-13);
# 1e-11 leaves two orders of magnitude of margin and is still 10^6 tighter
# than the float32 bar.
F64_TOL = 1e-11


def compare(gpu: torch.Tensor, ref: np.ndarray, dtype: torch.dtype, what: str = "", amp: float = 1.0):
    """Parity bar: float64 max-abs <= 1e-11; float32 max-abs <= 1e-5;
    bf16/f16 element-wise |gpu - ref| <= 1e-2 + ulp(ref) and tensor relative
    L2 <= 5e-3.

    The float32/float64 absolute bars are for inputs of unit variance.  With
    q, k and v scaled by ``amp`` the output error scales as amp^3: it is the
    rounding error of the score (proportional to |q| |k|, amp^2) carried into
    the output through the weights (times |v|, amp), so those bars are
    multiplied by max(1, amp)^3."""
    g = gpu.detach().to("cpu", torch.float64).numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    grow = max(1.0, amp) ** 3
    if dtype == torch.float64:
        tol = F64_TOL * grow
        assert err.max(initial=0.0) <= tol, f"{what}: max abs err {err.max():.3g} > {tol:.3g}"
        return err.max(initial=0.0)
    if dtype == torch.float32:
        tol = 1e-5 * grow
        assert err.max(initial=0.0) <= tol, f"{what}: max abs err {err.max():.3g} > {tol:.3g}"
        return err.max(initial=0.0)
    bound = 1e-2 + ulp_of(ref, dtype)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} elements over 1e-2 + ulp; worst at {idx}: "
                             f"gpu {g[idx]:.6g} ref {ref[idx]:.6g}")
    nref = np.linalg.norm(ref)
    if nref > 0:
        rel = np.linalg.norm(g - ref) / nref
        assert rel <= 5e-3, f"{what}: relative L2 {rel:.3g} > 5e-3"
    return err.max(initial=0.0)
