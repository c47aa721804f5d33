"""Helpers for the GPU parity tests (imported only by tests marked ``gpu``)."""
from __future__ import annotations

import sys

import numpy as np

# Tolerance for f32 attention outputs against the fp64 oracle: max-abs error
# <= 1e-4 and normwise relative error max|g - w| / max|w| <= 1e-3.
ABS_TOL = 1e-4
REL_TOL = 1e-3


def note(msg: str) -> None:
    """Name the case before a GPU step so a fault can be attributed."""
    print(msg, file=sys.stderr, flush=True)


def dev():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def nan_like(shape):
    import torch

    return torch.full(shape, float("nan"), dtype=torch.float32, device=dev())


def to_host(t) -> np.ndarray:
    import torch

    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_attn_close(got: np.ndarray, want: np.ndarray, what: str) -> dict:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    assert np.all(np.isfinite(got)), f"{what}: {np.count_nonzero(~np.isfinite(got))} non-finite outputs"
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    scale = float(np.max(np.abs(want))) if want.size else 0.0
    rel = err / scale if scale > 0 else err
    assert err <= ABS_TOL, f"{what}: max abs err {err:.3e} > {ABS_TOL:.0e}"
    assert rel <= REL_TOL, f"{what}: normwise rel err {rel:.3e} > {REL_TOL:.0e}"
    return {"max_abs": err, "rel": rel}


def bits(a) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint32)
