"""Helpers for the GPU parity tests: moving generated inputs to the device,
reading results back, and the comparison rules with their tolerances."""
from __future__ import annotations

import numpy as np

import workloads


def to_device(a: np.ndarray, dtype: str):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).cuda()
    raise ValueError(dtype)


def from_device(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return workloads.to_f64(a, dtype)


# Tolerances. fp32: 1e-5 relative (loss), and for gradient tensors a normwise
# 1e-5 plus an elementwise bound of 1e-5 relative to the element and to the
# tensor's largest magnitude (GEMM sums cancel, so a per-element relative bound
# alone cannot hold near zero). bf16 (the logits and dZ round to bf16 after
# fp32 arithmetic): 2e-2 relative / 1e-3 absolute elementwise as the pages'
# contract asks, and, because every gradient element is far below 1e-3 at
# batchmean, a normwise 2e-2 check that is not vacuous.
TOL = {
    "f32": {"loss_rel": 1e-5, "norm": 1e-5, "elem_rel": 1e-5, "elem_max": 1e-5, "elem_abs": 0.0},
    "bf16": {"loss_rel": 2e-2, "norm": 2e-2, "elem_rel": 2e-2, "elem_max": 0.0, "elem_abs": 1e-3},
}


def rel_err(got: float, ref: float) -> float:
    return abs(got - ref) / max(abs(ref), 1e-30)


def normwise(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else np.inf
    return num / den


def assert_loss_close(got, ref, tol, what="loss"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30))
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err <= tol["loss_rel"], f"{what}: relative error {err:.3e} > {tol['loss_rel']}"
    return err


def assert_tensor_close(got: np.ndarray, ref: np.ndarray, tol, what="tensor"):
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    nw = normwise(got, ref)
    assert nw <= tol["norm"], f"{what}: normwise error {nw:.3e} > {tol['norm']}"
    bound = tol["elem_abs"] + tol["elem_rel"] * np.abs(ref) + tol["elem_max"] * np.max(np.abs(ref))
    bad = np.abs(got - ref) > bound
    assert not np.any(bad), (f"{what}: {int(bad.sum())} elements outside the elementwise bound; "
                             f"worst |d|={np.max(np.abs(got - ref)):.3e}")
    return nw
