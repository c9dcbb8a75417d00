"""Helpers for the GPU parity tests: numpy <-> device tensors and the
elementwise tolerance check |gpu - ref| <= tol + tol * |ref|."""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch_dtype(io: str):
    import torch
    return torch.bfloat16 if io == "bf16" else torch.float32


def dev(a, dtype=None):
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda", dtype or torch.float32)


def host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def check(name: str, got, ref, tol: float):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} != {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    diff = np.abs(got - ref)
    excess = diff - (tol + tol * np.abs(ref))
    i = int(np.argmax(excess))
    max_abs = float(diff.max()) if diff.size else 0.0
    max_rel = float((diff / np.maximum(np.abs(ref), 1e-30)).max()) if diff.size else 0.0
    # the margin: worst |gpu - ref| / (tol + tol |ref|), <= 1 passes (shown with -s)
    margin = float((diff / (tol + tol * np.abs(ref))).max()) if diff.size else 0.0
    print(f"  {name}: margin {margin:.3f}")
    assert excess.flat[i] <= 0, (
        f"{name}: |gpu-ref| beyond {tol} at flat index {i}: gpu {got.flat[i]:.6g} ref "
        f"{ref.flat[i]:.6g} (max abs {max_abs:.3e}, max rel {max_rel:.3e})")
    return max_abs, max_rel
