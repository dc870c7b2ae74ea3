"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
from __future__ import annotations

import numpy as np

ATOL = 1e-3      # max |gpu - oracle|
RTOL_L2 = 1e-4   # ||gpu - oracle||_2 / ||oracle||_2
SENTINEL = 12345.0


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def errors(gpu: np.ndarray, ref: np.ndarray):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    d = g - r
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    nr = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(d)) / nr if nr > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_close(name: str, gpu, ref, atol: float = ATOL, rtol: float = RTOL_L2):
    max_abs, rel = errors(gpu, ref)
    finite = bool(np.isfinite(np.asarray(gpu)).all())
    print(f"    {name}: max_abs={max_abs:.3e} rel_l2={rel:.3e} finite={finite}", flush=True)
    assert finite, f"{name}: non-finite values"
    assert max_abs <= atol, f"{name}: max_abs {max_abs:.3e} > {atol}"
    assert rel <= rtol, f"{name}: rel_l2 {rel:.3e} > {rtol}"


def announce(msg: str):
    print(f"[gpu] {msg}", flush=True)
