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


def assert_close(name: str, gpu, ref, atol: float = ATOL, rtol: float = RTOL_L2, quiet: bool = False):
    max_abs, rel = errors(gpu, ref)
    finite = bool(np.isfinite(np.asarray(gpu)).all())
    if not quiet or not (finite and max_abs <= atol and rel <= rtol):
        print(f"    {name}: max_abs={max_abs:.3e} rel_l2={rel:.3e} finite={finite}", flush=True)
    assert finite, f"{name}: non-finite values"
    assert max_abs <= atol, f"{name}: max_abs {max_abs:.3e} > {atol}"
    assert rel <= rtol, f"{name}: rel_l2 {rel:.3e} > {rtol}"


def announce(msg: str):
    print(f"[gpu] {msg}", flush=True)


def assert_within_one_ulp(name, got, ref):
    """got: BF16 values as float64; ref: exact fp64 values.  Every finite element within one BF16
    unit in the last place of the exact value (what FP32 arithmetic and one rounding to nearest can
    guarantee), NaN where the exact value is NaN, and exact zeros kept."""
    import torch
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), name
    g, r = got[fin], ref[fin]
    a = np.abs(r)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.where(a > 0, 2.0 ** np.maximum(e - 7, -133), 2.0 ** -133)
    err = np.abs(g - r)
    worst = float(np.max(err / ulp)) if err.size else 0.0
    exact = torch.from_numpy(r).to(torch.bfloat16).double().numpy()
    n_exact = int(np.sum(g == exact))
    print(f"{name}: worst {worst:.3f} ulp, {n_exact}/{err.size} equal to the rounded exact value", flush=True)
    assert worst <= 1.0, name
    assert np.all(g[a == 0] == 0), name
