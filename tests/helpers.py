"""Shared helpers for the parity tests: moving generated inputs to the GPU and
the tolerance rule.

Tolerance rule (both conditions must hold, per tensor):
  max |x - ref| <= abs_tol   and   max |x - ref| / max |ref| <= rel_tol
bf16 paths: abs 2e-2, rel 1e-2.  fp32 paths: 1e-5 for both.
"""

import numpy as np

BF16_TOL = (2e-2, 1e-2)
F32_TOL = (1e-5, 1e-5)


from workloads import to_device  # noqa: F401  (re-exported for the tests)


def to_numpy64(x):
    import torch
    return x.detach().to(torch.float64).cpu().numpy()


def errors(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    err = float(np.max(np.abs(x - ref))) if x.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    return err, (err / scale if scale > 0 else err)


def assert_close(name, x, ref, tol):
    abs_tol, rel_tol = tol
    assert np.all(np.isfinite(x)), f"{name}: non-finite values"
    err, rel = errors(x, ref)
    assert err <= abs_tol and rel <= rel_tol, (
        f"{name}: max-abs {err:.3e} (tol {abs_tol}), max-rel {rel:.3e} "
        f"(tol {rel_tol})")
    return err, rel
