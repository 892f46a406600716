"""Shared helpers for the parity tests: moving generated inputs to the GPU and
the tolerance rule.

Tolerance rule (both conditions must hold, per tensor):
  max |x - ref| <= abs_tol   and   max |x - ref| / max |ref| <= rel_tol
bf16 paths: abs 2e-2, rel 1e-2.  fp32 paths: 1e-5 for both.

bf16 paths never take abs_tol below 2^-7 max |ref|, about one unit in the last
place of the tensor's largest value: bf16 keeps 8 significant bits, the
outputs are rounded to it and the products take bf16 operands (P, dS), so a
tensor whose values reach 2.56 or more carries rounding errors above 2e-2
however exact the arithmetic around them.  Gradients do (a key attended by
hundreds of queries collects their dO).  Below max |ref| = 2.56 the floor is
inactive, and above it the relative condition still holds with rel_tol.
"""

import numpy as np

BF16_TOL = (2e-2, 1e-2)
F32_TOL = (1e-5, 1e-5)
BF16_ULP_FLOOR = 2.0 ** -7   # of max |ref|


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
    if tol == BF16_TOL and np.size(ref):
        abs_tol = max(abs_tol,
                      BF16_ULP_FLOOR * float(np.max(np.abs(np.asarray(ref)))))
    assert err <= abs_tol and rel <= rel_tol, (
        f"{name}: max-abs {err:.3e} (tol {abs_tol}), max-rel {rel:.3e} "
        f"(tol {rel_tol})")
    return err, rel


def stored_forward(o, m, l):
    """The oracle's forward outputs as a backward reads them from HBM: o
    rounded to bf16 (returned as device bits and as the exact values of
    those bits), m and l as fp32 device tensors."""
    import torch
    from workloads import bf16_bits, bf16_value
    bits = bf16_bits(np.asarray(o, np.float32))
    o_exact = bf16_value(bits).astype(np.float64)
    o_dev = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).cuda()
    m_dev = torch.from_numpy(np.asarray(m, np.float32)).cuda()
    l_dev = torch.from_numpy(np.asarray(l, np.float32)).cuda()
    return o_dev, o_exact, m_dev, l_dev
