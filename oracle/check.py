"""Acceptance check of a GEMM output against the fp64 reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Tolerance: ``max|out - ref| <= 1e-2 * max|ref|`` and, per element,
``|out - ref| <= 2^-6 * |ref| + tau`` where tau is the fp32 summation bound of
the K-term accumulation (``summation_bound_*``), which only matters for outputs
that nearly cancel. The pages give no tolerance; the PR 34331 digest ("Risks
and impact") reports single-layer cosine similarity of about 0.9999 between two
backends whose accumulation order differs, which is reported here as a
diagnostic.
"""

import numpy as np


def check_gemm(out, ref, tau, rel: float = 2.0 ** -6, max_frac: float = 1e-2) -> dict:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tau = np.asarray(tau, dtype=np.float64)
    err = np.abs(out - ref)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    max_err = float(np.max(err)) if err.size else 0.0
    bound = rel * np.abs(ref) + tau
    elem_ok = err <= bound
    pure_rel_fail = float(np.mean(err > rel * np.abs(ref))) if err.size else 0.0
    denom = float(np.linalg.norm(out) * np.linalg.norm(ref))
    cosine = float(np.sum(out * ref) / denom) if denom > 0 else 1.0
    ok = bool(np.all(np.isfinite(out))) and max_err <= max_frac * scale and bool(np.all(elem_ok))
    return {
        "ok": ok,
        "max_err": max_err,
        "max_ref": scale,
        "n_elem_fail": int(np.sum(~elem_ok)),
        "frac_pure_rel_fail": pure_rel_fail,
        "cosine": cosine,
    }
