"""Acceptance check of a GEMM output against the fp64 reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Tolerance: ``max|out - ref| <= 1e-2 * max|ref|`` and, per element,
``|out - ref| <= 2^-6 * |ref| + tau`` where tau is the fp32 summation bound of
the K-term accumulation (``summation_bound_*``), which only matters for outputs
that nearly cancel. The pages give no tolerance; the PR 34331 digest ("Risks
and impact") reports single-layer cosine similarity of about 0.9999 between two
backends whose accumulation order differs, which is reported here as a
diagnostic.

The worst-case bound tau = K 2^-23 sum|terms| is rigorous but loose: on
N(0, 1)-like data it exceeds 2^-6 |ref| for most elements once K is a few
thousand, so on its own it would not enforce the per-element 2^-6 criterion.
Two tighter conditions are therefore also checked when the depth K of the sum
is passed:

* the probabilistic floor of Higham and Mary ("A new approach to
  probabilistic rounding error analysis", SIAM J. Sci. Comput. 41(5), 2019,
  Theorem 2.4): with independent, mean-zero rounding errors of unit roundoff u,
  a K-term sum errs by at most lambda sqrt(K) u sum|terms| with probability at
  least 1 - 2 exp(-lambda^2 / 2). With lambda = 8 (failure probability below
  3e-14 per element) and u = 2^-24 this floor is tau lambda / (2 sqrt(K)) for
  the worst-case tau above; every element must satisfy
  ``|out - ref| <= 2^-6 |ref| + floor``.
* the pure relative criterion ``|out - ref| <= 2^-6 |ref|`` may fail only on
  a small fraction of the elements (``max_pure_rel_frac``, 1%): those whose
  true value is cancelled far below the size of its terms.
"""

import math

import numpy as np

PROB_LAMBDA = 8.0


def check_gemm(out, ref, tau, rel: float = 2.0 ** -6, max_frac: float = 1e-2, k=None,
               max_pure_rel_frac: float = 1e-2) -> dict:
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
    finite = bool(np.all(np.isfinite(out)))
    ok = finite and max_err <= max_frac * scale and bool(np.all(elem_ok))
    res = {
        "ok": ok,
        "max_err": max_err,
        "max_ref": scale,
        "n_elem_fail": int(np.sum(~elem_ok)),
        "frac_pure_rel_fail": pure_rel_fail,
        "cosine": cosine,
    }
    if k is not None and err.size:
        floor = tau * (PROB_LAMBDA / (2.0 * math.sqrt(float(k))))
        excess = np.maximum(err - rel * np.abs(ref), 0.0)
        with np.errstate(divide="ignore", invalid="ignore"):
            used = np.where(floor > 0, excess / floor, np.where(excess > 0, np.inf, 0.0))
        prob_fail = int(np.sum(excess > floor))
        res["n_prob_floor_fail"] = prob_fail
        res["prob_floor_used"] = float(np.max(used))
        res["ok"] = res["ok"] and prob_fail == 0 and pure_rel_fail <= max_pure_rel_frac
    return res
