"""Reference CGLS and SIRT around the fp64 projector pair.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests, the smoke
check and the benchmark's CPU-baseline leg are the only callers.

What the solvers return and when they stop follows the diffct page
"Precision, training and reconstruction", section "Numerical solver API":
- a result with the volume, the number of completed iterations, the residual
  history, a converged flag and a stop reason;
- the history holds the residual norm of the initial iterate and then one
  value per completed iteration;
- the stop rule is ||y - A x|| <= atol + rtol ||y||, tested on the initial
  iterate too;
- SIRT has a relaxation factor (default 1) and a nonnegativity switch (default
  on), and feeds the residual of the last history entry into the next update,
  so one iteration costs one forward and one back projection;
- CGLS reads its two scalar norms of an iteration (the residual and the
  normal-equation residual) together, once per iteration;
- the inputs, x0 included, are left unchanged.

The page does not write the iterations out.  They are taken from the
textbooks, with every vector in fp64 and the projectors fed fp64 (no rounding
of iterates to fp32):
- CGLS: conjugate gradients on the normal equations A^T A x = A^T y, in the
  form of Hestenes and Stiefel (1952) as arranged for least squares by Bjorck
  ("Numerical Methods for Least Squares Problems", 1996, CGLS):
  r = y - A x, s = A^T r, p = s, gamma = ||s||^2; per iteration q = A p,
  alpha = gamma / ||q||^2, x += alpha p, r -= alpha q, s = A^T r,
  gamma' = ||s||^2, p = s + (gamma'/gamma) p.
- SIRT: x += lambda C A^T R (y - A x), with R = diag(1 / row sums of A) and
  C = diag(1 / column sums of A) (zero where a sum is zero), the simultaneous
  iterative reconstruction technique in the normalised form of Gregor and
  Benson (IEEE TMI 2008); with nonnegativity each iterate is clamped at 0.
Extra stop reasons (the page names none): "stationary" when ||A^T r|| is
exactly 0 (the least-squares normal equations hold, nothing further changes),
"breakdown" when ||A p|| is exactly 0.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from . import Geometry, back_f64, forward_f64


@dataclass
class SolverResult:
    volume: np.ndarray
    iterations: int
    residual_history: List[float] = field(default_factory=list)
    converged: bool = False
    reason: str = "iterations"


def _start(g: Geometry, y, x0):
    y = np.asarray(y, dtype=np.float64).reshape(g.sino_shape)
    x = np.zeros(g.recon_shape, np.float64) if x0 is None else \
        np.array(x0, dtype=np.float64).reshape(g.recon_shape)
    return y, x


def cgls(g: Geometry, y, iterations: int, atol: float = 0.0, rtol: float = 0.0, x0=None) -> SolverResult:
    y, x = _start(g, y, x0)
    tol = atol + rtol * float(np.linalg.norm(y))
    r = y - forward_f64(g, x)
    s = back_f64(g, r)
    p = s.copy()
    gamma = float(np.vdot(s, s))
    out = SolverResult(x, 0, [float(np.linalg.norm(r))])
    if out.residual_history[0] <= tol:
        out.converged, out.reason = True, "converged"
        return out
    for _ in range(iterations):
        if gamma == 0.0:
            out.reason = "stationary"
            return out
        q = forward_f64(g, p)
        qq = float(np.vdot(q, q))
        if qq == 0.0:
            out.reason = "breakdown"
            return out
        alpha = gamma / qq
        x += alpha * p
        r -= alpha * q
        s = back_f64(g, r)
        gamma_new = float(np.vdot(s, s))
        out.iterations += 1
        out.residual_history.append(float(np.linalg.norm(r)))
        if out.residual_history[-1] <= tol:
            out.converged, out.reason = True, "converged"
            return out
        p = s + (gamma_new / gamma) * p if gamma_new != 0.0 else s
        gamma = gamma_new
    if gamma == 0.0:
        out.reason = "stationary"
    return out


def sirt_weights(g: Geometry):
    """R = 1 / (A 1) over the sinogram and C = 1 / (A^T 1) over the volume,
    0 where the sum is 0 (a ray that meets no voxel, a voxel no ray meets)."""
    rs = forward_f64(g, np.ones(g.recon_shape))
    cs = back_f64(g, np.ones(g.sino_shape))
    with np.errstate(divide="ignore"):
        rw = np.where(rs > 0, 1.0 / rs, 0.0)
        cw = np.where(cs > 0, 1.0 / cs, 0.0)
    return rw, cw


def sirt(g: Geometry, y, iterations: int, atol: float = 0.0, rtol: float = 0.0, x0=None,
         relaxation: float = 1.0, nonnegative: bool = True) -> SolverResult:
    y, x = _start(g, y, x0)
    tol = atol + rtol * float(np.linalg.norm(y))
    rw, cw = sirt_weights(g)
    r = y - forward_f64(g, x)
    out = SolverResult(x, 0, [float(np.linalg.norm(r))])
    if out.residual_history[0] <= tol:
        out.converged, out.reason = True, "converged"
        return out
    for _ in range(iterations):
        x += relaxation * (cw * back_f64(g, rw * r))
        if nonnegative:
            np.maximum(x, 0.0, out=x)
        r = y - forward_f64(g, x)
        out.iterations += 1
        out.residual_history.append(float(np.linalg.norm(r)))
        if out.residual_history[-1] <= tol:
            out.converged, out.reason = True, "converged"
            return out
    return out
