"""Pins of the reference solvers (``oracle/solvers.py``) against facts fixed
outside their code: the least-squares and nonnegative least-squares solutions
of tiny problems computed by LAPACK (numpy.linalg.lstsq) and by
scipy.optimize.nnls from the explicit matrix A (assembled column by column
from projections of unit voxels), the row and column sums of that matrix, and
the stop rule and history layout the diffct page "Precision, training and
reconstruction" ("Numerical solver API") states."""
import math

import numpy as np
import pytest
from scipy.optimize import nnls

import workloads as W

solvers = pytest.importorskip("oracle.solvers")


def geom(kind, angles, sid=0.0, sdd=0.0, dch=1.0):
    return dict(kind=kind, num_views=len(angles), angles=np.asarray(angles, np.float64), channel_shift=None,
                source_z=None, delta_voxel=1.0, delta_channel=dch, delta_row=dch if kind else 1.0,
                source_iso=sid, source_detector=sdd, det_channel_offset=0.0, det_row_offset=0.0, psf_radius=1)


TINY = {
    "parallel": (geom(W.PARALLEL, np.arange(7) * math.pi / 7), (3, 4, 2), (7, 2, 8)),
    "cone": (geom(W.CONE_FLAT, np.arange(6) * 2 * math.pi / 6, sid=20.0, sdd=30.0, dch=1.2), (3, 3, 3), (6, 6, 8)),
}


def tiny(orc, name):
    geo, rs, ss = TINY[name]
    g = orc.Geometry(geo, rs, ss)
    n = int(np.prod(rs))
    a = np.empty((int(np.prod(ss)), n))
    for c in range(n):
        e = np.zeros(n)
        e[c] = 1.0
        a[:, c] = orc.forward_f64(g, e.reshape(rs)).ravel()
    return g, a


@pytest.mark.parametrize("name", list(TINY))
def test_fp64_projectors_are_the_adjoint_pair(orc, name):
    """The fp64-input projectors read their inputs unrounded (a value below
    fp32 resolution changes the result) and are each other's adjoint: the
    back projection equals A^T of the matrix assembled from the forward."""
    g, a = tiny(orc, name)
    rng = np.random.default_rng(1)
    y = rng.standard_normal(g.sino_shape)
    assert np.allclose(orc.back_f64(g, y).ravel(), a.T @ y.ravel(), rtol=0, atol=1e-13)
    x = np.full(g.recon_shape, 1.0)
    x2 = x + 2.0 ** -40
    assert not np.array_equal(orc.forward_f64(g, x), orc.forward_f64(g, x2))
    x32 = rng.standard_normal(g.recon_shape).astype(np.float32)
    assert np.array_equal(orc.forward_f64(g, x32.astype(np.float64)), orc.forward(g, x32))


@pytest.mark.parametrize("name", list(TINY))
def test_cgls_reaches_the_minimum_norm_least_squares_solution(orc, name):
    """CGLS from x0 = 0 stays in the range of A^T and converges to the
    minimum-norm least-squares solution (LAPACK's lstsq); in exact arithmetic
    within rank(A) iterations."""
    g, a = tiny(orc, name)
    rng = np.random.default_rng(2)
    y = rng.standard_normal(g.sino_shape)
    ref = np.linalg.lstsq(a, y.ravel(), rcond=None)[0]
    res = solvers.cgls(g, y, iterations=3 * a.shape[1])
    assert np.linalg.norm(res.volume.ravel() - ref) <= 1e-8 * np.linalg.norm(ref)
    h = np.array(res.residual_history)
    assert h[0] == pytest.approx(np.linalg.norm(y), rel=1e-15)
    assert np.all(np.diff(h) <= 1e-12 * h[0])                   # CGLS residuals never grow
    assert h[-1] == pytest.approx(np.linalg.norm(y.ravel() - a @ ref), rel=1e-8)


def test_cgls_history_stop_rule_and_inputs_preserved(orc):
    g, a = tiny(orc, "parallel")
    rng = np.random.default_rng(3)
    xt = rng.standard_normal(g.recon_shape)
    y = (a @ xt.ravel()).reshape(g.sino_shape)                  # consistent data
    x0 = rng.standard_normal(g.recon_shape)
    y_in, x0_in = y.copy(), x0.copy()
    res = solvers.cgls(g, y, iterations=4, x0=x0)
    assert np.array_equal(y, y_in) and np.array_equal(x0, x0_in)
    assert res.iterations == 4 and len(res.residual_history) == 5 and not res.converged
    assert res.reason == "iterations"
    assert res.residual_history[0] == pytest.approx(np.linalg.norm(y - orc.forward_f64(g, x0)), rel=1e-14)
    # the rule holds at the initial iterate: no iteration runs
    res0 = solvers.cgls(g, y, iterations=10, x0=xt, atol=1e-9 * np.linalg.norm(y))
    assert res0.iterations == 0 and res0.converged and res0.reason == "converged"
    assert len(res0.residual_history) == 1
    # a relative tolerance met at iteration k stops there
    h = res.residual_history
    rtol = 0.5 * (h[2] + h[3]) / np.linalg.norm(y)
    res3 = solvers.cgls(g, y, iterations=10, x0=x0, rtol=rtol)
    assert res3.converged and res3.iterations == 3 and res3.residual_history == pytest.approx(h[:4], rel=1e-14)


@pytest.mark.parametrize("name", list(TINY))
def test_sirt_weights_are_the_row_and_column_sums(orc, name):
    g, a = tiny(orc, name)
    rw, cw = solvers.sirt_weights(g)
    rs, cs = a.sum(axis=1), a.sum(axis=0)
    assert np.allclose(rw.ravel(), np.where(rs > 0, 1 / np.where(rs > 0, rs, 1), 0), rtol=1e-13, atol=0)
    assert np.allclose(cw.ravel(), np.where(cs > 0, 1 / np.where(cs > 0, cs, 1), 0), rtol=1e-13, atol=0)
    assert np.any(rs == 0) and np.all(rw.ravel()[rs == 0] == 0)   # rays that miss the volume


@pytest.mark.parametrize("name,relax", [("parallel", 1.0), ("parallel", 0.5), ("cone", 1.0)])
def test_sirt_reaches_the_row_weighted_least_squares_solution(orc, name, relax):
    """Unconstrained SIRT is gradient descent on ||y - A x||^2_R scaled by C;
    its fixed point (for 0 < relaxation < 2) solves A^T R (y - A x) = 0, the
    least-squares problem weighted by R (unique: A has full column rank)."""
    g, a = tiny(orc, name)
    assert np.linalg.matrix_rank(a) == a.shape[1]
    rw, _ = solvers.sirt_weights(g)
    rng = np.random.default_rng(4)
    y = rng.standard_normal(g.sino_shape)
    sq = np.sqrt(rw.ravel())
    ref = np.linalg.lstsq(sq[:, None] * a, sq * y.ravel(), rcond=None)[0]
    res = solvers.sirt(g, y, iterations=6000, relaxation=relax, nonnegative=False)
    assert np.linalg.norm(res.volume.ravel() - ref) <= 1e-7 * np.linalg.norm(ref)
    assert len(res.residual_history) == 6001


def test_sirt_nonnegative_reaches_the_weighted_nnls_solution(orc):
    """With nonnegativity SIRT is a projected scaled gradient method (the
    clamp is the projection onto x >= 0 in the C-scaled norm, C diagonal), so
    it converges to argmin_{x >= 0} ||y - A x||_R (scipy's nnls); the data are
    chosen so that the bound is active."""
    g, a = tiny(orc, "parallel")
    rw, _ = solvers.sirt_weights(g)
    rng = np.random.default_rng(5)
    xt = rng.standard_normal(a.shape[1])
    y = (a @ xt + 0.1 * rng.standard_normal(a.shape[0])).reshape(g.sino_shape)
    sq = np.sqrt(rw.ravel())
    ref, _ = nnls(sq[:, None] * a, sq * y.ravel(), maxiter=10000)
    assert np.sum(ref == 0) >= 3                                  # the constraint binds
    res = solvers.sirt(g, y, iterations=20000)
    assert res.volume.min() >= 0.0
    assert np.linalg.norm(res.volume.ravel() - ref) <= 1e-6 * np.linalg.norm(ref)
