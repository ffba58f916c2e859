"""Parity metrics shared by the GPU tests, the smoke run and the benchmark.

relative L2     ||g - o||_2 / ||o||_2 over the whole array;
max relative    max_i |g_i - o_i| / A_i with A_i = sum |w * input| over the
                taps that reach entry i (the reference returns it); entries
                no tap reaches (A_i = 0) must be exactly 0;
adjoint gap     |<A x, y> - <x, A^T y>| / (||A x|| ||y||).
"""
from __future__ import annotations

import numpy as np

REL_L2 = 1e-5
MAX_REL = 1e-4
ADJOINT = 1e-5


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def max_rel(got, ref, absum) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    a = np.asarray(absum, np.float64)
    zero = a == 0
    if np.any(got[zero] != 0):
        return float("inf")
    nz = ~zero
    if not np.any(nz):
        return 0.0
    return float(np.max(np.abs(got[nz] - ref[nz]) / a[nz]))


def assert_close(got, ref, absum, what: str, rel=REL_L2, mrel=MAX_REL) -> dict:
    r = rel_l2(got, ref)
    m = max_rel(got, ref, absum)
    assert r <= rel, f"{what}: relative L2 {r:.3e} > {rel:.0e}"
    assert m <= mrel, f"{what}: max relative error {m:.3e} > {mrel:.0e}"
    return {"rel_l2": r, "max_rel": m}


def adjoint_gap(ax, y, x, aty) -> float:
    ax = np.asarray(ax, np.float64)
    y = np.asarray(y, np.float64)
    x = np.asarray(x, np.float64)
    aty = np.asarray(aty, np.float64)
    lhs = float(np.sum(ax * y))
    rhs = float(np.sum(x * aty))
    return abs(lhs - rhs) / (np.linalg.norm(ax) * np.linalg.norm(y))
