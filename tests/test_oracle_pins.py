"""Pins of the fp64 reference against facts fixed outside its own code.

Each test names what it pins.  None of them re-types the reference's formula
and compares it with itself: the expected values come from closed forms worked
by hand, exact rational arithmetic, invariants of the model (adjoint,
linearity, partition of unity, symmetry), the physics of a voxel's projection,
or limits where one geometry reduces to another.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads as W


def geom_dict(kind=W.PARALLEL, angles=(0.0,), shift=None, zsrc=None, dch=1.0, drow=1.0,
              sid=0.0, sdd=0.0, radius=1, ch_off=0.0, row_off=0.0, dv=1.0):
    return dict(kind=kind, num_views=len(angles), angles=np.asarray(angles, np.float64),
                channel_shift=None if shift is None else np.asarray(shift, np.float64),
                source_z=None if zsrc is None else np.asarray(zsrc, np.float64),
                delta_voxel=dv, delta_channel=dch, delta_row=drow, source_iso=sid,
                source_detector=sdd, det_channel_offset=ch_off, det_row_offset=row_off,
                psf_radius=radius)


def make(orc, w: W.Workload):
    return orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)


def adjoint_gap(orc, g, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(g.recon_shape).astype(np.float32)
    y = rng.standard_normal(g.sino_shape).astype(np.float32)
    ax = orc.forward(g, x)
    aty = orc.back(g, y)
    lhs = float((ax * y.astype(np.float64)).sum())
    rhs = float((x.astype(np.float64) * aty).sum())
    return abs(lhs - rhs) / (np.linalg.norm(ax) * np.linalg.norm(y))


SMALL_CONE = W.Workload("cone-24x20x12-17v", W.CONE_FLAT, 24, 20, 12, 17, 16, 30,
                        dch=1.5, drow=1.5, sid=60.0, sdd=90.0, seed_x=7, seed_y=8)
SMALL_HELIX = W.Workload("helical-20x20x10-23v", W.CONE_FLAT, 20, 20, 10, 23, 8, 28,
                         dch=11 / 6, drow=11 / 6, sid=30.0, sdd=55.0,
                         angle_step=2 * math.pi / 10, zsrc_step=0.4, seed_x=9, seed_y=10)
SMALL_TRANS = W.Workload("translation-16x24x4-9v", W.PARALLEL, 16, 24, 4, 9, 4, 64,
                         shift_step=3.0, seed_x=11, seed_y=12)

# A cone whose channel and row pitches differ, with a source close enough that
# off-centre pixels see the central ray at 5-25 degrees: the in-plane ray
# direction theta - gamma and theta + gamma then give clearly different box
# widths, and a magnification built from the wrong pitch moves every voxel.
PITCH_CONE = W.Workload("cone-20x24x10-9v-pitch", W.CONE_FLAT, 20, 24, 10, 9, 32, 120,
                        dch=1.3, drow=1.1, sid=40.0, sdd=70.0,
                        angle_step=0.61, seed_x=31, seed_y=32)


# --------------------------------------------------------------------- ov ---
def test_ov_closed_form_values(orc):
    """The overlap of a unit cell with a centred box, at hand-worked points."""
    assert orc.ov(0.0, 1.0) == 1.0
    assert orc.ov(1.0, 1.0) == 0.0
    assert orc.ov(0.5, 1.0) == 0.5
    assert orc.ov(0.25, 0.5) == 0.25 + 0.25 - 0.25 + 0.25  # cell [-.25,.75] vs box [-.25,.25]
    assert orc.ov(0.0, 3.0) == 1.0                    # box wider than the cell
    assert orc.ov(1.25, 3.0) == pytest.approx(0.75, abs=0)
    assert orc.ov(-2.0, 3.0) == 0.0


@pytest.mark.parametrize("a", [0.3, 0.70710678, 1.0, 1.37, 1.99])
def test_ov_partition_of_unity(orc, a):
    """Sum over integer shifts equals the box width (partition of unity)."""
    rng = np.random.default_rng(3)
    for u in rng.uniform(-3, 3, 50):
        s = sum(orc.ov(n - u, a) for n in range(-8, 9))
        assert abs(s - a) < 1e-14


def test_ov_matches_quadrature(orc):
    """B2: numerical integral of the box over each cell, Q = 1e4 midpoints."""
    q = 10_000
    rng = np.random.default_rng(5)
    for _ in range(40):
        d, a = rng.uniform(-1.6, 1.6), rng.uniform(0.2, 2.5)
        t = (np.arange(q) + 0.5) / q - 0.5 + d            # sample points of the cell
        quad = np.mean(np.abs(t) <= a / 2)
        assert abs(orc.ov(d, a) - quad) <= 2.0 / q


# ----------------------------------------------------------- single voxel ---
def one_voxel(orc, theta, u_off, radius=1, nc=11):
    """A 1x1x1 recon with its centre projecting to channel (nc-1)/2 + u_off."""
    g = orc.Geometry(geom_dict(angles=[theta], shift=[u_off], radius=radius), (1, 1, 1), (1, 1, nc))
    return g, orc.forward(g, np.ones((1, 1, 1), np.float32))[0, 0]


def test_single_voxel_axis_aligned(orc):
    """P4: at theta = 0 a unit voxel whose centre falls on a channel centre
    puts exactly dv into that channel and nothing elsewhere."""
    for theta in (0.0, math.pi):
        _, y = one_voxel(orc, theta, 0.0)
        assert y[5] == 1.0 and np.count_nonzero(y) == 1
    # the small disk workload: u = j + 16 at theta = 0, for every pixel
    w = W.get(W.SMALL)
    g = make(orc, w)
    x = np.zeros(w.recon_shape, np.float32)
    x[10, 37, 3] = 1.0
    y = orc.forward(g, x)
    assert y[0, 3, 37 + 16] == 1.0 and np.count_nonzero(y[0]) == 1


@pytest.mark.parametrize("d,expect", [
    (0.0, {5: 1.0}),
    (-0.5, {5: 0.5, 4: 0.5}),        # u = 4.5 rounds (ties to even) to 4
    (0.5, {5: 0.5, 6: 0.5}),         # u = 5.5 rounds to 6
    (-0.25, {5: 0.5 + math.sqrt(2) / 4, 4: 0.5 - math.sqrt(2) / 4}),
    (0.25, {5: 0.5 + math.sqrt(2) / 4, 6: 0.5 - math.sqrt(2) / 4}),
])
def test_single_voxel_45_degrees(orc, d, expect):
    """P4: at 45 degrees the box has width 1/sqrt2 and height sqrt2; the cell
    overlaps worked by hand give these tap weights."""
    _, y = one_voxel(orc, math.pi / 4, d)
    got = {n: y[n] for n in np.nonzero(y)[0]}
    assert set(got) == set(expect)
    for n, v in expect.items():
        assert abs(got[n] - v) < 1e-15


def test_single_voxel_golden_fixture(orc):
    """The hand-worked single-voxel taps of ``tests/golden/single_voxel_taps.txt``
    (0, 45 and 180 degrees, centred, half and quarter channel off)."""
    from golden_io import single_voxel_taps
    cases = single_voxel_taps()
    assert len(cases) == 7
    for (th, off), taps in cases.items():
        _, y = one_voxel(orc, math.radians(th), off)
        expect = np.zeros_like(y)
        for n, wgt in taps.items():
            expect[n] = wgt
        assert np.max(np.abs(y - expect)) < 1e-15, (th, off, y)


def test_tap_count_bounded_by_footprint(orc):
    """With W <= 1 at most two adjacent channels receive weight; the chosen
    channel n_c = rint(u) always carries weight."""
    w = W.get(W.BENCH)
    g = make(orc, w)
    rng = np.random.default_rng(0)
    for v, i, j in zip(rng.integers(0, w.nv, 200), rng.integers(0, w.ny, 200), rng.integers(0, w.nx, 200)):
        taps = orc.voxel_taps(g, int(v), int(i), int(j), 0)
        chans = sorted(t[1] for t in taps)
        assert 1 <= len(chans) <= 2 and chans == list(range(chans[0], chans[0] + len(chans)))
        nc = orc.vp_params(g, int(v), int(i), int(j))["nc"]
        assert nc in chans


# ----------------------------------------------------------------- adjoint ---
@pytest.mark.parametrize("w", [W.get(W.SMALL), SMALL_CONE, SMALL_HELIX, SMALL_TRANS],
                         ids=lambda w: w.name)
def test_adjoint_identity(orc, w):
    """P1: <Ax, y> = <x, A^T y> for the matched pair."""
    assert adjoint_gap(orc, make(orc, w), seed=11) < 1e-12


@pytest.mark.parametrize("w", [W.get(W.SMALL), SMALL_CONE], ids=lambda w: w.name)
def test_linearity(orc, w):
    """P2: A(alpha x + beta z) = alpha A x + beta A z (no hidden state)."""
    g = make(orc, w)
    rng = np.random.default_rng(4)
    # values on a 1/16 grid, so the combination is exact in fp32
    x = (rng.integers(-64, 64, w.recon_shape) / 16.0).astype(np.float32)
    z = (rng.integers(-64, 64, w.recon_shape) / 16.0).astype(np.float32)
    comb = (2.0 * x.astype(np.float64) - 3.0 * z.astype(np.float64))
    assert np.array_equal(comb.astype(np.float32).astype(np.float64), comb)  # exact in fp32
    lhs = orc.forward(g, comb.astype(np.float32))
    rhs = 2.0 * orc.forward(g, x) - 3.0 * orc.forward(g, z)
    assert np.linalg.norm(lhs - rhs) / np.linalg.norm(rhs) < 1e-13


# -------------------------------------------------------------------- mass ---
def test_parallel_mass_per_view_and_row(orc):
    """P3: every view of a parallel projection carries mass dv^2/dch times the
    slice's sum, when every tap lands on the detector (small disk workload:
    projected half-diagonal 45.3 < 47.5)."""
    w = W.get(W.SMALL)
    g = make(orc, w)
    x = w.recon_input()
    y = orc.forward(g, x)
    slice_sum = x.astype(np.float64).sum(axis=(0, 1))
    assert np.allclose(y.sum(axis=2), slice_sum[None, :], rtol=1e-13, atol=0)


@pytest.mark.slow
def test_parallel_mass_full_size_sampled_views(orc):
    """P3 at the 512x512x64, 720-view size: projected half-diagonal
    362 < 383.5, so each view's mass equals the slice sum."""
    w = W.get(W.BENCH)
    g = make(orc, w)
    rng = np.random.default_rng(2)
    x = rng.random(w.recon_shape).astype(np.float32)
    views = [0, 77, 180, 359, 540, 719]
    y = orc.forward_views(g, x, views)
    slice_sum = x.astype(np.float64).sum(axis=(0, 1))
    assert np.allclose(y.sum(axis=2), slice_sum[None, :], rtol=1e-12, atol=0)


@pytest.mark.parametrize("w", [W.get("cone-256x256x256-360v"), SMALL_CONE],
                         ids=lambda w: w.name)
def test_cone_voxel_mass_is_physical(orc, w):
    """P3 (cone): the detector integral of one voxel's cell-averaged line
    integrals equals the physical value dv^3 (SDD/D)^2 / cos(incidence), with
    cos(incidence) the ray's direction cosine on the detector normal.  The
    expected value is computed from the source/voxel/detector positions, not
    from the footprint formulas."""
    g = make(orc, w)
    rng = np.random.default_rng(9)
    ang = w.angles()
    zs = w.source_z()
    for _ in range(60):
        v, i, j = int(rng.integers(w.nv)), int(rng.integers(w.ny)), int(rng.integers(w.nx))
        k = int(rng.integers(w.ns))
        taps = orc.voxel_taps(g, v, i, j, k)
        if not taps:
            continue
        rows = [t[0] for t in taps]
        chans = [t[1] for t in taps]
        if min(rows) == 0 or max(rows) == w.nr - 1 or min(chans) == 0 or max(chans) == w.nc - 1:
            continue                          # tap possibly cut by the detector edge
        total = sum(t[2] for t in taps) * w.dch * w.drow
        # physics: source S, voxel P, detector normal e_b
        th = ang[v]
        e_a = np.array([math.cos(th), math.sin(th), 0.0])
        e_b = np.array([-math.sin(th), math.cos(th), 0.0])
        zsrc = 0.0 if zs is None else zs[v]
        src = -w.sid * e_b + np.array([0, 0, zsrc])
        p = np.array([j - (w.nx - 1) / 2, i - (w.ny - 1) / 2, k - (w.ns - 1) / 2])
        ray = p - src
        dist_plane = float(ray @ e_b)                   # D: source to voxel along the normal
        cos_inc = dist_plane / np.linalg.norm(ray)
        expect = (w.sdd / dist_plane) ** 2 / cos_inc
        assert abs(total - expect) < 1e-12 * expect


# --------------------------------------------------------- cone -> parallel ---
def test_cone_reduces_to_parallel(orc):
    """P7: a cone with its source 1e9 voxels away, unit pitches and R = S is
    the parallel projector."""
    base = W.get(W.SMALL)
    par = make(orc, base)
    cone = orc.Geometry(geom_dict(kind=W.CONE_FLAT, angles=base.angles(), sid=1e9, sdd=1e9),
                        base.recon_shape, base.sino_shape)
    x = base.recon_input()
    yp, yc = orc.forward(par, x), orc.forward(cone, x)
    assert np.linalg.norm(yp - yc) / np.linalg.norm(yp) < 1e-6
    rng = np.random.default_rng(1)
    s = rng.standard_normal(base.sino_shape).astype(np.float32)
    bp, bc = orc.back(par, s), orc.back(cone, s)
    assert np.linalg.norm(bp - bc) / np.linalg.norm(bp) < 1e-6


def _box_cell_quadrature(d, a, q=20000):
    """Overlap of the unit cell centred at d with the box [-a/2, a/2], by
    midpoint quadrature (independent of the reference's closed form)."""
    t = (np.arange(q) + 0.5) / q - 0.5 + d
    return float(np.mean(np.abs(t) <= a / 2))


@pytest.mark.parametrize("w", [W.get("cone-256x256x256-360v"), SMALL_HELIX, PITCH_CONE],
                         ids=lambda w: w.name)
def test_cone_rows_follow_perspective(orc, w):
    """The row profile of a voxel is its magnified height (SDD/D * dv) centred
    on the perspective projection of its centre onto the flat detector.  Row
    centre and width come from the source/voxel positions; the cell overlaps
    from quadrature.  Since the centre moves by SDD/D * dv per slice, this also
    pins the row as an affine function of the slice index."""
    g = make(orc, w)
    rng = np.random.default_rng(21)
    ang, zs = w.angles(), w.source_z()
    checked = 0
    for _ in range(200):
        v, i, j, k = (int(rng.integers(n)) for n in (w.nv, w.ny, w.nx, w.ns))
        taps = orc.voxel_taps(g, v, i, j, k)
        if not taps or min(t[0] for t in taps) == 0 or max(t[0] for t in taps) == w.nr - 1:
            continue
        th = ang[v]
        e_b = np.array([-math.sin(th), math.cos(th)])
        p = np.array([j - (w.nx - 1) / 2, i - (w.ny - 1) / 2])
        dplane = w.sid + float(p @ e_b)
        dz = (k - (w.ns - 1) / 2) - (0.0 if zs is None else zs[v])
        wrow = w.sdd * w.dv / (dplane * w.drow)
        if wrow > 2.0:
            continue                               # three taps do not cover it
        row_c = (w.nr - 1) / 2 + w.sdd * dz / (dplane * w.drow)
        tot = sum(t[2] for t in taps)
        rows = {}
        for r_, _, wt in taps:
            rows[r_] = rows.get(r_, 0.0) + wt / tot
        for r_ in range(min(rows) - 1, max(rows) + 2):
            expect = _box_cell_quadrature(r_ - row_c, wrow) / wrow
            assert abs(rows.get(r_, 0.0) - expect) < 3e-4
        checked += 1
    assert checked > 50


def _pixel_chords(src, ea, eb, cch, dch, sdd, sid, px, py, dv, t):
    """Length of the in-plane ray from the source to the detector point at
    channel coordinate t inside the square pixel centred at (px, py): slab
    clipping against the pixel's four edges, exact for straight rays."""
    q = ((t - cch) * dch)[:, None] * ea[None, :] + (sdd - sid) * eb[None, :]
    d = q - src[None, :]
    lo = np.array([px - dv / 2, py - dv / 2])
    hi = np.array([px + dv / 2, py + dv / 2])
    with np.errstate(divide="ignore", invalid="ignore"):
        t0 = (lo[None, :] - src[None, :]) / d
        t1 = (hi[None, :] - src[None, :]) / d
    enter = np.minimum(t0, t1).max(axis=1)
    leave = np.maximum(t0, t1).min(axis=1)
    return np.maximum(leave - enter, 0.0) * np.linalg.norm(d, axis=1)


def _half_max_window(t, prof):
    """Peak value and the two half-maximum crossings of a sampled profile
    (linear interpolation between samples)."""
    pk = float(prof.max())
    half = pk / 2
    above = np.flatnonzero(prof >= half)
    i0, i1 = above[0], above[-1]
    tl = t[i0 - 1] + (half - prof[i0 - 1]) * (t[i0] - t[i0 - 1]) / (prof[i0] - prof[i0 - 1])
    tr = t[i1] + (half - prof[i1]) * (t[i1 + 1] - t[i1]) / (prof[i1 + 1] - prof[i1])
    return pk, tl, tr


def cone_inplane_shadow_errors(vp_params, w: W.Workload, min_gamma_deg=5.0):
    """For every (view, pixel) of a cone workload whose centre sees the central
    ray at |gamma| >= min_gamma_deg, the exact in-plane shadow of the square
    pixel on the flat detector: chord lengths of the rays from the source
    through the pixel, sampled over the span of its four projected corners.
    Returns the worst deviations of the reference's box from that shadow:
    centre (channels) against the half-maximum window's midpoint, width
    (relative) against the full width at half maximum, and height (relative)
    against the longest chord.  vp_params(v, i, j) returns the reference's
    per-(view, pixel) parameters."""
    ang = w.angles()
    cch = (w.nc - 1) / 2
    worst = dict(centre=0.0, width=0.0, height=0.0, n=0)
    for v, th in enumerate(ang):
        ea = np.array([math.cos(th), math.sin(th)])
        eb = np.array([-math.sin(th), math.cos(th)])
        src = -w.sid * eb
        for i in range(w.ny):
            for j in range(w.nx):
                p = np.array([(j - (w.nx - 1) / 2) * w.dv, (i - (w.ny - 1) / 2) * w.dv])
                if abs(math.degrees(math.atan2(float(p @ ea), w.sid + float(p @ eb)))) < min_gamma_deg:
                    continue
                corners = np.array([[p[0] + sx * w.dv / 2, p[1] + sy * w.dv / 2]
                                    for sx in (-1, 1) for sy in (-1, 1)])
                tc = w.sdd * (corners @ ea) / (w.sid + corners @ eb) / w.dch + cch
                t = np.linspace(tc.min() - 0.05, tc.max() + 0.05, 4001)
                prof = _pixel_chords(src, ea, eb, cch, w.dch, w.sdd, w.sid, p[0], p[1], w.dv, t)
                pk, tl, tr = _half_max_window(t, prof)
                prm = vp_params(v, i, j)
                worst["centre"] = max(worst["centre"], abs((tl + tr) / 2 - prm["u"]))
                worst["width"] = max(worst["width"], abs((tr - tl) - prm["W"]) / prm["W"])
                worst["height"] = max(worst["height"], abs(pk - prm["L"]) / prm["L"])
                worst["n"] += 1
    return worst


# The shadow is the box only up to the perspective across one pixel: the
# deviations grow like dv / D (D between 24 and 56 voxels here).
INPLANE_TOL = dict(centre=0.02, width=0.01, height=0.01)


@pytest.mark.parametrize("w", [PITCH_CONE, SMALL_HELIX], ids=lambda w: w.name)
def test_cone_inplane_footprint_is_the_pixel_shadow(orc, w):
    """B3/P8 in the plane: the cone's channel box (centre u, width W_ch,
    height L_xy) is the pixel's shadow on the flat detector, traced from the
    source through the pixel's square.  The centre is where the shadow's
    half-maximum window sits, the width its full width at half maximum, the
    height its longest chord.  This fixes the in-plane ray direction used for
    the box (a sign slip in theta -/+ gamma changes the width and height by up
    to 40% here), the 1/cos(gamma) obliquity of the flat detector and the
    channel magnification's pitch (the channel pitch differs from the row
    pitch in the first geometry)."""
    g = make(orc, w)
    worst = cone_inplane_shadow_errors(lambda v, i, j: orc.vp_params(g, v, i, j), w)
    assert worst["n"] > 300
    for key, tol in INPLANE_TOL.items():
        assert worst[key] < tol, (key, worst)


def _mutant(orc, tmp_path, old, new):
    """A copy of the reference built on the CPU from its own source with one
    line changed, exposing the per-(view, pixel) parameters and the voxel taps
    through the same interface as the reference module."""
    import ctypes
    import subprocess
    import types
    src = open(os.path.join(os.path.dirname(orc.__file__), "proj_oracle.c")).read()
    assert src.count(old) == 1, "the planted line no longer matches the reference's source"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", *orc.CFLAGS, "-o", lib_path, str(path), "-lm"], check=True)
    lib = ctypes.CDLL(lib_path)
    f64 = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
    i32 = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
    lib.orc_vp_params.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, f64]
    lib.orc_voxel_taps.argtypes = [ctypes.c_void_p] + [ctypes.c_int32] * 4 + [i32, i32, f64, ctypes.c_int]
    lib.orc_voxel_taps.restype = ctypes.c_int

    def vp_params(g, v, i, j):
        out = np.zeros(7, np.float64)
        lib.orc_vp_params(ctypes.addressof(g.s), v, i, j, out)
        return dict(u=out[0], nc=int(out[1]), W=out[2], L=out[3], Mr=out[4], rho=out[5], Wrow=out[6])

    def voxel_taps(g, v, i, j, k):
        cap = (2 * g.s.radius + 1) ** 2
        rows, chans, w = np.zeros(cap, np.int32), np.zeros(cap, np.int32), np.zeros(cap, np.float64)
        n = lib.orc_voxel_taps(ctypes.addressof(g.s), v, i, j, k, rows, chans, w, cap)
        return [(int(rows[q]), int(chans[q]), float(w[q])) for q in range(n)]

    return types.SimpleNamespace(Geometry=orc.Geometry, vp_params=vp_params, voxel_taps=voxel_taps)


@pytest.mark.slow
@pytest.mark.parametrize("old,new", [
    ("double alpha = g->angles[v] - gam;", "double alpha = g->angles[v] + gam;"),
    ("double mc = g->sdd / dc;", "double mc = g->sdd / drw;"),
    ("o->w = mc * g->dv * m / cos(gam);", "o->w = mc * g->dv * m;"),
    ("double mr = g->sdd / drw;", "double mr = g->sdd / dc;"),
], ids=["theta_plus_gamma", "mc_from_row_pitch", "no_obliquity", "mr_from_channel_pitch"])
def test_cone_footprint_pins_catch_planted_mistakes(orc, tmp_path, old, new):
    """The cone footprint pins reject a copy of the reference with one
    plausible mistake planted in its footprint: the in-plane shadow pin or
    the perspective row pin fails on the geometry whose pitches differ."""
    mut = _mutant(orc, tmp_path, old, new)
    w = PITCH_CONE
    g = make(mut, w)
    worst = cone_inplane_shadow_errors(lambda v, i, j: mut.vp_params(g, v, i, j), w)
    inplane_caught = any(worst[k] > 2 * tol for k, tol in INPLANE_TOL.items())
    try:
        test_cone_rows_follow_perspective(mut, w)
        rows_caught = False
    except AssertionError:
        rows_caught = True
    assert inplane_caught or rows_caught, worst


# ---------------------------------------------------------------- symmetry ---
def test_symmetry_rotation_by_90_degrees(orc):
    """P9: rotating the image by +90 degrees and the view angle by +pi/2
    leaves the parallel projection unchanged."""
    w = W.get(W.SMALL)
    x = w.recon_input()
    xr = np.ascontiguousarray(x[::-1].transpose(1, 0, 2))
    ang = w.angles()[:10]
    g = orc.Geometry(geom_dict(angles=ang), w.recon_shape, (10, w.nr, w.nc))
    gr = orc.Geometry(geom_dict(angles=ang + math.pi / 2), w.recon_shape, (10, w.nr, w.nc))
    a, b = orc.forward(g, x), orc.forward(gr, xr)
    assert np.abs(a - b).max() < 1e-13 * np.abs(a).max()


def test_symmetry_mirror(orc):
    """P9: mirroring x -> -x and theta -> -theta reverses the channel axis."""
    w = W.get(W.SMALL)
    x = w.recon_input()
    xm = np.ascontiguousarray(x[:, ::-1, :])
    ang = w.angles()[1:12]
    g = orc.Geometry(geom_dict(angles=ang), w.recon_shape, (11, w.nr, w.nc))
    gm = orc.Geometry(geom_dict(angles=-ang), w.recon_shape, (11, w.nr, w.nc))
    a, b = orc.forward(g, x), orc.forward(gm, xm)
    assert np.abs(a - b[:, :, ::-1]).max() < 1e-13 * np.abs(a).max()


# ------------------------------------------------------------ tie canaries ---
def _exact_u(xv, yv, c, s, cch):
    """u of the parallel geometry with every rounding of the stated order
    carried out in exact rational arithmetic, rounding to double after each
    operation (the IEEE definition of the fp64 ops)."""
    xc = float(Fraction(xv) * Fraction(c))
    ys = float(Fraction(yv) * Fraction(s))
    t = float(Fraction(xc) + Fraction(ys))
    return float(Fraction(t) + Fraction(cch))


def test_tie_canaries_round_half_to_even(orc):
    """P10: in the 512x512, 720-view workload the views at 45 and 135 degrees
    hold 512 pixels each whose channel coordinate is exactly 383.5 (cos and sin
    of pi/4 differ by one ulp, and the products cancel exactly); rounding half
    to even sends every one to 384.  A fused multiply-add would move 28 and 21
    of them off the tie, so these entries also catch FMA contraction."""
    w = W.get(W.BENCH)
    g = make(orc, w)
    idx = orc.channel_index(g)
    ang = w.angles()
    coords = (np.arange(512) - 255.5)
    expected_flips = {180: 28, 540: 21}
    for v in (180, 540):
        c, s = math.cos(ang[v]), math.sin(ang[v])
        img = idx[v].reshape(512, 512)
        # the anti-diagonal (v=180) / diagonal (v=540) pixels
        pix = [(i, 511 - i) for i in range(512)] if v == 180 else [(i, i) for i in range(512)]
        flips = 0
        for i, j in pix:
            u = _exact_u(coords[j], coords[i], c, s, 383.5)
            assert u == 383.5
            assert img[i, j] == 384
            # the contracted form: t = fma(x, c, y*s), exact then one rounding
            ys = float(Fraction(coords[i]) * Fraction(s))
            t = float(Fraction(coords[j]) * Fraction(c) + Fraction(ys))
            if round(t + 383.5) != 384:   # python round: half to even
                flips += 1
        assert flips == expected_flips[v]


def test_tie_canaries_only_in_those_views(orc):
    """P10: no other view of the small, the 512x512x64 or the translation
    workloads has a channel coordinate within 1e-9 of a half-integer, except
    the translation geometry, whose coordinates are exact integers."""
    for name in (W.SMALL, W.BENCH):
        w = W.get(name)
        g = make(orc, w)
        near = []
        for v0 in range(0, w.nv, 90):
            sub = orc.Geometry(dict(w.geometry(), num_views=min(90, w.nv - v0),
                                    angles=w.angles()[v0:v0 + 90]),
                               w.recon_shape, (min(90, w.nv - v0), w.nr, w.nc))
            u = orc.channel_coord(sub)
            frac = np.abs(u - np.floor(u) - 0.5)
            vv = np.nonzero((frac < 1e-9).any(axis=1))[0] + v0
            near.extend(int(v) for v in vv)
        assert near == ([180, 540] if name == W.BENCH else [])
    w = W.get("translation-512x512x32-64v")
    u = orc.channel_coord(make(orc, w))
    assert np.array_equal(u, np.round(u))
    assert u.min() == 4.0 and u.max() == 1019.0


# ------------------------------------------------- squared-weight back ---
@pytest.mark.parametrize("w", [W.get(W.SMALL), SMALL_CONE, SMALL_HELIX, SMALL_TRANS],
                         ids=lambda w: w.name)
def test_squared_back_is_hessian_diagonal_weighting(orc, w):
    """P-H: the back projection with squared weights at voxel j is
    sum_i A_ij^2 y_i ("Gradient and Hessian can take different paths",
    coefficient power 2).  A_ij is read off the forward scatter of the unit
    voxel e_j -- a different loop from the back gather -- so a dropped square,
    a wrong tap or a transposed index in either shows up."""
    g = make(orc, w)
    ny, nx, ns = w.recon_shape
    rng = np.random.default_rng(21)
    y = rng.standard_normal(w.sino_shape).astype(np.float32)
    picks = [(ny // 2, nx // 2, ns // 2), (1, nx - 2, 0), (ny - 1, 0, ns - 1), (ny // 3, 2 * nx // 3, ns // 3)]
    for (i, j, k) in picks:
        e = np.zeros(w.recon_shape, np.float32)
        e[i, j, k] = 1.0
        col = orc.forward(g, e)                       # A e_j, fp64
        expect = float((col * col * y.astype(np.float64)).sum())
        got = orc.back_pixels(g, y, [i * nx + j], power=2)[0, k]
        scale = float((col * col * np.abs(y.astype(np.float64))).sum())
        assert scale > 0.0, (i, j, k)
        assert abs(got - expect) <= 1e-12 * scale, (i, j, k, got, expect)
        # and the plain adjoint on the same voxel is sum_i A_ij y_i
        got1 = orc.back_pixels(g, y, [i * nx + j], power=1)[0, k]
        assert abs(got1 - float((col * y.astype(np.float64)).sum())) <= 1e-12 * float(
            (np.abs(col) * np.abs(y.astype(np.float64))).sum()), (i, j, k)


def test_squared_back_single_voxel_axis_aligned(orc):
    """P-H closed form: at theta = 0 with unit pitches a voxel centred on a
    channel has one tap of weight dv/max(|cos|,|sin|) = 1, so its squared
    back projection of y is y at that channel, and a voxel half a channel off
    splits 1/2 + 1/2, whose squares sum to 1/2."""
    geo = geom_dict(angles=(0.0,), dch=1.0)
    g = orc.Geometry(geo, (1, 2, 1), (1, 1, 4))
    y = np.array([[[1.0, 2.0, 4.0, 8.0]]], np.float32)
    # Nx = 2: pixel centres at x = -0.5, +0.5; C = 4: channel centre 1.5, so
    # u = x + 1.5 lands on channels 1 and 2 exactly
    out = orc.back(g, y, power=2)
    assert out[0, 0, 0] == 2.0 and out[0, 1, 0] == 4.0
    g2 = orc.Geometry(dict(geo, det_channel_offset=0.5), (1, 2, 1), (1, 1, 4))
    # u = x + 2: pixel 0 at 1.5 (half in channel 1, half in 2), pixel 1 at 2.5
    out2 = orc.back(g2, y, power=2)
    assert out2[0, 0, 0] == 0.25 * 2.0 + 0.25 * 4.0
    assert out2[0, 1, 0] == 0.25 * 4.0 + 0.25 * 8.0


# ------------------------------------------------------- batches of cylinders ---
def _centroid(w, axis):
    idx = np.arange(w.shape[axis], dtype=np.float64)
    shape = [1] * w.ndim
    shape[axis] = -1
    return float((w * idx.reshape(shape)).sum() / w.sum())


def test_pixel_batch_parallel_centroid_and_mass(orc):
    """P-B: one listed pixel in a batch padded with NaN cylinders.  Per view
    and row, a parallel voxel's taps carry mass cyl[k] dv^2/dch (every tap on
    the detector).  With dch = cos 0.3 and views where max(|cos t|, |sin t|)
    = cos 0.3 the footprint box is exactly one channel wide; the cells it
    overlaps then have their weighted mean at the box centre
    u = (x cos t + y sin t)/dch + (C-1)/2, x = (j - (Nx-1)/2) dv,
    y = (i - (Ny-1)/2) dv, p = i Nx + j (for a box of whole width the offset
    of each point from its cell centre averages to zero).  Ny != Nx, so a
    transposed id fails."""
    ny, nx, ns, nc = 7, 9, 3, 40
    dch = math.cos(0.3)
    angles = (0.3, -0.3, math.pi / 2 - 0.3, math.pi + 0.3, 1.5 * math.pi + 0.3)
    g = orc.Geometry(geom_dict(angles=angles, dch=dch), (ny, nx, ns), (len(angles), ns, nc))
    i, j = 2, 6
    pix = np.array([-1, i * nx + j, ny * nx, -(2 ** 31), ny * nx + 5], np.int64)
    cyl = np.full((len(pix), ns), np.nan, np.float32)
    cyl[1] = [1.0, 2.5, 0.75]
    y = orc.forward_pixels(g, pix, cyl)
    assert np.isfinite(y).all()
    x0, y0 = (j - (nx - 1) / 2), (i - (ny - 1) / 2)
    for v, t in enumerate(angles):
        u = (x0 * math.cos(t) + y0 * math.sin(t)) / dch + (nc - 1) / 2
        for k in range(ns):
            row = y[v, k]
            assert abs(row.sum() - float(cyl[1, k]) / dch) < 1e-13
            assert abs(_centroid(row, 0) - u) < 1e-12


@pytest.mark.parametrize("w", [SMALL_CONE, SMALL_HELIX], ids=lambda w: w.name)
def test_pixel_batch_cone_is_the_scattered_volume(orc, w):
    """P-B (cone), the definition of a batch: listing pixel p = i Nx + j with
    cylinder c projects the volume that holds c at (i, j, 0..S-1) and zero
    elsewhere; the entries with ids outside [0, Ny Nx) hold inf and must
    change nothing.  Ny != Nx for the first workload, so a transposed id
    fails."""
    g = make(orc, w)
    ny, nx, ns = w.recon_shape
    rng = np.random.default_rng(8)
    i, j = ny - 3, 2
    c = rng.standard_normal(ns).astype(np.float32)
    x = np.zeros(w.recon_shape, np.float32)
    x[i, j] = c
    cyl = np.full((3, ns), np.inf, np.float32)
    cyl[1] = c
    got = orc.forward_pixels(g, [ny * nx, i * nx + j, -1], cyl)
    assert np.array_equal(got, orc.forward(g, x))


@pytest.mark.parametrize("w", [W.get(W.SMALL), SMALL_CONE, SMALL_HELIX], ids=lambda w: w.name)
def test_pixel_batch_adjoint_with_repeats_and_padding(orc, w):
    """P1 on batches: <A_B c, y> = <c, A_B^T y> for a batch B with repeated
    ids and padding; the forward runs through the per-view forward and the back
    through the per-pixel gather, two separate code paths."""
    g = make(orc, w)
    ny, nx, ns = w.recon_shape
    rng = np.random.default_rng(21)
    pix = rng.integers(0, ny * nx, 40)
    pix[5] = pix[9] = pix[30]            # a pixel listed three times
    pix[[3, 17, 38]] = [-1, ny * nx, 10 ** 9]
    cyl = rng.standard_normal((len(pix), ns)).astype(np.float32)
    y = rng.standard_normal(w.sino_shape).astype(np.float32)
    fwd = orc.forward_pixels(g, pix, cyl)
    bck = orc.back_pixels(g, y, pix)
    assert not bck[[3, 17, 38]].any()
    keep = np.ones(len(pix), bool)
    keep[[3, 17, 38]] = False
    lhs = float((fwd * y.astype(np.float64)).sum())
    rhs = float((cyl[keep].astype(np.float64) * bck[keep]).sum())
    assert abs(lhs - rhs) < 1e-12 * np.linalg.norm(fwd) * np.linalg.norm(y)


def test_pixel_batch_repeats_add_and_full_list_is_the_volume(orc):
    """P2 on batches: a pixel listed twice adds its cylinders (values on a
    1/16 grid, so the sum is exact in fp32), and listing every pixel once, in
    any order, is the forward of the whole volume."""
    w = W.get(W.SMALL)
    g = make(orc, w)
    ny, nx, ns = w.recon_shape
    rng = np.random.default_rng(5)
    c1 = (rng.integers(-64, 64, ns) / 16.0).astype(np.float32)
    c2 = (rng.integers(-64, 64, ns) / 16.0).astype(np.float32)
    p = 17 * nx + 40
    twice = orc.forward_pixels(g, [p, p], np.stack([c1, c2]))
    once = orc.forward_pixels(g, [p], (c1 + c2)[None])
    assert np.allclose(twice, once, rtol=0, atol=1e-12)
    x = w.recon_input()
    perm = rng.permutation(ny * nx)
    full = orc.forward_pixels(g, perm, x.reshape(ny * nx, ns)[perm])
    assert np.array_equal(full, orc.forward(g, x))
