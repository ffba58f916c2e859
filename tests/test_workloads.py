"""The seeded input recipes: shapes, determinism and the stated structure."""
import math

import numpy as np

import workloads as W


def test_all_workloads_have_consistent_shapes():
    for w in W.WORKLOADS.values():
        assert w.angles().shape == (w.nv,)
        if w.kind == W.PARALLEL:
            assert w.nr == w.ns                    # row r sees slice r
        g = w.geometry()
        assert g["num_views"] == w.nv
        assert w.nv * w.ny * w.nx < 2 ** 31        # index table below 2^31 entries


def test_angle_sets():
    par = W.get(W.BENCH)
    assert par.angles()[0] == 0.0 and par.angles()[-1] < math.pi
    assert np.allclose(np.diff(par.angles()), math.pi / 720)
    cone = W.get("cone-256x256x256-360v")
    assert cone.angles()[-1] < 2 * math.pi
    hel = W.get("helical-512x512x96-1338v")
    assert np.allclose(np.diff(hel.angles()), 2 * math.pi / 600)
    z = hel.source_z()
    assert np.allclose(np.diff(z), 0.1) and abs(z[0] + z[-1]) < 1e-12
    tr = W.get("translation-512x512x32-64v")
    assert np.all(tr.angles() == 0.0)
    assert np.array_equal(tr.channel_shift(), 8.0 * np.arange(64) - 252.0)


def test_disk_phantom():
    w = W.get(W.SMALL)
    x = w.recon_input()
    assert x.shape == (64, 64, 8) and x.dtype == np.float32
    assert np.array_equal(x, w.recon_input())                 # seeded
    c = np.arange(64) - 31.5
    inside = (c[None, :] ** 2 + c[:, None] ** 2) < 28 ** 2
    assert np.all(x[inside] >= 1.0) and np.all(x[inside] < 1.1)
    assert np.all(x[~inside] >= 0.0) and np.all(x[~inside] < 0.1)


def test_ellipsoid_phantom_structure():
    x = W.ellipsoid_phantom(64, 64, 16, seed=2)
    assert x.dtype == np.float32 and x.shape == (64, 64, 16)
    assert x.min() >= 0.0 and np.count_nonzero(x) > 0.01 * x.size
    params = W.ellipsoid_params(64, 64, 16, seed=2)
    assert len(params) == 10
    assert x.max() <= sum(p["val"] for p in params) + 1e-6
    for p in params:
        assert math.hypot(p["cx"], p["cy"]) <= 0.6 * 32 + 1e-9
        assert 0.08 * 32 <= p["ax"] <= 0.35 * 32 + 1e-9
    assert np.array_equal(x, W.ellipsoid_phantom(64, 64, 16, seed=2))


def test_back_inputs_are_seeded_normal():
    w = W.get("translation-512x512x32-64v")
    y = w.sino_input()
    assert y.shape == w.sino_shape and y.dtype == np.float32
    assert abs(float(y.mean())) < 0.01 and abs(float(y.std()) - 1) < 0.01
