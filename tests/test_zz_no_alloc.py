"""proj_forward_noalloc through the C ABI against proj_forward.

The allocation-free forward runs the same kernels with the parallel walk's
partial sums in the library's fixed device scratch.  Its sinogram must match
proj_forward's to the parity bar (relative L2 1e-5, max relative error 1e-4
with the reference's absolute sums as denominators) on two calls in a row, the
second on a smaller problem, so that it starts from what the first left in the
scratch.  Handles whose accumulation buffer exceeds the scratch are refused
before anything is written.
"""
import numpy as np
import pytest

import workloads as W
from metrics import assert_close, rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def note(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.fixture(scope="module")
def bp():
    import back_projectors_amd as m
    m.load_library()
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_against_forward(bp, orc, w, views, geo=None):
    """One proj_forward_noalloc call on workload w against proj_forward on the
    same handle and input: the whole sinogram in relative L2, and the views
    `views` to the parity bar with the reference's absolute sums."""
    geo = w.geometry() if geo is None else geo
    proj = bp.Projector(geo, w.recon_shape, w.sino_shape)
    x = w.recon_input() if w.phantom == "disk" else np.random.default_rng(w.seed_x).standard_normal(
        w.recon_shape).astype(np.float32)
    xd = dev(x)
    ref = host(proj.forward(xd))
    out = torch.full(w.sino_shape, float("nan"), device="cuda:0")
    got = host(proj.forward_noalloc(xd, out=out))
    assert np.isfinite(got).all()
    assert rel_l2(got, ref) < 1e-6, f"{w.name}: no-alloc forward differs from proj_forward"
    g = orc.Geometry(geo, w.recon_shape, w.sino_shape)
    yo, ay = orc.forward_views(g, x, views, with_abs=True)
    assert_close(got[views], ref[views].astype(np.float64), ay, f"{w.name} no-alloc vs proj_forward")
    assert_close(got[views], yo, ay, f"{w.name} no-alloc vs reference")
    proj.close()


def test_noalloc_forward_two_calls_second_smaller(bp, orc):
    """The 512x512x64, 720-view scan (142 MB of accumulation buffer, the
    largest workload the scratch holds), then the 64x64x8, 90-view one."""
    big = W.get("parallel-512x512x64-720v")
    note(f"no-alloc forward {big.name}")
    check_against_forward(bp, orc, big, [0, 180, 361, 540, 719])
    small = W.get(W.SMALL)
    note(f"no-alloc forward {small.name} after it")
    check_against_forward(bp, orc, small, list(range(small.nv)))


@pytest.mark.parametrize("name,strategy", [
    ("translation", 1), ("translation", 0), ("ragged-gather", 2), ("ragged-tile", 1), ("cone", 0), ("helical", 0)])
def test_noalloc_forward_strategies_and_geometries(bp, orc, name, strategy):
    """Both parallel strategies, a translation scan (forced region walk, and
    its own column forward, whose column sums then live in the scratch) and
    the cone geometries (which use no scratch) through the allocation-free
    entry point."""
    w = {
        "translation": W.scaled(W.get("translation-512x512x32-64v"), "translation-40x48x12-9v", ny=40, nx=48, ns=12,
                                nv=9, nr=12, nc=96, shift_step=3.0, seed_x=27),
        "ragged-gather": W.Workload("parallel-45x70x20-37v", W.PARALLEL, 45, 70, 20, 37, 20, 90, seed_x=21),
        "ragged-tile": W.Workload("parallel-45x70x20-37v", W.PARALLEL, 45, 70, 20, 37, 20, 90, seed_x=22),
        "cone": W.Workload("cone-37x40x30-23v", W.CONE_FLAT, 37, 40, 30, 23, 28, 60, dch=1.5, drow=1.5, sid=80.0,
                           sdd=120.0, seed_x=29),
        "helical": W.Workload("helical-36x36x40-47v", W.CONE_FLAT, 36, 36, 40, 47, 12, 60, dch=11 / 6,
                              drow=11 / 6, sid=45.0, sdd=82.5, angle_step=0.314159, zsrc_step=0.6, seed_x=33),
    }[name]
    note(f"no-alloc forward {w.name} strategy={strategy}")
    geo = dict(w.geometry(), forward_strategy=strategy)
    check_against_forward(bp, orc, w, list(range(w.nv)), geo=geo)


def test_noalloc_forward_refuses_a_buffer_over_the_scratch(bp):
    """A parallel handle whose accumulation buffer (100 views x 1026 channels
    x 512 slices, 210 MB) exceeds the 144 MiB scratch: PROJ_ERR_UNSUPPORTED,
    the sinogram untouched; proj_forward on the handle still works."""
    geo = dict(kind=0, num_views=100, angles=np.linspace(0.0, 3.0, 100), delta_channel=1.0)
    rs, ss = (8, 8, 512), (100, 512, 1024)
    note(f"no-alloc refusal recon={rs} sino={ss}")
    proj = bp.Projector(geo, rs, ss)
    x = torch.ones(rs, device="cuda:0")
    out = torch.full(ss, 5.0, device="cuda:0")
    with pytest.raises(bp.ProjError) as ei:
        proj.forward_noalloc(x, out=out)
    assert ei.value.status == -2 and "144 MiB" in str(ei.value)
    assert bool(torch.all(out == 5.0))
    y = proj.forward(x)
    # every voxel's taps land on the detector: each view and row carries the slice's mass (64 voxels)
    mass = host(y).sum(axis=2)
    assert np.allclose(mass, 64.0, rtol=1e-5)
    proj.close()
