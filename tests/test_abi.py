"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, and rejects bad requests with the documented status before
touching a GPU.  No compute call runs here."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "proj.h")


@pytest.fixture(scope="session")
def bp():
    import back_projectors_amd as m
    if not os.path.exists(m.LIB_PATH):
        from back_projectors_amd import build_lib
        build_lib.build()
    m.load_library()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(proj_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("proj_create", "proj_forward", "proj_back", "proj_channel_index", "proj_destroy"):
        assert must in names


def test_library_exports_every_declared_symbol(bp):
    names = declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", bp.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    lib = bp.load_library()
    for n in names:
        getattr(lib, n)                               # resolvable through ctypes
    assert set(bp.EXPORTS) == set(names)


def test_status_strings(bp):
    lib = bp.load_library()
    for code, name in bp.STATUS.items():
        assert lib.proj_status_string(code).decode() == name
    assert lib.proj_status_string(17).decode() == "PROJ_ERR_UNKNOWN"


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_every_workload_plans(bp, name):
    w = W.get(name)
    desc = bp.plan_query(w.geometry(), w.recon_shape, w.sino_shape)
    assert ("parallel" if w.kind == W.PARALLEL else "cone_flat") in desc
    assert f"V={w.nv}" in desc


def base_geo(**kw):
    g = dict(kind=0, num_views=4, angles=np.linspace(0, 3, 4), delta_voxel=1.0, delta_channel=1.0,
             delta_row=1.0, psf_radius=1)
    g.update(kw)
    return g


CONE = dict(kind=1, source_iso=100.0, source_detector=150.0, delta_channel=1.5, delta_row=1.5)

BAD = [
    ("kind", base_geo(kind=3), (8, 8, 4), (4, 4, 16), -1),
    ("column forward on a rotating scan", base_geo(forward_strategy=5), (8, 8, 4), (4, 4, 16), -2),
    ("column forward with one view off 0", base_geo(angles=np.array([0.0, 0.0, 1e-300, 0.0]), forward_strategy=5),
     (8, 8, 4), (4, 4, 16), -2),
    ("column forward on a cone", dict(base_geo(forward_strategy=5), **CONE), (8, 8, 4), (4, 4, 16), -1),
    ("views mismatch", base_geo(num_views=5, angles=np.zeros(5)), (8, 8, 4), (4, 4, 16), -1),
    ("nan angle", base_geo(angles=np.array([0.0, math.nan, 1.0, 2.0])), (8, 8, 4), (4, 4, 16), -1),
    ("inf shift", base_geo(channel_shift=np.array([0.0, math.inf, 0.0, 0.0])), (8, 8, 4), (4, 4, 16), -1),
    ("zero pitch", base_geo(delta_channel=0.0), (8, 8, 4), (4, 4, 16), -1),
    ("negative voxel", base_geo(delta_voxel=-1.0), (8, 8, 4), (4, 4, 16), -1),
    ("parallel R != S", base_geo(), (8, 8, 4), (4, 5, 16), -1),
    ("parallel drow != dv", base_geo(delta_row=2.0), (8, 8, 4), (4, 4, 16), -1),
    ("parallel source_z", base_geo(source_z=np.zeros(4)), (8, 8, 4), (4, 4, 16), -1),
    ("radius 0", base_geo(psf_radius=0), (8, 8, 4), (4, 4, 16), -1),
    ("radius 5", base_geo(psf_radius=5), (8, 8, 4), (4, 4, 16), -1),
    ("negative shape", base_geo(), (8, -8, 4), (4, 4, 16), -1),
    ("source inside volume", base_geo(**dict(CONE, source_iso=5.0, source_detector=9.0)), (8, 8, 4), (4, 6, 16), -1),
    ("detector before iso", base_geo(**dict(CONE, source_detector=90.0)), (8, 8, 4), (4, 6, 16), -1),
    ("nan distance", base_geo(**dict(CONE, source_iso=math.nan)), (8, 8, 4), (4, 6, 16), -1),
    ("index table too large", base_geo(num_views=40000, angles=np.zeros(40000)), (256, 256, 1),
     (40000, 1, 16), -2),
    ("recon of 2^31 elements", base_geo(), (2048, 2048, 512), (4, 512, 16), -2),
    ("sinogram of 2^31 elements", base_geo(num_views=8192, angles=np.zeros(8192)), (4, 4, 16), (8192, 16, 16384),
     -2),
    ("16384 channels", base_geo(), (8, 8, 4), (4, 4, 16384), -2),
    ("detector 10x finer than voxels", base_geo(delta_channel=0.1), (8, 8, 4), (4, 4, 160), -2),
    ("cone detector 20x finer", base_geo(**dict(CONE, delta_channel=0.05, delta_row=0.05)), (8, 8, 4), (4, 200, 400),
     -2),
    ("cone rows 8x coarser", base_geo(**dict(CONE, delta_row=8.0)), (8, 8, 4), (4, 6, 16), -2),
    ("cone detector of 2^28 / radius channels", base_geo(**dict(CONE, psf_radius=4)), (8, 8, 4), (4, 1, 1 << 26),
     -2),
    ("forward strategy 3", base_geo(forward_strategy=3), (8, 8, 4), (4, 4, 16), -1),
    ("forward strategy -1", base_geo(forward_strategy=-1), (8, 8, 4), (4, 4, 16), -1),
    ("cone forward strategy", base_geo(**dict(CONE, forward_strategy=2)), (8, 8, 4), (4, 6, 16), -1),
    ("cone forward strategy 5", base_geo(**dict(CONE, forward_strategy=5)), (8, 8, 4), (4, 6, 16), -1),
    ("parallel with a cone tile", base_geo(forward_strategy=3), (8, 8, 4), (4, 4, 16), -1),
]


def test_largest_shapes_plan(bp):
    """Shapes just inside the limits plan (no allocation here): a recon of
    2^31 - 2^20 elements, psf radius 4."""
    desc = bp.plan_query(base_geo(), (2048, 2047, 512), (4, 512, 4096))
    assert "Ny=2048 Nx=2047 S=512" in desc
    assert "radius=4" in bp.plan_query(base_geo(psf_radius=4), (8, 8, 4), (4, 4, 16))


@pytest.mark.parametrize("slices,words", [
    (16, ("48x48 px tile", "lanes=16 slices x 4 views", ", 16 slices,")),
    (17, ("40x32 px tile", "lanes=16 x 4 views with 2 slices each", ", 32 slices,")),
    (64, ("40x32 px tile", "lanes=16 x 4 views with 2 slices each", ", 32 slices,")),
])
def test_region_walk_slices_per_lane(bp, slices, words):
    """The tile forward walks two slices per lane (32-slice chunks over 40x32
    regions) unless the volume has 16 slices or fewer (one slice per lane,
    16-slice chunks over 48x48 regions)."""
    desc = bp.plan_query(base_geo(num_views=720, angles=np.arange(720) * np.pi / 720, forward_strategy=1),
                         (256, 256, slices), (720, slices, 384))
    for word in words:
        assert word in desc, (word, desc)


@pytest.mark.parametrize("w,stride", [
    (W.scaled(W.get("cone-256x256x256-360v"), "cone-22x26x30-13v-coarserows", ny=22, nx=26, ns=30, nv=13, nr=24,
              nc=40, dch=1.5, drow=3.0, sid=40.0, sdd=60.0), 3),
    (W.scaled(W.get("cone-256x256x256-360v"), "cone-20x24x100-12v-unitwalk", ny=20, nx=24, ns=100, nv=12, nr=128,
              nc=48, dch=1.5, drow=1.5, sid=40.0, sdd=60.0), 2),
    (W.scaled(W.get("cone-256x256x256-360v"), "cone-20x24x18-11v", ny=20, nx=24, ns=18, nv=11, nr=24, nc=48,
              dch=1.5, drow=0.9, sid=40.0, sdd=60.0), 1),
], ids=lambda v: v if isinstance(v, int) else v.name)
def test_cone_forward_slice_stride(bp, w, stride):
    """Lanes of one cone forward instruction take slices `stride` apart, the
    smallest stride at which the smallest row magnification over the scan
    (rows per slice, at the volume's corners) puts them on distinct rows: the
    chunk is 64 * stride slices."""
    desc = bp.plan_query(w.geometry(), w.recon_shape, w.sino_shape)
    assert f"channel ring accumulators, {64 * stride} slices," in desc.split("forward:")[1], desc


def test_cone_forward_window_wider_than_a_flush_step(bp):
    """Channels far finer than the magnified voxels: the cone forward's
    detector window spans more than the 64 lanes of one flush step, which
    then walks the window's cells in order (the GPU parity case of this
    geometry runs that flush)."""
    geo = dict(kind=1, num_views=5, angles=-0.05 + 0.025 * np.arange(5), delta_voxel=1.0, delta_channel=0.14,
               delta_row=4.0, source_iso=200.0, source_detector=300.0, psf_radius=1)
    desc = bp.plan_query(geo, (20, 24, 16), (5, 12, 300))
    nw = int(re.search(r"forward: .*? window (\d+) ch", desc).group(1))
    assert nw > 64, desc


def test_cone_forward_window_taller_than_a_row_group(bp):
    """Detector rows far finer than the voxels: the cone forward's windows
    hold more detector rows than the three 64-lane passes of one row group,
    so its walk takes several groups (the GPU parity case of this geometry,
    cone-20x24x64-9v-vtallrows, runs that walk)."""
    geo = dict(kind=1, num_views=9, angles=2 * np.pi / 9 * np.arange(9), delta_voxel=1.0, delta_channel=2.0,
               delta_row=0.45, source_iso=60.0, source_detector=120.0, psf_radius=1)
    desc = bp.plan_query(geo, (20, 24, 64), (9, 260, 40))
    nr = int(re.search(r"forward: .*? window \d+ ch x (\d+) rows", desc).group(1))
    assert min(nr, 260) > 3 * 64, desc


@pytest.mark.parametrize("drow,slices", [(0.8, 48), (0.7, 32), (0.5, 16)])
def test_cone_back_chunk_falls_back_when_the_window_overflows(bp, drow, slices):
    """96 slices take 48-slice back chunks (two, no padding) while their
    double-buffered window fits the workgroup's LDS; finer rows make the window
    taller and the planner steps down 48 -> 32 -> 16 slices."""
    geo = dict(kind=1, num_views=8, angles=2 * np.pi / 8 * np.arange(8), delta_voxel=1.0, delta_channel=1.0,
               delta_row=drow, source_iso=100.0, source_detector=150.0, psf_radius=1)
    desc = bp.plan_query(geo, (32, 32, 96), (8, 300, 80))
    assert f"back: 16x16 px tile, lanes=pixels, {slices} slices/lane" in desc, desc


def test_helical_radius2_plans(bp):
    """The helical scan at psf radius 2 (no truncated footprint) plans with
    5x5 taps."""
    w = W.scaled(W.get("helical-512x512x96-1338v"), "helical-r2", radius=2)
    desc = bp.plan_query(w.geometry(), w.recon_shape, w.sino_shape)
    assert "radius=2 taps=5" in desc, desc


@pytest.mark.parametrize("name,inter", [("cone-256x256x256-360v", False), ("helical-512x512x96-1338v", True)])
def test_cone_forward_profile_columns(bp, name, inter):
    """Interleaved row-profile columns only where they save slice passes: the
    helical scan's far pixels reach the detector with fewer than 64 slices of
    the 128-slice chunk, which then take one pass instead of two; every chunk
    of the 256^3 cone is active over nearly all its slices, so it keeps one
    column (and its LDS: a second column would cost a workgroup per CU)."""
    w = W.get(name)
    desc = bp.plan_query(w.geometry(), w.recon_shape, w.sino_shape)
    assert ("interleaved row-profile columns" in desc) == inter, desc


@pytest.mark.parametrize("name,rows_scale,tile", [("cone-256x256x256-360v", 1, "8x4"),
                                                  ("helical-512x512x96-1338v", 1, "8x4"),
                                                  ("cone-256x256x256-360v", 2, "8x8")])
def test_cone_forward_tile_choice(bp, name, rows_scale, tile):
    """The cone forward's tile from the planner's estimate: the 256^3 cone and
    the helical scan, both bound by their slice work, take 8 x 4 tiles; the
    256^3 cone on a detector with twice the rows at half the pitch, whose
    atomic adds from 8 x 4 tiles would bound the call, takes 8 x 8 (half the
    adds per voxel-view).  Either can be forced."""
    w = W.get(name)
    geo = dict(w.geometry(), delta_row=w.geometry()["delta_row"] / rows_scale)
    sino = (w.sino_shape[0], w.sino_shape[1] * rows_scale, w.sino_shape[2])
    fwd = lambda d: d.split("forward:")[1]
    assert f"{tile} px tile" in fwd(bp.plan_query(geo, w.recon_shape, sino))
    for code, forced in ((3, "8x4"), (4, "8x8")):
        desc = bp.plan_query(dict(geo, forward_strategy=code), w.recon_shape, sino)
        assert f"{forced} px tile" in fwd(desc), desc


@pytest.mark.parametrize("ny,ns,nv,kind,word", [
    (64, 8, 90, "parallel", "gather:"), (512, 64, 8, "parallel", "gather:"), (512, 64, 12, "parallel", "gather:"),
    (512, 64, 16, "parallel", "tile:"), (512, 32, 16, "translation", "column:"),
    (512, 32, 24, "translation", "column:"), (512, 32, 64, "translation", "column:"), (256, 32, 96, "parallel", "tile:"),
    (512, 64, 720, "parallel", "tile:"),
])
def test_forward_strategy_rule(bp, ny, ns, nv, kind, word):
    """The planner's parallel forward strategy on shapes of the gfx950 sweep:
    gather up to 1e8 voxel-views, and up to 2.5e8 with at most 32 views;
    translation scans (every view at angle 0) take the column forms."""
    base = W.get("translation-512x512x32-64v" if kind == "translation" else W.BENCH)
    w = W.scaled(base, "sweep", ny=ny, nx=ny, ns=ns, nr=ns, nv=nv, nc=int(ny * 1.5) + 16)
    desc = bp.plan_query(w.geometry(), w.recon_shape, w.sino_shape)
    assert word in desc.split("forward:")[1]
    assert ("back: column:" in desc) == (kind == "translation")


def test_translation_column_forward_is_chosen_and_can_be_overridden(bp):
    """A translation scan plans the column forward by itself; tile and gather
    can still be forced, and the back stays in its column form either way."""
    w = W.get("translation-512x512x32-64v")
    assert "column:" in bp.plan_query(w.geometry(), w.recon_shape, w.sino_shape).split("forward:")[1]
    assert "column:" in bp.plan_query(dict(w.geometry(), forward_strategy=5), w.recon_shape, w.sino_shape)
    for code, word in ((1, "tile:"), (2, "gather:")):
        desc = bp.plan_query(dict(w.geometry(), forward_strategy=code), w.recon_shape, w.sino_shape)
        assert word in desc.split("forward:")[1] and "back: column:" in desc


@pytest.mark.parametrize("strategy,word", [(1, "tile:"), (2, "gather:")])
def test_forward_strategy_is_honoured(bp, strategy, word):
    """A forced parallel forward strategy shows in the plan; AUTO picks one."""
    w = W.get("parallel-512x512x64-720v")
    desc = bp.plan_query(dict(w.geometry(), forward_strategy=strategy), w.recon_shape, w.sino_shape)
    assert word in desc
    auto = bp.plan_query(w.geometry(), w.recon_shape, w.sino_shape)
    assert ("tile:" in auto) != ("gather:" in auto)


@pytest.mark.parametrize("case", BAD, ids=lambda c: c[0])
def test_invalid_requests_rejected_before_any_device_call(bp, case):
    _, geo, rs, ss, code = case
    with pytest.raises(bp.ProjError) as ei:
        bp.plan_query(geo, rs, ss)
    assert ei.value.status == code
    # proj_create runs the same checks first, so it fails the same way on a
    # machine without a GPU
    lib = bp.load_library()
    ga = bp._GeomArgs(geo, rs, ss)
    h = ctypes.c_void_p(123)
    st = lib.proj_create(ctypes.byref(ga.s), ga.rs, ga.ss, 0, ctypes.byref(h))
    assert st == code and not h.value
    assert lib.proj_last_error().decode()


def test_null_arguments(bp):
    lib = bp.load_library()
    assert lib.proj_create(None, None, None, 0, None) == -1
    assert lib.proj_forward(None, None, None, None) == -1
    assert lib.proj_back(None, None, None, None) == -1
    assert lib.proj_channel_index(None, None, None) == -1
    assert lib.proj_back_squared(None, None, None, None) == -1
    assert lib.proj_forward_pixels(None, None, 0, None, None, None) == -1
    assert lib.proj_back_pixels(None, None, None, 0, None, None) == -1
    assert lib.proj_solver_workspace_size(None, None) == -1
    info = bp._SolverInfo()
    assert lib.proj_cgls(None, None, None, None, None, 0, 1, 0.0, 0.0, None, ctypes.byref(info), None) == -1
    assert lib.proj_sirt(None, None, None, None, None, 0, 1, 0.0, 0.0, 1.0, 1, None, ctypes.byref(info), None) == -1
    lib.proj_destroy(None)                           # ignored
    assert lib.proj_describe(None, None, 0) == -1


def test_valid_geometry_without_gpu_fails_only_at_the_device(bp):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lib = bp.load_library()
    w = W.get(W.SMALL)
    ga = bp._GeomArgs(w.geometry(), w.recon_shape, w.sino_shape)
    h = ctypes.c_void_p()
    st = lib.proj_create(ctypes.byref(ga.s), ga.rs, ga.ss, 0, ctypes.byref(h))
    assert st in (-1, -5)            # no device: invalid ordinal or HIP error
    assert not h.value


def test_product_path_fails_loudly_without_the_library(tmp_path):
    import back_projectors_amd as m
    saved = m._lib
    try:
        m._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            m.load_library(str(tmp_path / "missing.so"))
    finally:
        m._lib = saved
