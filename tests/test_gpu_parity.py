"""GPU parity: the HIP path through the C ABI against the fp64 CPU reference.

Channel indices must match bit for bit; fp32 projections must be within
relative L2 1e-5 and max relative error 1e-4 (denominator: the sum of
|tap weight * input| reaching the entry), and the GPU pair must satisfy the
adjoint identity within 1e-5.  Small geometries are compared element by
element (several tiles, ragged edges in pixels, slices and views); the full
benchmark sizes are compared on sampled views and pixels, which the reference
computes one at a time.
"""
import math

import numpy as np
import pytest

import workloads as W
from metrics import ADJOINT, adjoint_gap, assert_close, rel_l2

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


# Small geometries: ragged against the 16- and 32-pixel tiles and the slice
# chunks, a few dozen views, every entry compared.
PAR_RAGGED = W.Workload("parallel-45x70x20-37v", W.PARALLEL, 45, 70, 20, 37, 20, 90, seed_x=21, seed_y=22)
PAR_FINE = W.Workload("parallel-33x29x9-31v-fine-r2", W.PARALLEL, 33, 29, 9, 31, 9, 80, dch=0.6,
                      radius=2, seed_x=23, seed_y=24)
PAR_WIDE = W.Workload("parallel-40x40x70-13v", W.PARALLEL, 40, 40, 70, 13, 70, 64, seed_x=25, seed_y=26)
TRANS_SMALL = W.Workload("translation-40x48x12-9v", W.PARALLEL, 40, 48, 12, 9, 12, 96, shift_step=3.0,
                         seed_x=27, seed_y=28)
CONE_RAGGED = W.Workload("cone-37x40x30-23v", W.CONE_FLAT, 37, 40, 30, 23, 28, 60, dch=1.5, drow=1.5,
                         sid=80.0, sdd=120.0, seed_x=29, seed_y=30)
CONE_R2 = W.Workload("cone-20x24x18-11v-r2", W.CONE_FLAT, 20, 24, 18, 11, 30, 50, dch=0.9, drow=0.9,
                     sid=40.0, sdd=70.0, radius=2, seed_x=31, seed_y=32)
HELIX_SMALL = W.Workload("helical-36x36x40-47v", W.CONE_FLAT, 36, 36, 40, 47, 12, 60, dch=11 / 6,
                         drow=11 / 6, sid=45.0, sdd=82.5, angle_step=2 * math.pi / 20, zsrc_step=0.6,
                         seed_x=33, seed_y=34)
# larger psf radii: 4 channel taps on a fine parallel detector; cone radii 3
# and 4 (their outer taps carry no weight here, the code paths are what counts)
PAR_R4 = W.Workload("parallel-30x26x11-19v-fine-r4", W.PARALLEL, 30, 26, 11, 19, 11, 120, dch=0.45, radius=4,
                    seed_x=41, seed_y=42)
CONE_R3 = W.Workload("cone-22x26x20-13v-r3", W.CONE_FLAT, 22, 26, 20, 13, 40, 70, dch=1.0, drow=1.0, sid=50.0,
                     sdd=80.0, radius=3, seed_x=43, seed_y=44)
CONE_R4 = W.Workload("cone-22x26x20-13v-r4", W.CONE_FLAT, 22, 26, 20, 13, 40, 70, dch=1.5, drow=1.5, sid=50.0,
                     sdd=80.0, radius=4, seed_x=45, seed_y=46)
# rows much finer than the voxels (about 2 rows per slice): the cone back's
# window of a 32-slice chunk spans about 70 rows, its widest LDS row pitch
CONE_TALL = W.Workload("cone-30x34x64-17v-tallrows", W.CONE_FLAT, 30, 34, 64, 17, 128, 40, dch=2.0, drow=0.45,
                       sid=60.0, sdd=70.0, seed_x=47, seed_y=48)
# channels finer than the voxels at radius 1: footprints up to about 2.6
# channels wide are cut by the three taps (parallel, and cone with a row pitch
# close to the voxels')
PAR_TRUNC = W.Workload("parallel-26x30x18-21v-fine-r1", W.PARALLEL, 26, 30, 18, 21, 18, 90, dch=0.55, radius=1,
                       seed_x=61, seed_y=62)
# a translation scan with ragged sizes, two 64-slice chunks, a fine detector
# and five taps: the column forms (every view at angle 0) beyond one block
TRANS_R2 = W.Workload("translation-23x37x70-7v-fine-r2", W.PARALLEL, 23, 37, 70, 7, 70, 90, shift_step=2.5, dch=0.7,
                      radius=2, seed_x=65, seed_y=66)
CONE_FINECH = W.Workload("cone-24x28x20-15v-finech", W.CONE_FLAT, 24, 28, 20, 15, 30, 110, dch=0.45, drow=1.2,
                         sid=50.0, sdd=75.0, seed_x=63, seed_y=64)
# the same at radius 3: a batch forward's detector band (64 slices at up to
# about 4.2 rows each, 7 channel taps) outgrows the band the LDS holds in the
# high-magnification views, which then take the direct form
CONE_TALL_R3 = W.Workload("cone-30x34x64-17v-tallrows-r3", W.CONE_FLAT, 30, 34, 64, 17, 128, 40, dch=2.0, drow=0.45,
                          sid=60.0, sdd=70.0, radius=3, seed_x=49, seed_y=50)
# a short source distance: the planned stride is 2 (row magnification down to
# 0.73), while the tiles nearest the source (magnification at least 1) walk
# consecutive slices, over 64 of them, in as many passes as the stride; 128
# rows cut the longest cylinders
CONE_UNIT = W.Workload("cone-20x24x100-12v-unitwalk", W.CONE_FLAT, 20, 24, 100, 12, 128, 48, dch=1.5, drow=1.5,
                       sid=40.0, sdd=60.0, seed_x=65, seed_y=66)
# detector rows coarser than the voxels (row magnification 0.38 to 0.74): the
# cone forwards (full and batch) take slices three apart per instruction
CONE_COARSE = W.Workload("cone-22x26x30-13v-coarserows", W.CONE_FLAT, 22, 26, 30, 13, 24, 40, dch=1.5, drow=3.0,
                         sid=40.0, sdd=60.0, seed_x=67, seed_y=68)
# channels about 11 times finer than the magnified voxels and rows 2.7 times
# coarser, near-frontal views: the cone forward's detector window spans 89
# channels, over the 64 lanes of a flush step (the flush then walks the
# window's cells in order, 64 per step)
CONE_WIDEWIN = W.Workload("cone-20x24x16-5v-widewindow", W.CONE_FLAT, 20, 24, 16, 5, 12, 300, dch=0.14, drow=4.0,
                          sid=200.0, sdd=300.0, angle_step=0.025, angle_start=-0.05, seed_x=69, seed_y=70)
# the small helical scan at psf radius 2: its footprints near the source are
# up to 2.6 channels wide, which radius 1 truncates and radius 2 keeps whole
HELIX_R2 = W.scaled(HELIX_SMALL, "helical-36x36x40-47v-r2", radius=2, seed_x=71, seed_y=72)
# rows far finer than the voxels (about 4.4 rows per slice, footprints wider
# than the three row taps): the forward windows hold all 260 detector rows,
# more than the three passes of 64 lanes one row group keeps in registers, so
# the forward walks its pixels once per row group
CONE_VTALL = W.Workload("cone-20x24x64-9v-vtallrows", W.CONE_FLAT, 20, 24, 64, 9, 260, 40, dch=2.0, drow=0.45,
                        sid=60.0, sdd=120.0, seed_x=83, seed_y=84)
SMALL_CASES = [W.get(W.SMALL), PAR_RAGGED, PAR_FINE, PAR_WIDE, TRANS_SMALL, PAR_R4, CONE_RAGGED, CONE_R2, CONE_R3,
               CONE_R4, HELIX_SMALL, CONE_TALL, PAR_TRUNC, CONE_FINECH, CONE_TALL_R3, CONE_UNIT, CONE_COARSE,
               CONE_WIDEWIN, HELIX_R2, TRANS_R2, CONE_VTALL]


def inputs(w):
    rng = np.random.default_rng(w.seed_x)
    x = w.recon_input() if w.phantom == "disk" else rng.standard_normal(w.recon_shape).astype(np.float32)
    y = np.random.default_rng(w.seed_y).standard_normal(w.sino_shape).astype(np.float32)
    return x, y


@pytest.mark.parametrize("w", SMALL_CASES, ids=lambda w: w.name)
def test_small_parity(bp, orc, w):
    note(f"small parity {w.name} recon={w.recon_shape} sino={w.sino_shape}")
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    x, y = inputs(w)
    # channel indices: bit-exact
    assert np.array_equal(host(proj.channel_index()), orc.channel_index(g))
    # forward
    yo, ay = orc.forward(g, x, with_abs=True)
    yg = host(proj.forward(dev(x)))
    assert_close(yg, yo, ay, f"{w.name} forward")
    # back (of an independent sinogram; the small disk case backs up the reference forward of x)
    yin = yo.astype(np.float32) if w.phantom == "disk" else y
    xo, ax = orc.back(g, yin, with_abs=True)
    xg = host(proj.back(dev(yin)))
    assert_close(xg, xo, ax, f"{w.name} back")
    # adjoint identity of the GPU pair
    ygy = host(proj.back(dev(y)))
    gap = adjoint_gap(yg, y, x, ygy)
    assert gap < ADJOINT, f"adjoint gap {gap:.2e}"
    proj.close()


@pytest.mark.parametrize("w", [PAR_RAGGED, CONE_RAGGED, HELIX_SMALL], ids=lambda w: w.name)
def test_outputs_fully_overwritten_and_guards_untouched(bp, orc, w):
    """NaN-prefilled outputs come back fully written; canaries just outside
    the output ranges keep their values (adapted poison-the-padding test)."""
    note(f"guard bands {w.name}")
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    x, y = inputs(w)
    pad = 1024
    ns, nr = int(np.prod(w.sino_shape)), int(np.prod(w.recon_shape))
    sbuf = torch.full((ns + 2 * pad,), float("nan"), device="cuda:0")
    rbuf = torch.full((nr + 2 * pad,), float("nan"), device="cuda:0")
    sbuf[:pad] = 7.0
    sbuf[-pad:] = 7.0
    rbuf[:pad] = -3.0
    rbuf[-pad:] = -3.0
    sview = sbuf[pad:pad + ns].view(w.sino_shape)
    rview = rbuf[pad:pad + nr].view(w.recon_shape)
    proj.forward(dev(x), out=sview)
    proj.back(dev(y), out=rview)
    s, r = host(sbuf), host(rbuf)
    assert np.all(s[:pad] == 7.0) and np.all(s[-pad:] == 7.0)
    assert np.all(r[:pad] == -3.0) and np.all(r[-pad:] == -3.0)
    assert np.all(np.isfinite(s[pad:-pad])) and np.all(np.isfinite(r[pad:-pad]))
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    yo, ay = orc.forward(g, x, with_abs=True)
    assert_close(s[pad:-pad].reshape(w.sino_shape), yo, ay, "forward into a view")
    xo, ax = orc.back(g, y, with_abs=True)
    assert_close(r[pad:-pad].reshape(w.recon_shape), xo, ax, "back into a view")
    proj.close()


def test_overlapping_buffers_rejected_before_any_write(bp):
    """Every call that takes two caller buffers returns PROJ_ERR_ALIAS when
    they overlap, through the C ABI, and leaves both untouched (the check runs
    before any launch).  (proj_channel_index's alias check guards the
    handle's own table, whose address the ABI never hands out.)"""
    import ctypes
    w = CONE_RAGGED
    note(f"alias checks {w.name}")
    lib = bp.load_library()
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    h = proj._h
    nr, ns = int(np.prod(w.recon_shape)), int(np.prod(w.sino_shape))
    buf = torch.full((nr + ns,), 3.0, device="cuda:0")
    base = buf.data_ptr()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    # recon and sinogram sharing their last/first 4 bytes, or fully the same memory
    for rec, sino in ((base, base + 4 * (nr - 1)), (base, base)):
        assert lib.proj_forward(h, ctypes.c_void_p(rec), ctypes.c_void_p(sino), stream) == -3
        assert lib.proj_back(h, ctypes.c_void_p(sino), ctypes.c_void_p(rec), stream) == -3
        assert lib.proj_back_squared(h, ctypes.c_void_p(sino), ctypes.c_void_p(rec), stream) == -3
    # batches: pixel list, cylinders and sinogram, pairwise overlapping
    n = 8
    pix = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    cyl = torch.full((n, w.ns), 3.0, device="cuda:0")
    sino = torch.full(w.sino_shape, 3.0, device="cuda:0")
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)
    for pp, cc, ss in ((pix, cyl, cyl), (pix, pix, sino), (cyl, cyl, sino)):
        st_f = lib.proj_forward_pixels(h, P(pp), ctypes.c_int64(n), P(cc), P(ss), stream)
        st_b = lib.proj_back_pixels(h, P(ss), P(pp), ctypes.c_int64(n), P(cc), stream)
        assert st_f == -3 and st_b == -3, (st_f, st_b)
    assert "overlap" in lib.proj_last_error().decode()
    torch.cuda.synchronize()
    assert bool(torch.all(buf == 3.0)) and bool(torch.all(cyl == 3.0)) and bool(torch.all(sino == 3.0))
    # disjoint buffers still work on the same handle afterwards
    x, _ = inputs(w)
    out = proj.forward(dev(x))
    assert np.isfinite(host(out)).all()
    proj.close()


def test_repeat_calls_and_streams(bp):
    """Calls are stateless: the same input gives the same values on a side
    stream as on the default stream, and repeated calls agree."""
    w = CONE_RAGGED
    note(f"streams {w.name}")
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    x, y = inputs(w)
    xd = dev(x)
    a = proj.back(dev(y))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = proj.back(dev(y), stream=s)
    s.synchronize()
    c = proj.forward(xd)
    d = proj.forward(xd)
    assert np.array_equal(host(a), host(b))          # the gather is deterministic
    # the forward's atomic flushes may add in another order: equal up to rounding
    assert rel_l2(host(c), host(d)) < 1e-6
    proj.close()


@pytest.mark.parametrize("w,strategy", [(PAR_RAGGED, 1), (PAR_RAGGED, 2), (CONE_RAGGED, None), (HELIX_SMALL, None)],
                         ids=["tile", "gather", "cone", "helical"])
def test_forwards_on_two_streams(bp, orc, w, strategy):
    """Forwards share a handle buffer (the parallel accumulation buffer, the
    cone's transposed sinogram): forwards of different volumes issued on two
    streams back to back (no host sync between them) are ordered on the GPU
    and each gets its own correct sinogram; so do forwards interleaved with
    batch forwards on a third stream."""
    note(f"two-stream forwards {w.name} strategy={strategy}")
    geo = w.geometry() if strategy is None else dict(w.geometry(), forward_strategy=strategy)
    proj = bp.Projector(geo, w.recon_shape, w.sino_shape)
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    rng = np.random.default_rng(17)
    xs = [rng.standard_normal(w.recon_shape).astype(np.float32) for _ in range(4)]
    xd = [dev(x) for x in xs]
    outs = [torch.empty(w.sino_shape, device="cuda:0") for _ in range(4)]
    pix = dev(rng.permutation(w.ny * w.nx)[:100].astype(np.int32))
    cyl = dev(rng.standard_normal((100, w.ns)).astype(np.float32))
    bout = torch.empty(w.sino_shape, device="cuda:0")
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    for k in range(4):
        s = streams[k % 2]
        with torch.cuda.stream(s):
            proj.forward(xd[k], out=outs[k], stream=s)
        if k == 1:
            with torch.cuda.stream(streams[2]):
                proj.forward_pixels(pix, cyl, out=bout, stream=streams[2])
    torch.cuda.synchronize()
    for k in range(4):
        yo, ay = orc.forward(g, xs[k], with_abs=True)
        assert_close(host(outs[k]), yo, ay, f"forward {k} on stream {k % 2}")
    bo, ab = orc.forward_pixels(g, host(pix), host(cyl), with_abs=True)
    assert_close(host(bout), bo, ab, "batch forward on a third stream")
    proj.close()


def test_empty_and_degenerate_shapes(bp):
    """Zero views: back gives exact zeros.  Zero slices / pixels: nothing to
    write.  A single pixel and a single view still projects correctly."""
    note("empty shapes")
    geo = dict(kind=0, num_views=0, angles=np.zeros(0), delta_channel=1.0)
    p = bp.Projector(geo, (8, 8, 4), (0, 4, 16))
    out = torch.full((8, 8, 4), 5.0, device="cuda:0")
    p.back(torch.empty((0, 4, 16), device="cuda:0"), out=out)
    assert host(out).max() == 0.0 and host(out).min() == 0.0
    p.close()
    geo = dict(kind=0, num_views=3, angles=np.array([0.0, 1.0, 2.0]), delta_channel=1.0)
    p = bp.Projector(geo, (0, 5, 2), (3, 2, 10))
    sino = torch.full((3, 2, 10), 5.0, device="cuda:0")
    p.forward(torch.empty((0, 5, 2), device="cuda:0"), out=sino)
    assert np.all(host(sino) == 0.0)
    p.close()


FEW_VIEWS = [W.scaled(base, f"{base.name}-{nv}v-few", nv=nv)
             for base in (PAR_RAGGED, PAR_FINE, HELIX_SMALL) for nv in (1, 2, 3, 5, 7)]


@pytest.mark.parametrize("w", FEW_VIEWS, ids=lambda w: w.name)
def test_few_views_parity(bp, orc, w):
    """One to seven views: the back projections load the views ahead of the
    one they gather (two ahead for the parallel beam), so the first and last
    views of a scan take the prologue and the loop's early exits; forward and
    back against the reference, every entry."""
    note(f"few views {w.name}")
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    x, y = inputs(w)
    yo, ay = orc.forward(g, x, with_abs=True)
    assert_close(host(proj.forward(dev(x))), yo, ay, f"{w.name} forward")
    xo, ax = orc.back(g, y, with_abs=True)
    assert_close(host(proj.back(dev(y))), xo, ax, f"{w.name} back")
    proj.close()


def test_single_voxel_matches_hand_value(bp):
    """One unit voxel, the hand-worked taps of tests/golden/single_voxel_taps.txt:
    fp32 weights rounded once from the fp64 closed forms."""
    from golden_io import single_voxel_taps
    note("single voxel golden taps")
    for (th, off), taps in single_voxel_taps().items():
        geo = dict(kind=0, num_views=1, angles=np.array([np.radians(th)]), channel_shift=np.array([off]),
                   delta_channel=1.0)
        p = bp.Projector(geo, (1, 1, 1), (1, 1, 11))
        y = host(p.forward(torch.ones((1, 1, 1), device="cuda:0")))
        expect = np.zeros((1, 1, 11), np.float32)
        for n, wgt in taps.items():
            expect[0, 0, n] = np.float32(wgt)
        assert np.max(np.abs(y - expect)) <= 1e-7, (th, off, y)
        p.close()


# ------------------------------------------------------------ full sizes ---
FULL = ["parallel-512x512x64-720v", "cone-256x256x256-360v", "translation-512x512x32-64v",
        "helical-512x512x96-1338v"]


@pytest.fixture(scope="module")
def full_cache():
    return {}


def full_setup(bp, orc, name, cache):
    if name not in cache:
        cache.clear()
        torch.cuda.empty_cache()
        w = W.get(name)
        note(f"full setup {name}")
        proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
        g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
        cache[name] = (w, proj, g)
    return cache[name]


@pytest.mark.parametrize("name", FULL)
def test_full_index_bit_exact(bp, orc, name, full_cache):
    w, proj, g = full_setup(bp, orc, name, full_cache)
    note(f"full index {name}")
    idx = host(proj.channel_index())
    if w.nv * w.ny * w.nx <= 200_000_000:
        ref = orc.channel_index(g)
        assert np.array_equal(idx, ref)
    else:
        # the reference index of a view subset, through a geometry of those views
        views = np.unique(np.linspace(0, w.nv - 1, 24).astype(int))
        geo = w.geometry()
        sub = dict(geo, num_views=len(views), angles=geo["angles"][views],
                   source_z=None if geo["source_z"] is None else geo["source_z"][views],
                   channel_shift=None if geo["channel_shift"] is None else geo["channel_shift"][views])
        gs = orc.Geometry(sub, w.recon_shape, (len(views), w.nr, w.nc))
        assert np.array_equal(idx[views], orc.channel_index(gs))


def test_tie_canaries_on_gpu(bp, orc, full_cache):
    """The 45 and 135 degree views of the 512x512 parallel geometry hold 512
    exact half-integer channel coordinates each; they must round to even."""
    w, proj, g = full_setup(bp, orc, "parallel-512x512x64-720v", full_cache)
    idx = host(proj.channel_index())
    u = orc.channel_coord(orc.Geometry(dict(w.geometry(), num_views=2, angles=w.angles()[[180, 540]]),
                                       w.recon_shape, (2, w.nr, w.nc)))
    for row, v in ((0, 180), (1, 540)):
        ties = np.nonzero(u[row] == np.floor(u[row]) + 0.5)[0]
        assert len(ties) == 512
        assert np.all(idx[v, ties] % 2 == 0)


@pytest.mark.parametrize("name", FULL)
def test_full_forward_sampled_views(bp, orc, name, full_cache):
    w, proj, g = full_setup(bp, orc, name, full_cache)
    note(f"full forward {name}")
    x = w.recon_input()
    yg = host(proj.forward(dev(x)))
    views = sorted({0, w.nv // 4, w.nv // 2 + 1, w.nv - 1})
    if w.nv >= 720:
        views = sorted(set(views) | {180, 540})
    yo, ay = orc.forward_views(g, x, views, with_abs=True)
    assert_close(yg[views], yo, ay, f"{name} forward views {views}")


@pytest.mark.parametrize("name", ["cone-256x256x256-360v", "helical-512x512x96-1338v"])
def test_full_forward_dense_sampled_views(bp, orc, name, full_cache):
    """The cone forward of a dense N(0,1) volume (every solver iterate is
    dense; the phantom leaves most of each tile's detector window at zero and
    skips those cells' flushes) on sampled views, against the reference."""
    w, proj, g = full_setup(bp, orc, name, full_cache)
    note(f"full dense forward {name}")
    x = np.random.default_rng(101).standard_normal(w.recon_shape).astype(np.float32)
    yg = host(proj.forward(dev(x)))
    views = sorted({1, w.nv // 3, (2 * w.nv) // 3 + 1, w.nv - 2})
    yo, ay = orc.forward_views(g, x, views, with_abs=True)
    assert_close(yg[views], yo, ay, f"{name} dense forward views {views}")


@pytest.mark.parametrize("name", FULL)
def test_full_back_sampled_pixels(bp, orc, name, full_cache):
    w, proj, g = full_setup(bp, orc, name, full_cache)
    note(f"full back {name}")
    y = w.sino_input()
    xg = host(proj.back(dev(y))).reshape(w.ny * w.nx, w.ns)
    rng = np.random.default_rng(77)
    pix = np.unique(np.concatenate([rng.integers(0, w.ny * w.nx, 600),
                                    [0, w.nx - 1, w.ny * w.nx - w.nx, w.ny * w.nx - 1,
                                     (w.ny // 2) * w.nx + w.nx // 2]]))
    xo, ax = orc.back_pixels(g, y, pix, with_abs=True)
    assert_close(xg[pix], xo, ax, f"{name} back pixels")


@pytest.mark.parametrize("name", FULL)
def test_full_adjoint_identity(bp, orc, name, full_cache):
    w, proj, g = full_setup(bp, orc, name, full_cache)
    note(f"full adjoint {name}")
    x = w.recon_input()
    y = w.sino_input()
    ax = host(proj.forward(dev(x)))
    aty = host(proj.back(dev(y)))
    gap = adjoint_gap(ax, y, x, aty)
    assert gap < ADJOINT, f"{name}: adjoint gap {gap:.2e}"


def test_full_helical_radius2(bp, orc, full_cache):
    """The helical scan at psf radius 2, where no footprint is truncated (the
    widest, near the source, span about 2.5 channels): bit-exact index on
    sampled views, forward of the phantom and of a dense volume on sampled
    views, back on sampled pixels, adjoint identity."""
    full_cache.clear()
    torch.cuda.empty_cache()
    base = W.get("helical-512x512x96-1338v")
    w = W.scaled(base, "helical-512x512x96-1338v-r2", radius=2)
    note(f"full helical radius 2 {w.name}")
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    assert "radius=2 taps=5" in proj.describe()
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    views = [0, 335, 668, 1001, w.nv - 1]
    geo = w.geometry()
    sub = dict(geo, num_views=len(views), angles=geo["angles"][views], source_z=geo["source_z"][views])
    gs = orc.Geometry(sub, w.recon_shape, (len(views), w.nr, w.nc))
    assert np.array_equal(host(proj.channel_index())[views], orc.channel_index(gs))
    for label, x in (("phantom", w.recon_input()),
                     ("dense", np.random.default_rng(103).standard_normal(w.recon_shape).astype(np.float32))):
        yg = host(proj.forward(dev(x)))
        yo, ay = orc.forward_views(g, x, views, with_abs=True)
        assert_close(yg[views], yo, ay, f"{w.name} forward of the {label} on views {views}")
    y = w.sino_input()
    xg = host(proj.back(dev(y))).reshape(w.ny * w.nx, w.ns)
    rng = np.random.default_rng(79)
    pix = np.unique(np.concatenate([rng.integers(0, w.ny * w.nx, 300), [0, w.ny * w.nx - 1,
                                                                         (w.ny // 2) * w.nx + w.nx // 2]]))
    xo, ax = orc.back_pixels(g, y, pix, with_abs=True)
    assert_close(xg[pix], xo, ax, f"{w.name} back pixels")
    x = w.recon_input()
    gap = adjoint_gap(host(proj.forward(dev(x))), y, x, xg.reshape(w.recon_shape))
    assert gap < ADJOINT, f"adjoint gap {gap:.2e}"
    proj.close()
    torch.cuda.empty_cache()


# ---------------------------------------------- squared-weight back ---
@pytest.mark.parametrize("w", SMALL_CASES, ids=lambda w: w.name)
def test_small_back_squared(bp, orc, w):
    """proj_back_squared (every tap weight squared: the Hessian-diagonal back
    projection) against the reference, every entry; and with a sinogram of
    ones, sum_i A_ij^2 itself."""
    note(f"small back squared {w.name}")
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    _, y = inputs(w)
    xo, ax = orc.back(g, y, with_abs=True, power=2)
    xg = host(proj.back_squared(dev(y)))
    assert_close(xg, xo, ax, f"{w.name} back squared")
    ones = np.ones(w.sino_shape, np.float32)
    ho = orc.back(g, ones, power=2)
    hg = host(proj.back_squared(dev(ones)))
    assert_close(hg, ho, ho, f"{w.name} diagonal of A^T A")
    # the plain adjoint is untouched by the squared path (same handle, after it)
    xo1, ax1 = orc.back(g, y, with_abs=True)
    assert_close(host(proj.back(dev(y))), xo1, ax1, f"{w.name} back after squared")
    proj.close()


@pytest.mark.parametrize("name", FULL)
def test_full_back_squared_sampled_pixels(bp, orc, name, full_cache):
    w, proj, g = full_setup(bp, orc, name, full_cache)
    note(f"full back squared {name}")
    y = w.sino_input()
    xg = host(proj.back_squared(dev(y))).reshape(w.ny * w.nx, w.ns)
    rng = np.random.default_rng(78)
    pix = np.unique(np.concatenate([rng.integers(0, w.ny * w.nx, 300),
                                    [0, w.ny * w.nx - 1, (w.ny // 2) * w.nx + w.nx // 2]]))
    xo, ax = orc.back_pixels(g, y, pix, with_abs=True, power=2)
    assert_close(xg[pix], xo, ax, f"{name} back squared pixels")


# ------------------------------------------ forward strategies (a8) ---
PAR_SMALL = [W.get(W.SMALL), PAR_RAGGED, PAR_FINE, PAR_WIDE, TRANS_SMALL, PAR_TRUNC, TRANS_R2]


@pytest.mark.parametrize("w", [TRANS_SMALL, TRANS_R2], ids=lambda w: w.name)
def test_translation_column_forms(bp, orc, w):
    """A translation scan (every view at angle 0) takes the column forward and
    the column back.  The back gives the same bits as the general back: with
    every angle at 1e-300 instead of 0 (sine not 0, so the general kernels;
    cosine 1 and no pixel centre at x = 0, so the same tap records) the back
    is bitwise equal, and both forwards match the reference (where the
    width is even; an odd one has a column at x = 0, which the tilt moves)."""
    note(f"translation column forms {w.name}")
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    desc = proj.describe()
    assert "column:" in desc.split("forward:")[1] and "back: column:" in desc
    x, y = inputs(w)
    yo, ay = orc.forward(g, x, with_abs=True)
    yg = host(proj.forward(dev(x)))
    assert_close(yg, yo, ay, f"{w.name} column forward")
    xb = host(proj.back(dev(y)))
    xs = host(proj.back_squared(dev(y)))
    if w.nx % 2 == 0:
        tilted = dict(w.geometry(), angles=np.full(w.nv, 1e-300))
        gen = bp.Projector(tilted, w.recon_shape, w.sino_shape)
        gdesc = gen.describe()
        assert "column:" not in gdesc
        assert np.array_equal(xb, host(gen.back(dev(y)))), "column back differs from the general back"
        assert np.array_equal(xs, host(gen.back_squared(dev(y)))), "column squared back differs"
        assert_close(host(gen.forward(dev(x))), yo, ay, f"{w.name} general forward, angles 1e-300")
        gen.close()
    xo, ax = orc.back(g, y, with_abs=True)
    assert_close(xb, xo, ax, f"{w.name} column back")
    proj.close()


@pytest.mark.parametrize("strategy", [1, 2], ids=["tile", "gather"])
@pytest.mark.parametrize("w", PAR_SMALL, ids=lambda w: w.name)
def test_small_forward_strategies(bp, orc, w, strategy):
    """Both parallel forward strategies, forced, against the reference."""
    note(f"forward strategy {strategy} {w.name}")
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    proj = bp.Projector(dict(w.geometry(), forward_strategy=strategy), w.recon_shape, w.sino_shape)
    assert ("gather:" if strategy == 2 else "tile:") in proj.describe()
    x, y = inputs(w)
    yo, ay = orc.forward(g, x, with_abs=True)
    yg = host(proj.forward(dev(x)))
    assert_close(yg, yo, ay, f"{w.name} forward strategy {strategy}")
    gap = adjoint_gap(yg, y, x, host(proj.back(dev(y))))
    assert gap < ADJOINT, f"adjoint gap {gap:.2e}"
    proj.close()


CONE_SMALL = [w for w in SMALL_CASES if w.kind == W.CONE_FLAT]


@pytest.mark.parametrize("tile", [3, 4], ids=["8x4", "8x8"])
@pytest.mark.parametrize("w", CONE_SMALL, ids=lambda w: w.name)
def test_small_cone_forward_tiles(bp, orc, w, tile):
    """Both cone forward tiles (8 x 4 and 8 x 8 pixels), forced, against the
    reference: forward of the whole sinogram and the adjoint identity."""
    note(f"cone forward tile {tile} {w.name}")
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    proj = bp.Projector(dict(w.geometry(), forward_strategy=tile), w.recon_shape, w.sino_shape)
    assert ("8x4 px tile" if tile == 3 else "8x8 px tile") in proj.describe().split("forward:")[1]
    x, y = inputs(w)
    yo, ay = orc.forward(g, x, with_abs=True)
    yg = host(proj.forward(dev(x)))
    assert_close(yg, yo, ay, f"{w.name} forward tile {tile}")
    gap = adjoint_gap(yg, y, x, host(proj.back(dev(y))))
    assert gap < ADJOINT, f"adjoint gap {gap:.2e}"
    proj.close()


@pytest.mark.parametrize("name,tile", [("cone-256x256x256-360v", 3), ("helical-512x512x96-1338v", 4)],
                         ids=["cone-8x4", "helical-8x8"])
def test_full_cone_forward_other_tile(bp, orc, name, tile, full_cache):
    """The full-size cone workloads with the tile the planner does not pick
    for them, dense volume, sampled views against the reference."""
    full_cache.clear()
    torch.cuda.empty_cache()
    w = W.get(name)
    note(f"full cone forward tile {tile} {name}")
    proj = bp.Projector(dict(w.geometry(), forward_strategy=tile), w.recon_shape, w.sino_shape)
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    x = np.random.default_rng(105).standard_normal(w.recon_shape).astype(np.float32)
    yg = host(proj.forward(dev(x)))
    views = sorted({2, w.nv // 2, w.nv - 3})
    yo, ay = orc.forward_views(g, x, views, with_abs=True)
    assert_close(yg[views], yo, ay, f"{name} forward tile {tile} views {views}")
    proj.close()


@pytest.mark.parametrize("name", ["parallel-512x512x64-720v", "translation-512x512x32-64v"])
def test_full_forward_gather_sampled_views(bp, orc, name, full_cache):
    full_cache.clear()
    torch.cuda.empty_cache()
    w = W.get(name)
    note(f"full gather forward {name}")
    proj = bp.Projector(dict(w.geometry(), forward_strategy=2), w.recon_shape, w.sino_shape)
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    x = w.recon_input()
    yg = host(proj.forward(dev(x)))
    views = sorted({0, w.nv // 4 + 1, w.nv // 2, w.nv - 1})
    yo, ay = orc.forward_views(g, x, views, with_abs=True)
    assert_close(yg[views], yo, ay, f"{name} gather forward views {views}")
    proj.close()


# ------------------------------------------------ batches of voxel cylinders ---
PADDING_IDS = (-1, -(2 ** 31), 2 ** 31 - 1)


def batch(w, n, seed, repeats=True):
    """n listed pixels of w: random ids (one pixel three times when
    `repeats`), the first and last pixel, and padding entries (ids outside
    [0, Ny*Nx)) whose cylinders hold NaN, inf and huge values."""
    rng = np.random.default_rng(seed)
    np_ = w.ny * w.nx
    pix = rng.integers(0, np_, n).astype(np.int32)
    pix[0], pix[-1] = 0, np_ - 1
    if repeats:
        pix[4] = pix[11] = pix[n // 2]
    pad = np.array([1, 7, n - 3, n // 3])
    pix[pad] = [np_, PADDING_IDS[0], PADDING_IDS[1], PADDING_IDS[2]]
    cyl = rng.standard_normal((n, w.ns)).astype(np.float32)
    cyl[pad[0]] = np.nan
    cyl[pad[1]] = np.inf
    cyl[pad[2]] = -3e38
    cyl[pad[3], ::2] = np.nan
    return pix, cyl, pad


@pytest.mark.parametrize("w", SMALL_CASES, ids=lambda w: w.name)
def test_small_pixel_batches(bp, orc, w):
    note(f"pixel batches {w.name}")
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    pix, cyl, pad = batch(w, 203, seed=w.seed_x)       # 203: ragged against the waves per workgroup
    _, y = inputs(w)
    yo, ay = orc.forward_pixels(g, pix, cyl, with_abs=True)
    yg = host(proj.forward_pixels(dev(pix), dev(cyl)))
    assert np.isfinite(yg).all(), "padding leaked into the forward"
    assert_close(yg, yo, ay, f"{w.name} forward of a batch")
    xo, ax = orc.back_pixels(g, y, pix, with_abs=True)
    xg = host(proj.back_pixels(dev(y), dev(pix)))
    assert not xg[pad].any(), "padding rows must be zero"
    assert_close(xg, xo, ax, f"{w.name} back at a batch")
    keep = np.ones(len(pix), bool)
    keep[pad] = False
    lhs = float((yg.astype(np.float64) * y).sum())
    rhs = float((cyl[keep].astype(np.float64) * xg[keep]).sum())
    gap = abs(lhs - rhs) / (np.linalg.norm(yg) * np.linalg.norm(y))
    assert gap < ADJOINT, f"batch adjoint gap {gap:.2e}"
    proj.close()


@pytest.mark.parametrize("w", [PAR_RAGGED, CONE_RAGGED, HELIX_SMALL], ids=lambda w: w.name)
def test_pixel_batch_poison_padding_bitwise(bp, w):
    """Padding is exactly inert: a single listed voxel among poisoned padding
    entries gives the same bits as the voxel listed alone and as a batch with
    zero padding (each sinogram cell then receives one contribution, so no
    summation order is involved)."""
    note(f"poisoned padding {w.name}")
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    p = (w.ny // 2) * w.nx + w.nx // 3
    k = w.ns // 2
    one = np.zeros((1, w.ns), np.float32)
    one[0, k] = 1.75
    alone = host(proj.forward_pixels(dev(np.array([p], np.int32)), dev(one)))
    assert np.count_nonzero(alone) > 0
    pix = np.full(64, -1, np.int32)
    pix[1::3] = w.ny * w.nx
    pix[37] = p
    clean = np.zeros((64, w.ns), np.float32)
    clean[37] = one[0]
    poison = np.full((64, w.ns), np.nan, np.float32)
    poison[::2] = np.inf
    poison[37] = one[0]
    a = host(proj.forward_pixels(dev(pix), dev(clean)))
    b = host(proj.forward_pixels(dev(pix), dev(poison)))
    assert np.array_equal(a, alone) and np.array_equal(b, alone)
    # the back: the listed pixel's row does not depend on its neighbours in the list
    _, y = inputs(w)
    r1 = host(proj.back_pixels(dev(y), dev(np.array([p], np.int32))))
    r64 = host(proj.back_pixels(dev(y), dev(pix)))
    assert np.array_equal(r64[37], r1[0]) and not np.delete(r64, 37, axis=0).any()
    proj.close()


@pytest.mark.parametrize("w", [PAR_RAGGED, CONE_R2], ids=lambda w: w.name)
def test_pixel_batch_of_every_pixel_is_the_volume(bp, orc, w):
    """Listing every pixel once (shuffled) is the whole-volume projection: the
    batch path matches the reference forward and back of the volume."""
    note(f"every pixel as a batch {w.name}")
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    x, y = inputs(w)
    perm = np.random.default_rng(3).permutation(w.ny * w.nx).astype(np.int32)
    cyl = x.reshape(-1, w.ns)[perm]
    yo, ay = orc.forward(g, x, with_abs=True)
    assert_close(host(proj.forward_pixels(dev(perm), dev(cyl))), yo, ay, f"{w.name} batch of every pixel")
    xo, ax = orc.back(g, y, with_abs=True)
    xg = host(proj.back_pixels(dev(y), dev(perm)))
    assert_close(xg, xo.reshape(-1, w.ns)[perm], ax.reshape(-1, w.ns)[perm], f"{w.name} back of every pixel")
    proj.close()


def test_pixel_batch_empty_and_all_padding(bp):
    note("empty and all-padding batches")
    for w in (PAR_RAGGED, CONE_RAGGED):
        proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
        empty_i = torch.zeros(0, dtype=torch.int32, device="cuda:0")
        empty_c = torch.zeros((0, w.ns), dtype=torch.float32, device="cuda:0")
        out = torch.full(w.sino_shape, float("nan"), device="cuda:0")
        proj.forward_pixels(empty_i, empty_c, out=out)
        assert not host(out).any()
        assert host(proj.back_pixels(dev(inputs(w)[1]), empty_i)).shape == (0, w.ns)
        pix = np.array([-5, w.ny * w.nx, -1], np.int32)
        out.fill_(float("nan"))
        proj.forward_pixels(dev(pix), dev(np.full((3, w.ns), np.nan, np.float32)), out=out)
        assert not host(out).any()
        cyl = torch.full((3, w.ns), float("nan"), device="cuda:0")
        proj.back_pixels(dev(inputs(w)[1]), dev(pix), out=cyl)
        assert not host(cyl).any()
        proj.close()


PAR_BATCH = [w for w in SMALL_CASES if w.kind == W.PARALLEL]


@pytest.mark.parametrize("w", PAR_BATCH, ids=lambda w: w.name)
def test_pixel_batch_back_direct_and_packed_agree(bp, orc, w):
    """The parallel batch back reads the sinogram itself for a few entries and
    a slice-fastest copy of it for many: three listed pixels alone (the first
    form) and the same three inside a batch of 203 (the second) give the same
    bits, and match the reference."""
    note(f"batch back forms {w.name}")
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    _, y = inputs(w)
    np_ = w.ny * w.nx
    few = np.array([0, np_ // 2 + 3, np_ - 1], np.int32)
    big, _, _ = batch(w, 203, seed=w.seed_y)
    at = [5, 100, 202]
    big[at] = few
    r_few = host(proj.back_pixels(dev(y), dev(few)))
    r_big = host(proj.back_pixels(dev(y), dev(big)))
    assert np.array_equal(r_few, r_big[at]), "the two batch back forms differ"
    xo, ax = orc.back_pixels(g, y, few, with_abs=True)
    assert_close(r_few, xo, ax, f"{w.name} back at three pixels")
    proj.close()


@pytest.mark.parametrize("w", [PAR_RAGGED, PAR_FINE], ids=lambda w: w.name)
def test_pixel_batch_forward_in_passes(bp, orc, w):
    """A parallel batch forward longer than one sort pass (4096 entries): 9000
    entries, ids repeated many times, padding in every pass; the passes after
    the first add to the sinogram."""
    note(f"batch forward in passes {w.name}")
    g = orc.Geometry(w.geometry(), w.recon_shape, w.sino_shape)
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    rng = np.random.default_rng(w.seed_x + 5)
    n = 9000
    pix = rng.integers(0, w.ny * w.nx, n).astype(np.int32)
    pad = np.array([2, 4100, 8999, 6000])
    pix[pad] = [-1, w.ny * w.nx, 2 ** 31 - 1, -7]
    cyl = rng.standard_normal((n, w.ns)).astype(np.float32)
    cyl[pad] = np.nan
    yg = host(proj.forward_pixels(dev(pix), dev(cyl)))
    assert np.isfinite(yg).all(), "padding leaked into the forward"
    yo, ay = orc.forward_pixels(g, pix, cyl, with_abs=True)
    assert_close(yg, yo, ay, f"{w.name} forward of 9000 entries")
    _, y = inputs(w)
    xg = host(proj.back_pixels(dev(y), dev(pix)))
    keep = np.ones(n, bool)
    keep[pad] = False
    lhs = float((yg.astype(np.float64) * y).sum())
    rhs = float((cyl[keep].astype(np.float64) * xg[keep]).sum())
    gap = abs(lhs - rhs) / (np.linalg.norm(yg) * np.linalg.norm(y))
    assert gap < ADJOINT, f"batch adjoint gap {gap:.2e}"
    proj.close()


@pytest.mark.parametrize("name", FULL)
def test_full_pixel_batch_sampled(bp, orc, name, full_cache):
    """A batch of 1000 distinct pixels (plus padding) at the full sizes: the
    forward on sampled views against the reference forward of the scattered
    volume, the back on sampled rows of the batch."""
    w, proj, g = full_setup(bp, orc, name, full_cache)
    note(f"full pixel batch {name}")
    rng = np.random.default_rng(91)
    pix = rng.permutation(w.ny * w.nx)[:1000].astype(np.int32)
    pix[[10, 500]] = [-1, w.ny * w.nx]
    cyl = rng.standard_normal((len(pix), w.ns)).astype(np.float32)
    cyl[[10, 500]] = np.nan
    yg = host(proj.forward_pixels(dev(pix), dev(cyl)))
    x = np.zeros((w.ny * w.nx, w.ns), np.float32)
    keep = (pix >= 0) & (pix < w.ny * w.nx)
    x[pix[keep]] = cyl[keep]
    views = sorted({0, w.nv // 3, w.nv - 1})
    yo, ay = orc.forward_views(g, x.reshape(w.recon_shape), views, with_abs=True)
    assert_close(yg[views], yo, ay, f"{name} batch forward views {views}")
    y = w.sino_input()
    xg = host(proj.back_pixels(dev(y), dev(pix)))
    rows = np.r_[0:40, 500, len(pix) - 40:len(pix)]
    xo, ax = orc.back_pixels(g, y, pix[rows], with_abs=True)
    assert_close(xg[rows], xo, ax, f"{name} batch back rows")
    assert not xg[[10, 500]].any()


def test_largest_volume_mass_and_back_of_ones(bp):
    """The largest parallel volume the planner accepts, 2048 x 2047 x 512
    (2^31 - 2^20 voxels, so every address above 2^31 bytes is exercised), 4
    views, a 4096-channel detector that every tap lands on: per view and row
    the forward carries the slice's mass (dv^2/dch = 1 per voxel), and the back
    projection of ones is 4 (the view count) at every voxel."""
    geo = dict(kind=0, num_views=4, angles=np.array([0.0, 0.4, 1.3, 2.2]), delta_channel=1.0)
    rs, ss = (2048, 2047, 512), (4, 512, 4096)
    note(f"largest volume {rs} sino {ss}")
    proj = bp.Projector(geo, rs, ss)
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(11)
    x = torch.rand(rs, device="cuda:0", generator=gen)
    y = proj.forward(x)
    slice_mass = torch.sum(x, dim=(0, 1), dtype=torch.float64)          # [S]
    row_mass = torch.sum(y, dim=2, dtype=torch.float64)                 # [V, R]
    err = float(torch.max(torch.abs(row_mass - slice_mass[None, :]) / slice_mass[None, :]))
    assert err < 1e-5, f"mass per view and row off by {err:.2e}"
    del x
    torch.cuda.empty_cache()
    b = proj.back(torch.ones(ss, device="cuda:0"))
    dev_max = float(torch.max(torch.abs(b - 4.0)))
    assert dev_max < 1e-5, f"back projection of ones deviates from 4 by {dev_max:.2e}"
    del b, y
    proj.close()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("w,dv", [(CONE_RAGGED, 1.25), (HELIX_SMALL, 0.9), (PAR_RAGGED, 0.8)],
                         ids=["cone", "helical", "parallel"])
def test_offsets_shifts_and_voxel_pitch(bp, orc, w, dv):
    """Geometry parameters the workloads leave at their defaults: a voxel pitch
    other than 1, detector channel and row offsets, and a lateral detector
    shift per view."""
    note(f"offsets {w.name} dv={dv}")
    rng = np.random.default_rng(51)
    geo = dict(w.geometry(), delta_voxel=dv, det_channel_offset=2.3,
               det_row_offset=-1.7 if w.kind == W.CONE_FLAT else 0.0,
               channel_shift=rng.uniform(-3.0, 3.0, w.nv))
    if w.kind == W.PARALLEL:
        geo["delta_row"] = dv                      # parallel: one row per slice
    g = orc.Geometry(geo, w.recon_shape, w.sino_shape)
    proj = bp.Projector(geo, w.recon_shape, w.sino_shape)
    x, y = inputs(w)
    assert np.array_equal(host(proj.channel_index()), orc.channel_index(g))
    yo, ay = orc.forward(g, x, with_abs=True)
    yg = host(proj.forward(dev(x)))
    assert_close(yg, yo, ay, f"{w.name} forward with offsets")
    xo, ax = orc.back(g, y, with_abs=True)
    xg = host(proj.back(dev(y)))
    assert_close(xg, xo, ax, f"{w.name} back with offsets")
    gap = adjoint_gap(yg, y, x, xg)
    assert gap < ADJOINT, f"adjoint gap {gap:.2e}"
    proj.close()
