"""Capture of the projector calls into a HIP graph (torch.cuda.CUDAGraph is a
hipGraph on ROCm).  The calls allocate, copy and synchronise nothing and use
fill kernels instead of memset nodes, so a forward + back pair can be captured
once and replayed.  Every replay is checked against the eager result, with
eager work on the same handle between replays (clobbered outputs, an eager
forward that reuses the handle's accumulation buffer)."""
import numpy as np
import pytest

import workloads as W
from metrics import rel_l2
from test_gpu_parity import CONE_RAGGED, HELIX_SMALL, PAR_RAGGED, TRANS_SMALL, dev, host, inputs, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def bp():
    import back_projectors_amd as m
    m.load_library()
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return m


def _geometry(w, strategy):
    geo = w.geometry()
    if strategy is not None:
        geo = dict(geo, forward_strategy=strategy)
    return geo


@pytest.mark.parametrize("w,strategy", [(W.get(W.SMALL), 2), (PAR_RAGGED, 1), (TRANS_SMALL, None),
                                        (CONE_RAGGED, None), (HELIX_SMALL, None)],
                         ids=["small-gather", "ragged-tile", "translation", "cone", "helical"])
def test_forward_back_graph_replays(bp, w, strategy):
    note(f"graph capture {w.name} strategy={strategy}")
    proj = bp.Projector(_geometry(w, strategy), w.recon_shape, w.sino_shape)
    x, y = inputs(w)
    xs, ys = dev(x), dev(y)
    ref_y = host(proj.forward(xs))
    ref_x = host(proj.back(ys))
    out_y = torch.empty(w.sino_shape, device="cuda:0")
    out_x = torch.empty(w.recon_shape, device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm-up on the capture stream
        proj.forward(xs, out=out_y)
        proj.back(ys, out=out_x)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        proj.forward(xs, out=out_y)
        proj.back(ys, out=out_x)
    for rep in range(3):
        out_y.fill_(float("nan"))
        out_x.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        gy, gx = host(out_y), host(out_x)
        assert np.isfinite(gy).all() and np.isfinite(gx).all(), f"replay {rep} left outputs unwritten"
        # the back is deterministic; the forward's atomic flushes may add in another order
        assert np.array_equal(gx, ref_x), f"replay {rep}: back differs from eager"
        assert rel_l2(gy, ref_y) < 1e-6, f"replay {rep}: forward differs from eager"
        # eager work on the same handle between replays
        e = host(proj.forward(xs * 2.0))
        assert rel_l2(e, 2.0 * ref_y) < 1e-6
    proj.close()


@pytest.mark.parametrize("w,strategy", [(PAR_RAGGED, 1), (PAR_RAGGED, 2), (CONE_RAGGED, None)],
                         ids=["tile", "gather", "cone"])
def test_replay_and_eager_forward_on_other_streams(bp, w, strategy):
    """A replayed forward and an eager one on another stream share a handle
    buffer (the parallel accumulation buffer, the cone's transposed sinogram),
    and inside a graph the library cannot order them: the caller does, with an
    event after the replay and a stream wait before the next replay.  Done
    that way, replay / eager / replay on alternating streams all give the
    eager result."""
    note(f"replay then eager on another stream {w.name} strategy={strategy}")
    proj = bp.Projector(_geometry(w, strategy), w.recon_shape, w.sino_shape)
    x, _ = inputs(w)
    xs, x2 = dev(x), dev(3.0 * x)
    ref = host(proj.forward(xs))
    out_g = torch.empty(w.sino_shape, device="cuda:0")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        proj.forward(xs, out=out_g, stream=s1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s1):
        proj.forward(xs, out=out_g, stream=s1)
    outs = [torch.empty(w.sino_shape, device="cuda:0") for _ in range(3)]
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(s1):
            g.replay()
            done = torch.cuda.Event()
            done.record(s1)
        s2.wait_event(done)                        # the caller orders the eager forward after the replay
        with torch.cuda.stream(s2):
            proj.forward(x2, out=outs[rep], stream=s2)
        s1.wait_stream(s2)                         # and the next replay after the eager forward
        if rep == 1:
            torch.cuda.synchronize()
            assert rel_l2(host(out_g), ref) < 1e-6, "replay result"
    torch.cuda.synchronize()
    assert rel_l2(host(out_g), ref) < 1e-6
    for rep in range(3):
        assert rel_l2(host(outs[rep]), 3.0 * ref) < 1e-6, f"eager forward {rep} on the second stream"
    proj.close()


def test_pixel_batch_graph_replays(bp):
    w = PAR_RAGGED
    note(f"graph capture of batches {w.name}")
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    rng = np.random.default_rng(5)
    pix = dev(rng.permutation(w.ny * w.nx)[:300].astype(np.int32))
    cyl = dev(rng.standard_normal((300, w.ns)).astype(np.float32))
    _, y = inputs(w)
    ys = dev(y)
    ref_f = host(proj.forward_pixels(pix, cyl))
    ref_b = host(proj.back_pixels(ys, pix))
    of = torch.empty(w.sino_shape, device="cuda:0")
    ob = torch.empty((300, w.ns), device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        proj.forward_pixels(pix, cyl, out=of)
        proj.back_pixels(ys, pix, out=ob)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        proj.forward_pixels(pix, cyl, out=of)
        proj.back_pixels(ys, pix, out=ob)
    for rep in range(3):
        of.fill_(float("nan"))
        ob.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert rel_l2(host(of), ref_f) < 1e-6 and np.array_equal(host(ob), ref_b), f"replay {rep}"
        proj.forward(dev(inputs(w)[0]))             # eager use of the accumulation buffer in between
    proj.close()


def test_graph_replay_time_small(bp):
    """Launch overhead: the small 64x64x8 workload, 20 forward + back pairs
    eager against one graph of 20 pairs (reported, not asserted)."""
    w = W.get(W.SMALL)
    proj = bp.Projector(w.geometry(), w.recon_shape, w.sino_shape)
    xs = dev(w.recon_input())
    ys = proj.forward(xs)
    oy = torch.empty_like(ys)
    ox = torch.empty_like(xs)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            proj.forward(xs, out=oy)
            proj.back(ys, out=ox)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(20):
            proj.forward(xs, out=oy)
            proj.back(ys, out=ox)
    g.replay()
    torch.cuda.synchronize()
    import time
    t0 = time.perf_counter()
    for _ in range(20):
        proj.forward(xs, out=oy)
        proj.back(ys, out=ox)
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / 20
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    graph = (time.perf_counter() - t0) / 20
    note(f"small workload forward+back: eager {eager * 1e3:.3f} ms, graph replay {graph * 1e3:.3f} ms per pair")
    assert np.isfinite(host(ox)).all()
    proj.close()
