"""ctypes front end of the fp64 CPU reference (``proj_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports this
package, and this package never imports the product.

Arrays in: float32 recon ``(Ny, Nx, S)`` / sinogram ``(V, R, C)``, C order.
Arrays out: float64, plus the absolute-sum arrays ``A = sum |w * input|`` used as
the denominators of the max-relative-error metric.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "proj_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = True) -> str:
    """Compile the reference with gcc (plain IEEE fp64, no contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    tmp = _LIB + f".tmp{os.getpid()}"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


class _Geom(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("nviews", ctypes.c_int32),
        ("angles", ctypes.POINTER(ctypes.c_double)),
        ("shift", ctypes.POINTER(ctypes.c_double)),
        ("zsrc", ctypes.POINTER(ctypes.c_double)),
        ("dv", ctypes.c_double), ("dch", ctypes.c_double), ("drow", ctypes.c_double),
        ("sid", ctypes.c_double), ("sdd", ctypes.c_double),
        ("ch_off", ctypes.c_double), ("row_off", ctypes.c_double),
        ("radius", ctypes.c_int32),
        ("ny", ctypes.c_int32), ("nx", ctypes.c_int32), ("ns", ctypes.c_int32),
        ("nr", ctypes.c_int32), ("nc", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER
        g = P(_Geom)
        f32, f64, i32, i64 = (np.ctypeslib.ndpointer(t, flags="C_CONTIGUOUS")
                              for t in (np.float32, np.float64, np.int32, np.int64))
        lib.orc_channel_index.argtypes = [g, i32]
        lib.orc_channel_coord.argtypes = [g, f64]
        lib.orc_forward.argtypes = [g, f32, f64, ctypes.c_void_p]
        lib.orc_back.argtypes = [g, f32, f64, ctypes.c_void_p]
        lib.orc_forward_views.argtypes = [g, f32, ctypes.c_int32, i32, f64, ctypes.c_void_p]
        lib.orc_back_pixels.argtypes = [g, f32, ctypes.c_int32, i64, f64, ctypes.c_void_p]
        lib.orc_back_power.argtypes = [g, f32, ctypes.c_int, f64, ctypes.c_void_p]
        lib.orc_forward_f64.argtypes = [g, f64, f64]
        lib.orc_back_f64.argtypes = [g, f64, f64]
        lib.orc_back_pixels_power.argtypes = [g, f32, ctypes.c_int, ctypes.c_int32, i64, f64, ctypes.c_void_p]
        lib.orc_voxel_taps.argtypes = [g, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       i32, i32, f64, ctypes.c_int]
        lib.orc_voxel_taps.restype = ctypes.c_int
        lib.orc_vp_params.argtypes = [g, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, f64]
        lib.orc_ov.argtypes = [ctypes.c_double, ctypes.c_double]
        lib.orc_ov.restype = ctypes.c_double
        lib.orc_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


class Geometry:
    """Owns the ctypes struct and keeps its arrays alive."""

    def __init__(self, geom: dict, recon_shape, sino_shape):
        ny, nx, ns = (int(v) for v in recon_shape)
        nv, nr, nc = (int(v) for v in sino_shape)
        self.recon_shape = (ny, nx, ns)
        self.sino_shape = (nv, nr, nc)
        self._angles = np.ascontiguousarray(geom["angles"], dtype=np.float64)
        if self._angles.shape != (nv,):
            raise ValueError("angles must have one entry per view")

        def opt(key):
            a = geom.get(key)
            return None if a is None else np.ascontiguousarray(a, dtype=np.float64)

        self._shift = opt("channel_shift")
        self._zsrc = opt("source_z")
        dp = ctypes.POINTER(ctypes.c_double)
        ptr = (lambda a: a.ctypes.data_as(dp) if a is not None else ctypes.cast(None, dp))
        self.s = _Geom(
            int(geom["kind"]), nv, ptr(self._angles), ptr(self._shift), ptr(self._zsrc),
            float(geom.get("delta_voxel", 1.0)), float(geom["delta_channel"]),
            float(geom.get("delta_row", 1.0)), float(geom.get("source_iso", 0.0)),
            float(geom.get("source_detector", 0.0)), float(geom.get("det_channel_offset", 0.0)),
            float(geom.get("det_row_offset", 0.0)), int(geom.get("psf_radius", 1)),
            ny, nx, ns, nr, nc)

    @property
    def ref(self):
        return ctypes.byref(self.s)


def _f32(a, shape):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.shape != tuple(shape):
        raise ValueError(f"expected shape {shape}, got {a.shape}")
    return a


def channel_index(g: Geometry) -> np.ndarray:
    nv = g.sino_shape[0]
    ny, nx, _ = g.recon_shape
    out = np.empty((nv, ny * nx), dtype=np.int32)
    _load().orc_channel_index(g.ref, out)
    return out


def channel_coord(g: Geometry) -> np.ndarray:
    nv = g.sino_shape[0]
    ny, nx, _ = g.recon_shape
    out = np.empty((nv, ny * nx), dtype=np.float64)
    _load().orc_channel_coord(g.ref, out)
    return out


def forward(g: Geometry, x, with_abs: bool = False):
    x = _f32(x, g.recon_shape)
    y = np.empty(g.sino_shape, dtype=np.float64)
    a = np.empty(g.sino_shape, dtype=np.float64) if with_abs else None
    _load().orc_forward(g.ref, x, y, a.ctypes.data if with_abs else None)
    return (y, a) if with_abs else y


def back(g: Geometry, y, with_abs: bool = False, power: int = 1):
    """Back projection; power 2 squares every tap weight (the Hessian-diagonal
    back projection)."""
    if power not in (1, 2):
        raise ValueError("power must be 1 or 2")
    y = _f32(y, g.sino_shape)
    x = np.empty(g.recon_shape, dtype=np.float64)
    a = np.empty(g.recon_shape, dtype=np.float64) if with_abs else None
    _load().orc_back_power(g.ref, y, power, x, a.ctypes.data if with_abs else None)
    return (x, a) if with_abs else x


def forward_f64(g: Geometry, x) -> np.ndarray:
    """Forward projection of an fp64 volume, read without rounding to fp32
    (for solver iterates); the arithmetic is ``forward``'s."""
    x = np.ascontiguousarray(x, dtype=np.float64).reshape(g.recon_shape)
    y = np.empty(g.sino_shape, dtype=np.float64)
    _load().orc_forward_f64(g.ref, x, y)
    return y


def back_f64(g: Geometry, y) -> np.ndarray:
    """Back projection of an fp64 sinogram, read without rounding to fp32."""
    y = np.ascontiguousarray(y, dtype=np.float64).reshape(g.sino_shape)
    x = np.empty(g.recon_shape, dtype=np.float64)
    _load().orc_back_f64(g.ref, y, x)
    return x


def forward_views(g: Geometry, x, views, with_abs: bool = False):
    x = _f32(x, g.recon_shape)
    views = np.ascontiguousarray(views, dtype=np.int32)
    shape = (len(views),) + g.sino_shape[1:]
    y = np.empty(shape, dtype=np.float64)
    a = np.empty(shape, dtype=np.float64) if with_abs else None
    _load().orc_forward_views(g.ref, x, len(views), views, y, a.ctypes.data if with_abs else None)
    return (y, a) if with_abs else y


def back_pixels(g: Geometry, y, pixels, with_abs: bool = False, power: int = 1):
    """Back projection at the listed flat pixel ids p = i*Nx + j: row q is
    pixel pixels[q]'s column of ``back``.  An id outside [0, Ny*Nx) is batch
    padding (MBIRJAX "Sharding Overview", "Why cone beam projects whole
    cylinders": padding must stay inert) and its row is zero."""
    if power not in (1, 2):
        raise ValueError("power must be 1 or 2")
    y = _f32(y, g.sino_shape)
    pixels = np.asarray(pixels, dtype=np.int64).reshape(-1)
    ny, nx, ns = g.recon_shape
    keep = np.flatnonzero((pixels >= 0) & (pixels < ny * nx))
    sel = np.ascontiguousarray(pixels[keep])
    shape = (len(pixels), ns)
    x = np.zeros(shape, dtype=np.float64)
    a = np.zeros(shape, dtype=np.float64) if with_abs else None
    xs = np.empty((len(sel), ns), dtype=np.float64)
    as_ = np.empty((len(sel), ns), dtype=np.float64) if with_abs else None
    if len(sel):
        _load().orc_back_pixels_power(g.ref, y, power, len(sel), sel, xs, as_.ctypes.data if with_abs else None)
    x[keep] = xs
    if with_abs:
        a[keep] = as_
    return (x, a) if with_abs else x


def forward_pixels(g: Geometry, pixels, cylinders, with_abs: bool = False):
    """Forward projection of a batch of voxel cylinders (MBIRJAX "Sharding
    Overview", "Why cone beam projects whole cylinders"): A x for the volume x
    that is zero except that pixel pixels[q] (flat id i*Nx + j) holds
    cylinders[q] (S voxels).  Ids outside [0, Ny*Nx) are padding and add
    nothing, whatever their cylinders hold.  A repeated id adds its cylinders:
    the q-th occurrence of each id goes into volume number q, each volume is
    projected on its own and the projections are summed in fp64, so no input
    is rounded on the way."""
    ny, nx, ns = g.recon_shape
    pixels = np.asarray(pixels, dtype=np.int64).reshape(-1)
    cylinders = np.asarray(cylinders, dtype=np.float32).reshape(len(pixels), ns)
    keep = np.flatnonzero((pixels >= 0) & (pixels < ny * nx))
    y = np.zeros(g.sino_shape, dtype=np.float64)
    ay = np.zeros(g.sino_shape, dtype=np.float64) if with_abs else None
    seen: dict = {}
    layers: list = []
    for q in keep:
        p = int(pixels[q])
        r = seen.get(p, 0)
        seen[p] = r + 1
        if r == len(layers):
            layers.append(np.zeros((ny * nx, ns), dtype=np.float32))
        layers[r][p] = cylinders[q]
    for layer in layers:
        out = forward(g, layer.reshape(ny, nx, ns), with_abs=with_abs)
        if with_abs:
            y += out[0]
            ay += out[1]
        else:
            y += out
    return (y, ay) if with_abs else y


def voxel_taps(g: Geometry, v, i, j, k):
    """List of (row, channel, weight) for one voxel-view."""
    cap = (2 * g.s.radius + 1) ** 2
    rows = np.zeros(cap, np.int32)
    chans = np.zeros(cap, np.int32)
    w = np.zeros(cap, np.float64)
    n = _load().orc_voxel_taps(g.ref, v, i, j, k, rows, chans, w, cap)
    return [(int(rows[q]), int(chans[q]), float(w[q])) for q in range(n)]


def vp_params(g: Geometry, v, i, j) -> dict:
    out = np.zeros(7, np.float64)
    _load().orc_vp_params(g.ref, v, i, j, out)
    return dict(u=out[0], nc=int(out[1]), W=out[2], L=out[3], Mr=out[4], rho=out[5], Wrow=out[6])


def ov(d: float, a: float) -> float:
    return _load().orc_ov(d, a)


def num_threads() -> int:
    return _load().orc_num_threads()
