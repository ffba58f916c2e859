"""Python binding of the gfx950 projector library (``_lib/libbpamd.so``).

Argument marshalling only: every step of forward and back projection runs in
the HIP kernels behind the C ABI declared in ``include/proj.h``.  PyTorch
supplies device memory and the current HIP stream.  There is no CPU path: if
the library has not been built, or a tensor is not on the handle's GPU, the
call raises.

Names follow the C ABI: ``proj_create`` -> :class:`Projector`,
``proj_forward`` -> :meth:`Projector.forward`, ``proj_forward_noalloc`` ->
:meth:`Projector.forward_noalloc`, ``proj_back`` ->
:meth:`Projector.back`, ``proj_back_squared`` -> :meth:`Projector.back_squared`,
``proj_channel_index`` -> :meth:`Projector.channel_index`,
``proj_forward_pixels`` -> :meth:`Projector.forward_pixels`,
``proj_back_pixels`` -> :meth:`Projector.back_pixels`, ``proj_cgls`` ->
:meth:`Projector.cgls`, ``proj_sirt`` -> :meth:`Projector.sirt` (with
``proj_solver_workspace_size`` for their workspace).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

PROJ_PARALLEL = 0
PROJ_CONE_FLAT = 1
PROJ_FORWARD_AUTO = 0
PROJ_FORWARD_TILE = 1
PROJ_FORWARD_GATHER = 2
PROJ_FORWARD_CONE_TILE_8X4 = 3
PROJ_FORWARD_CONE_TILE_8X8 = 4

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libbpamd.so")

STATUS = {
    0: "PROJ_OK",
    -1: "PROJ_ERR_INVALID_ARGUMENT",
    -2: "PROJ_ERR_UNSUPPORTED",
    -3: "PROJ_ERR_ALIAS",
    -4: "PROJ_ERR_OUT_OF_MEMORY",
    -5: "PROJ_ERR_DEVICE",
}

# Every entry point include/proj.h declares.
EXPORTS = ("proj_create", "proj_forward", "proj_forward_noalloc", "proj_back", "proj_back_squared", "proj_channel_index",
           "proj_forward_pixels", "proj_back_pixels", "proj_solver_workspace_size", "proj_cgls", "proj_sirt",
           "proj_plan_query", "proj_destroy", "proj_status_string", "proj_last_error", "proj_describe")


class _SolverInfo(ctypes.Structure):
    _fields_ = [("iterations", ctypes.c_int32), ("converged", ctypes.c_int32), ("reason", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


STOP_REASONS = ("converged", "iterations", "stationary", "breakdown")


@dataclass
class SolverResult:
    """What ``Projector.cgls`` and ``Projector.sirt`` return: the last iterate
    (a device tensor), completed iterations, the residual norms (initial, then
    one per iteration), whether the stop rule held, and why the loop ended."""
    volume: object
    iterations: int
    residual_history: List[float] = field(default_factory=list)
    converged: bool = False
    reason: str = "iterations"


class ProjError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


class _Geometry(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("num_views", ctypes.c_int32),
        ("angles", ctypes.POINTER(ctypes.c_double)),
        ("channel_shift", ctypes.POINTER(ctypes.c_double)),
        ("source_z", ctypes.POINTER(ctypes.c_double)),
        ("delta_voxel", ctypes.c_double),
        ("delta_channel", ctypes.c_double),
        ("delta_row", ctypes.c_double),
        ("source_iso", ctypes.c_double),
        ("source_detector", ctypes.c_double),
        ("det_channel_offset", ctypes.c_double),
        ("det_row_offset", ctypes.c_double),
        ("psf_radius", ctypes.c_int32),
        ("forward_strategy", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"the HIP projector library is not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    i64x3 = P(ctypes.c_int64)
    lib.proj_create.argtypes = [P(_Geometry), i64x3, i64x3, ctypes.c_int, P(ctypes.c_void_p)]
    lib.proj_create.restype = ctypes.c_int
    for name in ("proj_forward", "proj_forward_noalloc", "proj_back", "proj_back_squared"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.proj_channel_index.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    vp = ctypes.c_void_p
    lib.proj_forward_pixels.argtypes = [vp, vp, ctypes.c_int64, vp, vp, vp]
    lib.proj_forward_pixels.restype = ctypes.c_int
    lib.proj_back_pixels.argtypes = [vp, vp, vp, ctypes.c_int64, vp, vp]
    lib.proj_back_pixels.restype = ctypes.c_int
    lib.proj_solver_workspace_size.argtypes = [vp, P(ctypes.c_int64)]
    lib.proj_solver_workspace_size.restype = ctypes.c_int
    d, i32, i64 = ctypes.c_double, ctypes.c_int32, ctypes.c_int64
    lib.proj_cgls.argtypes = [vp, vp, vp, vp, vp, i64, i32, d, d, P(d), P(_SolverInfo), vp]
    lib.proj_cgls.restype = ctypes.c_int
    lib.proj_sirt.argtypes = [vp, vp, vp, vp, vp, i64, i32, d, d, d, i32, P(d), P(_SolverInfo), vp]
    lib.proj_sirt.restype = ctypes.c_int
    lib.proj_channel_index.restype = ctypes.c_int
    lib.proj_plan_query.argtypes = [P(_Geometry), i64x3, i64x3, ctypes.c_char_p, ctypes.c_int]
    lib.proj_plan_query.restype = ctypes.c_int
    lib.proj_destroy.argtypes = [ctypes.c_void_p]
    lib.proj_destroy.restype = None
    lib.proj_status_string.argtypes = [ctypes.c_int]
    lib.proj_status_string.restype = ctypes.c_char_p
    lib.proj_last_error.argtypes = []
    lib.proj_last_error.restype = ctypes.c_char_p
    lib.proj_describe.argtypes = [ctypes.c_void_p, ctypes.c_char_p, ctypes.c_int]
    lib.proj_describe.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        detail = load_library().proj_last_error().decode(errors="replace")
        raise ProjError(status, where, detail)


class _GeomArgs:
    """Owns the ctypes geometry struct and the arrays it points into."""

    def __init__(self, geometry: dict, recon_shape: Sequence[int], sino_shape: Sequence[int]):
        self.recon_shape = tuple(int(v) for v in recon_shape)
        self.sino_shape = tuple(int(v) for v in sino_shape)
        if len(self.recon_shape) != 3 or len(self.sino_shape) != 3:
            raise ValueError("recon_shape and sino_shape have three entries each")

        def arr(key):
            a = geometry.get(key)
            return None if a is None else np.ascontiguousarray(a, dtype=np.float64).ravel()

        self._angles = arr("angles")
        self._shift = arr("channel_shift")
        self._zsrc = arr("source_z")
        dp = ctypes.POINTER(ctypes.c_double)

        def ptr(a):
            return a.ctypes.data_as(dp) if a is not None and a.size else ctypes.cast(None, dp)

        nv = int(geometry.get("num_views", self.sino_shape[0]))
        for name, a in (("angles", self._angles), ("channel_shift", self._shift), ("source_z", self._zsrc)):
            if a is not None and a.size != nv:
                raise ValueError(f"{name} must have num_views entries")
        self.s = _Geometry(
            int(geometry["kind"]), nv, ptr(self._angles), ptr(self._shift), ptr(self._zsrc),
            float(geometry.get("delta_voxel", 1.0)), float(geometry.get("delta_channel", 1.0)),
            float(geometry.get("delta_row", 1.0)), float(geometry.get("source_iso", 0.0)),
            float(geometry.get("source_detector", 0.0)), float(geometry.get("det_channel_offset", 0.0)),
            float(geometry.get("det_row_offset", 0.0)), int(geometry.get("psf_radius", 1)),
            int(geometry.get("forward_strategy", 0)))
        self.rs = (ctypes.c_int64 * 3)(*self.recon_shape)
        self.ss = (ctypes.c_int64 * 3)(*self.sino_shape)


def plan_query(geometry: dict, recon_shape, sino_shape) -> str:
    """Validate and plan without a GPU; returns the plan description."""
    lib = load_library()
    ga = _GeomArgs(geometry, recon_shape, sino_shape)
    buf = ctypes.create_string_buffer(1024)
    _check(lib.proj_plan_query(ctypes.byref(ga.s), ga.rs, ga.ss, buf, len(buf)), "proj_plan_query")
    return buf.value.decode()


def _stream_ptr(torch, device: int, stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


class Projector:
    """A matched forward/back projector pair on one GPU (``proj_create``)."""

    def __init__(self, geometry: dict, recon_shape, sino_shape, device: int = 0):
        import torch  # device memory and streams only

        self._torch = torch
        self._lib = load_library()
        self._ga = _GeomArgs(geometry, recon_shape, sino_shape)
        self.recon_shape = self._ga.recon_shape
        self.sino_shape = self._ga.sino_shape
        self.device = int(device)
        self._work = None          # solver workspace, allocated on first use
        h = ctypes.c_void_p()
        _check(self._lib.proj_create(ctypes.byref(self._ga.s), self._ga.rs, self._ga.ss, self.device,
                                     ctypes.byref(h)), "proj_create")
        self._h = h

    # ---------------------------------------------------------------- helpers
    def _tensor(self, t, shape, dtype, what):
        torch = self._torch
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{what} must be a torch tensor on the GPU")
        if t.device.type != "cuda" or (t.device.index or 0) != self.device:
            raise ValueError(f"{what} must live on cuda:{self.device}")
        if t.dtype != dtype:
            raise TypeError(f"{what} must be {dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous (C order)")
        return t

    def _empty(self, shape, dtype):
        return self._torch.empty(shape, dtype=dtype, device=f"cuda:{self.device}")

    # -------------------------------------------------------------- projectors
    def forward(self, recon, out=None, stream=None):
        """``proj_forward``: sinogram (V, R, C) = A recon (Ny, Nx, S)."""
        torch = self._torch
        self._tensor(recon, self.recon_shape, torch.float32, "recon")
        out = self._empty(self.sino_shape, torch.float32) if out is None else \
            self._tensor(out, self.sino_shape, torch.float32, "out")
        _check(self._lib.proj_forward(self._h, ctypes.c_void_p(recon.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                      ctypes.c_void_p(_stream_ptr(torch, self.device, stream))), "proj_forward")
        return out

    def forward_noalloc(self, recon, out=None, stream=None):
        """``proj_forward_noalloc``: the same sinogram as :meth:`forward`, with
        the parallel walk's partial sums in the library's fixed device scratch
        (at most 144 MiB, shared by every call on the GPU) instead of the
        handle's buffer.  The call itself allocates nothing; pass ``out`` to
        keep the whole call allocation-free."""
        torch = self._torch
        self._tensor(recon, self.recon_shape, torch.float32, "recon")
        out = self._empty(self.sino_shape, torch.float32) if out is None else \
            self._tensor(out, self.sino_shape, torch.float32, "out")
        _check(self._lib.proj_forward_noalloc(self._h, ctypes.c_void_p(recon.data_ptr()),
                                              ctypes.c_void_p(out.data_ptr()),
                                              ctypes.c_void_p(_stream_ptr(torch, self.device, stream))),
               "proj_forward_noalloc")
        return out

    def back(self, sino, out=None, stream=None):
        """``proj_back``: recon (Ny, Nx, S) = A^T sinogram (V, R, C)."""
        torch = self._torch
        self._tensor(sino, self.sino_shape, torch.float32, "sino")
        out = self._empty(self.recon_shape, torch.float32) if out is None else \
            self._tensor(out, self.recon_shape, torch.float32, "out")
        _check(self._lib.proj_back(self._h, ctypes.c_void_p(sino.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                   ctypes.c_void_p(_stream_ptr(torch, self.device, stream))), "proj_back")
        return out

    def back_squared(self, sino, out=None, stream=None):
        """``proj_back_squared``: the back projection with every tap weight
        squared (the Hessian-diagonal weighting), recon (Ny, Nx, S)."""
        torch = self._torch
        self._tensor(sino, self.sino_shape, torch.float32, "sino")
        out = self._empty(self.recon_shape, torch.float32) if out is None else \
            self._tensor(out, self.recon_shape, torch.float32, "out")
        _check(self._lib.proj_back_squared(self._h, ctypes.c_void_p(sino.data_ptr()),
                                           ctypes.c_void_p(out.data_ptr()),
                                           ctypes.c_void_p(_stream_ptr(torch, self.device, stream))),
               "proj_back_squared")
        return out

    def forward_pixels(self, pixels, cylinders, out=None, stream=None):
        """``proj_forward_pixels``: sinogram (V, R, C) of a volume that is zero
        except at the listed pixels.  ``pixels`` int32 (n,) flat ids i*Nx + j,
        ids outside [0, Ny*Nx) are inert padding; ``cylinders`` (n, S)."""
        torch = self._torch
        n = int(pixels.shape[0]) if isinstance(pixels, torch.Tensor) and pixels.dim() == 1 else -1
        self._tensor(pixels, (n,), torch.int32, "pixels")
        self._tensor(cylinders, (n, self.recon_shape[2]), torch.float32, "cylinders")
        out = self._empty(self.sino_shape, torch.float32) if out is None else \
            self._tensor(out, self.sino_shape, torch.float32, "out")
        _check(self._lib.proj_forward_pixels(self._h, ctypes.c_void_p(pixels.data_ptr()), n,
                                             ctypes.c_void_p(cylinders.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                             ctypes.c_void_p(_stream_ptr(torch, self.device, stream))),
               "proj_forward_pixels")
        return out

    def back_pixels(self, sino, pixels, out=None, stream=None):
        """``proj_back_pixels``: the cylinders (n, S) of A^T sinogram at the
        listed pixels; a padding id (outside [0, Ny*Nx)) gets zeros."""
        torch = self._torch
        self._tensor(sino, self.sino_shape, torch.float32, "sino")
        n = int(pixels.shape[0]) if isinstance(pixels, torch.Tensor) and pixels.dim() == 1 else -1
        self._tensor(pixels, (n,), torch.int32, "pixels")
        shape = (n, self.recon_shape[2])
        out = self._empty(shape, torch.float32) if out is None else self._tensor(out, shape, torch.float32, "out")
        _check(self._lib.proj_back_pixels(self._h, ctypes.c_void_p(sino.data_ptr()),
                                          ctypes.c_void_p(pixels.data_ptr()), n, ctypes.c_void_p(out.data_ptr()),
                                          ctypes.c_void_p(_stream_ptr(torch, self.device, stream))),
               "proj_back_pixels")
        return out

    def _solve(self, name, sino, iterations, atol, rtol, x0, out, stream, extra):
        torch = self._torch
        self._tensor(sino, self.sino_shape, torch.float32, "sino")
        if x0 is not None:
            self._tensor(x0, self.recon_shape, torch.float32, "x0")
        out = self._empty(self.recon_shape, torch.float32) if out is None else \
            self._tensor(out, self.recon_shape, torch.float32, "out")
        nbytes = ctypes.c_int64()
        _check(self._lib.proj_solver_workspace_size(self._h, ctypes.byref(nbytes)), "proj_solver_workspace_size")
        if self._work is None or self._work.numel() < nbytes.value:
            self._work = torch.empty(nbytes.value, dtype=torch.uint8, device=f"cuda:{self.device}")
        iterations = int(iterations)
        hist = (ctypes.c_double * (max(iterations, 0) + 1))()
        info = _SolverInfo()
        fn = getattr(self._lib, name)
        _check(fn(self._h, ctypes.c_void_p(sino.data_ptr()), ctypes.c_void_p(x0.data_ptr() if x0 is not None else 0),
                  ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(self._work.data_ptr()), self._work.numel(),
                  iterations, float(atol), float(rtol), *extra, hist, ctypes.byref(info),
                  ctypes.c_void_p(_stream_ptr(torch, self.device, stream))), name)
        return SolverResult(out, info.iterations, list(hist[:info.iterations + 1]), bool(info.converged),
                            STOP_REASONS[info.reason])

    def cgls(self, sino, iterations, atol=0.0, rtol=0.0, x0=None, out=None, stream=None) -> SolverResult:
        """``proj_cgls``: least squares by conjugate gradients, stopping when
        ||y - A x|| <= atol + rtol ||y|| (the initial iterate included)."""
        return self._solve("proj_cgls", sino, iterations, atol, rtol, x0, out, stream, ())

    def sirt(self, sino, iterations, atol=0.0, rtol=0.0, x0=None, relaxation=1.0, nonnegative=True, out=None,
             stream=None) -> SolverResult:
        """``proj_sirt``: x += relaxation * C A^T R (y - A x), clamped at 0 when
        ``nonnegative``; the same stop rule as ``cgls``."""
        return self._solve("proj_sirt", sino, iterations, atol, rtol, x0, out, stream,
                           (float(relaxation), int(bool(nonnegative))))

    def channel_index(self, out=None, stream=None):
        """``proj_channel_index``: int32 (V, Ny*Nx) channel index table."""
        torch = self._torch
        shape = (self.sino_shape[0], self.recon_shape[0] * self.recon_shape[1])
        out = self._empty(shape, torch.int32) if out is None else self._tensor(out, shape, torch.int32, "out")
        _check(self._lib.proj_channel_index(self._h, ctypes.c_void_p(out.data_ptr()),
                                            ctypes.c_void_p(_stream_ptr(torch, self.device, stream))),
               "proj_channel_index")
        return out

    def describe(self) -> str:
        buf = ctypes.create_string_buffer(1024)
        self._lib.proj_describe(self._h, buf, len(buf))
        return buf.value.decode()

    @property
    def handle(self) -> int:
        return int(self._h.value or 0)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.proj_destroy(self._h)
            self._h = ctypes.c_void_p()
        self._work = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
