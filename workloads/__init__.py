"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke run.

This module only *describes* inputs: acquisition parameters (angles, detector
shifts, source heights, pitches, shapes) and seeded phantoms / sinograms.  It
holds none of the projector's arithmetic, so both the HIP path and the CPU
reference can take their inputs from here without sharing any of the method.

Geometry conventions (the projector pages leave these open, see the notes on
each workload):

* Recon arrays are ``(Ny, Nx, S)`` float32, slices fastest (voxel cylinders, as
  in the MBIRJAX "Sharding Overview" page, section "The two shardings").
* Sinogram arrays are ``(V, R, C)`` float32, channels fastest (one view block
  per view-owner, same section).
* Angles are radians; parallel views spread evenly over ``[0, pi)`` and
  circular cone views over ``[0, 2 pi)``, endpoint excluded.
* Every workload has unit voxel pitch and a trapezoid PSF radius of one
  channel (and one row for cone beam).

Phantoms are drawn with ``numpy.random.default_rng(seed)`` in float64 and then
cast to float32; both projector implementations consume the same float32
values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

PARALLEL = 0
CONE_FLAT = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    """One acquisition: geometry, shapes and the seeds of its inputs."""

    name: str
    kind: int                      # PARALLEL or CONE_FLAT
    ny: int
    nx: int
    ns: int                        # slices S
    nv: int                        # views V
    nr: int                        # detector rows R
    nc: int                        # detector channels C
    dch: float = 1.0               # channel pitch, voxel units
    drow: float = 1.0              # row pitch, voxel units
    sid: float = 0.0               # source to iso distance (cone)
    sdd: float = 0.0               # source to detector distance (cone)
    angle_step: Optional[float] = None   # None -> span/V (span = pi or 2 pi)
    zsrc_step: float = 0.0         # helical source advance per view, voxel units
    shift_step: float = 0.0        # translation: detector shift per view, channels
    phantom: str = "ellipsoids"    # "disk" or "ellipsoids"
    seed_x: int = 0
    seed_y: int = 0                # 0 -> the back input is the forward of x
    dv: float = 1.0
    radius: int = 1
    angle_start: float = 0.0       # first view angle when angle_step is given

    # ----------------------------------------------------------- geometry ---
    def angles(self) -> np.ndarray:
        v = np.arange(self.nv, dtype=np.float64)
        if self.shift_step != 0.0:
            return np.zeros(self.nv, dtype=np.float64)
        if self.angle_step is not None:
            return self.angle_start + v * self.angle_step
        span = math.pi if self.kind == PARALLEL else 2.0 * math.pi
        return v * span / self.nv

    def channel_shift(self) -> Optional[np.ndarray]:
        if self.shift_step == 0.0:
            return None
        v = np.arange(self.nv, dtype=np.float64)
        # centred so the shifted detector positions are symmetric about view (V-1)/2
        return self.shift_step * (v - (self.nv - 1) / 2.0)

    def source_z(self) -> Optional[np.ndarray]:
        if self.zsrc_step == 0.0:
            return None
        v = np.arange(self.nv, dtype=np.float64)
        return self.zsrc_step * (v - (self.nv - 1) / 2.0)

    @property
    def recon_shape(self):
        return (self.ny, self.nx, self.ns)

    @property
    def sino_shape(self):
        return (self.nv, self.nr, self.nc)

    @property
    def voxel_views(self) -> int:
        return self.nv * self.ny * self.nx * self.ns

    def geometry(self) -> dict:
        """Plain-dict description consumed by both bindings."""
        return dict(
            kind=self.kind, num_views=self.nv, angles=self.angles(),
            channel_shift=self.channel_shift(), source_z=self.source_z(),
            delta_voxel=self.dv, delta_channel=self.dch, delta_row=self.drow,
            source_iso=self.sid, source_detector=self.sdd,
            det_channel_offset=0.0, det_row_offset=0.0, psf_radius=self.radius,
        )

    # ------------------------------------------------------------- inputs ---
    def recon_input(self) -> np.ndarray:
        if self.phantom == "disk":
            return disk_phantom(self.ny, self.nx, self.ns, 28.0, 0.1, self.seed_x)
        return ellipsoid_phantom(self.ny, self.nx, self.ns, self.seed_x)

    def sino_input(self) -> np.ndarray:
        """N(0,1) back-projection input.  Seed 0 means "use the forward of x"
        instead; the caller then supplies it (from the reference forward)."""
        if self.seed_y == 0:
            raise ValueError(f"{self.name}: back input is the forward of the phantom")
        rng = np.random.default_rng(self.seed_y)
        return rng.standard_normal(self.sino_shape).astype(np.float32)


def disk_phantom(ny, nx, ns, radius, noise, seed) -> np.ndarray:
    """Uniform disk of value 1 (pixel centres strictly inside ``radius``) in
    every slice, plus U[0, noise) on every voxel drawn in C order."""
    rng = np.random.default_rng(seed)
    y = np.arange(ny, dtype=np.float64) - (ny - 1) / 2.0
    x = np.arange(nx, dtype=np.float64) - (nx - 1) / 2.0
    inside = (x[None, :] ** 2 + y[:, None] ** 2) < radius * radius
    vol = np.repeat(inside[:, :, None].astype(np.float64), ns, axis=2)
    vol += noise * rng.random((ny, nx, ns))
    return vol.astype(np.float32)


def ellipsoid_params(nx, ny, ns, seed, count=10):
    """Ten random ellipsoids; draws in a fixed order, one ``rng.random()`` each."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        rho = 0.6 * math.sqrt(rng.random())
        phi = 2.0 * math.pi * rng.random()
        czf = 0.7 * rng.random() - 0.35
        axf = 0.08 + 0.27 * rng.random()
        ayf = 0.08 + 0.27 * rng.random()
        azf = 0.08 + 0.27 * rng.random()
        psi = math.pi * rng.random()
        val = rng.random()
        out.append(dict(
            cx=rho * (nx / 2.0) * math.cos(phi), cy=rho * (nx / 2.0) * math.sin(phi),
            cz=czf * ns, ax=axf * nx / 2.0, ay=ayf * ny / 2.0, az=azf * ns / 2.0,
            psi=psi, val=val))
    return out


def ellipsoid_phantom(ny, nx, ns, seed) -> np.ndarray:
    """Sum of ten uniform ellipsoids evaluated at voxel centres, float32."""
    y = np.arange(ny, dtype=np.float64) - (ny - 1) / 2.0
    x = np.arange(nx, dtype=np.float64) - (nx - 1) / 2.0
    z = np.arange(ns, dtype=np.float64) - (ns - 1) / 2.0
    vol = np.zeros((ny, nx, ns), dtype=np.float64)
    for e in ellipsoid_params(nx, ny, ns, seed):
        cp, sp = math.cos(e["psi"]), math.sin(e["psi"])
        dx = x[None, :] - e["cx"]
        dy = y[:, None] - e["cy"]
        xr = cp * dx + sp * dy          # rotate by -psi
        yr = -sp * dx + cp * dy
        q2 = (xr / e["ax"]) ** 2 + (yr / e["ay"]) ** 2          # (ny, nx)
        qz = ((z - e["cz"]) / e["az"]) ** 2                       # (ns,)
        vol += e["val"] * ((q2[:, :, None] + qz[None, None, :]) <= 1.0)
    return vol.astype(np.float32)


# Workloads.  The first is small enough for the reference to finish in well
# under a second; the others are the full single-GPU sizes.
WORKLOADS = {
    w.name: w for w in [
        Workload("parallel-64x64x8-90v", PARALLEL, 64, 64, 8, 90, 8, 96,
                 phantom="disk", seed_x=1, seed_y=0),
        Workload("parallel-512x512x64-720v", PARALLEL, 512, 512, 64, 720, 64, 768,
                 seed_x=2, seed_y=12),
        Workload("cone-256x256x256-360v", CONE_FLAT, 256, 256, 256, 360, 256, 384,
                 dch=1.5, drow=1.5, sid=1000.0, sdd=1500.0, seed_x=3, seed_y=13),
        Workload("translation-512x512x32-64v", PARALLEL, 512, 512, 32, 64, 32, 1024,
                 shift_step=8.0, seed_x=4, seed_y=14),
        Workload("helical-512x512x96-1338v", CONE_FLAT, 512, 512, 96, 1338, 64, 736,
                 dch=1100.0 / 600.0, drow=1100.0 / 600.0, sid=600.0, sdd=1100.0,
                 angle_step=2.0 * math.pi / 600.0, zsrc_step=0.1, seed_x=5, seed_y=15),
    ]
}

SMALL = "parallel-64x64x8-90v"
BENCH = "parallel-512x512x64-720v"


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(base: Workload, name: str, **changes) -> Workload:
    """A variant of ``base`` (used for small test geometries)."""
    return dataclasses.replace(base, name=name, **changes)
