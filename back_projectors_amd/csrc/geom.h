// Geometry shared by the host planner and the gfx950 kernels.
//
// Model (MBIRJAX "Projector kernels" page, paragraph "Shared machinery, and
// the rounding defense": a geometry contributes only its coordinate math and a
// weight scale; the trapezoid taps are common to all geometries):
//
//   pixel centre      x = (j - (Nx-1)/2) dv,  y = (i - (Ny-1)/2) dv,
//                     z = (k - (S-1)/2) dv
//   parallel          u = (x cos t + y sin t)/dch + c_ch + shift_v,
//                     W = dv m/dch, L = dv/m, m = max(|cos t|, |sin t|);
//                     row r <-> slice r
//   flat cone         a = x cos t + y sin t, d = SID + y cos t - x sin t,
//                     u = SDD a/(d dch) + c_ch + shift_v,
//                     W_ch = SDD dv M/(d^2 dch), M = max(|y + SID cos t|, |SID sin t - x|),
//                     row w_k = SDD (z_k - zsrc_v)/(d drow) + c_row, W_row = SDD dv/(d drow),
//                     L_k = dv sqrt(d^2 + a^2 + (z_k - zsrc_v)^2)/M
//   taps              n_c = rint(u) (ties to even), tap n in [n_c - r, n_c + r]
//                     has weight L * ov(n - u; W), ov(e; a) the overlap of the
//                     unit cell centred at e with the centred box of width a
//                     (the same in rows for the cone), off-detector taps dropped.
//
// The channel index n_c is computed by a separate fp64 pass with every product
// and sum rounded in the written order (no contraction), so it is reproducible
// bit for bit; the projection kernels only read it.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace bpamd {

// Per-view constants, fp64, computed once on the host at creation.
struct ViewK {
    double c, s;      // cos and sin of the view angle (C library, fp64)
    double shift;     // lateral detector shift, channels
    double zsrc;      // source height (cone), voxel units
    double cd, sd;    // parallel: c/dch, s/dch
    double u0;        // c_ch + shift
    double W, L;      // parallel: footprint width (channels) and chord scale
};

// Shapes and scalar geometry, passed by value to every kernel.
struct Geo {
    int32_t kind;     // 0 parallel, 1 flat-detector cone
    int32_t radius;   // taps on each side, 1..4
    int32_t ny, nx, ns, nv, nr, nc;
    double dv, dch, drow, sid, sdd;
    double cx, cy, cz;     // (N-1)/2 of the recon axes
    double cch, crow;      // detector centres including offsets
};

__host__ __device__ inline double pix_x(const Geo &g, int j) { return ((double)j - g.cx) * g.dv; }
__host__ __device__ inline double pix_y(const Geo &g, int i) { return ((double)i - g.cy) * g.dv; }
__host__ __device__ inline double slice_z(const Geo &g, int k) { return ((double)k - g.cz) * g.dv; }

// Conservative window of detector cells a rectangular pixel tile (and, for
// the cone, a run of slices) can reach in one view, including the r taps on
// each side, clipped to the detector plus 2r cells.  nw <= 0 or nrw <= 0
// means the tile sees nothing of the detector in that view.  Used by the host
// planner to size LDS and by the kernels to place their windows; both call
// this same code.
struct Window {
    int n0, nw;   // channels [n0, n0 + nw)
    int m0, nrw;  // rows [m0, m0 + nrw) (cone) ; unused for parallel
};
static_assert(sizeof(Window) == 16, "windows are read by the kernels as int4 tables");

__host__ __device__ inline double cone_u_approx(const Geo &g, const ViewK &vk, double x, double y) {
    double a = x * vk.c + y * vk.s;
    double d = g.sid + (y * vk.c - x * vk.s);
    return g.sdd * a / (d * g.dch) + vk.u0;
}

// Tile = pixels [i0, i1] x [j0, j1] (inclusive); slices [k0, k1] (cone rows).
__host__ __device__ inline Window tile_window(const Geo &g, const ViewK &vk, int i0, int i1, int j0, int j1,
                                              int k0, int k1) {
    Window w;
    const double xa = pix_x(g, j0), xb = pix_x(g, j1), ya = pix_y(g, i0), yb = pix_y(g, i1);
    double umin, umax;
    if (g.kind == 0) {
        const double p0 = xa * vk.cd, p1 = xb * vk.cd, q0 = ya * vk.sd, q1 = yb * vk.sd;
        umin = fmin(p0, p1) + fmin(q0, q1) + vk.u0;
        umax = fmax(p0, p1) + fmax(q0, q1) + vk.u0;
        w.m0 = k0;
        w.nrw = k1 - k0 + 1;
    } else {
        // a/d is linear-fractional with d > 0, so its extremes over the
        // rectangle sit at the corners; the same holds for dz/d over the box.
        const double u00 = cone_u_approx(g, vk, xa, ya), u01 = cone_u_approx(g, vk, xb, ya);
        const double u10 = cone_u_approx(g, vk, xa, yb), u11 = cone_u_approx(g, vk, xb, yb);
        umin = fmin(fmin(u00, u01), fmin(u10, u11));
        umax = fmax(fmax(u00, u01), fmax(u10, u11));
        const double d00 = g.sid + (ya * vk.c - xa * vk.s), d01 = g.sid + (ya * vk.c - xb * vk.s);
        const double d10 = g.sid + (yb * vk.c - xa * vk.s), d11 = g.sid + (yb * vk.c - xb * vk.s);
        const double dmin = fmin(fmin(d00, d01), fmin(d10, d11));
        const double dmax = fmax(fmax(d00, d01), fmax(d10, d11));
        const double mlo = g.sdd / (dmax * g.drow), mhi = g.sdd / (dmin * g.drow);
        const double z0 = slice_z(g, k0) - vk.zsrc, z1 = slice_z(g, k1) - vk.zsrc;
        const double a0 = mlo * z0, a1 = mlo * z1, b0 = mhi * z0, b1 = mhi * z1;
        const double wmin = fmin(fmax(fmin(fmin(a0, a1), fmin(b0, b1)) + g.crow, -1e9), 1e9);
        const double wmax = fmin(fmax(fmax(fmax(a0, a1), fmax(b0, b1)) + g.crow, -1e9), 1e9);
        w.m0 = (int)floor(wmin) - 1 - g.radius;
        w.nrw = (int)ceil(wmax) + 1 + g.radius - w.m0 + 1;
    }
    umin = fmin(fmax(umin, -1e9), 1e9);
    umax = fmin(fmax(umax, -1e9), 1e9);
    w.n0 = (int)floor(umin) - 1 - g.radius;
    w.nw = (int)ceil(umax) + 1 + g.radius - w.n0 + 1;
    // Clip to the detector plus 2r cells: a voxel whose centre cell lies more
    // than r cells off the detector has no tap on it and is skipped, so the
    // taps that are kept always fall inside the clipped window.
    {
        const int lo = -2 * g.radius, hi = g.nc - 1 + 2 * g.radius;
        const int a = w.n0 > lo ? w.n0 : lo;
        const int b0 = w.n0 + w.nw - 1, b = b0 < hi ? b0 : hi;
        w.n0 = a;
        w.nw = b - a + 1;
    }
    if (g.kind != 0) {
        const int lo = -2 * g.radius, hi = g.nr - 1 + 2 * g.radius;
        const int a = w.m0 > lo ? w.m0 : lo;
        const int b0 = w.m0 + w.nrw - 1, b = b0 < hi ? b0 : hi;
        w.m0 = a;
        w.nrw = b - a + 1;
    }
    return w;
}

// The (tile, chunk) work item of this workgroup in a gx x gy grid, ordered for
// the L2 caches: workgroups are dispatched to the 8 XCDs in turn by linear id
// (id mod 8), and each XCD has its own L2, so the ids one XCD receives are
// mapped to a contiguous run of the chunk-major, row-major tile list.  Tiles
// that run together on one XCD are then neighbours whose detector windows
// overlap, and they read them through one L2.  A bijection of the grid: any
// other placement by the hardware is still correct, only slower.
__device__ inline void xcd_work_item(int gx, int gy, int &tile, int &chunk) {
    const int n = gx * gy;
    const int lin = (int)blockIdx.y * gx + (int)blockIdx.x;
    const int xcd = lin & 7, slot = lin >> 3;
    const int q = n >> 3, r = n & 7;
    const int w = xcd * q + (xcd < r ? xcd : r) + slot;
    tile = w % gx;
    chunk = w / gx;
}

// Tile t of a tx x ty tile grid in blocked order: blocks of 8 x 8 tiles, the
// blocks row-major and the tiles of a block row-major (the blocks of the last
// block row and column are cut to the grid).  A run of consecutive t is then
// a compact patch of tiles instead of a strip across the volume.  A
// bijection of [0, tx ty).
__device__ inline int blocked_tile(int t, int tx, int ty) {
    const int br = t / (8 * tx);              // block row
    const int h = min(8, ty - 8 * br);        // its height in tiles
    const int o = t - br * 8 * tx;
    const int bc = o / (8 * h);               // block column (all before it are 8 wide)
    const int bw = min(8, tx - 8 * bc);       // its width in tiles
    const int oo = o - bc * 8 * h;
    const int r = oo / bw, c = oo - r * bw;
    return (8 * br + r) * tx + 8 * bc + c;
}

// The (tile, chunk) work item of this workgroup in a grid of gx = tx ty tiles
// by gy chunks, for kernels whose chunks read disjoint detector rows and whose
// neighbouring tiles share detector channels.  Where gx is a multiple of 8,
// XCD x takes the same eighth of the tiles in every chunk, chunk by chunk
// (each XCD gets an equal share of every chunk's work, and the chunks' work
// can differ), and its tiles are consecutive in blocked order, so that the
// workgroups resident on one XCD at a time form a compact patch whose
// windows overlap in its L2.  Otherwise the grid is split as by
// xcd_work_item, with the tiles in blocked order.  A bijection of the grid.
__device__ inline void xcd_work_item_blocked(int gx, int gy, int tx, int ty, int &tile, int &chunk) {
    const int lin = (int)blockIdx.y * gx + (int)blockIdx.x;
    const int xcd = lin & 7, slot = lin >> 3;
    int t;
    if ((gx & 7) == 0) {
        const int per = gx >> 3;
        chunk = slot / per;
        t = xcd * per + slot % per;
    } else {
        const int n = gx * gy;
        const int q = n >> 3, r = n & 7;
        const int w = xcd * q + (xcd < r ? xcd : r) + slot;
        t = w % gx;
        chunk = w / gx;
    }
    tile = blocked_tile(t, tx, ty);
}

}  // namespace bpamd
