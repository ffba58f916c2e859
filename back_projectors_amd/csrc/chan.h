// The exact channel coordinate of a pixel centre and the parallel-beam tap
// record derived from it (MBIRJAX "Projector kernels" page, paragraph "Shared
// machinery, and the rounding defense": each voxel's channel is computed once,
// in a step of its own, and handed on as data).  Shared by the creation passes
// and by the batch kernels, which evaluate the same records for the pixels they
// list instead of reading the table: every operation below is one IEEE fp64
// operation rounded in the written order (-ffp-contract=off, and the pragma
// forbids fusing a product into a sum), and fp64 division on gfx950 is
// correctly rounded, so every caller gets the same bits.
#pragma once

#include "geom.h"

#pragma clang fp contract(off)

namespace bpamd {

__device__ __forceinline__ double channel_coord_exact(const Geo &g, const ViewK &vk, int i, int j) {
    const double x = pix_x(g, j);
    const double y = pix_y(g, i);
    if (g.kind == 0) {
        const double xc = x * vk.c;
        const double ys = y * vk.s;
        const double t = xc + ys;
        const double tq = t / g.dch;
        const double u = tq + g.cch;
        return u + vk.shift;
    }
    const double xc = x * vk.c;
    const double ys = y * vk.s;
    const double yc = y * vk.c;
    const double xs = x * vk.s;
    const double a = xc + ys;
    const double b = yc - xs;
    const double d = g.sid + b;
    const double dc = d * g.dch;
    const double mc = g.sdd / dc;
    const double ma = mc * a;
    const double u = ma + g.cch;
    return u + vk.shift;
}

// Overlap of the unit cell centred at e with the centred box [-a/2, a/2].
__device__ __forceinline__ double cell_overlap(double e, double a) {
    const double hi = fmin(e + 0.5, a / 2.0);
    const double lo = fmax(e - 0.5, -a / 2.0);
    const double r = hi - lo;
    return r > 0.0 ? r : 0.0;
}

// Parallel-beam tap record of pixel (i, j) in view vk: the first channel that
// can carry weight, n_f, and the fp32 weights of channels n_f .. n_f + ntap -
// 1.  The weights are L ov(n - u; W) evaluated in fp64 from the exact channel
// coordinate and rounded once; taps outside [n_c - r, n_c + r] (the PSF
// radius) or off the detector get weight 0, and a pixel none of whose taps
// reaches the detector gets n_f = INT_MAX (the projectors skip it).
template <int NT>
__device__ __forceinline__ int par_tap_record(const Geo &g, const ViewK &vk, int i, int j, int ntap,
                                              float (&w)[NT]) {
    const double u = channel_coord_exact(g, vk, i, j);
    const int nc = (int)rint(u);
    // first cell with positive overlap, kept so that all ntap taps stay
    // inside the PSF radius [n_c - r, n_c + r]
    int nf = (int)floor(u - 0.5 * vk.W - 0.5) + 1;
    if (nf < nc - g.radius) nf = nc - g.radius;
    if (nf > nc + g.radius - ntap + 1) nf = nc + g.radius - ntap + 1;
    bool any = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        double wd = 0.0;
        const int n = nf + t;
        if (t < ntap && n <= nc + g.radius && n >= 0 && n < g.nc) wd = vk.L * cell_overlap((double)n - u, vk.W);
        w[t] = (float)wd;
        any = any || w[t] != 0.f;
    }
    return any ? nf : INT32_MAX;
}

}  // namespace bpamd
