// Trapezoid tap weights, evaluated in fp64 and rounded once to fp32.
//
// ov(e; a), the overlap of the unit detector cell centred at e with the
// centred box [-a/2, a/2], equals G(e + 1/2) - G(e - 1/2) with
// G(t) = clamp(t, -a/2, a/2).  For the 2R+1 taps around n_c the cell edges
// are shared, so 2R+2 clamps give all weights, and clamping the outermost
// edges drops whatever part of a wide box falls beyond the last tap.  The
// small weights near the box edges come out of a subtraction of nearby
// numbers, which is why it runs in fp64 (as fast as fp32 on CDNA vector ALUs).
#pragma once

#include <hip/hip_runtime.h>

namespace bpamd {

// w[t + R] = scale * ov(t - f; a), t = -R..R, with f = u - n_c in [-1/2, 1/2].
template <int R>
__device__ __forceinline__ void tap_weights(double f, double a, double scale, float (&w)[2 * R + 1]) {
    const double h = 0.5 * a;
    double gp = fmin(fmax(-0.5 - (double)R - f, -h), h);
#pragma unroll
    for (int t = -R; t <= R; ++t) {
        const double gn = fmin(fmax((double)t + 0.5 - f, -h), h);
        w[t + R] = (float)(scale * (gn - gp));
        gp = gn;
    }
}

// Same, unscaled, into fp64 (for products of row and channel weights).
template <int R>
__device__ __forceinline__ void tap_weights_d(double f, double a, double (&w)[2 * R + 1]) {
    const double h = 0.5 * a;
    double gp = fmin(fmax(-0.5 - (double)R - f, -h), h);
#pragma unroll
    for (int t = -R; t <= R; ++t) {
        const double gn = fmin(fmax((double)t + 0.5 - f, -h), h);
        w[t + R] = gn - gp;
        gp = gn;
    }
}

}  // namespace bpamd
