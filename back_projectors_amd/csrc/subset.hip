// Projection of a batch of voxel cylinders: the forward of a volume that is
// zero except at the listed pixels, and the back projection evaluated at the
// listed pixels only.  A view owner that collects full cylinders for a batch
// of pixels and projects them is how the MBIRJAX "Sharding Overview" page
// ("Why cone beam projects whole cylinders") runs the cone projectors; the
// same page holds zero padding of a batch to be exactly inert.  Here a list
// entry outside [0, Ny*Nx) is padding: it contributes nothing to the forward
// whatever its cylinder holds, and its back projected cylinder is written as
// zeros.
//
// One wave per (listed pixel, 64-slice chunk), lanes are slices.  The
// per-(view, pixel) quantities are the handle's tables (parallel: the fp64
// tap records; cone: the channel index, then the same fp64 footprint as the
// full projectors).  These kernels serve batches, not whole volumes: they read
// and add the sinogram cell by cell.
#include "launch.h"
#include "taps.h"

#pragma clang fp contract(off)

namespace bpamd {

namespace {

constexpr int SW = 4;   // waves (listed pixels) per workgroup

__device__ __forceinline__ int listed_pixel(const int32_t *pix, int i, int np) {
    const int p = __builtin_amdgcn_readfirstlane(pix[i]);
    return (p >= 0 && p < np) ? p : -1;
}

}  // namespace

template <int NTAP>
__global__ __launch_bounds__(SW * 64) void par_back_pixels_kernel(const float *__restrict__ sino,
                                                                  const int32_t *__restrict__ pix, int n,
                                                                  float *__restrict__ cyl,
                                                                  const int32_t *__restrict__ rec, Geo g) {
    const int lane = (int)threadIdx.x & 63;
    const int i = (int)blockIdx.x * SW + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (i >= n) return;
    const int np = g.ny * g.nx;
    const int k = (int)blockIdx.y * 64 + lane;
    const int p = listed_pixel(pix, i, np);
    float acc = 0.f;
    if (p >= 0 && k < g.ns) {
        for (int v = 0; v < g.nv; ++v) {
            const int32_t *r = rec + ((int64_t)v * np + p) * (1 + NTAP);
            const int nf = r[0];
            if (nf == INT32_MAX) continue;
            const float *row = sino + ((int64_t)v * g.nr + k) * g.nc;   // parallel: row k sees slice k
#pragma unroll
            for (int t = 0; t < NTAP; ++t) {
                const int c = nf + t;
                if (c >= 0 && c < g.nc) acc = fmaf(__int_as_float(r[1 + t]), row[c], acc);
            }
        }
    }
    if (k < g.ns) cyl[(int64_t)i * g.ns + k] = acc;
}

template <int NTAP>
__global__ __launch_bounds__(SW * 64) void par_forward_pixels_kernel(const int32_t *__restrict__ pix, int n,
                                                                     const float *__restrict__ cyl,
                                                                     float *__restrict__ facc,
                                                                     const int32_t *__restrict__ rec, Geo g, int cb,
                                                                     int s16) {
    const int lane = (int)threadIdx.x & 63;
    const int i = (int)blockIdx.x * SW + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (i >= n) return;
    const int np = g.ny * g.nx;
    const int k = (int)blockIdx.y * 64 + lane;
    const int p = listed_pixel(pix, i, np);
    if (p < 0 || k >= g.ns) return;                 // padding contributes nothing
    const float x = cyl[(int64_t)i * g.ns + k];
    for (int v = 0; v < g.nv; ++v) {
        const int32_t *r = rec + ((int64_t)v * np + p) * (1 + NTAP);
        const int nf = r[0];
        if (nf == INT32_MAX) continue;
        // the slice-fastest buffer keeps NTAP - 1 guard channels on each side
        float *col = facc + ((int64_t)v * cb + (NTAP - 1) + nf) * s16 + k;
#pragma unroll
        for (int t = 0; t < NTAP; ++t) unsafeAtomicAdd(col + (int64_t)t * s16, __int_as_float(r[1 + t]) * x);
    }
}

// The cone footprint of one voxel-view: channel taps h (from the channel
// index), the row mk and row taps gd of slice k, and the chord scale lk, with
// the same fp64 arithmetic as the full cone projectors.
template <int R>
__device__ __forceinline__ bool cone_voxel(const Geo &g, const ViewK &vk, double x, double y, int ncv, int k,
                                           float (&h)[2 * R + 1], double (&gd)[2 * R + 1], int &mk, float &lk) {
    const double xc = x * vk.c, ys = y * vk.s, yc = y * vk.c, xs = x * vk.s;
    const double a = xc + ys;
    const double b = yc - xs;
    const double d = g.sid + b;
    const double drw = d * g.drow;
    const double mr = g.sdd / drw;
    const double mc = g.sdd / (d * g.dch);
    const double f = (mc * a + g.cch + vk.shift) - (double)ncv;
    const double mm = fmax(fabs(y + vk.c * g.sid), fabs(vk.s * g.sid - x));
    const double wch = mc * g.dv * mm / d;
    double hd[2 * R + 1];
    tap_weights_d<R>(f, wch, hd);
#pragma unroll
    for (int t = 0; t < 2 * R + 1; ++t) h[t] = (float)hd[t];
    const double dz = slice_z(g, k) - vk.zsrc;
    const double t0 = mr * dz;
    const double wk = t0 + g.crow;
    const double mkd = rint(wk);
    if (mkd < -R || mkd > g.nr - 1 + R) return false;
    tap_weights_d<R>(wk - mkd, mr * g.dv, gd);
    mk = (int)mkd;
    lk = (float)(g.dv / mm) * sqrtf((float)(d * d + a * a + dz * dz));
    return true;
}

template <int R>
__global__ __launch_bounds__(SW * 64) void cone_back_pixels_kernel(const float *__restrict__ sino,
                                                                   const int32_t *__restrict__ pix, int n,
                                                                   float *__restrict__ cyl,
                                                                   const int32_t *__restrict__ idx,
                                                                   const ViewK *__restrict__ views, Geo g) {
    constexpr int NTAP = 2 * R + 1;
    const int lane = (int)threadIdx.x & 63;
    const int i = (int)blockIdx.x * SW + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (i >= n) return;
    const int np = g.ny * g.nx;
    const int k = (int)blockIdx.y * 64 + lane;
    const int p = listed_pixel(pix, i, np);
    float acc = 0.f;
    if (p >= 0 && k < g.ns) {
        const double x = pix_x(g, p % g.nx), y = pix_y(g, p / g.nx);
        for (int v = 0; v < g.nv; ++v) {
            const int ncv = idx[(int64_t)v * np + p];
            if (ncv < -R || ncv > g.nc - 1 + R) continue;
            float h[NTAP], lk;
            double gd[NTAP];
            int mk;
            if (!cone_voxel<R>(g, views[v], x, y, ncv, k, h, gd, mk, lk)) continue;
            const float *sv = sino + (int64_t)v * g.nr * g.nc;
            float s = 0.f;
#pragma unroll
            for (int sg = 0; sg < NTAP; ++sg) {
                const int m = mk - R + sg;
                if (m < 0 || m >= g.nr) continue;
                float rv = 0.f;
#pragma unroll
                for (int t = 0; t < NTAP; ++t) {
                    const int c = ncv - R + t;
                    if (c >= 0 && c < g.nc) rv = fmaf(h[t], sv[(int64_t)m * g.nc + c], rv);
                }
                s = fmaf(lk * (float)gd[sg], rv, s);
            }
            acc += s;
        }
    }
    if (k < g.ns) cyl[(int64_t)i * g.ns + k] = acc;
}

// Cone forward of a batch: per view the wave first adds its slices' taps into
// an LDS band of the detector (the rows its 64 slices reach times the 2R + 1
// channel taps; a slice's row never decreases with the slice, so the rows in
// range form one band, from the first to the last lane in range), as plain
// read-modify-writes in `stride` passes, each taking the lanes whose slice is
// that pass's residue (the plan's stride puts the rows of one pass on distinct
// rows, as in the full cone forward; LDS float atomics cost tens of times
// more).  Then it adds the band to the sinogram, one global atomic per touched
// cell, the channels of a row adjacent (about 66 requests per view at 256^3
// against 9 per slice when every tap is its own global atomic).  A band taller
// than the LDS holds (magnification far above one) takes the direct form.
constexpr int CPB_CELLS = 1536;         // LDS band cells per wave (rows x taps)

template <int R>
__global__ __launch_bounds__(SW * 64) void cone_forward_pixels_kernel(const int32_t *__restrict__ pix, int n,
                                                                      const float *__restrict__ cyl,
                                                                      float *__restrict__ sino,
                                                                      const int32_t *__restrict__ idx,
                                                                      const ViewK *__restrict__ views, Geo g,
                                                                      int stride) {
    constexpr int NTAP = 2 * R + 1;
    constexpr int PROW = CPB_CELLS / NTAP;      // band rows at most
    __shared__ float band_all[SW * CPB_CELLS];
    const int lane = (int)threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int i = (int)blockIdx.x * SW + wave;
    if (i >= n) return;                             // whole waves only: no workgroup barrier below
    const int np = g.ny * g.nx;
    const int k = (int)blockIdx.y * 64 + lane;
    const int p = listed_pixel(pix, i, np);
    if (p < 0) return;                              // padding contributes nothing
    const bool kin = k < g.ns;
    const float xv = kin ? cyl[(int64_t)i * g.ns + k] : 0.f;
    const double x = pix_x(g, p % g.nx), y = pix_y(g, p / g.nx);
    float *band = band_all + wave * CPB_CELLS;
    for (int e = lane; e < CPB_CELLS; e += 64) band[e] = 0.f;
    for (int v = 0; v < g.nv; ++v) {
        const int ncv = idx[(int64_t)v * np + p];
        if (ncv < -R || ncv > g.nc - 1 + R) continue;   // uniform
        float h[NTAP], lk = 0.f;
        double gd[NTAP];
        int mk = 0;
        const bool ok = kin && cone_voxel<R>(g, views[v], x, y, ncv, k, h, gd, mk, lk);
        const uint64_t act = __builtin_amdgcn_ballot_w64(ok);
        if (!act) continue;
        const int first = (int)__builtin_ctzll(act), last = 63 - (int)__builtin_clzll(act);
        const int lo = max(__builtin_amdgcn_readlane(mk, first) - R, 0);
        const int hi = min(__builtin_amdgcn_readlane(mk, last) + R, g.nr - 1);
        float *sv = sino + (int64_t)v * g.nr * g.nc;
        if (hi - lo + 1 > PROW) {                    // uniform: the direct form
            if (ok) {
#pragma unroll
                for (int sg = 0; sg < NTAP; ++sg) {
                    const int m = mk - R + sg;
                    if (m < 0 || m >= g.nr) continue;
                    const float c = lk * (float)gd[sg] * xv;
#pragma unroll
                    for (int t = 0; t < NTAP; ++t) {
                        const int ch = ncv - R + t;
                        if (ch >= 0 && ch < g.nc && h[t] != 0.f)
                            unsafeAtomicAdd(&sv[(int64_t)m * g.nc + ch], h[t] * c);
                    }
                }
            }
            continue;
        }
        for (int ph = 0; ph < stride; ++ph) {        // uniform
            if (ok && lane % stride == ph) {
#pragma unroll
                for (int sg = 0; sg < NTAP; ++sg) {
                    const int m = mk - R + sg;
                    if (m >= lo && m <= hi) {
                        const float c = lk * (float)gd[sg] * xv;
                        float *cell = band + (m - lo) * NTAP;
#pragma unroll
                        for (int t = 0; t < NTAP; ++t) cell[t] = fmaf(h[t], c, cell[t]);
                    }
                    // a lane's next row is its neighbour's (in the pass) current
                    // one: LDS operations of a wave run in order, and the fence
                    // keeps the compiler from moving the next round up
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                }
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
        }
        // the band's adds are done (LDS operations of a wave complete in
        // order; the fence keeps the compiler from moving the reads up)
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const int cells = (hi - lo + 1) * NTAP;
        for (int e = lane; e < cells; e += 64) {
            const float val = band[e];
            band[e] = 0.f;
            const int m = lo + e / NTAP, ch = ncv - R + e % NTAP;
            if (val != 0.f && ch >= 0 && ch < g.nc) unsafeAtomicAdd(&sv[(int64_t)m * g.nc + ch], val);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
}

#define BPAMD_SUBSET_NTAP(KERN, ...)                                                                          \
    switch (p.ntap) {                                                                                         \
    case 2: hipLaunchKernelGGL((KERN<2>), __VA_ARGS__); break;                                                \
    case 3: hipLaunchKernelGGL((KERN<3>), __VA_ARGS__); break;                                                \
    case 4: hipLaunchKernelGGL((KERN<4>), __VA_ARGS__); break;                                                \
    case 5: hipLaunchKernelGGL((KERN<5>), __VA_ARGS__); break;                                                \
    case 6: hipLaunchKernelGGL((KERN<6>), __VA_ARGS__); break;                                                \
    case 7: hipLaunchKernelGGL((KERN<7>), __VA_ARGS__); break;                                                \
    default: return hipErrorInvalidValue;                                                                     \
    }

#define BPAMD_SUBSET_R(KERN, ...)                                                                             \
    switch (g.radius) {                                                                                       \
    case 1: hipLaunchKernelGGL((KERN<1>), __VA_ARGS__); break;                                                \
    case 2: hipLaunchKernelGGL((KERN<2>), __VA_ARGS__); break;                                                \
    case 3: hipLaunchKernelGGL((KERN<3>), __VA_ARGS__); break;                                                \
    case 4: hipLaunchKernelGGL((KERN<4>), __VA_ARGS__); break;                                                \
    default: return hipErrorInvalidValue;                                                                     \
    }

hipError_t launch_back_pixels(const Plan &p, const float *sino, const int32_t *pix, int n, float *cyl,
                              hipStream_t st) {
    const Geo &g = p.g;
    if (n == 0 || g.ns == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + SW - 1) / SW), (unsigned)((g.ns + 63) / 64));
    if (g.kind == 0) {
        BPAMD_SUBSET_NTAP(par_back_pixels_kernel, grid, dim3(SW * 64), 0, st, sino, pix, n, cyl, p.rec, g)
    } else {
        BPAMD_SUBSET_R(cone_back_pixels_kernel, grid, dim3(SW * 64), 0, st, sino, pix, n, cyl, p.idx, p.views, g)
    }
    return hipGetLastError();
}

hipError_t launch_forward_pixels(const Plan &p, const int32_t *pix, int n, const float *cyl, float *sino,
                                 hipStream_t st) {
    const Geo &g = p.g;
    if (g.kind == 0) {
        hipError_t e = launch_fill_zero(p.facc, (int64_t)g.nv * p.fwd_cb * p.fwd_s16, st);
        if (e != hipSuccess) return e;
        if (n > 0) {
            const dim3 grid((unsigned)((n + SW - 1) / SW), (unsigned)((g.ns + 63) / 64));
            BPAMD_SUBSET_NTAP(par_forward_pixels_kernel, grid, dim3(SW * 64), 0, st, pix, n, cyl, p.facc, p.rec, g,
                              p.fwd_cb, p.fwd_s16)
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return launch_par_unpack(p, sino, st);
    }
    hipError_t e = launch_fill_zero(sino, (int64_t)g.nv * g.nr * g.nc, st);
    if (e != hipSuccess || n == 0) return e;
    const dim3 grid((unsigned)((n + SW - 1) / SW), (unsigned)((g.ns + 63) / 64));
    BPAMD_SUBSET_R(cone_forward_pixels_kernel, grid, dim3(SW * 64), 0, st, pix, n, cyl, sino, p.idx, p.views, g,
                   p.cone_stride)
    return hipGetLastError();
}

}  // namespace bpamd
