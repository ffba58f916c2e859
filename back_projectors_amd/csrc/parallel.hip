// Parallel-beam projector pair on gfx950.
//
// Detector row r sees slice r only (MBIRJAX "Projector kernels" page,
// paragraph "Geometry decides whether a slice can stream"), so every
// (view, pixel) pair has one set of channel taps shared by all slices of the
// voxel cylinder.  Both kernels give each lane one pixel and loop over a chunk
// of SL slices held in registers, so the fp64 tap weights of a (view, pixel)
// pair are computed once per lane and reused SL times.
//
// Back (gather; paragraph "Forward scatters, back gathers"): a workgroup owns
// a BT x BT pixel tile and one slice chunk.  For each view it stages the
// sinogram cells the tile can reach (a channel window, SL rows) in LDS with
// coalesced reads, then every lane gathers its taps from LDS into per-slice
// register accumulators.  Each voxel is written once; nothing collides.
//
// Forward (scatter without colliding global atomics): a workgroup owns an
// FT x FT tile, keeps the tile's voxels in registers and, for each view of its
// range, adds the taps into an LDS-private channel window.  Lanes of a 32-lane
// half cover one tile row (or column, whichever runs across the rays), so in
// one LDS atomic at most two lanes share an address.  The window is then added
// to the sinogram with one coalesced global atomic per nonzero cell, i.e.
// about 1.3/FT atomics per voxel-view instead of one per tap.
#include "launch.h"
#include "taps.h"

namespace bpamd {

template <int SL, int R>
__global__ __launch_bounds__(BT *BT) void par_back_kernel(const float *__restrict__ sino,
                                                           float *__restrict__ recon,
                                                           const int32_t *__restrict__ idx,
                                                           const ViewK *__restrict__ views, Geo g) {
    constexpr int NT = BT * BT;
    constexpr int SLP = SL + 1;           // LDS pitch of one channel column
    extern __shared__ float win[];        // [nwcap][SLP], slices fastest

    const int tiles_x = (g.nx + BT - 1) / BT;
    const int tj0 = (int)(blockIdx.x % tiles_x) * BT;
    const int ti0 = (int)(blockIdx.x / tiles_x) * BT;
    const int tj1 = min(tj0 + BT, g.nx) - 1;
    const int ti1 = min(ti0 + BT, g.ny) - 1;
    const int k0 = (int)blockIdx.y * SL;
    const int nk = min(SL, g.ns - k0);

    const int i = ti0 + (int)threadIdx.x / BT;
    const int j = tj0 + (int)threadIdx.x % BT;
    const bool valid = (i < g.ny) && (j < g.nx);
    const int np = g.ny * g.nx;
    const int p = valid ? i * g.nx + j : 0;
    const double x = pix_x(g, j), y = pix_y(g, i);

    float acc[SL];
#pragma unroll
    for (int k = 0; k < SL; ++k) acc[k] = 0.f;

    const int lane = (int)threadIdx.x & 31;
    const int grp = (int)threadIdx.x >> 5;

    for (int v = 0; v < g.nv; ++v) {
        const ViewK vk = views[v];
        const Window wd = tile_window(g, vk, ti0, ti1, tj0, tj1, k0, k0 + nk - 1);
        if (wd.nw <= 0) continue;          // the tile misses the detector in this view
        __syncthreads();
        // stage rows k0..k0+nk-1, channels n0..n0+nw-1 (zeros off the detector)
        for (int r = grp; r < SL; r += NT / 32) {
            const float *srow = sino + ((int64_t)v * g.nr + (k0 + r)) * g.nc;
            for (int c = lane; c < wd.nw; c += 32) {
                const int n = wd.n0 + c;
                float val = 0.f;
                if (r < nk && n >= 0 && n < g.nc) val = srow[n];
                win[c * SLP + r] = val;
            }
        }
        __syncthreads();
        const int ncv = valid ? idx[(int64_t)v * np + p] : 0;
        if (valid && ncv >= -R && ncv <= g.nc - 1 + R) {
            const double u = x * vk.cd + y * vk.sd + vk.u0;
            float w[2 * R + 1];
            tap_weights<R>(u - (double)ncv, vk.W, vk.L, w);
            const float *col = win + (ncv - R - wd.n0) * SLP;
#pragma unroll
            for (int k = 0; k < SL; ++k) {
                float s = acc[k];
#pragma unroll
                for (int t = 0; t <= 2 * R; ++t) s = fmaf(w[t], col[t * SLP + k], s);
                acc[k] = s;
            }
        }
    }
    if (valid) {
        float *out = recon + (int64_t)p * g.ns + k0;
#pragma unroll
        for (int k = 0; k < SL; ++k)
            if (k < nk) out[k] = acc[k];
    }
}

template <int SL, int R>
__global__ __launch_bounds__(FT *FT) void par_forward_kernel(const float *__restrict__ recon,
                                                              float *__restrict__ sino,
                                                              const int32_t *__restrict__ idx,
                                                              const ViewK *__restrict__ views, Geo g,
                                                              int nwcap, int vsplit) {
    constexpr int NT = FT * FT;
    constexpr int SLP = SL + 1;
    extern __shared__ float win[];        // two buffers of [nwcap][SLP]

    const int tiles_x = (g.nx + FT - 1) / FT;
    const int tj0 = (int)(blockIdx.x % tiles_x) * FT;
    const int ti0 = (int)(blockIdx.x / tiles_x) * FT;
    const int tj1 = min(tj0 + FT, g.nx) - 1;
    const int ti1 = min(ti0 + FT, g.ny) - 1;
    const int k0 = (int)blockIdx.y * SL;
    const int nk = min(SL, g.ns - k0);
    const int np = g.ny * g.nx;

    // lane -> pixel in the two orientations: along a row, or along a column
    const int a = (int)threadIdx.x % FT, b = (int)threadIdx.x / FT;
    const int ir = ti0 + b, jr = tj0 + a;     // row mode
    const int ic = ti0 + a, jc = tj0 + b;     // column mode
    const bool vr = ir < g.ny && jr < g.nx;
    const bool vc = ic < g.ny && jc < g.nx;
    float xr[SL], xc[SL];
    {
        const float *pr = recon + (int64_t)(vr ? ir * g.nx + jr : 0) * g.ns + k0;
        const float *pc = recon + (int64_t)(vc ? ic * g.nx + jc : 0) * g.ns + k0;
#pragma unroll
        for (int k = 0; k < SL; ++k) {
            xr[k] = (vr && k < nk) ? pr[k] : 0.f;
            xc[k] = (vc && k < nk) ? pc[k] : 0.f;
        }
    }

    const int cap = nwcap * SLP;
    for (int e = (int)threadIdx.x; e < 2 * cap; e += NT) win[e] = 0.f;
    __syncthreads();

    // this block's view range, visited from a staggered start so that tiles
    // along one ray do not hit the same sinogram rows at the same time
    const int vper = (g.nv + vsplit - 1) / vsplit;
    const int vbeg = (int)blockIdx.z * vper;
    const int vend = min(g.nv, vbeg + vper);
    const int cnt = vend - vbeg;
    const int start = cnt > 0 ? (int)((blockIdx.x * 7u + blockIdx.y * 3u) % (unsigned)cnt) : 0;

    for (int it = 0; it < cnt; ++it) {
        int v = vbeg + start + it;
        if (v >= vend) v -= cnt;
        const ViewK vk = views[v];
        const Window wd = tile_window(g, vk, ti0, ti1, tj0, tj1, k0, k0 + nk - 1);
        float *buf = win + (it & 1) * cap;
        const bool rowmode = fabs(vk.cd) >= fabs(vk.sd);
        const int i = rowmode ? ir : ic, j = rowmode ? jr : jc;
        const bool valid = (rowmode ? vr : vc) && wd.nw > 0;
        const int ncv = valid ? idx[(int64_t)v * np + i * g.nx + j] : 0;
        if (valid && ncv >= -R && ncv <= g.nc - 1 + R) {
            const double u = pix_x(g, j) * vk.cd + pix_y(g, i) * vk.sd + vk.u0;
            float w[2 * R + 1];
            tap_weights<R>(u - (double)ncv, vk.W, vk.L, w);
            float *col = buf + (ncv - R - wd.n0) * SLP;
            if (rowmode) {
#pragma unroll
                for (int k = 0; k < SL; ++k)
#pragma unroll
                    for (int t = 0; t <= 2 * R; ++t) atomicAdd(&col[t * SLP + k], w[t] * xr[k]);
            } else {
#pragma unroll
                for (int k = 0; k < SL; ++k)
#pragma unroll
                    for (int t = 0; t <= 2 * R; ++t) atomicAdd(&col[t * SLP + k], w[t] * xc[k]);
            }
        }
        __syncthreads();
        // flush: rows k (slices), channels n0..n0+nw-1; clear as we go
        const int lane = (int)threadIdx.x & 31;
        for (int r = (int)threadIdx.x >> 5; r < nk; r += NT / 32) {
            float *srow = sino + ((int64_t)v * g.nr + (k0 + r)) * g.nc;
            for (int c = lane; c < wd.nw; c += 32) {
                const float val = buf[c * SLP + r];
                buf[c * SLP + r] = 0.f;
                const int n = wd.n0 + c;
                if (val != 0.f && n >= 0 && n < g.nc) unsafeAtomicAdd(&srow[n], val);
            }
        }
    }
}

template <int SL, int R>
static hipError_t par_back_t(const Plan &p, const float *sino, float *recon, hipStream_t st) {
    const Geo &g = p.g;
    const int tiles = ((g.nx + BT - 1) / BT) * ((g.ny + BT - 1) / BT);
    const int chunks = (g.ns + SL - 1) / SL;
    hipLaunchKernelGGL((par_back_kernel<SL, R>), dim3(tiles, chunks), dim3(BT * BT), p.back_lds, st, sino, recon,
                       p.idx, p.views, g);
    return hipGetLastError();
}

template <int SL, int R>
static hipError_t par_fwd_t(const Plan &p, const float *recon, float *sino, hipStream_t st) {
    const Geo &g = p.g;
    const int tiles = ((g.nx + FT - 1) / FT) * ((g.ny + FT - 1) / FT);
    const int chunks = (g.ns + SL - 1) / SL;
    hipLaunchKernelGGL((par_forward_kernel<SL, R>), dim3(tiles, chunks, p.fwd_vsplit), dim3(FT * FT), p.fwd_lds,
                       st, recon, sino, p.idx, p.views, g, p.fwd_nwcap, p.fwd_vsplit);
    return hipGetLastError();
}

#define BPAMD_DISPATCH_R(FN, SLV, ...)                         \
    switch (p.g.radius) {                                      \
    case 1: return FN<SLV, 1>(__VA_ARGS__);                    \
    case 2: return FN<SLV, 2>(__VA_ARGS__);                    \
    case 3: return FN<SLV, 3>(__VA_ARGS__);                    \
    case 4: return FN<SLV, 4>(__VA_ARGS__);                    \
    default: return hipErrorInvalidValue;                      \
    }

hipError_t launch_par_back(const Plan &p, const float *sino, float *recon, hipStream_t st) {
    switch (p.back_sl) {
    case 8: BPAMD_DISPATCH_R(par_back_t, 8, p, sino, recon, st)
    case 16: BPAMD_DISPATCH_R(par_back_t, 16, p, sino, recon, st)
    case 32: BPAMD_DISPATCH_R(par_back_t, 32, p, sino, recon, st)
    case 64: BPAMD_DISPATCH_R(par_back_t, 64, p, sino, recon, st)
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_par_forward(const Plan &p, const float *recon, float *sino, hipStream_t st) {
    switch (p.fwd_sl) {
    case 8: BPAMD_DISPATCH_R(par_fwd_t, 8, p, recon, sino, st)
    case 16: BPAMD_DISPATCH_R(par_fwd_t, 16, p, recon, sino, st)
    case 32: BPAMD_DISPATCH_R(par_fwd_t, 32, p, recon, sino, st)
    default: return hipErrorInvalidValue;
    }
}

}  // namespace bpamd
