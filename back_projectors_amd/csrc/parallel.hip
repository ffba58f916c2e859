// Parallel-beam projector pair on gfx950.
//
// Detector row r sees slice r only (MBIRJAX "Projector kernels" page,
// paragraph "Geometry decides whether a slice can stream"), so every
// (view, pixel) pair has one set of channel taps shared by all slices of the
// voxel cylinder.  Those taps -- the first channel n_f and NTAP fp32 weights --
// come from the tap records the creation pass wrote in fp64; the projectors
// do no geometry arithmetic and never round a coordinate.
//
// Back (gather; paragraph "Forward scatters, back gathers"): a workgroup owns
// a BT x BT pixel tile and a chunk of SL slices; lanes are pixels, each with
// SL register accumulators.  Per view the sinogram cells the tile can reach
// (a channel window of SL rows) are staged in LDS, channel-major with slices
// fastest, by coalesced reads; each lane then reads its NTAP taps per slice
// (adjacent channels, so pairs come in one ds_read2) and accumulates.  Every
// voxel is written once and nothing collides.
//
// Forward (scatter with no colliding LDS or register updates): a workgroup
// owns an FTX x FTY pixel tile and a chunk of 64 slices; lanes are slices and
// each wave works on one view at a time.  The tile's voxels sit in LDS.  A
// wave walks the tile's pixels in the order of their first tap channel, which
// the creation pass fixed per (view, tile) together with how far the walk's
// channel window moves after each pixel, so the walk has no comparisons: NTAP
// registers hold the current channels and a channel the walk leaves behind is
// stored once into the wave's own LDS window.  The window is then added to the
// sinogram with coalesced global atomics, one per cell per view and tile.
// Float atomics in LDS are avoided on purpose: on gfx950 they cost tens of
// times a plain read-modify-write.
#include "launch.h"

namespace bpamd {

template <int SL, int NTAP, int NCG>
__global__ __launch_bounds__(BT *BT) void par_back_kernel(const float *__restrict__ sino,
                                                           float *__restrict__ recon,
                                                           const int32_t *__restrict__ rec,
                                                           const int4 *__restrict__ wtab, Geo g, int nwcap) {
    constexpr int SLP = SL + 1;           // LDS pitch of one channel column
    constexpr int NREC = 1 + NTAP;
    constexpr int RPT = (SL + 7) / 8;     // staged rows per thread: 8 row groups of 32 lanes
    extern __shared__ float lds[];        // two windows of [nwcap][SLP], slices fastest

    const int tiles_x = (g.nx + BT - 1) / BT;
    const int ntiles = tiles_x * ((g.ny + BT - 1) / BT);
    const int tile = (int)blockIdx.x;
    const int tj0 = (tile % tiles_x) * BT;
    const int ti0 = (tile / tiles_x) * BT;
    const int k0 = (int)blockIdx.y * SL;
    const int nk = min(SL, g.ns - k0);

    const int i = ti0 + (int)threadIdx.x / BT;
    const int j = tj0 + (int)threadIdx.x % BT;
    const bool valid = (i < g.ny) && (j < g.nx);
    const int np = g.ny * g.nx;
    const int p = valid ? i * g.nx + j : 0;
    const int clane = (int)threadIdx.x & 31;       // staging: channel within a 32-wide group
    const int rgrp = (int)threadIdx.x >> 5;        // staging: rows rgrp, rgrp + 8, ...

    // the sinogram cells of one view the tile can reach, into registers
    auto load_view = [&](int v, const int4 &w, float (&st)[NCG][RPT]) {
        const float *base = sino + ((int64_t)v * g.nr + k0) * g.nc;
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) {
            const int c = clane + 32 * cg;
            const int n = w.x + c;
            const bool cok = c < w.y && n >= 0 && n < g.nc;
#pragma unroll
            for (int u = 0; u < RPT; ++u) {
                const int r = rgrp + 8 * u;
                st[cg][u] = (cok && r < nk) ? base[(int64_t)r * g.nc + n] : 0.f;
            }
        }
    };
    auto store_view = [&](float *buf, const float (&st)[NCG][RPT]) {
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) {
            const int c = clane + 32 * cg;
            if (c < nwcap) {
#pragma unroll
                for (int u = 0; u < RPT; ++u) {
                    const int r = rgrp + 8 * u;
                    if (r < SL) buf[c * SLP + r] = st[cg][u];
                }
            }
        }
    };
    auto load_taps = [&](int v, int &nf, float (&w)[NTAP]) {
        const int32_t *r = rec + ((int64_t)v * np + p) * NREC;
        nf = valid ? r[0] : INT32_MAX;
#pragma unroll
        for (int t = 0; t < NTAP; ++t) w[t] = valid ? __int_as_float(r[1 + t]) : 0.f;
    };

    float acc[SL];
#pragma unroll
    for (int k = 0; k < SL; ++k) acc[k] = 0.f;
    if (g.nv == 0) return;

    // double-buffered pipeline: view v + 1 is fetched while view v is gathered
    float st[NCG][RPT];
    int4 wcur = wtab[tile];
    load_view(0, wcur, st);
    store_view(lds, st);
    int nf;
    float w[NTAP];
    load_taps(0, nf, w);
    __syncthreads();
    for (int v = 0; v < g.nv; ++v) {
        const float *buf = lds + (v & 1) * nwcap * SLP;
        const bool more = v + 1 < g.nv;
        int4 wnext = wcur;
        float nst[NCG][RPT];
        int nnf = INT32_MAX;
        float nw[NTAP];
        if (more) {
            wnext = wtab[(int64_t)(v + 1) * ntiles + tile];
            load_view(v + 1, wnext, nst);
            load_taps(v + 1, nnf, nw);
        }
        if (nf != INT32_MAX && wcur.y > 0) {
            const float *col = buf + (nf - wcur.x) * SLP;
#pragma unroll
            for (int k = 0; k < SL; ++k) {
                float sacc = acc[k];
#pragma unroll
                for (int t = 0; t < NTAP; ++t) sacc = fmaf(w[t], col[t * SLP + k], sacc);
                acc[k] = sacc;
            }
        }
        if (more) {
            store_view(lds + ((v + 1) & 1) * nwcap * SLP, nst);
            wcur = wnext;
            nf = nnf;
#pragma unroll
            for (int t = 0; t < NTAP; ++t) w[t] = nw[t];
        }
        __syncthreads();
    }
    if (valid) {
        float *out = recon + (int64_t)p * g.ns + k0;
#pragma unroll
        for (int k = 0; k < SL; ++k)
            if (k < nk) out[k] = acc[k];
    }
}

template <int NTAP, int NREC>
__global__ __launch_bounds__(FW * 64) void par_forward_kernel(const float *__restrict__ recon,
                                                               float *__restrict__ sino,
                                                               const int32_t *__restrict__ wrec,
                                                               const int4 *__restrict__ wtab, Geo g, int nwcap,
                                                               int vsplit) {
    constexpr int TP = FTX * FTY;         // pixels per tile, one walk record per lane
    static_assert(TP == 64, "the walk keeps the tile's records one per lane");
    constexpr int XP = 64;                // LDS pitch of one voxel cylinder chunk
    constexpr int WP = 65;                // LDS pitch of one window channel (slices fastest)
    extern __shared__ float lds[];
    float *xt = lds;                                   // [TP + 1][XP]; row TP stays zero
    const int lane = (int)threadIdx.x & 63;
    // wave index, made visibly uniform so per-view work stays on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    float *win = lds + (TP + 1) * XP + wave * nwcap * WP;   // this wave's window [nwcap][WP]

    const int tiles_x = (g.nx + FTX - 1) / FTX;
    const int ntiles = tiles_x * ((g.ny + FTY - 1) / FTY);
    const int tile = (int)blockIdx.x;
    const int tj0 = (tile % tiles_x) * FTX;
    const int ti0 = (tile / tiles_x) * FTY;
    const int k0 = (int)blockIdx.y * 64;
    const int nk = min(64, g.ns - k0);

    // the tile's voxels, one 64-slice chunk per pixel, plus a zero row
    for (int e = (int)threadIdx.x; e < (TP + 1) * 64; e += FW * 64) {
        const int q = e >> 6, k = e & 63;
        const int i = ti0 + q / FTX, j = tj0 + q % FTX;
        float val = 0.f;
        if (q < TP && i < g.ny && j < g.nx && k < nk) val = recon[(int64_t)(i * g.nx + j) * g.ns + k0 + k];
        xt[q * XP + k] = val;
    }
    for (int e = lane; e < nwcap * WP; e += 64) win[e] = 0.f;
    __syncthreads();

    const int vper = (g.nv + vsplit - 1) / vsplit;
    const int vbeg = (int)blockIdx.z * vper;
    const int vend = min(g.nv, vbeg + vper);
    const int cnt = vend - vbeg;
    // staggered start, so that tiles along one ray reach a view at different times
    const int start = cnt > 0 ? (int)((blockIdx.x * 37u + blockIdx.y * 11u) % (unsigned)cnt) : 0;
    auto view_of = [&](int it) {
        int v = vbeg + start + it;
        return v >= vend ? v - cnt : v;
    };
    // the (view, tile) records: lane l holds walk step l
    auto load_records = [&](int v, int (&ra)[NREC]) {
        const int32_t *base = wrec + ((int64_t)v * ntiles + tile) * TP * NREC;
#pragma unroll
        for (int t = 0; t < NREC; ++t) ra[t] = base[lane * NREC + t];
    };

    int ra[NREC];
    int it = wave;
    int v = it < cnt ? view_of(it) : 0;
    if (it < cnt) load_records(v, ra);
    for (; it < cnt; it += FW) {
        const int vc = v;
        int na[NREC];
        if (it + FW < cnt) {              // prefetch the next view's records
            v = view_of(it + FW);
            load_records(v, na);
        }
        const int4 w4 = wtab[(int64_t)vc * ntiles + tile];
        Window wd;
        wd.n0 = w4.x;
        wd.nw = w4.y;
        const int p0 = __builtin_amdgcn_readlane(ra[0], 0);
        if (wd.nw > 0 && (p0 & 255) != TP) {
            // acc[t] holds channel cur + t; the records say when to move on, and
            // a channel left behind is finished, so it is stored, not added
            float acc[NTAP];
#pragma unroll
            for (int t = 0; t < NTAP; ++t) acc[t] = 0.f;
            int cur = (p0 >> 11) - 65536;
            auto store = [&](int n, float a) { win[(n - wd.n0) * WP + lane] = a; };
#pragma unroll
            for (int s = 0; s < TP; s += 4) {
                int pk[4];
                float w[4][NTAP], xv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    pk[u] = __builtin_amdgcn_readlane(ra[0], s + u);
#pragma unroll
                    for (int t = 0; t < NTAP; ++t) w[u][t] = __int_as_float(__builtin_amdgcn_readlane(ra[1 + t], s + u));
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) xv[u] = xt[(pk[u] & 255) * XP + lane];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
#pragma unroll
                    for (int t = 0; t < NTAP; ++t) acc[t] = fmaf(w[u][t], xv[u], acc[t]);
                    const int adv = (pk[u] >> 8) & 7;
                    if (adv != 0) {
                        if (adv == 7) {
#pragma unroll
                            for (int t = 0; t < NTAP; ++t) {
                                store(cur + t, acc[t]);
                                acc[t] = 0.f;
                            }
                            if (s + u + 1 < TP) cur = (__builtin_amdgcn_readlane(ra[0], s + u + 1) >> 11) - 65536;
                        } else {
#pragma unroll
                            for (int t = 0; t < NTAP - 1; ++t)
                                if (t < adv) store(cur + t, acc[t]);
#pragma unroll
                            for (int t = 0; t < NTAP; ++t) {
                                float nv = 0.f;
#pragma unroll
                                for (int dd = 1; dd < NTAP; ++dd)
                                    if (adv == dd && t + dd < NTAP) nv = acc[t + dd];
                                acc[t] = nv;
                            }
                            cur += adv;
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < NTAP; ++t) store(cur + t, acc[t]);
            // add the window to the sinogram: lanes run along channels, coalesced
            const int total = wd.nw * nk;
            const float rnw = 1.0f / (float)wd.nw;
            for (int e = lane; e < total; e += 64) {
                const int k = (int)(((float)e + 0.5f) * rnw);   // exact: e < 2^22 and nw is small
                const int c = e - k * wd.nw;
                const float val = win[c * WP + k];
                win[c * WP + k] = 0.f;
                const int n = wd.n0 + c;
                if (val != 0.f && n >= 0 && n < g.nc)
                    unsafeAtomicAdd(&sino[((int64_t)vc * g.nr + (k0 + k)) * g.nc + n], val);
            }
        }
#pragma unroll
        for (int t = 0; t < NREC; ++t) ra[t] = na[t];
    }
}

template <int SL, int NTAP>
static hipError_t par_back_t(const Plan &p, const float *sino, float *recon, hipStream_t st) {
    const Geo &g = p.g;
    const int tiles = ((g.nx + BT - 1) / BT) * ((g.ny + BT - 1) / BT);
    const int chunks = (g.ns + SL - 1) / SL;
    if (p.back_ncg == 1)
        hipLaunchKernelGGL((par_back_kernel<SL, NTAP, 1>), dim3(tiles, chunks), dim3(BT * BT), p.back_lds, st, sino,
                           recon, p.rec, p.bwin, g, p.back_nwcap);
    else
        hipLaunchKernelGGL((par_back_kernel<SL, NTAP, 2>), dim3(tiles, chunks), dim3(BT * BT), p.back_lds, st, sino,
                           recon, p.rec, p.bwin, g, p.back_nwcap);
    return hipGetLastError();
}

template <int NTAP>
static hipError_t par_fwd_t(const Plan &p, const float *recon, float *sino, hipStream_t st) {
    const Geo &g = p.g;
    const int tiles = ((g.nx + FTX - 1) / FTX) * ((g.ny + FTY - 1) / FTY);
    const int chunks = (g.ns + 63) / 64;
    constexpr int NREC = NTAP <= 3 ? 4 : 8;
    hipLaunchKernelGGL((par_forward_kernel<NTAP, NREC>), dim3(tiles, chunks, p.fwd_vsplit), dim3(FW * 64), p.fwd_lds,
                       st, recon, sino, p.wrec, p.fwin, g, p.fwd_nwcap, p.fwd_vsplit);
    return hipGetLastError();
}

#define BPAMD_DISPATCH_NTAP(FN, ...)                                                                          \
    switch (p.ntap) {                                                                                         \
    case 2: return FN<2>(__VA_ARGS__);                                                                        \
    case 3: return FN<3>(__VA_ARGS__);                                                                        \
    case 4: return FN<4>(__VA_ARGS__);                                                                        \
    case 5: return FN<5>(__VA_ARGS__);                                                                        \
    case 6: return FN<6>(__VA_ARGS__);                                                                        \
    case 7: return FN<7>(__VA_ARGS__);                                                                        \
    default: return hipErrorInvalidValue;                                                                     \
    }

template <int SL>
static hipError_t par_back_sl(const Plan &p, const float *sino, float *recon, hipStream_t st) {
    switch (p.ntap) {
    case 2: return par_back_t<SL, 2>(p, sino, recon, st);
    case 3: return par_back_t<SL, 3>(p, sino, recon, st);
    case 4: return par_back_t<SL, 4>(p, sino, recon, st);
    case 5: return par_back_t<SL, 5>(p, sino, recon, st);
    case 6: return par_back_t<SL, 6>(p, sino, recon, st);
    case 7: return par_back_t<SL, 7>(p, sino, recon, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_par_back(const Plan &p, const float *sino, float *recon, hipStream_t st) {
    switch (p.back_sl) {
    case 8: return par_back_sl<8>(p, sino, recon, st);
    case 16: return par_back_sl<16>(p, sino, recon, st);
    case 32: return par_back_sl<32>(p, sino, recon, st);
    case 64: return par_back_sl<64>(p, sino, recon, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_par_forward(const Plan &p, const float *recon, float *sino, hipStream_t st) {
    BPAMD_DISPATCH_NTAP(par_fwd_t, p, recon, sino, st)
}

// Dynamic LDS above the default limit needs the opt-in attribute; called once
// per kernel by the planner when a plan asks for more.
hipError_t par_forward_allow_lds(int ntap, size_t bytes) {
    const void *f = nullptr;
    switch (ntap) {
    case 2: f = (const void *)par_forward_kernel<2, 4>; break;
    case 3: f = (const void *)par_forward_kernel<3, 4>; break;
    case 4: f = (const void *)par_forward_kernel<4, 8>; break;
    case 5: f = (const void *)par_forward_kernel<5, 8>; break;
    case 6: f = (const void *)par_forward_kernel<6, 8>; break;
    case 7: f = (const void *)par_forward_kernel<7, 8>; break;
    default: return hipErrorInvalidValue;
    }
    return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace bpamd
