// Flat-detector cone-beam projector pair (circular and helical orbits) on gfx950.
//
// In the cone geometry one slice spreads over a band of detector rows, and
// the row of a voxel is an affine function of its slice index, so a kernel
// that holds a whole voxel cylinder walks up the slices and recomputes the row
// as it goes; the taps form a 3x3 block (MBIRJAX "Projector kernels" page,
// "The cone back kernel: a fused vertical fan"; "Sharding overview" page,
// "Why cone beam projects whole cylinders").
//
// Lanes are pixels (a tile of them per workgroup), each lane walks a chunk of
// SL slices.  Per (view, pixel) the lane computes, in fp64, the channel
// taps and the row magnification; per slice it computes the row coordinate
// w_k = Mr dz_k + c_row (rounded to the tap row exactly as the reference
// model does, product then sum, no contraction), the row taps and the chord
// scale L_k.  The sinogram window a tile and slice chunk can reach in one view
// is staged in LDS (rows fastest); the forward adds into an LDS-private window
// and flushes it with coalesced global atomics, exactly as the parallel pair.
#include <type_traits>

#include "launch.h"
#include "taps.h"

#pragma clang fp contract(off)

namespace bpamd {

// Word 3 of a raw buffer resource on gfx950: 32-bit data format, no swizzle,
// no index stride (the loads below address bytes directly).
constexpr int kRawDwordRsrc = 0x00020000;
// A byte offset past any buffer range the back sets up (each is one view of
// the sinogram, below 2^31 bytes): the range check makes its load a zero.
constexpr unsigned kOffRange = 0x80000000u;
// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt at their maxima):
// every global load of this wave, the direct global-to-LDS ones included, done.
constexpr int kWaitVm0 = 0x0F70;

// Per (view, pixel) quantities of the flat cone.
struct ConeVP {
    double f;      // u - n_c
    double mr;     // SDD / (d drow): row magnification in rows per voxel unit
    double wch;    // channel footprint width
    double lsc;    // dv / M
    double r2;     // d^2 + a^2 (squared in-plane source distance)
};

__device__ __forceinline__ ConeVP cone_vp(const Geo &g, const ViewK &vk, double x, double y, int ncv) {
    ConeVP o;
    const double xc = x * vk.c, ys = y * vk.s, yc = y * vk.c, xs = x * vk.s;
    const double a = xc + ys;
    const double b = yc - xs;
    const double d = g.sid + b;
    const double drw = d * g.drow;
    o.mr = g.sdd / drw;
    const double mc = g.sdd / (d * g.dch);
    o.f = (mc * a + g.cch + vk.shift) - (double)ncv;
    const double mm = fmax(fabs(y + vk.c * g.sid), fabs(vk.s * g.sid - x));
    o.wch = mc * g.dv * mm / d;
    o.lsc = g.dv / mm;
    o.r2 = d * d + a * a;
    return o;
}

// The same per (view, pixel) quantities for the back projection, with two
// fp64 divisions instead of four: the row magnification stays the exact
// quotient (the back's fp64 row placement uses it), while the channel
// magnification and footprint width take one reciprocal of the source
// distance (a relative error of about 1e-16 that only moves tap values), and
// the chord factor dv / M, which only enters fp32 weights, takes the fp32
// hardware reciprocal (about 1e-7 relative).
struct ConeVPB {
    double f, mr, wch, r2;
    float lsc;
};

__device__ __forceinline__ ConeVPB cone_vp_back(const Geo &g, const ViewK &vk, double x, double y, int ncv) {
    ConeVPB o;
    const double xc = x * vk.c, ys = y * vk.s, yc = y * vk.c, xs = x * vk.s;
    const double a = xc + ys;
    const double b = yc - xs;
    const double d = g.sid + b;
    o.mr = g.sdd / (d * g.drow);
    const double rd = 1.0 / d;
    const double mc = (g.sdd / g.dch) * rd;
    o.f = (mc * a + g.cch + vk.shift) - (double)ncv;
    const double mm = fmax(fabs(y + vk.c * g.sid), fabs(vk.s * g.sid - x));
    o.wch = mc * g.dv * mm * rd;
    o.lsc = (float)g.dv * __builtin_amdgcn_rcpf((float)mm);   // hardware reciprocal, about 1 ulp
    o.r2 = d * d + a * a;
    return o;
}

// Back: lanes are the pixels of a BT x BT tile, each with SL slice
// accumulators.  Per view the sinogram window the tile and slice chunk can reach
// is staged in LDS, double buffered: view v + 1's window rows are copied from
// the sinogram straight into LDS (one direct global-to-LDS load per window row
// and 64 channels, no registers held) while view v is gathered, and one wait
// and barrier per view publishes them.  The window keeps the sinogram's
// layout, channels fastest, with an odd channel pitch PC fixed at compile time,
// so the (2R+1)^2 tap reads of a slice share one address with immediate
// offsets, and lanes on one row but different channels hit different banks.
// The per-view constants and window travel as one register (lanes 0-17 the
// view's 18 dwords, lanes 18-21 its window) fetched two views ahead; the
// channel index of each lane's pixel one view ahead.
//
// Per (view, pixel) the row coordinate w_k = Mr dz_k + c_row is affine in the
// slice index, so it is carried in 32.32 fixed point (from the fp64 value at
// the chunk's first slice, advanced by one 64-bit add per slice: about 4e-9
// of a row off after 32 slices, 6e-9 after 48): the high word is the tap row
// m_k = floor(w_k + 1/2) (plus R + 1) and the low word the position inside
// it.  A row chosen differently at an exact half (round half up here, half to
// even in the model) moves no weight while the footprint is no wider than 2R
// rows: every tap is the overlap of one cell with the footprint.  The row taps
// run in fp32 (clamped edges by v_med3).  Two cases take the row in fp64, in
// the model's operation order, with each tap the model's own fp64 overlap of
// its cell with the footprint (exact for thin taps): a tap cell off the
// detector's top or bottom edge, and a footprint wider than 2R rows (its
// outermost taps cut it, so the tap row must be the model's even at an exact
// half).  The chord scale
// sqrt(d^2 + a^2 + dz^2) runs in fp32, with the per-pixel factor dv / M folded
// into the channel taps.
template <int SL, int R, int POW, int PC>
__global__ __launch_bounds__(BT *BT, 3) void cone_back_kernel(const float *__restrict__ sino,
                                                            float *__restrict__ recon,
                                                            const int32_t *__restrict__ idx,
                                                            const ViewK *__restrict__ views,
                                                            const int4 *__restrict__ wtab, Geo g, int nrcap) {
    constexpr int NT = BT * BT;
    constexpr int NTAP = 2 * R + 1;
    static_assert(PC % 2 == 1, "odd channel pitch");
    extern __shared__ float win[];        // two windows of [nrcap][PC], channels fastest
    static_assert(sizeof(ViewK) == 72, "ViewK is read as 18 dwords");

    const int tiles_x = (g.nx + BT - 1) / BT;
    const int ntiles = tiles_x * ((g.ny + BT - 1) / BT);
    const int nch = (g.ns + SL - 1) / SL;
    int tile, chunk;
    xcd_work_item_blocked((int)gridDim.x, (int)gridDim.y, tiles_x, (g.ny + BT - 1) / BT, tile, chunk);
    const int tj0 = (tile % tiles_x) * BT;
    const int ti0 = (tile / tiles_x) * BT;
    const int k0 = chunk * SL;
    const int nk = min(SL, g.ns - k0);
    const int tid = (int)threadIdx.x;
    const int wl = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wsz = nrcap * PC;           // floats per window
    // rows m with m + R in [0, nr - 1 + 2R] have a tap on the detector; those
    // with m + R in [2R, nr - 1] have every tap on it (none if ib < 0)
    const unsigned rlim = (unsigned)(g.nr - 1 + 2 * R);
    const int ib = g.nr - 1 - 2 * R;

    const int i = ti0 + tid / BT;
    const int j = tj0 + tid % BT;
    const bool valid = (i < g.ny) && (j < g.nx);
    const int np = g.ny * g.nx;
    const int p = valid ? i * g.nx + j : 0;
    const double x = pix_x(g, j), y = pix_y(g, i);

    float acc[SL];
#pragma unroll
    for (int k = 0; k < SL; ++k) acc[k] = 0.f;

    auto fetch_view = [&](int v, uint32_t &pv) {
        const uint32_t *vkd = reinterpret_cast<const uint32_t *>(views + v);
        const uint32_t *wd = reinterpret_cast<const uint32_t *>(wtab + ((int64_t)v * ntiles + tile) * nch + chunk);
        pv = wl < 18 ? vkd[wl] : (wl < 22 ? wd[wl - 18] : 0u);
    };
    auto win_of = [](uint32_t pv) {
        Window w;
        w.n0 = __builtin_amdgcn_readlane((int)pv, 18);
        w.nw = __builtin_amdgcn_readlane((int)pv, 19);
        w.m0 = __builtin_amdgcn_readlane((int)pv, 20);
        w.nrw = __builtin_amdgcn_readlane((int)pv, 21);
        return w;
    };
    auto rd = [](uint32_t pv, int e) {
        const int lo = __builtin_amdgcn_readlane((int)pv, 2 * e), hi = __builtin_amdgcn_readlane((int)pv, 2 * e + 1);
        return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
    };
    // View v's window into buf: wave w copies window rows w, w + 4, ..., each
    // as direct global-to-LDS loads of 64 channels (lane c: channel n0 + c to
    // LDS cell [row][c]).  A cell off the detector gets an offset past the
    // view's buffer range, which the range check turns into a zero: a channel
    // off the detector is given such an offset outright; a row off it needs no
    // test, since 4 (row nc + n) taken modulo 2^32 is then at least the
    // view's nr nc floats (rows below the detector wrap to at least 2^31, and
    // the view is under 2^31 bytes), so the offset just advances by one row
    // step per load.  Lanes past the window's width write nothing (no tap
    // reads there).
    const int64_t vfl = (int64_t)g.nr * g.nc;    // floats per view (bytes below 2^31, checked by the plan)
    auto stage = [&](int v, const Window &w, float *buf) {
        if (w.nw <= 0 || w.nrw <= 0) return;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(sino + (int64_t)v * vfl), (short)0, (int)(vfl * 4), kRawDwordRsrc);
        for (int c0 = 0; c0 < w.nw; c0 += 64) {
            const int c = c0 + wl, n = w.n0 + c;
            const bool nok = (unsigned)n < (unsigned)g.nc;
            if (c < w.nw) {
                unsigned off = nok ? (unsigned)((w.m0 + wave) * g.nc + n) * 4u : kOffRange;
                const unsigned step = nok ? (unsigned)(NT / 64 * g.nc) * 4u : 0u;
                for (int m = wave; m < w.nrw; m += NT / 64, off += step)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(buf + m * PC + c0),
                                                             4, off, 0, 0, 0);
            }
        }
    };

    if (g.nv > 0) {
        uint32_t pcur, pnext;
        fetch_view(0, pcur);
        fetch_view(min(1, g.nv - 1), pnext);
        int ncur = valid ? idx[p] : INT32_MIN;
        stage(0, win_of(pcur), win);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
        for (int v = 0; v < g.nv; ++v) {
            const bool more = v + 1 < g.nv;
            const Window wv = win_of(pcur);
            const Window wn = win_of(pnext);
            int nnext = INT32_MIN;
            uint32_t pafter = pnext;
            if (more) {
                stage(v + 1, wn, win + ((v + 1) & 1) * wsz);
                nnext = valid ? idx[(int64_t)(v + 1) * np + p] : INT32_MIN;
                fetch_view(min(v + 2, g.nv - 1), pafter);
            }
            if (wv.nw > 0 && wv.nrw > 0 && ncur >= -R && ncur <= g.nc - 1 + R) {
                ViewK vk;
                vk.c = rd(pcur, 0);
                vk.s = rd(pcur, 1);
                vk.shift = rd(pcur, 2);
                vk.zsrc = rd(pcur, 3);
                const ConeVPB q = cone_vp_back(g, vk, x, y, ncur);
                double hd[NTAP];
                tap_weights_d<R>(q.f, q.wch, hd);
                // channel taps with the chord factor dv / M folded in (squared
                // for the Hessian-diagonal back projection)
                float h[NTAP];
#pragma unroll
                for (int t = 0; t < NTAP; ++t)
                    h[t] = POW == 2 ? ((float)(hd[t] * hd[t]) * (q.lsc * q.lsc)) : ((float)hd[t] * q.lsc);
                // window cell of row offset sg, channel tap t at slice k:
                // col[(m_k + R + 1) PC + sg PC + t]
                const float *col = win + (v & 1) * wsz + (ncur - R - wv.n0) - (wv.m0 + 2 * R + 1) * PC;
                const double wrow = q.mr * g.dv;        // footprint width in rows = row advance per slice
                const double hrowd = 0.5 * wrow;
                const float hrow = (float)hrowd;
                // the fast row taps' offsets: tap t != R is clamp(ct[t] -+ phi,
                // 0, 1) (below), the centre one what remains of the width wf
                float ct[NTAP];
#pragma unroll
                for (int t = 0; t < NTAP; ++t)
                    ct[t] = t < R ? hrow - (float)(R - 1 - t) : hrow - (float)(t - R);
                const float wf = 2.f * hrow;
                // a footprint wider than the 2R + 1 tap rows loses a sliver to the
                // outermost taps, which one it loses depends on the tap row, so
                // that row must be the model's own rounding even at an exact
                // half: such pixels take the fp64 placement for every slice
                const bool wide = wrow > 2.0 * R;
                // slice k0 sits dz0 above the source; w + R + 3/2 in 32.32 fixed point
                const double dz0 = slice_z(g, k0) - vk.zsrc;
                // (clamped into the integer range first: a row that far off is off
                // the detector for every slice of the chunk either way)
                const double t0 = fmin(fmax((q.mr * dz0 + g.crow) + (1.5 + (double)R), -1e9), 1e9);
                const double fl0 = floor(t0);
                uint64_t wfx = ((uint64_t)(uint32_t)(int)fl0 << 32) | (uint64_t)(uint32_t)((t0 - fl0) * 4294967296.0);
                const uint64_t afx = (uint64_t)(fmin(wrow, 1e6) * 4294967296.0 + 0.5);
                const float r2f = (float)q.r2, dvf = (float)g.dv;
                float dzf = (float)dz0;
                // the slice count, re-read per view so that the per-slice tests
                // stay scalar compares instead of 32 hoisted lane masks,
                int nkv, k0v;
                asm volatile("s_mov_b32 %0, %1" : "=s"(nkv) : "s"(nk));
                // and the chunk's first slice, so that the edge branch's slice
                // heights are not hoisted out of the view loop into registers
                asm volatile("s_mov_b32 %0, %1" : "=s"(k0v) : "s"(k0));
#pragma unroll
                for (int k = 0; k < SL; ++k) {
                    const int hk = (int)(wfx >> 32);            // m_k + R + 1
                    const uint32_t fr = (uint32_t)wfx;          // (w_k - m_k + 1/2) 2^32
                    const float dzk = dzf;
                    wfx += afx;
                    dzf += dvf;
                    // slices past the chunk's last one get an empty row range
                    // (a uniform bound, so the test stays one compare); the
                    // range is one row wider each side than the taps need, and
                    // the edge branch below decides those rows in fp64, as it
                    // decides every slice of a wide footprint
                    const unsigned rl1 = k < nkv ? rlim + 3u : 0u;
                    if ((unsigned)hk < rl1 || (wide && k < nkv)) {
                        // inside the detector, a footprint no wider than 2R
                        // rows: with phi = fr 2^-32 = w_k - m_k + 1/2 it spans
                        // [R + phi - W/2, R + phi + W/2] in units of the tap
                        // cells [t, t + 1], and never leaves them, so a cell
                        // below the centre one overlaps it by clamp(W/2 - (R -
                        // 1 - t) - phi, 0, 1), one above by clamp(W/2 - (t - R)
                        // + phi, 0, 1), and the centre one by what remains of
                        // W: one fma with the clamp modifier per outer tap,
                        // about 1e-7 absolute error, far below the tolerance.
                        // Formed for every lane (straight-line code); the
                        // branch below replaces it where it does not apply.
                        float gw[NTAP];
                        {
                            const float phr = (float)fr;
                            float mid = wf;
#pragma unroll
                            for (int t = 0; t < NTAP; ++t) {
                                if (t == R) continue;
                                gw[t] = __builtin_amdgcn_fmed3f(fmaf(phr, t < R ? -0x1p-32f : 0x1p-32f, ct[t]), 0.f, 1.f);
                                mid -= gw[t];
                            }
                            gw[R] = mid;
                        }
                        int hr = hk;                            // tap centre row + R + 1
                        bool ok = true;
                        if (wide || ib < 0 || (unsigned)(hk - (2 * R + 1)) > (unsigned)ib) {
                            // a footprint wider than the taps, or a tap cell off
                            // the top or bottom detector edge: the row is placed
                            // in fp64 in the model's operation order, so that
                            // the tap row is the model's at an exact half, and a
                            // footprint edge on a cell boundary gives an exactly
                            // empty tap there (a voxel that only grazes the
                            // detector then adds exactly nothing).  A voxel whose
                            // rows graze that edge sums nothing but thin edge
                            // taps, so each tap is the model's own overlap of
                            // cell m = mk + t - R with the footprint, in the
                            // model's operations (d = m - w_k, then the clipped
                            // interval [d - 1/2, d + 1/2] against [-W/2, W/2]):
                            // a thin tap is then an exact difference of nearby
                            // numbers, rounded once
                            const double dz = slice_z(g, k0v + k) - vk.zsrc;
                            const double wk = q.mr * dz + g.crow;    // product, then sum (no contraction)
                            const double mk = rint(wk);
                            ok = mk >= -R && mk <= g.nr - 1 + R;
                            hr = ok ? (int)mk + (R + 1) : R + 1;
#pragma unroll
                            for (int t = 0; t < NTAP; ++t) {
                                const double d = (mk + (double)(t - R)) - wk;
                                const double hi = fmin(d + 0.5, hrowd), lo = fmax(d - 0.5, -hrowd);
                                gw[t] = hi > lo ? (float)(hi - lo) : 0.f;
                            }
                        }
                        if (ok) {
                            const float qk = fmaf(dzk, dzk, r2f);   // d^2 + a^2 + dz^2
                            float lk;
                            if (POW == 2) {             // squared weights: the Hessian-diagonal back projection
                                lk = qk;
#pragma unroll
                                for (int t = 0; t < NTAP; ++t) gw[t] = gw[t] * gw[t];
                            } else {
                                lk = __builtin_amdgcn_sqrtf(qk);
                            }
                            const float *cell = col + hr * PC;
                            float s = 0.f;
#pragma unroll
                            for (int sg = 0; sg < NTAP; ++sg) {
                                float rv = 0.f;
#pragma unroll
                                for (int t = 0; t < NTAP; ++t) rv = fmaf(h[t], cell[sg * PC + t], rv);
                                s = fmaf(gw[sg], rv, s);
                            }
                            acc[k] = fmaf(lk, s, acc[k]);
                        }
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the next window has landed in LDS
            __syncthreads();
            pcur = pnext;
            pnext = pafter;
            ncur = nnext;
        }
    }
    if (valid) {
        float *out = recon + (int64_t)p * g.ns + k0;
#pragma unroll
        for (int k = 0; k < SL; ++k)
            if (k < nk) out[k] = acc[k];
    }
}

// Forward: a workgroup owns a CTX x CTY pixel tile and a chunk of 64*P slices;
// each wave works on one view at a time.  The 3x3 (generally (2R+1)^2) tap
// block of a voxel is the product of its row taps and its channel taps, so a
// pixel's cylinder is projected in two steps:
//   1. slices -> rows.  Lanes are slices (lane l takes slices l*P + ph, or
//      consecutive slices where the slab allows); each computes its row w_k
//      (fp64, the model's operation order), its 2R+1 row taps and the chord,
//      and adds L_k x_k g_sg into a one-column row profile of the window in
//      LDS, one row offset per round.  P is chosen at creation so that the
//      slices of one instruction fall on distinct rows: every add is a plain
//      read-modify-write with no two lanes on one cell (float atomics in LDS
//      cost tens of times a plain update on gfx950).
//   2. rows -> channels.  Lanes are the window's rows on the detector (64
//      per pass; the flush drops the others); each reads and clears its
//      profile cell and adds h_t times it into 2R+1 register accumulators,
//      one per channel of the pixel's taps.  The tile's
//      pixels are walked in the order of their channel index, so a channel is
//      finished once the walk has passed it: it is written into its window
//      column once (rows of the pass) and the accumulators shift down by one
//      channel (slot t holds channel lo + t, so every register index is
//      fixed at compile time).
// A finished channel goes straight from the ring to memory: one global atomic
// add per nonzero cell per (view, tile, chunk), lanes along the channel's
// rows.  Into the handle's transposed sinogram [view][channel][row] (then
// unpacked) those are whole 64-byte lines, four per pass; the row-major
// sinogram takes the same adds one line per row (cst, rst: the destination's
// channel and row strides).  So a wave keeps only its row profile in LDS, and
// LDS no longer bounds the workgroups per CU.  Per voxel-view this does 2R+1 LDS
// read-modify-writes on one column instead of (2R+1)^2 on the block, and the
// (2R+1)^2 products become 2R+1 per slice and 2R+1 per row.
// Waves per SIMD the compiler must fit (registers capped at 512 / waves).
// Without a window in LDS the registers bound the occupancy, and more waves
// hide more of the walk's LDS and memory latency, at the price of spilled
// registers, whose traffic goes through the caches: six at radius 1 and 2
// (12-36 bytes spilled per lane).  Measured, 5 / 6 / 7 or 8 waves: 256^3 cone
// forward 8.92 / 8.68 / 8.42 ms with 1.2 / 3.7 / 9.1 GB fetched per call;
// helical 47.2 / 45.0 / 43.8 ms with 8.8 / 10.8 / 66 GB.  Radius 3 and 4 hold
// too many taps for that and are left free.
template <int R, int NPG>
constexpr int cone_fwd_waves() {
    return R <= 2 ? 6 : 1;
}

template <int R, int P, bool U, int TY, int NPG>
__global__ __launch_bounds__(CFW * 64, (cone_fwd_waves<R, NPG>())) void cone_forward_kernel(const float *__restrict__ recon,
                                                                 float *__restrict__ sino,
                                                                 const int32_t *__restrict__ idx,
                                                                 const ViewK *__restrict__ views,
                                                                 const int4 *__restrict__ wtab,
                                                                 const int4 *__restrict__ stab, Geo g, int nrp,
                                                                 int ncol, int vsplit, int cst, int rst) {
    constexpr int NTAP = 2 * R + 1;
    constexpr int CH = 64 * P;            // slices per chunk
    constexpr int NPX = CTX * TY;         // pixels per tile (at most one per lane)
    static_assert(NPX <= 64, "one pixel per lane");
    extern __shared__ float lds[];
    const int lane = (int)threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    float *prof = lds + wave * cone_fwd_wave_words(nrp, ncol);   // this wave's row profile columns [ncol][nrp]

    const int tiles_x = (g.nx + CTX - 1) / CTX;
    const int ntiles = tiles_x * ((g.ny + TY - 1) / TY);
    const int nch = (g.ns + CH - 1) / CH;
    const int tj0 = (int)(blockIdx.x % tiles_x) * CTX;
    const int ti0 = (int)(blockIdx.x / tiles_x) * TY;
    const int k0 = (int)blockIdx.y * CH;
    const int nk = min(CH, g.ns - k0);
    const int np = g.ny * g.nx;

    // the profile starts at zero; the second step clears every cell it reads
    for (int e = lane; e < ncol * nrp; e += 64) prof[e] = 0.f;

    const int vper = (g.nv + vsplit - 1) / vsplit;
    const int vbeg = (int)blockIdx.z * vper;
    const int vend = min(g.nv, vbeg + vper);
    const int cnt = vend - vbeg;
    const int start = cnt > 0 ? (int)((blockIdx.x * 37u + blockIdx.y * 11u) % (unsigned)cnt) : 0;
    auto view_of = [&](int it) {
        const int v = vbeg + start + it;
        return v >= vend ? v - cnt : v;
    };
    // this lane's pixel of the tile (lanes past the tile's CTX * TY pixels
    // hold none)
    const int il = ti0 + lane / CTX, jl = tj0 + lane % CTX;
    const bool lin = lane < NPX && il < g.ny && jl < g.nx;
    const double xl = pix_x(g, jl), yl = pix_y(g, il);
    // this lane's voxel cylinder in the chunk (clamped into the volume for
    // lanes without a pixel, which are never walked), as two dwords the walk
    // reads out per pixel
    const uint64_t cyl = reinterpret_cast<uint64_t>(
        recon + ((int64_t)min(il, g.ny - 1) * g.nx + min(jl, g.nx - 1)) * g.ns + k0);
    const int cyl_lo = (int)(uint32_t)cyl, cyl_hi = (int)(uint32_t)(cyl >> 32);

    // Per-view data, fetched one view ahead with vector loads: lanes 0-17
    // hold the view's constants (ViewK, 18 dwords), lanes 18-21 its window,
    // lanes 22-25 its slab, and every lane the channel index of its pixel.
    static_assert(sizeof(ViewK) == 72, "ViewK is read as 18 dwords");
    auto prefetch = [&](int it, uint32_t &pv, int &pn) {
        const int v = view_of(min(it, cnt - 1));    // always issued, for a static wait count
        const uint32_t *vkd = reinterpret_cast<const uint32_t *>(views + v);
        const int64_t te = ((int64_t)v * ntiles + blockIdx.x) * nch + blockIdx.y;
        const uint32_t *wd = reinterpret_cast<const uint32_t *>(wtab + te);
        const uint32_t *sd = reinterpret_cast<const uint32_t *>(stab + te);
        if (U)
            pv = lane < 18 ? vkd[lane] : (lane < 22 ? wd[lane - 18] : (lane < 26 ? sd[lane - 22] : 0u));
        else
            pv = lane < 18 ? vkd[lane] : (lane < 22 ? wd[lane - 18] : 0u);
        pn = lin ? idx[(int64_t)v * np + il * g.nx + jl] : INT32_MIN;
    };
    auto rl_d = [](double d, int q) {           // lane q's double, as a wave-uniform value
        const long long b = __double_as_longlong(d);
        const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), q);
        const int hi = __builtin_amdgcn_readlane((int)(b >> 32), q);
        return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
    };

    auto walk_view = [&](int it, uint32_t pv, int pn) {
        const int v = view_of(it);
        ViewK vk;
        {
            double vd[9];
#pragma unroll
            for (int e = 0; e < 9; ++e) {
                const int lo = __builtin_amdgcn_readlane((int)pv, 2 * e), hi = __builtin_amdgcn_readlane((int)pv, 2 * e + 1);
                vd[e] = __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
            }
            vk.c = vd[0]; vk.s = vd[1]; vk.shift = vd[2]; vk.zsrc = vd[3]; vk.cd = vd[4]; vk.sd = vd[5];
            vk.u0 = vd[6]; vk.W = vd[7]; vk.L = vd[8];
        }
        Window wd;
        wd.n0 = __builtin_amdgcn_readlane((int)pv, 18);
        wd.nw = __builtin_amdgcn_readlane((int)pv, 19);
        wd.m0 = __builtin_amdgcn_readlane((int)pv, 20);
        wd.nrw = __builtin_amdgcn_readlane((int)pv, 21);
        if (wd.nw <= 0 || wd.nrw <= 0) return;
        // The chunk's slices that can reach the detector rows in this view
        // (the slab, from the creation pass): with `unit`, lanes take
        // consecutive slices from the first one, in `nit` passes of 64, and
        // with `inter` as well lane l adds into profile column l mod P (its
        // slices are P apart, so on distinct rows; only where the plan gave
        // the wave P columns); otherwise lane l takes
        // slices l*P + ph over the whole chunk.  (Without slabs, U false:
        // every chunk walks all its slices with stride P.)
        const int klo = U ? __builtin_amdgcn_readlane((int)pv, 22) : 0;
        const int nit = U ? __builtin_amdgcn_readlane((int)pv, 23) : P;
        const int smode = U ? __builtin_amdgcn_readlane((int)pv, 24) : 0;
        const bool unit = smode != 0;
        const bool inter = P > 1 && smode == 2;
        if (nit <= 0) return;                                 // no slice reaches the detector
        const int pcol = inter ? (lane % P) * nrp : 0;        // this lane's profile column
        // this lane's pixel: channel taps and the per-(view, pixel) constants, fp64
        const bool act = pn >= -R && pn <= g.nc - 1 + R;
        const uint64_t actb = __builtin_amdgcn_ballot_w64(act);
        if (!actb) return;
        // (the chord factor dv / M and d^2 + a^2 only ever enter the fp32
        // chord, so they are carried in fp32)
        float hq[NTAP];
        double mrq = 0.0;
        float lscq = 0.f, r2q = 0.f;
#pragma unroll
        for (int t = 0; t < NTAP; ++t) hq[t] = 0.f;
        if (act) {
            const ConeVP cv = cone_vp(g, vk, xl, yl, pn);
            double hd[NTAP];
            tap_weights_d<R>(cv.f, cv.wch, hd);
#pragma unroll
            for (int t = 0; t < NTAP; ++t) hq[t] = (float)hd[t];
            mrq = cv.mr;
            lscq = (float)cv.lsc;
            r2q = (float)cv.r2;
        }
        // Walk order: the active pixels by channel index, then by pixel.  The
        // rank of each comes from counting over the channel keys; the lanes
        // of the order are filled by a forward permute (inactive lanes take
        // the ranks after the active ones).
        const int kq = act ? pn : INT32_MAX;
        int kmin = INT32_MAX, kmax = INT32_MIN;
        {
            uint64_t rest = actb;
            while (rest) {
                const int q = (int)__builtin_ctzll(rest);
                rest &= rest - 1;
                const int kk2 = __builtin_amdgcn_readlane(kq, q);
                kmin = min(kmin, kk2);
                kmax = max(kmax, kk2);
            }
        }
        const int npix = (int)__builtin_popcountll(actb);
        int rank = npix + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(~actb >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)~actb, 0u));
        {
            int base = 0;
            for (int c = kmin; c <= kmax; ++c) {
                const uint64_t b = __builtin_amdgcn_ballot_w64(kq == c);
                if (!b) continue;
                const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
                if (kq == c) rank = base + below;
                base += (int)__builtin_popcountll(b);
            }
        }
        const int order = __builtin_amdgcn_ds_permute(rank * 4, lane);   // lane r: the pixel of rank r
        const int korder = __builtin_amdgcn_ds_permute(rank * 4, kq);    // and its channel index

        int kkv[P];                                           // this lane's slice in each pass
        double dzs[P];
#pragma unroll
        for (int ph = 0; ph < P; ++ph) {
            kkv[ph] = unit ? klo + ph * 64 + lane : lane * P + ph;
            dzs[ph] = slice_z(g, k0 + kkv[ph]) - vk.zsrc;
        }
        float dz2[P];
        bool kok[P];                                          // slice inside the chunk
        int kkc[P];                                           // and clamped into it, for the loads
#pragma unroll
        for (int ph = 0; ph < P; ++ph) {
            dz2[ph] = (float)(dzs[ph] * dzs[ph]);
            kok[ph] = kkv[ph] < nk && (!U || ph < nit);
            kkc[ph] = min(kkv[ph], nk - 1);
        }

        const int nrw = wd.nrw;
        // Only the window rows on the detector are ever flushed, so step 2
        // walks those alone: rows rb .. re - 1 of the window, in passes of 64
        // lanes.  (Step 1 also adds into the profile rows off the detector;
        // they are never read, and are cleared when the view is done.)
        const int rb = max(0, -wd.m0);
        const int re = min(nrw, g.nr - wd.m0);
        const int npass = re > rb ? (re - rb + 63) >> 6 : 0;
        const int cbase = kmin - R;                          // first channel of the walk
        const int clast = kmax + R;                          // last channel of the walk
        float *const dview = sino + (int64_t)v * g.nr * g.nc;   // this view of the destination

        // Step 1 for one pixel: its cylinder's slices into the row profile.
        // Per slice: the row (fp64, bit-exact with the model), the row taps
        // (fp64; with a box no wider than the 2R+1 taps the outermost clamps
        // are the box edges themselves, so they are skipped), the chord, then
        // 2R+1 read-modify-writes, one row offset per round: within a round
        // the active lanes hold distinct rows, and a lane's next row may be
        // its neighbour's previous one, hence the ordering fence between
        // rounds (LDS operations of a wave issue in order; the fence keeps
        // the compiler from hoisting the next round's reads).
        auto to_rows = [&](int q, const float (&xv)[P]) {
            const double mr = rl_d(mrq, q);
            const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r2q), q));
            const float lscf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lscq), q));
            const double wbox = mr * g.dv;
            const double hw = 0.5 * wbox, nhw = -hw;
            const double hwm = hw - 0.5;                      // exact for hw in [1/4, 1] (Sterbenz)
            const float wboxf = (float)wbox;
            float *const pr = prof + pcol - wd.m0 - R;        // pr[mk + sg]: row offset sg - R of row mk
            auto slices = [&](auto narrow_c) {
                constexpr bool NARROW = decltype(narrow_c)::value;
#pragma unroll
                for (int ph = 0; ph < P; ++ph) {
                    if (U && ph >= nit) break;                    // uniform
                    const double t0 = mr * dzs[ph];
                    const double wk = t0 + g.crow;
                    const double mk = rint(wk);
                    const int mi = (int)mk;                       // saturates far off the detector
                    const bool ok = kok[ph] && (unsigned)mi + (unsigned)R <= (unsigned)(g.nr - 1 + 2 * R);
                    const double f = wk - mk;
                    float gf[NTAP];
                    if constexpr (R == 1 && NARROW) {
                        // the box [-h, h] and the cells around it, whose inner
                        // edges sit at -(1/2 + f) and 1/2 - f: the outer taps
                        // are max((h - 1/2) - f, 0) and max((h - 1/2) + f, 0),
                        // each one rounding of the exact value (h - 1/2 is
                        // exact for h >= 1/4), as the model's overlap gives it
                        // (a tap of a footprint that only touches its cell can
                        // be 1e-15 and alone in its sinogram cell); the middle
                        // one is never thin (at least min(2h, 1) minus the
                        // outer two), so the box width minus the outer two in
                        // fp32 is accurate.  (hwm -+ f is at most 1, so the
                        // upper clamp never binds: the clamp to [0, 1] is the
                        // add's own output modifier.)
                        gf[0] = (float)fmin(fmax(hwm - f, 0.0), 1.0);
                        gf[2] = (float)fmin(fmax(hwm + f, 0.0), 1.0);
                        gf[1] = (wboxf - gf[0]) - gf[2];
                    } else {
                        double gp = NARROW ? nhw : fmin(fmax((-0.5 - (double)R) - f, nhw), hw);
#pragma unroll
                        for (int t = 0; t < NTAP; ++t) {
                            const double gn =
                                (NARROW && t == NTAP - 1) ? hw : fmin(fmax(((double)(t - R) + 0.5) - f, nhw), hw);
                            gf[t] = (float)(gn - gp);
                            gp = gn;
                        }
                    }
                    const float lkx = lscf * __builtin_amdgcn_sqrtf(r2 + dz2[ph]) * xv[ph];
                    // one exec mask for the 2R + 1 rounds (the lanes of a round
                    // are the same in every round)
                    if (ok) {
                        float *const cell = pr + mi;
#pragma unroll
                        for (int sg = 0; sg < NTAP; ++sg) {
                            cell[sg] = fmaf(lkx, gf[sg], cell[sg]);
                            __atomic_signal_fence(__ATOMIC_SEQ_CST);
                        }
                    }
                }
            };
            if (R == 1 ? (hw <= 1.0 && hw >= 0.25) : hw <= (double)R)
                slices(std::true_type{});
            else
                slices(std::false_type{});
        };

        // The voxels come from memory (L2: the tile's cylinders are read by
        // every view), the next pixel's while this one is projected, in two
        // alternating register buffers (no copies, so the loads are waited for
        // only where used).  Every lane loads, from its slice clamped into the
        // chunk: lanes past the chunk's last slice never use the value, and
        // loads that are all unconditional let the compiler wait for the
        // current pixel's alone, not for the prefetch behind them.
        // (through a global address-space pointer: a generic one would make
        // these flat loads, which the LDS waits of the walk also wait for)
        auto load_px = [&](int q, float (&xv)[P]) {
            const __attribute__((address_space(1))) float *src =
                reinterpret_cast<const __attribute__((address_space(1))) float *>(
                    ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(cyl_hi, q) << 32) |
                    (uint64_t)(uint32_t)__builtin_amdgcn_readlane(cyl_lo, q));
#pragma unroll
            for (int ph = 0; ph < P; ++ph) xv[ph] = src[kkc[ph]];
        };

        // Row groups of NPG passes: the ring accumulators of one group live
        // in registers; a window taller than 64 * NPG detector rows walks the
        // pixels once per group (the profile is cleared in full every time).
        // Row passes that lie inside the profile column and the window column
        // whatever this view's window (a single group, and passes below the
        // plan's row pitch nrp) read, clear and write without a row guard:
        // rows past the detector rows of this view's window are never flushed
        // from the window, and reading them only clears them.  The last pass
        // of a group is guarded.
        auto walk_groups = [&](auto full_c) {
            constexpr bool FULL = decltype(full_c)::value;
            for (int grp = 0; grp * NPG < npass; ++grp) {
                float acc[NPG][NTAP];
#pragma unroll
                for (int ps = 0; ps < NPG; ++ps)
#pragma unroll
                    for (int s = 0; s < NTAP; ++s) acc[ps][s] = 0.f;
                bool rowin[NPG], rowok[NPG];     // a detector row of the window; and read in step 2
#pragma unroll
                for (int ps = 0; ps < NPG; ++ps) {
                    rowin[ps] = rb + (grp * NPG + ps) * 64 + lane < re;
                    rowok[ps] = (FULL && ps + 1 < NPG) || rowin[ps];
                }
                // this lane's first detector row, as a destination offset
                const int dro = (wd.m0 + rb + grp * NPG * 64 + lane) * rst;
                int lo = cbase;                                   // channel of ring slot 0
                // write channel lo's accumulators into its window column and
                // shift the ring down by one channel (slot t holds channel lo + t)
                auto finish = [&]() {
                    if ((unsigned)lo < (unsigned)g.nc) {            // uniform: a channel on the detector
                        float *dcol = dview + lo * cst + dro;
#pragma unroll
                        for (int ps = 0; ps < NPG; ++ps) {
                            const float val = acc[ps][0];
                            if (rowin[ps] && val != 0.f) unsafeAtomicAdd(dcol + ps * 64 * rst, val);
                        }
                    }
#pragma unroll
                    for (int ps = 0; ps < NPG; ++ps) {
#pragma unroll
                        for (int t = 0; t + 1 < NTAP; ++t) acc[ps][t] = acc[ps][t + 1];
                        acc[ps][NTAP - 1] = 0.f;
                    }
                    ++lo;
                };
                // Step 2 for one pixel, whose taps cover channels lo .. lo + 2R:
                // every profile row of the window is read, cleared and added into
                // the ring.
                auto to_channels = [&](int q) {
                    float h[NTAP];
#pragma unroll
                    for (int t = 0; t < NTAP; ++t)
                        h[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hq[t]), q));
#pragma unroll
                    for (int ps = 0; ps < NPG; ++ps) {
                        float *cell = prof + rb + (grp * NPG + ps) * 64 + lane;
                        float r = 0.f;
                        if (rowok[ps]) {
                            r = *cell;
                            *cell = 0.f;
                            if (inter) {
#pragma unroll
                                for (int c = 1; c < P; ++c) {
                                    r += cell[c * nrp];
                                    cell[c * nrp] = 0.f;
                                }
                            }
                        }
#pragma unroll
                        for (int t = 0; t < NTAP; ++t) acc[ps][t] = fmaf(h[t], r, acc[ps][t]);
                    }
                    if (!FULL && npass > NPG) {                   // the other groups' rows: cleared only
                        for (int pp = 0; pp < npass; ++pp)
                            if (pp / NPG != grp && rb + pp * 64 + lane < re)
                                for (int c = 0; c < (inter ? P : 1); ++c) prof[c * nrp + rb + pp * 64 + lane] = 0.f;
                    }
                };
                auto visit = [&](int i, const float (&xv)[P]) {
                    const int q = __builtin_amdgcn_readlane(order, i);
                    const int n = __builtin_amdgcn_readlane(korder, i);
                    while (lo < n - R) finish();                  // channels the walk has passed
                    to_rows(q, xv);
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    to_channels(q);
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                };
                {
                    float xa[P], xb[P];
                    int i = 0;
                    // (the prefetch is always issued, the last pixel's again at
                    // the end, so that the wait counts stay static)
                    load_px(__builtin_amdgcn_readlane(order, 0), xa);
                    for (;;) {
                        load_px(__builtin_amdgcn_readlane(order, min(i + 1, npix - 1)), xb);
                        visit(i, xa);
                        if (++i >= npix) break;
                        load_px(__builtin_amdgcn_readlane(order, min(i + 1, npix - 1)), xa);
                        visit(i, xb);
                        if (++i >= npix) break;
                    }
                }
                while (lo <= clast) finish();
            }
        };
        if (npass <= NPG && nrp >= rb + (NPG - 1) * 64)
            walk_groups(std::true_type{});
        else
            walk_groups(std::false_type{});
        // the profile rows off the detector, which step 1 added into and
        // step 2 never read
        for (int m = lane; m < nrw; m += 64)
            if (m < rb || m >= re)
                for (int c = 0; c < (inter ? P : 1); ++c) prof[c * nrp + m] = 0.f;
    };

    // two prefetch buffers in turn: the next view's data is loaded while this
    // one is walked (no copies, so the waits stay narrow; a third buffer, two
    // views ahead, gained nothing and held two more registers)
    if (wave >= cnt) return;
    uint32_t pvA, pvB;
    int pnA, pnB;
    prefetch(wave, pvA, pnA);
    for (int it = wave; it < cnt; it += 2 * CFW) {
        prefetch(it + CFW, pvB, pnB);
        walk_view(it, pvA, pnA);
        if (it + CFW >= cnt) break;
        prefetch(it + 2 * CFW, pvA, pnA);
        walk_view(it + CFW, pvB, pnB);
    }
}

template <int SL, int R, int PC>
static hipError_t cone_back_n(const Plan &p, const float *sino, float *recon, int power, hipStream_t st) {
    const Geo &g = p.g;
    const int tiles = ((g.nx + BT - 1) / BT) * ((g.ny + BT - 1) / BT);
    const int chunks = (g.ns + SL - 1) / SL;
    if (power == 2)
        hipLaunchKernelGGL((cone_back_kernel<SL, R, 2, PC>), dim3(tiles, chunks), dim3(BT * BT), p.back_lds, st,
                           sino, recon, p.idx, p.views, p.bwin, g, p.back_nrcap);
    else
        hipLaunchKernelGGL((cone_back_kernel<SL, R, 1, PC>), dim3(tiles, chunks), dim3(BT * BT), p.back_lds, st,
                           sino, recon, p.idx, p.views, p.bwin, g, p.back_nrcap);
    return hipGetLastError();
}

template <int SL, int R>
static hipError_t cone_back_t(const Plan &p, const float *sino, float *recon, int power, hipStream_t st) {
    switch (p.back_pc) {
    case 33: return cone_back_n<SL, R, 33>(p, sino, recon, power, st);
    case 65: return cone_back_n<SL, R, 65>(p, sino, recon, power, st);
    case 129: return cone_back_n<SL, R, 129>(p, sino, recon, power, st);
    case 257: return cone_back_n<SL, R, 257>(p, sino, recon, power, st);
    default: return hipErrorInvalidValue;
    }
}

// Row passes of 64 lanes held in registers per row group, from the most
// detector rows a window can hold (the window's rows, at most the detector's):
// 1 where that is at most 64, 2 where at most 128 (radius 1), else 3.
template <int R>
constexpr int cone_fwd_npg(int rows) {
    return rows <= 64 ? 1 : ((R == 1 && rows <= 128) ? 2 : 3);
}

template <int R, int P, bool U, int TY, int NPG>
static hipError_t cone_fwd_u(const Plan &p, const float *recon, float *sino, bool tr, hipStream_t st) {
    const Geo &g = p.g;
    const int tiles = ((g.nx + CTX - 1) / CTX) * ((g.ny + TY - 1) / TY);
    const int chunks = (g.ns + 64 * P - 1) / (64 * P);
    hipLaunchKernelGGL((cone_forward_kernel<R, P, U, TY, NPG>), dim3(tiles, chunks, p.fwd_vsplit), dim3(CFW * 64),
                       p.fwd_lds, st, recon, sino, p.idx, p.views, p.fwin, p.fslab, g, p.fwd_nrcap, p.cone_ncol,
                       p.fwd_vsplit, tr ? g.nr : 1, tr ? 1 : g.nc);
    return hipGetLastError();
}

template <int R, int P, int NPG>
static hipError_t cone_fwd_n(const Plan &p, const float *recon, float *sino, bool tr, hipStream_t st) {
    if (p.cone_ty == 8) {
        if (p.cone_unit) return cone_fwd_u<R, P, true, 8, NPG>(p, recon, sino, tr, st);
        return cone_fwd_u<R, P, false, 8, NPG>(p, recon, sino, tr, st);
    }
    if (p.cone_unit) return cone_fwd_u<R, P, true, 4, NPG>(p, recon, sino, tr, st);
    return cone_fwd_u<R, P, false, 4, NPG>(p, recon, sino, tr, st);
}

template <int R, int P>
static hipError_t cone_fwd_t(const Plan &p, const float *recon, float *sino, bool tr, hipStream_t st) {
    const int npg = cone_fwd_npg<R>(std::min(p.fwd_nrcap, p.g.nr));
    if (npg == 1) return cone_fwd_n<R, P, 1>(p, recon, sino, tr, st);
    if constexpr (R == 1) {
        if (npg == 2) return cone_fwd_n<R, P, 2>(p, recon, sino, tr, st);
    }
    return cone_fwd_n<R, P, 3>(p, recon, sino, tr, st);
}

template <int R>
static hipError_t cone_fwd_r(const Plan &p, const float *recon, float *sino, bool tr, hipStream_t st) {
    switch (p.cone_stride) {
    case 1: return cone_fwd_t<R, 1>(p, recon, sino, tr, st);
    case 2: return cone_fwd_t<R, 2>(p, recon, sino, tr, st);
    case 3: return cone_fwd_t<R, 3>(p, recon, sino, tr, st);
    default: return hipErrorInvalidValue;
    }
}

#define BPAMD_DISPATCH_R(FN, SLV, ...)                         \
    switch (p.g.radius) {                                      \
    case 1: return FN<SLV, 1>(__VA_ARGS__);                    \
    case 2: return FN<SLV, 2>(__VA_ARGS__);                    \
    case 3: return FN<SLV, 3>(__VA_ARGS__);                    \
    case 4: return FN<SLV, 4>(__VA_ARGS__);                    \
    default: return hipErrorInvalidValue;                      \
    }

hipError_t launch_cone_back(const Plan &p, const float *sino, float *recon, int power, hipStream_t st) {
    switch (p.back_sl) {
    case 8: BPAMD_DISPATCH_R(cone_back_t, 8, p, sino, recon, power, st)
    case 16: BPAMD_DISPATCH_R(cone_back_t, 16, p, sino, recon, power, st)
    case 32: BPAMD_DISPATCH_R(cone_back_t, 32, p, sino, recon, power, st)
    case 48: BPAMD_DISPATCH_R(cone_back_t, 48, p, sino, recon, power, st)
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_cone_forward(const Plan &p, const float *recon, float *sino, bool transposed, hipStream_t st) {
    switch (p.g.radius) {
    case 1: return cone_fwd_r<1>(p, recon, sino, transposed, st);
    case 2: return cone_fwd_r<2>(p, recon, sino, transposed, st);
    case 3: return cone_fwd_r<3>(p, recon, sino, transposed, st);
    case 4: return cone_fwd_r<4>(p, recon, sino, transposed, st);
    default: return hipErrorInvalidValue;
    }
}

// Dynamic LDS above the default limit needs the opt-in attribute.
hipError_t cone_forward_allow_lds(int radius, int stride, int ty, int rows, size_t bytes) {
    const void *f = nullptr;
    const void *fu = nullptr;
#define BPAMD_CFN(RR, PP, NN)                                                                                 \
    {                                                                                                         \
        f = ty == 8 ? (const void *)cone_forward_kernel<RR, PP, false, 8, NN>                                 \
                    : (const void *)cone_forward_kernel<RR, PP, false, 4, NN>;                                \
        fu = ty == 8 ? (const void *)cone_forward_kernel<RR, PP, true, 8, NN>                                 \
                     : (const void *)cone_forward_kernel<RR, PP, true, 4, NN>;                                \
    }
#define BPAMD_CF(RR, PP)                                                                                      \
    if (radius == RR && stride == PP) {                                                                       \
        if (cone_fwd_npg<RR>(rows) == 1)                                                                      \
            BPAMD_CFN(RR, PP, 1)                                                                              \
        else if constexpr (RR == 1) {                                                                         \
            if (cone_fwd_npg<RR>(rows) == 2) BPAMD_CFN(RR, PP, 2) else BPAMD_CFN(RR, PP, 3)                   \
        } else                                                                                                \
            BPAMD_CFN(RR, PP, 3)                                                                              \
    }
    BPAMD_CF(1, 1) BPAMD_CF(1, 2) BPAMD_CF(1, 3) BPAMD_CF(2, 1) BPAMD_CF(2, 2) BPAMD_CF(2, 3)
    BPAMD_CF(3, 1) BPAMD_CF(3, 2) BPAMD_CF(3, 3) BPAMD_CF(4, 1) BPAMD_CF(4, 2) BPAMD_CF(4, 3)
#undef BPAMD_CF
#undef BPAMD_CFN
    if (!f) return hipErrorInvalidValue;
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(fu, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace bpamd
