// C ABI of the projector library: validation, the launch plan, the device
// tables a handle owns, and the entry points declared in include/proj.h.
//
// Creation runs once per geometry (the projectors themselves are called every
// solver iteration, MBIRJAX "Projector kernels" page, introduction), so all
// checks, table uploads, the fp64 channel-index pass and the choice of tile
// and window sizes happen here.  The per-call entry points then do nothing on
// the host but argument checks and one or two kernel launches on the caller's
// stream: no allocation, no copy, no synchronisation (page section "The rules
// a Pallas kernel must follow": shapes from arrays, never data; no host round
// trips; build each kernel once).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "api_common.h"

using namespace bpamd;

namespace bpamd {

thread_local std::string g_last_error;

proj_status fail(proj_status s, const std::string &why) {
    g_last_error = why;
    return s;
}

proj_status ok() {
    g_last_error.clear();
    return PROJ_OK;
}

}  // namespace bpamd

namespace {


constexpr size_t kMaxLds = 64 * 1024;                 // dynamic LDS per workgroup without opt-in
constexpr size_t kMaxLdsOptIn = 160 * 1024;           // gfx950 LDS per workgroup

bool finite(double v) { return std::isfinite(v); }

}  // namespace


namespace {

// Smallest slice chunk from `opts` (ascending) that covers S with the least
// padding; chunks larger than S are not considered once one covers it.
int pick_chunk(int64_t s, const std::vector<int> &opts) {
    for (int o : opts)
        if (s <= o) return o;
    int best = opts.back();
    int64_t best_pad = ((s + best - 1) / best) * best - s;
    for (auto it = opts.rbegin(); it != opts.rend(); ++it) {
        const int o = *it;
        const int64_t pad = ((s + o - 1) / o) * o - s;
        if (pad < best_pad) {
            best = o;
            best_pad = pad;
        }
    }
    return best;
}

struct WinMax {
    int nw = 0, nr = 0;
};

// Windows of every (view, tile, slice chunk), in that order (tiles row-major,
// as the kernels number them), and their maxima.
WinMax window_table(const Geo &g, const std::vector<ViewK> &views, int tx_, int ty_, int sl,
                    std::vector<Window> *out) {
    WinMax m;
    const int ty = (g.ny + ty_ - 1) / ty_, tx = (g.nx + tx_ - 1) / tx_;
    const int nch = g.kind == 0 ? 1 : (g.ns + sl - 1) / sl;
    if (out) out->resize((size_t)g.nv * ty * tx * nch);
    size_t e = 0;
    for (int v = 0; v < g.nv; ++v)
        for (int a = 0; a < ty; ++a)
            for (int b = 0; b < tx; ++b) {
                const int i0 = a * ty_, i1 = std::min(i0 + ty_, g.ny) - 1;
                const int j0 = b * tx_, j1 = std::min(j0 + tx_, g.nx) - 1;
                for (int c = 0; c < nch; ++c, ++e) {
                    const int k0 = c * sl, k1 = std::min(k0 + sl, g.ns) - 1;
                    const Window w = tile_window(g, views[v], i0, i1, j0, j1, k0, k1);
                    m.nw = std::max(m.nw, w.nw);
                    m.nr = std::max(m.nr, w.nrw);
                    if (out) (*out)[e] = w;
                }
            }
    return m;
}

// Cone forward slab of one (view, tile, slice chunk): the chunk's slices
// whose rows can reach the detector in that view, conservatively for every
// pixel of the tile (rows within half a row of [-r, R - 1 + r], a slice of
// margin each side; the kernel still tests each slice exactly), as (first
// slice, passes, mode, 0).  Lanes of one instruction adding into one profile
// column must hold slices on distinct rows:
//   mode 1 (unit): the tile's smallest row advance per slice (magnification
//     times the voxel pitch) is at least one, so lane l takes consecutive
//     slices from the first one, all into one column;
//   mode 2 (interleaved): lane l takes consecutive slices from the first one
//     and adds into profile column l mod stride, whose slices are then
//     `stride` apart (stride times the smallest advance is at least one);
//     used where it takes fewer passes than the stride, if the plan gives
//     each wave `stride` profile columns;
//   mode 0 (strided): lane l takes slices l * stride + ph over the whole
//     chunk, one column (as many passes as mode 2 would take there, with
//     one profile column to read instead of `stride`).
// Zero passes: no slice of the chunk reaches the detector in that view.
struct SlabRange {
    double kglo, kghi;   // the tile's slices that can reach the detector (all chunks)
    double mlo;          // the tile's smallest row magnification
};

SlabRange slab_range(const Geo &g, const ViewK &vk, int i0, int i1, int j0, int j1) {
    const double wlo = (-0.5 - g.radius) - g.crow, whi = (g.nr - 1 + g.radius + 0.5) - g.crow;
    double dmin = 1e300, dmax = -1e300;
    for (int ii : {i0, i1})
        for (int jj : {j0, j1}) {
            const double d = g.sid + (pix_y(g, ii) * vk.c - pix_x(g, jj) * vk.s);
            dmin = std::min(dmin, d);
            dmax = std::max(dmax, d);
        }
    const double mlo = g.sdd / (dmax * g.drow), mhi = g.sdd / (dmin * g.drow);
    const double dz[4] = {wlo / mlo, wlo / mhi, whi / mlo, whi / mhi};
    const double zlo = *std::min_element(dz, dz + 4) + vk.zsrc;
    const double zhi = *std::max_element(dz, dz + 4) + vk.zsrc;
    return {std::floor(zlo / g.dv + g.cz) - 1.0, std::ceil(zhi / g.dv + g.cz) + 1.0, mlo};
}

Window slab_of(const Geo &g, const SlabRange &sr, int k0, int nk, int stride, bool inter_ok) {
    Window s;
    s.n0 = 0;
    s.nw = 0;
    s.m0 = 0;
    s.nrw = 0;
    const double lo = std::max(sr.kglo - k0, 0.0), hi = std::min(sr.kghi - k0, (double)nk - 1.0);
    if (hi >= lo) {
        const int klo = (int)lo, nact = (int)hi - klo + 1;
        const int nit_unit = (nact + 63) / 64;
        // consecutive slices are dv apart: their rows differ by mr dv.
        // Unit stride also where it takes as many passes: the rows of one
        // instruction then sit about mr apart instead of stride * mr
        const bool unit = stride > 1 && sr.mlo * g.dv >= 1.0 + 1e-9 && nit_unit <= stride;
        const bool inter = inter_ok && !unit && stride > 1 && nit_unit < stride;
        s.n0 = unit || inter ? klo : 0;
        s.nw = unit || inter ? nit_unit : stride;
        s.m0 = unit ? 1 : (inter ? 2 : 0);
    }
    return s;
}

// Slabs of every (view, tile, slice chunk), in the window table's order.
void slab_table(const Geo &g, const std::vector<ViewK> &views, int tx_, int ty_, int sl, int stride,
                bool inter_ok, std::vector<Window> *out) {
    const int ty = (g.ny + ty_ - 1) / ty_, tx = (g.nx + tx_ - 1) / tx_;
    const int nch = (g.ns + sl - 1) / sl;
    out->resize((size_t)g.nv * ty * tx * nch);
    size_t e = 0;
    for (int v = 0; v < g.nv; ++v)
        for (int a = 0; a < ty; ++a)
            for (int b = 0; b < tx; ++b) {
                const int i0 = a * ty_, i1 = std::min(i0 + ty_, g.ny) - 1;
                const int j0 = b * tx_, j1 = std::min(j0 + tx_, g.nx) - 1;
                const SlabRange sr = slab_range(g, views[v], i0, i1, j0, j1);
                for (int c = 0; c < nch; ++c, ++e) {
                    const int k0 = c * sl, nk = std::min(sl, g.ns - k0);
                    (*out)[e] = slab_of(g, sr, k0, nk, stride, inter_ok);
                }
            }
}

// Estimated time of a cone forward call with CTX x ty tiles, from the same
// windows and slabs the call uses, on a sample of at most about 64 views:
// the slice-to-row work (tile pixels times slab passes, about 0.12 ns each
// on gfx950) and the atomic adds of a dense volume (64-byte requests: each
// window channel's rows on the detector, contiguous in the transposed
// sinogram, about 21.6 G per second).  The two overlap, so the call takes
// about the larger; the 8 x 8 tiles cost about 5% more work per pass.
// (Measured when the windows were flushed row by row into the sinogram
// itself: the 256^3 cone forward of a dense volume 15.0 ms at 8 x 4,
// flush-bound, and 11.3 ms at 8 x 8; with the direct adds into the transposed
// sinogram 8.90 ms at 8 x 4 and 9.05 ms at 8 x 8, both bound by the work.)
// With `passes`, the sampled pixel-passes instead (slab passes times tile pixels).
double cone_forward_cost(const Geo &g, const std::vector<ViewK> &views, int ty_, int sl, int stride, bool inter_ok,
                         bool passes = false) {
    const int ty = (g.ny + ty_ - 1) / ty_, tx = (g.nx + CTX - 1) / CTX;
    const int nch = (g.ns + sl - 1) / sl;
    const int step = std::max(1, g.nv / 64);
    double pixpass = 0.0, lines = 0.0;
    int nsample = 0;
    for (int v = 0; v < g.nv; v += step, ++nsample)
        for (int a = 0; a < ty; ++a)
            for (int b = 0; b < tx; ++b) {
                const int i0 = a * ty_, i1 = std::min(i0 + ty_, g.ny) - 1;
                const int j0 = b * CTX, j1 = std::min(j0 + CTX, g.nx) - 1;
                const double npx = (double)(i1 - i0 + 1) * (j1 - j0 + 1);
                const SlabRange sr = slab_range(g, views[v], i0, i1, j0, j1);
                for (int c = 0; c < nch; ++c) {
                    const int k0 = c * sl, nk = std::min(sl, g.ns - k0);
                    const Window w = tile_window(g, views[v], i0, i1, j0, j1, k0, k0 + nk - 1);
                    if (w.nw <= 0 || w.nrw <= 0) continue;
                    pixpass += npx * slab_of(g, sr, k0, nk, stride, inter_ok).nw;
                    const int r0 = std::max(w.m0, 0), r1 = std::min(w.m0 + w.nrw - 1, g.nr - 1);
                    const int c0 = std::max(w.n0, 0), c1 = std::min(w.n0 + w.nw - 1, g.nc - 1);
                    // the forward adds a finished channel's rows into the
                    // transposed sinogram, where they are contiguous: about
                    // (rows + 15) / 16 lines of 64 bytes per channel
                    if (r1 >= r0 && c1 >= c0) lines += (double)(c1 - c0 + 1) * (r1 - r0 + 16) / 16.0;
                }
            }
    if (passes) return pixpass;
    const double scale = nsample > 0 ? (double)g.nv / nsample : 0.0;
    const double work = pixpass * scale * 0.12e-9 * (ty_ == 8 ? 1.05 : 1.0);
    const double flush = lines * scale / 21.6e9;
    return std::max(work, flush);
}

WinMax max_window(const Geo &g, const std::vector<ViewK> &views, int tx_, int ty_, int sl) {
    return window_table(g, views, tx_, ty_, sl, nullptr);
}

// The parallel-beam forward strategy from the shapes alone (no data), from
// a sweep of both strategies on gfx950 (bench.py --op sweep): the gather walk
// wins at up to 1e8 voxel-views (64^2 x 8 at 90 views, 128^2 x 16 at 90 views
// with radius 1 to 4, 512^2 x 32 translation at 8 views: 1.5x to 7x), and at
// up to about 2.5e8 when there are few views (512^2 x 32 translation at 16 and
// 24 views, 512^2 x 64 at 8 and 12 views: 1.1x to 1.5x), where the region
// walk has too few views per region to amortise loading it and too few
// regions to fill the chip.  The region walk wins from there on (512^2 x 64
// at 16 views and more, 256^2 x 32 at 96 views and more, every 3.8e8 shape
// with radius 1 to 4 and fine detectors: 1.2x to 6x).  The one shape of the
// sweep the rule misplaces, 512^2 x 32 translation at 32 views, loses 9%.
int choose_forward(const Geo &g, const Plan &plan) {
    (void)plan;
    const double vu = (double)g.nv * g.ny * g.nx * g.ns;
    return (vu <= 1e8 || (vu <= 2.5e8 && g.nv <= 32)) ? PROJ_FORWARD_GATHER : PROJ_FORWARD_TILE;
}

// Validation and planning without touching the GPU.  Fills geo/views/plan.
proj_status plan_geometry(const proj_geometry *gp, const int64_t rs[3], const int64_t ss[3], Geo &g,
                          std::vector<ViewK> &views, Plan &plan) {
    if (!gp || !rs || !ss) return fail(PROJ_ERR_INVALID_ARGUMENT, "null geometry or shape pointer");
    for (int d = 0; d < 3; ++d)
        if (rs[d] < 0 || ss[d] < 0 || rs[d] >= kMaxElems || ss[d] >= kMaxElems)
            return fail(PROJ_ERR_INVALID_ARGUMENT, "shape entries must lie in [0, 2^31)");
    if (gp->kind != PROJ_PARALLEL && gp->kind != PROJ_CONE_FLAT)
        return fail(PROJ_ERR_INVALID_ARGUMENT, "kind must be PROJ_PARALLEL or PROJ_CONE_FLAT");
    if (gp->num_views != ss[0])
        return fail(PROJ_ERR_INVALID_ARGUMENT, "num_views must equal sino_shape[0]");
    const int64_t V = ss[0], R = ss[1], C = ss[2], Ny = rs[0], Nx = rs[1], S = rs[2];
    if (V > 0 && !gp->angles) return fail(PROJ_ERR_INVALID_ARGUMENT, "angles is required");
    for (int64_t v = 0; v < V; ++v) {
        if (!finite(gp->angles[v])) return fail(PROJ_ERR_INVALID_ARGUMENT, "non-finite angle");
        if (gp->channel_shift && !finite(gp->channel_shift[v]))
            return fail(PROJ_ERR_INVALID_ARGUMENT, "non-finite channel_shift");
        if (gp->source_z && !finite(gp->source_z[v]))
            return fail(PROJ_ERR_INVALID_ARGUMENT, "non-finite source_z");
    }
    const double dv = gp->delta_voxel, dch = gp->delta_channel, drow = gp->delta_row;
    if (!(finite(dv) && dv > 0) || !(finite(dch) && dch > 0) || !(finite(drow) && drow > 0))
        return fail(PROJ_ERR_INVALID_ARGUMENT, "pitches must be finite and positive");
    if (!finite(gp->det_channel_offset) || !finite(gp->det_row_offset))
        return fail(PROJ_ERR_INVALID_ARGUMENT, "non-finite detector offset");
    if (gp->psf_radius < 1 || gp->psf_radius > 4)
        return fail(PROJ_ERR_INVALID_ARGUMENT, "psf_radius must be in [1, 4]");
    if (gp->kind == PROJ_PARALLEL && gp->forward_strategy != PROJ_FORWARD_AUTO &&
        gp->forward_strategy != PROJ_FORWARD_TILE && gp->forward_strategy != PROJ_FORWARD_GATHER &&
        gp->forward_strategy != PROJ_FORWARD_COLUMN)
        return fail(PROJ_ERR_INVALID_ARGUMENT,
                    "parallel forward_strategy must be PROJ_FORWARD_AUTO, _TILE, _GATHER or _COLUMN");
    if (gp->kind != PROJ_PARALLEL && gp->forward_strategy != PROJ_FORWARD_AUTO &&
        gp->forward_strategy != PROJ_FORWARD_CONE_TILE_8X4 && gp->forward_strategy != PROJ_FORWARD_CONE_TILE_8X8)
        return fail(PROJ_ERR_INVALID_ARGUMENT, "cone forward_strategy must be PROJ_FORWARD_AUTO, _CONE_TILE_8X4 or _8X8");
    const double half_diag = 0.5 * std::sqrt((double)Nx * Nx + (double)Ny * Ny) * dv;
    if (gp->kind == PROJ_PARALLEL) {
        if (R != S) return fail(PROJ_ERR_INVALID_ARGUMENT, "parallel beam needs one detector row per slice (R == S)");
        if (drow != dv) return fail(PROJ_ERR_INVALID_ARGUMENT, "parallel beam needs delta_row == delta_voxel");
        if (gp->source_z) return fail(PROJ_ERR_INVALID_ARGUMENT, "source_z is for cone beam only");
    } else {
        const double sid = gp->source_iso, sdd = gp->source_detector;
        if (!finite(sid) || !finite(sdd)) return fail(PROJ_ERR_INVALID_ARGUMENT, "non-finite source distances");
        if (!(sid > half_diag))
            return fail(PROJ_ERR_INVALID_ARGUMENT, "source_iso must exceed the in-plane radius of the volume");
        if (!(sdd > sid)) return fail(PROJ_ERR_INVALID_ARGUMENT, "source_detector must exceed source_iso");
    }
    if (V * Ny * Nx >= kMaxElems || Ny * Nx * S >= kMaxElems || V * R * C >= kMaxElems)
        return fail(PROJ_ERR_UNSUPPORTED, "an array or the index table would reach 2^31 elements");
    // the back projections copy window rows out of one view of the sinogram
    // with 32-bit byte offsets below 2^31
    if (R * C * 4 >= ((int64_t)1 << 31))
        return fail(PROJ_ERR_UNSUPPORTED, "one view of the sinogram is 2 GiB or more");
    // the cone back stages a window row at the byte offset 4 (row C + n)
    // modulo 2^32, which lies past the view for every row off the detector a
    // window can reach (from -2r to R - 1 + 2r) while 8 r C < 2^31
    if (gp->kind != PROJ_PARALLEL && 8 * (int64_t)gp->psf_radius * C >= ((int64_t)1 << 31))
        return fail(PROJ_ERR_UNSUPPORTED, "cone detector of 2^28 / psf_radius channels or more");

    g.kind = gp->kind;
    g.radius = gp->psf_radius;
    g.ny = (int)Ny; g.nx = (int)Nx; g.ns = (int)S;
    g.nv = (int)V; g.nr = (int)R; g.nc = (int)C;
    g.dv = dv; g.dch = dch; g.drow = drow;
    g.sid = gp->kind == PROJ_CONE_FLAT ? gp->source_iso : 0.0;
    g.sdd = gp->kind == PROJ_CONE_FLAT ? gp->source_detector : 0.0;
    g.cx = ((double)Nx - 1.0) / 2.0;
    g.cy = ((double)Ny - 1.0) / 2.0;
    g.cz = ((double)S - 1.0) / 2.0;
    g.cch = ((double)C - 1.0) / 2.0 + gp->det_channel_offset;
    g.crow = ((double)R - 1.0) / 2.0 + gp->det_row_offset;

    views.resize((size_t)V);
    for (int64_t v = 0; v < V; ++v) {
        ViewK &k = views[(size_t)v];
        k.c = std::cos(gp->angles[v]);
        k.s = std::sin(gp->angles[v]);
        k.shift = gp->channel_shift ? gp->channel_shift[v] : 0.0;
        k.zsrc = gp->source_z ? gp->source_z[v] : 0.0;
        k.cd = k.c / dch;
        k.sd = k.s / dch;
        k.u0 = g.cch + k.shift;
        const double m = std::max(std::fabs(k.c), std::fabs(k.s));
        k.W = dv * m / dch;
        k.L = dv / m;
    }

    plan = Plan();
    plan.g = g;
    if (V == 0 || Ny * Nx == 0 || S == 0 || R == 0 || C == 0) return ok();   // nothing to launch

    // Slice chunk per lane: the least padding first, then smaller chunks while
    // the detector window of a tile does not fit in LDS.
    const bool par = g.kind == 0;
    if (par) {
        // taps that can carry weight: a box of width W covers at most ceil(W) + 1 cells
        double wmax = 0.0;
        for (const ViewK &k : views) wmax = std::max(wmax, k.W);
        plan.ntap = (int)std::min<double>(2.0 * g.radius + 1.0, std::ceil(wmax) + 1.0);
        plan.ntap = std::max(plan.ntap, 2);
        if (plan.ntap > 7) return fail(PROJ_ERR_UNSUPPORTED, "more than 7 channel taps per voxel (detector far finer than the voxels)");
        if (C + plan.ntap > 16384) return fail(PROJ_ERR_UNSUPPORTED, "more than 16384 - taps detector channels");
        for (int sl = pick_chunk(S, {8, 16, 32, 64});; sl /= 2) {
            const WinMax w = max_window(g, views, BT, BT, sl);
            plan.back_sl = sl;
            plan.back_nwcap = w.nw + 2;
            // two raw windows [sl][rp] and two transposed ones [rp][sl + 4], rp =
            // 32 or 64 channels (static arrays of par_back_kernel)
            const size_t rp = w.nw + 2 <= 32 ? 32 : 64;
            plan.back_lds = (2 * (size_t)sl * rp + 2 * rp * (sl + 4)) * sizeof(float);
            if (plan.back_lds <= kMaxLds || sl == 8) break;
        }
        if (plan.back_nwcap > 64)
            return fail(PROJ_ERR_UNSUPPORTED, "back projection window wider than 64 channels (detector far finer than the voxels)");
        plan.back_ncg = plan.back_nwcap <= 32 ? 1 : 2;
        // region walk: two slices per lane, 16 apart (one paired LDS read per
        // step for 32 slices of four views) unless the volume has 16 slices or
        // fewer, which one slice per lane covers without idle lanes
        plan.fwd_spl = S > 16 ? 2 : 1;
        plan.fwd_sl = 16 * plan.fwd_spl;
        plan.rsx = (int)std::min<int64_t>(plan.fwd_spl == 2 ? FRS2X : FRS, Nx);
        plan.rsy = (int)std::min<int64_t>(plan.fwd_spl == 2 ? FRS2Y : FRS, Ny);
        plan.fwd_lds = (size_t)plan.rsx * plan.rsy * 16 * plan.fwd_spl * sizeof(float);
        plan.fwd_cb = (int)C + 2 * (plan.ntap - 1);
        plan.fwd_s16 = (int)(((S + 16 * plan.fwd_spl - 1) / (16 * plan.fwd_spl)) * 16 * plan.fwd_spl);
        // the walk addresses the views of one workgroup with 32-bit byte offsets
        if ((int64_t)(plan.fwd_cb + 2 * plan.ntap) * plan.fwd_s16 * 4 >= ((int64_t)1 << 30))
            return fail(PROJ_ERR_UNSUPPORTED, "forward accumulation buffer too large per view");
        // gather strategy: every pixel of a view, in groups of 16 steps padded to
        // a multiple of 4 groups, walked in segments of up to 144 groups; small
        // problems take shorter segments (multiples of 4 groups) so that the
        // grid of (64-view block, segment, 16-slice chunk) workgroups still
        // counts about 512 where it can
        plan.gat_ng = (int)(((Ny * Nx + 63) / 64) * 4);
        {
            const int64_t nvb = (V + 63) / 64, nchk = (S + 15) / 16;
            const int64_t want = (plan.gat_ng * nvb * nchk + 511) / 512;
            const int64_t segg = std::max<int64_t>(4, std::min<int64_t>(((want + 3) / 4) * 4, 144));
            plan.gat_segg = (int)std::min<int64_t>(segg, plan.gat_ng);
        }
        plan.gat_nseg = (plan.gat_ng + plan.gat_segg - 1) / plan.gat_segg;
        const bool gather_ok = Ny * Nx * S * 4 < ((int64_t)1 << 32) &&
                               64 * (int64_t)(plan.fwd_cb + 2 * plan.ntap) * plan.fwd_s16 * 4 < ((int64_t)1 << 31);
        // every view at angle 0 exactly (sine 0): a pixel's channel does not
        // depend on its row, and the column forms apply (translation scans)
        plan.colmode = V > 0 && Ny * Nx > 0 && S > 0;
        for (const ViewK &vk : views) plan.colmode = plan.colmode && vk.s == 0.0;
        if (gp->forward_strategy == PROJ_FORWARD_COLUMN && !plan.colmode)
            return fail(PROJ_ERR_UNSUPPORTED, "column forward: needs every view angle at 0 (sine exactly 0)");
        plan.fwd_strategy = gp->forward_strategy == PROJ_FORWARD_AUTO
                                ? (plan.colmode ? PROJ_FORWARD_COLUMN : choose_forward(g, plan))
                                : gp->forward_strategy;
        if (plan.fwd_strategy == PROJ_FORWARD_GATHER && !gather_ok) {
            if (gp->forward_strategy == PROJ_FORWARD_GATHER)
                return fail(PROJ_ERR_UNSUPPORTED, "gather forward: volume or detector too large for its 32-bit offsets");
            plan.fwd_strategy = PROJ_FORWARD_TILE;
        }
        // walk-order sort bins: the first tap channels of a region span at most its window
        plan.fwd_nbin = max_window(g, views, plan.rsx, plan.rsy, 64).nw + 2;
        if (plan.fwd_strategy == PROJ_FORWARD_TILE && plan.fwd_nbin > 8192)
            return fail(PROJ_ERR_UNSUPPORTED, "a forward region spans more than 8190 channels");
        if (plan.fwd_strategy == PROJ_FORWARD_GATHER || plan.fwd_strategy == PROJ_FORWARD_COLUMN) plan.fwd_lds = 0;
    } else {
        // two windows (double buffer) of [rows][channels], channels fastest with
        // an odd pitch of 33, 65, 129 or 257 floats (a compile-time constant of the
        // kernel)
        auto back_bytes = [&](int sl, int &nwcap, int &nrcap, int &pc) {
            const WinMax w = max_window(g, views, BT, BT, sl);
            nwcap = w.nw + 2;
            nrcap = w.nr + 2;
            pc = nwcap <= 33 ? 33 : (nwcap <= 65 ? 65 : (nwcap <= 129 ? 129 : 257));
            return 2 * (size_t)nrcap * pc * sizeof(float);
        };
        // (48-slice chunks: a 96-slice volume in two chunks instead of three,
        // each view's window staged twice instead of three times; the larger
        // accumulator file costs no occupancy where the window's LDS already
        // limits the kernel to four workgroups per CU)
        for (int sl = pick_chunk(S, {8, 16, 32, 48});; sl = sl == 48 ? 32 : sl / 2) {
            plan.back_sl = sl;
            plan.back_lds = back_bytes(sl, plan.back_nwcap, plan.back_nrcap, plan.back_pc);
            if ((plan.back_lds <= kMaxLds && plan.back_nwcap <= 257) || sl == 8) break;
        }
        if (plan.back_nwcap > 257)
            return fail(PROJ_ERR_UNSUPPORTED, "cone back window wider than 257 channels (detector far finer than the voxels)");
        // smallest row magnification (rows per slice) over the whole scan: lanes
        // of one forward instruction take slices `stride` apart, so that their
        // rows differ
        double amin = 1e300;
        const double xs[2] = {pix_x(g, 0), pix_x(g, g.nx - 1)}, ys[2] = {pix_y(g, 0), pix_y(g, g.ny - 1)};
        for (const ViewK &k : views)
            for (double xx : xs)
                for (double yy : ys) {
                    const double d = g.sid + (yy * k.c - xx * k.s);
                    amin = std::min(amin, g.sdd * g.dv / (d * g.drow));
                }
        int stride = 1;
        while (stride * amin < 1.0 + 1e-9 && stride <= 3) ++stride;
        if (stride > 3)
            return fail(PROJ_ERR_UNSUPPORTED, "row magnification below 1/3 (detector rows far coarser than the voxels)");
        plan.cone_stride = stride;
        plan.fwd_sl = 64 * stride;
        // tile rows: 8 x 4 pixels, or 8 x 8 where the atomic adds of the
        // narrower tiles would bound the call (forced by forward_strategy)
        if (gp->forward_strategy == PROJ_FORWARD_CONE_TILE_8X4)
            plan.cone_ty = 4;
        else if (gp->forward_strategy == PROJ_FORWARD_CONE_TILE_8X8)
            plan.cone_ty = 8;
        else
            plan.cone_ty = cone_forward_cost(g, views, 8, plan.fwd_sl, stride, false) <
                                   cone_forward_cost(g, views, 4, plan.fwd_sl, stride, false)
                               ? 8
                               : 4;
        // `stride` profile columns per wave where the interleaved slabs save a
        // tenth of the slice passes or more (each column costs a little LDS
        // and one more read and clear per row in step 2)
        plan.cone_ncol = 1;
        if (stride > 1 && cone_forward_cost(g, views, plan.cone_ty, plan.fwd_sl, stride, true, true) <=
                              0.9 * cone_forward_cost(g, views, plan.cone_ty, plan.fwd_sl, stride, false, true))
            plan.cone_ncol = stride;
        const WinMax wf = max_window(g, views, CTX, plan.cone_ty, plan.fwd_sl);
        plan.fwd_nwcap = wf.nw;
        plan.fwd_nrcap = wf.nr | 1;
        plan.fwd_lds = (size_t)CFW * cone_fwd_wave_words(plan.fwd_nrcap, plan.cone_ncol) * sizeof(float);
    }
    if (plan.back_lds > kMaxLds || plan.fwd_lds > kMaxLdsOptIn) {
        char buf[160];
        std::snprintf(buf, sizeof buf, "detector window too large for LDS (back %zu B, forward %zu B)",
                      plan.back_lds, plan.fwd_lds);
        return fail(PROJ_ERR_UNSUPPORTED, buf);
    }
    const int64_t chunks_b = (S + plan.back_sl - 1) / plan.back_sl;
    const int64_t chunks_f = (S + plan.fwd_sl - 1) / plan.fwd_sl;
    if (chunks_b > 65535 || chunks_f > 65535) return fail(PROJ_ERR_UNSUPPORTED, "too many slices");
    if (par) {
        // one region workgroup per CU: a few per CU over the whole grid, each
        // split keeping at least one view per row of every wave
        const int64_t nreg = ((Nx + plan.rsx - 1) / plan.rsx) * ((Ny + plan.rsy - 1) / plan.rsy);
        int64_t vs = (1024 + nreg * chunks_f - 1) / (nreg * chunks_f);
        vs = std::max<int64_t>(1, std::min<int64_t>(vs, std::max<int64_t>(1, V / (FRW * 4))));
        vs = std::min<int64_t>(vs, 64);
        // and few enough views per workgroup for 32-bit offsets into the buffer
        const int64_t view_bytes = (int64_t)(plan.fwd_cb + 2 * plan.ntap) * plan.fwd_s16 * 4;
        const int64_t vmax = ((int64_t)1 << 31) / view_bytes;       // >= 2 by the check above
        vs = std::max<int64_t>(vs, (V + vmax - 1) / vmax);
        if (vs * 8 * ((nreg + 7) / 8) * chunks_f >= ((int64_t)1 << 31))
            return fail(PROJ_ERR_UNSUPPORTED, "too many forward workgroups");
        plan.fwd_vsplit = (int)vs;
    } else {
        const int64_t ftiles = ((Nx + CTX - 1) / CTX) * ((Ny + plan.cone_ty - 1) / plan.cone_ty);
        // enough workgroups to fill 256 CUs a few times over; each split re-reads its tile
        int64_t vs = (2048 + ftiles * chunks_f - 1) / (ftiles * chunks_f);
        vs = std::max<int64_t>(1, std::min<int64_t>(vs, std::min<int64_t>(V, 64)));
        plan.fwd_vsplit = (int)vs;
    }
    return ok();
}

int describe(const Plan &p, int64_t table_bytes, char *buf, int len) {
    const Geo &g = p.g;
    const bool par = g.kind == 0;
    return std::snprintf(
        buf, (size_t)std::max(len, 0),
        "kind=%s V=%d R=%d C=%d Ny=%d Nx=%d S=%d radius=%d taps=%d | back: %s%dx%d px tile, lanes=pixels, %d "
        "slices/lane, window %d ch x %d rows, %zu B LDS%s | forward: %dx%d px tile, %s, %d slices, window %d ch x %d "
        "rows, %zu B LDS, %d view ranges | tables and buffers %lld B",
        par ? "parallel" : "cone_flat", g.nv, g.nr, g.nc, g.ny, g.nx, g.ns, g.radius, par ? p.ntap : 2 * g.radius + 1,
        p.colmode ? "column: one value per (column, slice) over the views, written to every row (else " : "", BT, BT,
        p.back_sl, p.back_nwcap, par ? p.back_sl : p.back_nrcap, p.back_lds, p.colmode ? ")" : "",
        par ? p.rsx : CTX, par ? p.rsy : p.cone_ty,
        par ? (p.fwd_strategy == PROJ_FORWARD_COLUMN
                   ? "column: every view at angle 0, column sums over rows, then per view a channel gather of the columns"
               : p.fwd_strategy == PROJ_FORWARD_GATHER
                   ? "gather: per-view sorted walk of all pixels, lanes=16 slices x 4 views, voxels from memory"
                   : (p.fwd_spl == 2 ? "tile: channel-ordered region walk, lanes=16 x 4 views with 2 slices each, ring accumulators"
                                     : "tile: channel-ordered region walk, lanes=16 slices x 4 views, ring accumulators"))
            : (p.cone_ncol > 1 ? "wave per view: lanes=slices into interleaved row-profile columns, then lanes=rows into channel ring accumulators"
                               : "wave per view: lanes=strided slices into a row profile, then lanes=rows into channel ring accumulators"),
        p.fwd_sl,
        p.fwd_nwcap, par ? p.fwd_sl : p.fwd_nrcap, p.fwd_lds, p.fwd_vsplit, (long long)table_bytes);
}

}  // namespace

extern "C" {

const char *proj_status_string(proj_status s) {
    switch (s) {
    case PROJ_OK: return "PROJ_OK";
    case PROJ_ERR_INVALID_ARGUMENT: return "PROJ_ERR_INVALID_ARGUMENT";
    case PROJ_ERR_UNSUPPORTED: return "PROJ_ERR_UNSUPPORTED";
    case PROJ_ERR_ALIAS: return "PROJ_ERR_ALIAS";
    case PROJ_ERR_OUT_OF_MEMORY: return "PROJ_ERR_OUT_OF_MEMORY";
    case PROJ_ERR_DEVICE: return "PROJ_ERR_DEVICE";
    }
    return "PROJ_ERR_UNKNOWN";
}

const char *proj_last_error(void) { return g_last_error.c_str(); }

proj_status proj_plan_query(const proj_geometry *g, const int64_t recon_shape[3], const int64_t sino_shape[3],
                            char *buf, int len) {
    try {
        Geo geo;
        std::vector<ViewK> views;
        Plan plan;
        const proj_status s = plan_geometry(g, recon_shape, sino_shape, geo, views, plan);
        if (s != PROJ_OK) return s;
        if (buf && len > 0)
            describe(plan, (int64_t)geo.nv * geo.ny * geo.nx * (int64_t)sizeof(int32_t), buf, len);
        return ok();
    } catch (const std::bad_alloc &) {
        return fail(PROJ_ERR_OUT_OF_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(PROJ_ERR_DEVICE, "unexpected internal error");
    }
}

proj_status proj_create(const proj_geometry *gp, const int64_t recon_shape[3], const int64_t sino_shape[3],
                        int hip_device, proj_handle *out) {
    if (!out) return fail(PROJ_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    try {
        Geo geo;
        std::vector<ViewK> views;
        Plan plan;
        proj_status s = plan_geometry(gp, recon_shape, sino_shape, geo, views, plan);
        if (s != PROJ_OK) return s;
        int ndev = 0;
        hipError_t e = hipGetDeviceCount(&ndev);
        if (e != hipSuccess) return device_fail(e, "hipGetDeviceCount");
        if (hip_device < 0 || hip_device >= ndev) return fail(PROJ_ERR_INVALID_ARGUMENT, "no such HIP device");
        DeviceGuard dg(hip_device);
        if (dg.err != hipSuccess) return device_fail(dg.err, "hipSetDevice");

        proj_handle h = new proj_handle_s();
        h->device = hip_device;
        h->plan = plan;
        h->recon_elems = recon_shape[0] * recon_shape[1] * recon_shape[2];
        h->sino_elems = sino_shape[0] * sino_shape[1] * sino_shape[2];
        h->index_elems = sino_shape[0] * recon_shape[0] * recon_shape[1];
        auto cleanup = [&](proj_status st, hipError_t he, const char *what) {
            proj_destroy(h);
            return he != hipSuccess ? device_fail(he, what) : st;
        };
        if (!views.empty()) {
            e = hipMalloc((void **)&h->d_views, views.size() * sizeof(ViewK));
            if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(views)");
            e = hipMemcpy(h->d_views, views.data(), views.size() * sizeof(ViewK), hipMemcpyHostToDevice);
            if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMemcpy(views)");
        }
        size_t rec_bytes = 0;
        if (h->index_elems > 0) {
            e = hipMalloc((void **)&h->d_idx, (size_t)h->index_elems * sizeof(int32_t));
            if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(index table)");
            e = launch_channel_index(geo, h->d_views, h->d_idx, nullptr);
            if (e != hipSuccess) return cleanup(PROJ_OK, e, "channel index pass");
            if (geo.kind == 0 && plan.ntap > 0) {
                rec_bytes = (size_t)h->index_elems * (1 + plan.ntap) * sizeof(int32_t);
                e = hipMalloc((void **)&h->d_rec, rec_bytes);
                if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(tap records)");
                e = launch_par_taps(geo, h->d_views, h->d_rec, plan.ntap, nullptr);
                if (e != hipSuccess) return cleanup(PROJ_OK, e, "tap record pass");
                if (plan.fwd_strategy == PROJ_FORWARD_COLUMN) {
                    // the column sums (the records of row 0 serve for every row)
                    const size_t col_bytes = (size_t)geo.nx * geo.ns * sizeof(float);
                    e = hipMalloc((void **)&h->d_col, col_bytes);
                    if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(column sums)");
                    rec_bytes += col_bytes;
                } else if (plan.fwd_strategy == PROJ_FORWARD_GATHER) {
                    const int64_t per_view = (int64_t)plan.gat_ng * (2 + plan.ntap) * 16;
                    const size_t wrec_bytes = (size_t)(geo.nv + 1) * per_view * sizeof(uint32_t);
                    e = hipMalloc((void **)&h->d_wrec, wrec_bytes);
                    if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(walk records)");
                    e = launch_fill_zero(reinterpret_cast<float *>(h->d_wrec) + (int64_t)geo.nv * per_view, per_view,
                                         nullptr);
                    if (e != hipSuccess) return cleanup(PROJ_OK, e, "zero fill");
                    int32_t *order = nullptr;         // the per-view pixel order, only while building
                    e = hipMalloc((void **)&order, (size_t)h->index_elems * sizeof(int32_t));
                    if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(pixel order)");
                    e = launch_par_view_records(geo, h->d_rec, order, h->d_wrec, plan.ntap, plan.gat_ng, plan.gat_segg,
                                                nullptr);
                    const hipError_t e2 = hipDeviceSynchronize();
                    (void)hipFree(order);
                    if (e != hipSuccess) return cleanup(PROJ_OK, e, "walk record pass");
                    if (e2 != hipSuccess) return cleanup(PROJ_OK, e2, "walk record pass");
                    rec_bytes += wrec_bytes;
                } else {
                    const int64_t nreg = (int64_t)((geo.nx + plan.rsx - 1) / plan.rsx) * ((geo.ny + plan.rsy - 1) / plan.rsy);
                    const int64_t per_view = nreg * fwd_groups(plan.rsx, plan.rsy) * (2 + plan.ntap) * 16;
                    // one more view of all-zero records for the rows of a wave past the last view
                    const size_t wrec_bytes = (size_t)(geo.nv + 1) * per_view * sizeof(uint32_t);
                    e = hipMalloc((void **)&h->d_wrec, wrec_bytes);
                    if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(walk records)");
                    e = launch_fill_zero(reinterpret_cast<float *>(h->d_wrec) + (int64_t)geo.nv * per_view, per_view,
                                         nullptr);
                    if (e != hipSuccess) return cleanup(PROJ_OK, e, "zero fill");
                    e = launch_par_region_records(geo, h->d_rec, h->d_wrec, plan.ntap, plan.rsx, plan.rsy, plan.fwd_nbin,
                                                  plan.fwd_spl, nullptr);
                    if (e != hipSuccess) return cleanup(PROJ_OK, e, "walk record pass");
                    rec_bytes += wrec_bytes;
                    if (plan.fwd_lds > kMaxLds) {
                        int lim = 0;
                        e = hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, hip_device);
                        if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipDeviceGetAttribute");
                        if ((size_t)lim < plan.fwd_lds) {
                            proj_destroy(h);
                            return fail(PROJ_ERR_UNSUPPORTED, "device LDS per workgroup below the forward plan's need");
                        }
                        e = par_forward_allow_lds(plan.ntap, plan.fwd_spl, plan.fwd_lds);
                        if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipFuncSetAttribute(LDS)");
                    }
                }
                const size_t facc_bytes = (size_t)geo.nv * plan.fwd_cb * plan.fwd_s16 * sizeof(float);
                e = hipMalloc((void **)&h->d_facc, facc_bytes);
                if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(forward accumulation buffer)");
                rec_bytes += facc_bytes;
                // the batch forward's sort: its LDS holds a count per key
                // (fwd_cb + 1 of them) and a pass's sorted records; those take
                // at most about 128 MiB in memory
                int lds_max = 0;
                e = hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, hip_device);
                if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipDeviceGetAttribute");
                const int64_t rs = 2 + plan.ntap;
                int64_t nb = ((int64_t)128 << 20) / ((int64_t)geo.nv * rs * 4);
                // (less 256 bytes: the sort's static LDS, its scan's wave sums)
                nb = std::min<int64_t>(nb, (((int64_t)lds_max - 256) / 4 - plan.fwd_cb - 1) / rs);
                nb = std::min<int64_t>(kBatchPass, nb / 256 * 256);
                if (nb >= 256) {
                    const size_t sort_bytes =
                        ((size_t)geo.nv * rs * nb + (size_t)geo.nv * (plan.fwd_cb + 1)) * sizeof(int32_t);
                    const size_t sort_lds = batch_sort_lds(plan.fwd_cb, plan.ntap, (int)nb);
                    // (a device that refuses the LDS keeps the atomic batch forward)
                    if (sort_lds <= kMaxLds || batch_sort_allow_lds(plan.ntap, sort_lds) == hipSuccess) {
                        e = hipMalloc((void **)&h->d_bsort, sort_bytes);
                        if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(batch sort)");
                        h->bsort_nb = (int)nb;
                        rec_bytes += sort_bytes;
                    } else {
                        (void)hipGetLastError();
                    }
                }
                e = hipEventCreateWithFlags(&h->fwd_done, hipEventDisableTiming);
                if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipEventCreateWithFlags");
            }
            if (geo.kind != 0 && h->sino_elems > 0) {
                // the cone batches' transposed sinogram, and the event that
                // orders the calls sharing it
                e = hipMalloc((void **)&h->d_ctr, (size_t)h->sino_elems * sizeof(float));
                if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(batch buffer)");
                rec_bytes += (size_t)h->sino_elems * sizeof(float);
                e = hipEventCreateWithFlags(&h->fwd_done, hipEventDisableTiming);
                if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipEventCreateWithFlags");
            }
            e = hipDeviceSynchronize();
            if (e != hipSuccess) return cleanup(PROJ_OK, e, "table passes");
        }
        if (plan.back_sl > 0) {
            // every (view, tile, chunk) window, from the same code that sized the plan
            std::vector<Window> bw, fw, fs;
            window_table(geo, views, BT, BT, plan.back_sl, &bw);
            if (geo.kind != 0) {
                window_table(geo, views, CTX, plan.cone_ty, plan.fwd_sl, &fw);
                slab_table(geo, views, CTX, plan.cone_ty, plan.fwd_sl, plan.cone_stride, plan.cone_ncol > 1, &fs);
                // the slab-reading kernel when some slab saves work (a walk of
                // consecutive slices, or a chunk that misses the detector in a view)
                for (const Window &w : fs) h->plan.cone_unit |= (w.m0 != 0 || w.nw == 0) ? 1 : 0;
            }
            e = hipMalloc((void **)&h->d_bwin, bw.size() * sizeof(Window));
            if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(windows)");
            e = hipMemcpy(h->d_bwin, bw.data(), bw.size() * sizeof(Window), hipMemcpyHostToDevice);
            if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMemcpy(windows)");
            if (!fw.empty()) {
                e = hipMalloc((void **)&h->d_fwin, fw.size() * sizeof(Window));
                if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(windows)");
                e = hipMemcpy(h->d_fwin, fw.data(), fw.size() * sizeof(Window), hipMemcpyHostToDevice);
                if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMemcpy(windows)");
                e = hipMalloc((void **)&h->d_fslab, fs.size() * sizeof(Window));
                if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMalloc(slabs)");
                e = hipMemcpy(h->d_fslab, fs.data(), fs.size() * sizeof(Window), hipMemcpyHostToDevice);
                if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipMemcpy(slabs)");
            }
            rec_bytes += (bw.size() + fw.size() + fs.size()) * sizeof(Window);
        }
        if (geo.kind != 0 && plan.fwd_sl > 0 && plan.fwd_lds > kMaxLds) {
            int lim = 0;
            e = hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, hip_device);
            if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipDeviceGetAttribute");
            if ((size_t)lim < plan.fwd_lds) {
                proj_destroy(h);
                return fail(PROJ_ERR_UNSUPPORTED, "device LDS per workgroup below the forward plan's need");
            }
            e = cone_forward_allow_lds(geo.radius, plan.cone_stride, plan.cone_ty, std::min(plan.fwd_nrcap, geo.nr),
                                       plan.fwd_lds);
            if (e != hipSuccess) return cleanup(PROJ_OK, e, "hipFuncSetAttribute(LDS)");
        }
        h->table_bytes = (size_t)h->index_elems * sizeof(int32_t) + views.size() * sizeof(ViewK) + rec_bytes;
        h->plan.views = h->d_views;
        h->plan.idx = h->d_idx;
        h->plan.rec = h->d_rec;
        h->plan.wrec = h->d_wrec;
        h->plan.facc = h->d_facc;
        h->plan.ctr = h->d_ctr;
        h->plan.col = h->d_col;
        if (h->d_bsort) {
            h->plan.bsort = h->d_bsort;
            h->plan.boff = h->d_bsort + (int64_t)geo.nv * (2 + plan.ntap) * h->bsort_nb;
            h->plan.bsort_nb = h->bsort_nb;
        }
        h->plan.bwin = reinterpret_cast<const int4 *>(h->d_bwin);
        h->plan.fwin = reinterpret_cast<const int4 *>(h->d_fwin);
        h->plan.fslab = reinterpret_cast<const int4 *>(h->d_fslab);
        if (std::getenv("PROJ_LOG")) {
            char buf[512];
            describe(h->plan, (int64_t)h->table_bytes, buf, sizeof buf);
            std::fprintf(stderr, "[proj] %s\n", buf);
        }
        *out = h;
        return ok();
    } catch (const std::bad_alloc &) {
        return fail(PROJ_ERR_OUT_OF_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(PROJ_ERR_DEVICE, "unexpected internal error");
    }
}

proj_status proj_forward(proj_handle h, const float *recon_dev, float *sino_dev, void *hip_stream) {
    if (!h) return fail(PROJ_ERR_INVALID_ARGUMENT, "null handle");
    if ((h->recon_elems > 0 && !recon_dev) || (h->sino_elems > 0 && !sino_dev))
        return fail(PROJ_ERR_INVALID_ARGUMENT, "null data pointer");
    if (overlaps(recon_dev, h->recon_elems * 4, sino_dev, h->sino_elems * 4))
        return fail(PROJ_ERR_ALIAS, "recon and sino buffers overlap");
    if (h->sino_elems == 0) return ok();
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return device_fail(dg.err, "hipSetDevice");
    hipStream_t st = (hipStream_t)hip_stream;
    hipError_t e;
    const bool cone_tr = h->plan.g.kind != 0 && h->plan.back_sl != 0 && h->plan.ctr;
    if (h->plan.back_sl == 0 || (h->plan.g.kind != 0 && !cone_tr)) {
        e = launch_fill_zero(sino_dev, h->sino_elems, st);
        if (e != hipSuccess) return device_fail(e, "zero fill");
    }
    if (h->plan.back_sl == 0) return ok();     // empty volume or no views: the sinogram is zero
    if (cone_tr) {
        // into the handle's transposed sinogram (zeroed first), then unpacked
        // into sino_dev; the buffer belongs to the handle, so a call on another
        // stream waits on the GPU for the previous user
        bool capturing = false;
        e = stream_capturing(st, capturing);
        if (e != hipSuccess) return device_fail(e, "hipStreamIsCapturing");
        if (!capturing) {
            e = hipStreamWaitEvent(st, h->fwd_done, 0);
            if (e != hipSuccess) return device_fail(e, "hipStreamWaitEvent");
        }
        const Geo &g = h->plan.g;
        e = launch_fill_zero(h->plan.ctr, h->sino_elems, st);
        if (e != hipSuccess) return device_fail(e, "zero fill");
        e = launch_cone_forward(h->plan, recon_dev, h->plan.ctr, true, st);
        if (e != hipSuccess) return device_fail(e, "forward projection launch");
        e = launch_unpack_rows(h->plan.ctr, sino_dev, g.nv, g.nr, g.nc, g.nc, g.nr, 0, st);
        if (e != hipSuccess) return device_fail(e, "forward unpack launch");
        if (!capturing) {
            e = hipEventRecord(h->fwd_done, st);
            if (e != hipSuccess) return device_fail(e, "hipEventRecord");
        }
        return ok();
    }
    if (h->plan.g.kind == 0) {
        // the accumulation buffer belongs to the handle: a call on another
        // stream waits on the GPU for the previous one
        bool capturing = false;
        e = stream_capturing(st, capturing);
        if (e != hipSuccess) return device_fail(e, "hipStreamIsCapturing");
        if (!capturing) {
            e = hipStreamWaitEvent(st, h->fwd_done, 0);
            if (e != hipSuccess) return device_fail(e, "hipStreamWaitEvent");
        }
        e = launch_par_forward(h->plan, recon_dev, sino_dev, st);
        if (e != hipSuccess) return device_fail(e, "forward projection launch");
        if (!capturing) {
            e = hipEventRecord(h->fwd_done, st);
            if (e != hipSuccess) return device_fail(e, "hipEventRecord");
        }
        return ok();
    }
    e = launch_cone_forward(h->plan, recon_dev, sino_dev, false, st);
    if (e != hipSuccess) return device_fail(e, "forward projection launch");
    return ok();
}

static proj_status back_power(proj_handle h, const float *sino_dev, float *recon_dev, int power, void *hip_stream) {
    if (!h) return fail(PROJ_ERR_INVALID_ARGUMENT, "null handle");
    if ((h->recon_elems > 0 && !recon_dev) || (h->sino_elems > 0 && !sino_dev))
        return fail(PROJ_ERR_INVALID_ARGUMENT, "null data pointer");
    if (overlaps(recon_dev, h->recon_elems * 4, sino_dev, h->sino_elems * 4))
        return fail(PROJ_ERR_ALIAS, "recon and sino buffers overlap");
    if (h->recon_elems == 0) return ok();
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return device_fail(dg.err, "hipSetDevice");
    hipStream_t st = (hipStream_t)hip_stream;
    hipError_t e;
    if (h->plan.back_sl == 0) {
        e = launch_fill_zero(recon_dev, h->recon_elems, st);      // no views or empty detector
        if (e != hipSuccess) return device_fail(e, "zero fill");
        return ok();
    }
    e = h->plan.g.kind == 0 ? launch_par_back(h->plan, sino_dev, recon_dev, power, st)
                            : launch_cone_back(h->plan, sino_dev, recon_dev, power, st);
    if (e != hipSuccess) return device_fail(e, "back projection launch");
    return ok();
}

proj_status proj_back(proj_handle h, const float *sino_dev, float *recon_dev, void *hip_stream) {
    return back_power(h, sino_dev, recon_dev, 1, hip_stream);
}

proj_status proj_back_squared(proj_handle h, const float *sino_dev, float *recon_dev, void *hip_stream) {
    return back_power(h, sino_dev, recon_dev, 2, hip_stream);
}

proj_status proj_channel_index(proj_handle h, int32_t *index_dev, void *hip_stream) {
    if (!h) return fail(PROJ_ERR_INVALID_ARGUMENT, "null handle");
    if (h->index_elems == 0) return ok();
    if (!index_dev) return fail(PROJ_ERR_INVALID_ARGUMENT, "null index pointer");
    if (overlaps(index_dev, h->index_elems * 4, h->d_idx, h->index_elems * 4))
        return fail(PROJ_ERR_ALIAS, "destination overlaps the handle's table");
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return device_fail(dg.err, "hipSetDevice");
    const hipError_t e = hipMemcpyAsync(index_dev, h->d_idx, (size_t)h->index_elems * sizeof(int32_t),
                                        hipMemcpyDeviceToDevice, (hipStream_t)hip_stream);
    if (e != hipSuccess) return device_fail(e, "hipMemcpyAsync(index)");
    return ok();
}

void proj_destroy(proj_handle h) {
    if (!h) return;
    {
        DeviceGuard dg(h->device);
        if (h->d_idx) (void)hipFree(h->d_idx);
        if (h->d_rec) (void)hipFree(h->d_rec);
        if (h->d_wrec) (void)hipFree(h->d_wrec);
        if (h->d_facc) (void)hipFree(h->d_facc);
        if (h->d_bsort) (void)hipFree(h->d_bsort);
        if (h->d_ctr) (void)hipFree(h->d_ctr);
        if (h->d_col) (void)hipFree(h->d_col);
        if (h->fwd_done) (void)hipEventDestroy(h->fwd_done);
        if (h->d_bwin) (void)hipFree(h->d_bwin);
        if (h->d_fwin) (void)hipFree(h->d_fwin);
        if (h->d_fslab) (void)hipFree(h->d_fslab);
        if (h->d_views) (void)hipFree(h->d_views);
    }
    delete h;
}

int proj_describe(proj_handle h, char *buf, int len) {
    if (!h) return -1;
    return describe(h->plan, (int64_t)h->table_bytes, buf, len);
}

}  // extern "C"
