// C ABI of the batch and solver entry points: projection of voxel-cylinder
// batches (proj_forward_pixels, proj_back_pixels) and the CGLS and SIRT loops
// around the pair (proj_cgls, proj_sirt, proj_solver_workspace_size).
#include <cmath>

#include "api_common.h"

using namespace bpamd;

extern "C" {

static proj_status check_batch(proj_handle h, const int32_t *pix, int64_t n, const void *cyl, const void *sino) {
    if (!h) return fail(PROJ_ERR_INVALID_ARGUMENT, "null handle");
    const int64_t ns = h->plan.g.ns;
    if (n < 0) return fail(PROJ_ERR_INVALID_ARGUMENT, "negative batch size");
    if (ns > 0 && n > (kMaxElems - 1) / ns) return fail(PROJ_ERR_UNSUPPORTED, "batch of n*S elements above 2^31");
    if (n > 0 && !pix) return fail(PROJ_ERR_INVALID_ARGUMENT, "null pixel list");
    if ((n * ns > 0 && !cyl) || (h->sino_elems > 0 && !sino))
        return fail(PROJ_ERR_INVALID_ARGUMENT, "null data pointer");
    const int64_t cb = n * ns * 4, pb = n * 4, sb = h->sino_elems * 4;
    if (overlaps(cyl, cb, sino, sb) || overlaps(pix, pb, cyl, cb) || overlaps(pix, pb, sino, sb))
        return fail(PROJ_ERR_ALIAS, "pixel list, cylinders and sino buffers overlap");
    return ok();
}

proj_status proj_forward_pixels(proj_handle h, const int32_t *pixels_dev, int64_t n, const float *cyl_dev,
                                float *sino_dev, void *hip_stream) {
    const proj_status s0 = check_batch(h, pixels_dev, n, cyl_dev, sino_dev);
    if (s0 != PROJ_OK) return s0;
    if (h->sino_elems == 0) return ok();
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return device_fail(dg.err, "hipSetDevice");
    hipStream_t st = (hipStream_t)hip_stream;
    hipError_t e;
    if (h->plan.back_sl == 0 || n == 0 || h->plan.g.ns == 0) {
        e = launch_fill_zero(sino_dev, h->sino_elems, st);       // nothing to project
        if (e != hipSuccess) return device_fail(e, "zero fill");
        return ok();
    }
    // (parallel: the accumulation and sort buffers; cone: the transposed
    // sinogram)
    const bool shared = h->plan.g.kind == 0 || h->plan.ctr;
    bool capturing = false;
    if (shared) {
        e = stream_capturing(st, capturing);
        if (e != hipSuccess) return device_fail(e, "hipStreamIsCapturing");
        if (!capturing) {
            e = hipStreamWaitEvent(st, h->fwd_done, 0);
            if (e != hipSuccess) return device_fail(e, "hipStreamWaitEvent");
        }
    }
    e = launch_forward_pixels(h->plan, pixels_dev, (int)n, cyl_dev, sino_dev, st);
    if (e != hipSuccess) return device_fail(e, "batch forward projection launch");
    if (shared && !capturing) {
        e = hipEventRecord(h->fwd_done, st);
        if (e != hipSuccess) return device_fail(e, "hipEventRecord");
    }
    return ok();
}

proj_status proj_back_pixels(proj_handle h, const float *sino_dev, const int32_t *pixels_dev, int64_t n,
                             float *cyl_dev, void *hip_stream) {
    const proj_status s0 = check_batch(h, pixels_dev, n, cyl_dev, sino_dev);
    if (s0 != PROJ_OK) return s0;
    if (n == 0 || h->plan.g.ns == 0) return ok();
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return device_fail(dg.err, "hipSetDevice");
    hipStream_t st = (hipStream_t)hip_stream;
    hipError_t e;
    if (h->plan.back_sl == 0) {
        e = launch_fill_zero(cyl_dev, n * h->plan.g.ns, st);     // no views or empty detector
        if (e != hipSuccess) return device_fail(e, "zero fill");
        return ok();
    }
    // a large batch reads a copy of the sinogram packed into the handle's
    // accumulation buffer (parallel) or its transposed sinogram (cone), so it
    // is ordered like the forwards that share it
    const bool packs = back_pixels_packs(h->plan, n);
    bool capturing = false;
    if (packs) {
        e = stream_capturing(st, capturing);
        if (e != hipSuccess) return device_fail(e, "hipStreamIsCapturing");
        if (!capturing) {
            e = hipStreamWaitEvent(st, h->fwd_done, 0);
            if (e != hipSuccess) return device_fail(e, "hipStreamWaitEvent");
        }
    }
    e = launch_back_pixels(h->plan, sino_dev, pixels_dev, (int)n, cyl_dev, st);
    if (e != hipSuccess) return device_fail(e, "batch back projection launch");
    if (packs && !capturing) {
        e = hipEventRecord(h->fwd_done, st);
        if (e != hipSuccess) return device_fail(e, "hipEventRecord");
    }
    return ok();
}

// ------------------------------------------------------------------ solvers
namespace {

constexpr int SC_R2 = 0, SC_Y2 = 1, SC_Q2 = 2, SC_G = 3;   // SC_G and SC_G + 1: gamma, alternating

int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

int64_t solver_bytes(const proj_handle_s *h) {
    return 256 + align256((int64_t)kVecMaxBlocks * 8) + 2 * align256(h->sino_elems * 4) +
           2 * align256(h->recon_elems * 4);
}

struct Work {
    double *sc, *red;
    float *sa, *sb;   // sinogram-sized
    float *ra, *rb;   // volume-sized
};

Work carve(void *base, const proj_handle_s *h) {
    char *b = (char *)base;
    Work w;
    w.sc = (double *)b;
    b += 256;
    w.red = (double *)b;
    b += align256((int64_t)kVecMaxBlocks * 8);
    w.sa = (float *)b;
    b += align256(h->sino_elems * 4);
    w.sb = (float *)b;
    b += align256(h->sino_elems * 4);
    w.ra = (float *)b;
    b += align256(h->recon_elems * 4);
    w.rb = (float *)b;
    return w;
}

proj_status solver_checks(proj_handle h, const float *y, const float *x0, float *x, void *work, int64_t wbytes,
                          int32_t iterations, double atol, double rtol, proj_solver_info *info) {
    if (!h) return fail(PROJ_ERR_INVALID_ARGUMENT, "null handle");
    if (!info) return fail(PROJ_ERR_INVALID_ARGUMENT, "null info");
    if (iterations < 0) return fail(PROJ_ERR_INVALID_ARGUMENT, "negative iteration count");
    if (!std::isfinite(atol) || !std::isfinite(rtol) || atol < 0 || rtol < 0)
        return fail(PROJ_ERR_INVALID_ARGUMENT, "atol and rtol must be finite and >= 0");
    if ((h->sino_elems > 0 && !y) || (h->recon_elems > 0 && !x))
        return fail(PROJ_ERR_INVALID_ARGUMENT, "null data pointer");
    if (!work || ((uintptr_t)work & 255)) return fail(PROJ_ERR_INVALID_ARGUMENT, "workspace null or not 256-byte aligned");
    if (wbytes < solver_bytes(h)) return fail(PROJ_ERR_INVALID_ARGUMENT, "workspace smaller than proj_solver_workspace_size");
    const int64_t sb = h->sino_elems * 4, rb = h->recon_elems * 4, wb = solver_bytes(h);
    if (overlaps(y, sb, x, rb) || overlaps(y, sb, work, wb) || overlaps(x, rb, work, wb))
        return fail(PROJ_ERR_ALIAS, "sino, recon and workspace overlap");
    if (x0 && x0 != x && (overlaps(x0, rb, x, rb) || overlaps(x0, rb, y, sb) || overlaps(x0, rb, work, wb)))
        return fail(PROJ_ERR_ALIAS, "x0 overlaps another buffer");
    return ok();
}

// Host reads of the device scalars: the one synchronisation of an iteration.
proj_status read_scalars(const Work &w, double *hs, hipStream_t st) {
    hipError_t e = hipMemcpyAsync(hs, w.sc, 8 * sizeof(double), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    return e == hipSuccess ? ok() : device_fail(e, "reading solver scalars");
}

#define BPAMD_TRY(call, what)                                                                                 \
    do {                                                                                                      \
        const hipError_t e_ = (call);                                                                         \
        if (e_ != hipSuccess) return device_fail(e_, what);                                                   \
    } while (0)
#define BPAMD_TRYS(call)                                                                                      \
    do {                                                                                                      \
        const proj_status s_ = (call);                                                                        \
        if (s_ != PROJ_OK) return s_;                                                                         \
    } while (0)

// x = x0, or 0 without x0
hipError_t start_iterate(proj_handle h, const float *x0, float *x, hipStream_t st) {
    if (x0 == x) return hipSuccess;
    if (!x0) return launch_vec(V_FILL, x, nullptr, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, h->recon_elems, nullptr, -1,
                               nullptr, st);
    return launch_vec(V_COPY, x, x0, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, h->recon_elems, nullptr, -1, nullptr, st);
}

}  // namespace

proj_status proj_solver_workspace_size(proj_handle h, int64_t *bytes) {
    if (!h || !bytes) return fail(PROJ_ERR_INVALID_ARGUMENT, "null handle or output");
    *bytes = solver_bytes(h);
    return ok();
}

proj_status proj_cgls(proj_handle h, const float *sino_dev, const float *x0_dev, float *recon_dev, void *work_dev,
                      int64_t work_bytes, int32_t iterations, double atol, double rtol, double *residual_history,
                      proj_solver_info *info, void *hip_stream) {
    BPAMD_TRYS(solver_checks(h, sino_dev, x0_dev, recon_dev, work_dev, work_bytes, iterations, atol, rtol, info));
    *info = proj_solver_info{0, 0, PROJ_STOP_ITERATIONS, 0};
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return device_fail(dg.err, "hipSetDevice");
    hipStream_t st = (hipStream_t)hip_stream;
    const Work w = carve(work_dev, h);
    const int64_t nr = h->recon_elems, ns = h->sino_elems;
    float *r = w.sa, *q = w.sb, *s = w.ra, *p = w.rb, *x = recon_dev;
    double hs[8];
    BPAMD_TRY(start_iterate(h, x0_dev, x, st), "initial iterate");
    BPAMD_TRY(launch_vec(V_NORM, nullptr, sino_dev, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, ns, w.red, SC_Y2, w.sc, st),
              "norm");
    if (x0_dev) {       // r = y - A x0
        BPAMD_TRYS(proj_forward(h, x, q, st));
        BPAMD_TRY(launch_vec(V_SUB_NORM, r, sino_dev, q, nullptr, 0, 0, 0.0, 0.f, 0, ns, w.red, SC_R2, w.sc, st),
                  "residual");
    } else {            // r = y
        BPAMD_TRY(launch_vec(V_COPY, r, sino_dev, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, ns, nullptr, -1, nullptr, st),
                  "copy");
        BPAMD_TRY(launch_vec(V_NORM, nullptr, r, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, ns, w.red, SC_R2, w.sc, st),
                  "norm");
    }
    BPAMD_TRYS(proj_back(h, r, s, st));
    BPAMD_TRY(launch_vec(V_NORM, nullptr, s, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, nr, w.red, SC_G, w.sc, st), "norm");
    BPAMD_TRY(launch_vec(V_COPY, p, s, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, nr, nullptr, -1, nullptr, st), "copy");
    BPAMD_TRYS(read_scalars(w, hs, st));
    const double tol = atol + rtol * std::sqrt(hs[SC_Y2]);
    double res = std::sqrt(hs[SC_R2]);
    double gamma = hs[SC_G];
    if (residual_history) residual_history[0] = res;
    if (res <= tol) {
        info->converged = 1;
        info->reason = PROJ_STOP_CONVERGED;
        return ok();
    }
    for (int it = 0; it < iterations; ++it) {
        const int gs = SC_G + (it & 1), gn = SC_G + ((it + 1) & 1);
        if (gamma == 0.0) {
            info->reason = PROJ_STOP_STATIONARY;
            return ok();
        }
        BPAMD_TRYS(proj_forward(h, p, q, st));
        BPAMD_TRY(launch_vec(V_NORM, nullptr, q, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, ns, w.red, SC_Q2, w.sc, st),
                  "norm");
        // x += alpha p and r -= alpha q, alpha = gamma / ||q||^2 read on the device
        BPAMD_TRY(launch_vec(V_AXPY, x, nullptr, p, w.sc, gs, SC_Q2, 1.0, 0.f, 0, nr, nullptr, -1, nullptr, st),
                  "update");
        BPAMD_TRY(launch_vec(V_AXPY, r, nullptr, q, w.sc, gs, SC_Q2, -1.0, 0.f, 0, ns, w.red, SC_R2, w.sc, st),
                  "update");
        BPAMD_TRYS(proj_back(h, r, s, st));
        BPAMD_TRY(launch_vec(V_NORM, nullptr, s, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, nr, w.red, gn, w.sc, st),
                  "norm");
        BPAMD_TRYS(read_scalars(w, hs, st));   // the residual and the normal-equation norm, together
        if (hs[SC_Q2] == 0.0) {                // alpha was 0: nothing changed
            info->reason = PROJ_STOP_BREAKDOWN;
            return ok();
        }
        res = std::sqrt(hs[SC_R2]);
        info->iterations = it + 1;
        if (residual_history) residual_history[it + 1] = res;
        if (res <= tol) {
            info->converged = 1;
            info->reason = PROJ_STOP_CONVERGED;
            return ok();
        }
        const double gamma_new = hs[gn];
        if (gamma_new != 0.0)   // p = s + (gamma_new / gamma) p
            BPAMD_TRY(launch_vec(V_XPBY, p, s, nullptr, w.sc, gn, gs, 1.0, 0.f, 0, nr, nullptr, -1, nullptr, st),
                      "update");
        gamma = gamma_new;
    }
    info->reason = gamma == 0.0 ? PROJ_STOP_STATIONARY : PROJ_STOP_ITERATIONS;
    return ok();
}

proj_status proj_sirt(proj_handle h, const float *sino_dev, const float *x0_dev, float *recon_dev, void *work_dev,
                      int64_t work_bytes, int32_t iterations, double atol, double rtol, double relaxation,
                      int32_t nonnegative, double *residual_history, proj_solver_info *info, void *hip_stream) {
    BPAMD_TRYS(solver_checks(h, sino_dev, x0_dev, recon_dev, work_dev, work_bytes, iterations, atol, rtol, info));
    if (!std::isfinite(relaxation) || relaxation <= 0) return fail(PROJ_ERR_INVALID_ARGUMENT, "relaxation must be finite and > 0");
    *info = proj_solver_info{0, 0, PROJ_STOP_ITERATIONS, 0};
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return device_fail(dg.err, "hipSetDevice");
    hipStream_t st = (hipStream_t)hip_stream;
    const Work w = carve(work_dev, h);
    const int64_t nr = h->recon_elems, ns = h->sino_elems;
    float *rw = w.sa, *t = w.sb, *cw = w.ra, *u = w.rb, *x = recon_dev;
    const int nn = nonnegative ? 1 : 0;
    double hs[8];
    BPAMD_TRY(start_iterate(h, x0_dev, x, st), "initial iterate");
    BPAMD_TRY(launch_vec(V_NORM, nullptr, sino_dev, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, ns, w.red, SC_Y2, w.sc, st),
              "norm");
    // R = 1 / (A 1), C = 1 / (A^T 1)
    BPAMD_TRY(launch_vec(V_FILL, u, nullptr, nullptr, nullptr, 0, 0, 0.0, 1.f, 0, nr, nullptr, -1, nullptr, st), "fill");
    BPAMD_TRYS(proj_forward(h, u, rw, st));
    BPAMD_TRY(launch_vec(V_RECIP, rw, nullptr, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, ns, nullptr, -1, nullptr, st),
              "weights");
    BPAMD_TRY(launch_vec(V_FILL, t, nullptr, nullptr, nullptr, 0, 0, 0.0, 1.f, 0, ns, nullptr, -1, nullptr, st), "fill");
    BPAMD_TRYS(proj_back(h, t, cw, st));
    BPAMD_TRY(launch_vec(V_RECIP, cw, nullptr, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, nr, nullptr, -1, nullptr, st),
              "weights");
    // t = R (y - A x), ||y - A x||^2
    if (x0_dev)
        BPAMD_TRYS(proj_forward(h, x, t, st));
    else
        BPAMD_TRY(launch_vec(V_FILL, t, nullptr, nullptr, nullptr, 0, 0, 0.0, 0.f, 0, ns, nullptr, -1, nullptr, st),
                  "fill");
    BPAMD_TRY(launch_vec(V_SIRT_RES, t, sino_dev, rw, nullptr, 0, 0, 0.0, 0.f, 0, ns, w.red, SC_R2, w.sc, st),
              "residual");
    BPAMD_TRYS(read_scalars(w, hs, st));
    const double tol = atol + rtol * std::sqrt(hs[SC_Y2]);
    double res = std::sqrt(hs[SC_R2]);
    if (residual_history) residual_history[0] = res;
    if (res <= tol) {
        info->converged = 1;
        info->reason = PROJ_STOP_CONVERGED;
        return ok();
    }
    for (int it = 0; it < iterations; ++it) {
        BPAMD_TRYS(proj_back(h, t, u, st));
        BPAMD_TRY(launch_vec(V_SIRT_UPD, x, u, cw, nullptr, 0, 0, 0.0, relaxation, nn, nr, nullptr, -1,
                             nullptr, st),
                  "update");
        BPAMD_TRYS(proj_forward(h, x, t, st));
        BPAMD_TRY(launch_vec(V_SIRT_RES, t, sino_dev, rw, nullptr, 0, 0, 0.0, 0.f, 0, ns, w.red, SC_R2, w.sc, st),
                  "residual");
        BPAMD_TRYS(read_scalars(w, hs, st));
        res = std::sqrt(hs[SC_R2]);
        info->iterations = it + 1;
        if (residual_history) residual_history[it + 1] = res;
        if (res <= tol) {
            info->converged = 1;
            info->reason = PROJ_STOP_CONVERGED;
            return ok();
        }
    }
    return ok();
}

}  // extern "C"
