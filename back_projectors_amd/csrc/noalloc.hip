// proj_forward_noalloc: the forward projection for callers that cannot
// allocate device memory.  It runs the kernels of proj_forward; the one
// difference is where the parallel-beam walk adds its partial sums: into a
// fixed device array of this file instead of the accumulation buffer the
// handle allocated.  The cone forward adds straight into the sinogram and
// needs no scratch.
#include <mutex>

#include "api_common.h"

using namespace bpamd;

// Largest accumulation buffer the fixed array holds, [V][C + 2 (taps - 1)]
// [S rounded up to 16 or 32] fp32: 144 MiB covers the 512 x 512 x 64,
// 720-view scan (142 MB).  Every GPU the library runs a kernel on holds one
// copy until the process ends.
constexpr int64_t kNoallocScratchBytes = (int64_t)144 << 20;

static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch[kMaxDevices] = {};

// The device address of `scratch` on device `dev`, which must be current.
// Resolved once per device: host code never passes the array's own name to a
// kernel or a copy (on the host that name is a stand-in, not the GPU address).
hipError_t scratch_address(int dev, float **out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = static_cast<float *>(p);
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" proj_status proj_forward_noalloc(proj_handle h, const float *recon_dev, float *sino_dev,
                                            void *hip_stream) {
    if (!h) return fail(PROJ_ERR_INVALID_ARGUMENT, "null handle");
    if ((h->recon_elems > 0 && !recon_dev) || (h->sino_elems > 0 && !sino_dev))
        return fail(PROJ_ERR_INVALID_ARGUMENT, "null data pointer");
    if (overlaps(recon_dev, h->recon_elems * 4, sino_dev, h->sino_elems * 4))
        return fail(PROJ_ERR_ALIAS, "recon and sino buffers overlap");
    if (h->device < 0 || h->device >= kMaxDevices)
        return fail(PROJ_ERR_UNSUPPORTED, "device ordinal above 63");
    const Plan &plan = h->plan;
    const bool par = plan.g.kind == 0;
    const bool work = plan.back_sl != 0;      // 0: empty volume or no views, the sinogram is zero
    // (the column forward of a translation scan needs only its column sums)
    const bool colf = par && plan.fwd_strategy == kForwardColumn;
    const int64_t need = !(par && work) ? 0
                         : colf         ? (int64_t)plan.g.nx * plan.g.ns * (int64_t)sizeof(float)
                                        : (int64_t)plan.g.nv * plan.fwd_cb * plan.fwd_s16 * (int64_t)sizeof(float);
    if (need > kNoallocScratchBytes)
        return fail(PROJ_ERR_UNSUPPORTED, "the forward needs " + std::to_string(need) +
                                              " bytes of accumulation buffer, more than the fixed 144 MiB "
                                              "scratch of proj_forward_noalloc (use proj_forward)");
    if (h->sino_elems == 0) return ok();
    DeviceGuard dg(h->device);
    if (dg.err != hipSuccess) return device_fail(dg.err, "hipSetDevice");
    hipStream_t st = (hipStream_t)hip_stream;
    float *ptr = nullptr;
    hipError_t e = hipSuccess;
    if (par && work) {
        e = scratch_address(h->device, &ptr);
        if (e != hipSuccess) return device_fail(e, "hipGetSymbolAddress(scratch)");
    }
    if (!work || !par) {
        e = launch_fill_zero(sino_dev, h->sino_elems, st);
        if (e != hipSuccess) return device_fail(e, "zero fill");
    }
    if (!work) return ok();
    if (!par) {
        e = launch_cone_forward(plan, recon_dev, sino_dev, false, st);
        if (e != hipSuccess) return device_fail(e, "forward projection launch");
        return ok();
    }
    // the walk, its zero fill and the unpack (or the column sums) use the
    // fixed array in place of the handle's buffer (the fill clears what the
    // last call left there; the column sums overwrite it)
    Plan p = plan;
    p.facc = ptr;
    p.col = ptr;
    e = launch_par_forward(p, recon_dev, sino_dev, st);
    if (e != hipSuccess) return device_fail(e, "forward projection launch");
    return ok();
}
