// Internals shared by the C-ABI sources: the handle, and the error and
// argument helpers every entry point uses.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "../../include/proj.h"
#include "launch.h"

namespace bpamd {

constexpr int64_t kMaxElems = (int64_t)1 << 31;      // work arrays stay below 2^31 elements

// Record `why` as the calling thread's last error and return `s`.
proj_status fail(proj_status s, const std::string &why);
// Clear the last error and return PROJ_OK.
proj_status ok();

inline bool overlaps(const void *a, int64_t na, const void *b, int64_t nb) {
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return na > 0 && nb > 0 && pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

struct DeviceGuard {
    int prev = -1;
    bool switched = false;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) {
            err = hipSetDevice(dev);
            switched = err == hipSuccess;
        }
    }
    ~DeviceGuard() {
        if (switched) (void)hipSetDevice(prev);
    }
};

inline proj_status device_fail(hipError_t e, const char *what) {
    return fail(e == hipErrorOutOfMemory ? PROJ_ERR_OUT_OF_MEMORY : PROJ_ERR_DEVICE,
                std::string(what) + ": " + hipGetErrorString(e));
}

// The parallel forward's accumulation buffer belongs to the handle, so a
// forward first waits on the GPU for the handle's previous one (an event; no
// host synchronisation) and then records its own end.  While `st` is being
// captured into a graph neither happens: an event recorded outside a capture
// cannot be waited on inside it, and within a graph the captured launches are
// ordered by the graph itself (two forwards on one handle must then not run
// concurrently, the caller's ordering).
inline hipError_t stream_capturing(hipStream_t st, bool &capturing) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(st, &cs);
    capturing = e == hipSuccess && cs != hipStreamCaptureStatusNone;
    return e;
}

}  // namespace bpamd

struct proj_handle_s {
    int device = 0;
    bpamd::Plan plan;
    int64_t recon_elems = 0, sino_elems = 0, index_elems = 0;
    bpamd::ViewK *d_views = nullptr;
    int32_t *d_idx = nullptr;
    int32_t *d_rec = nullptr;       // parallel tap records
    uint32_t *d_wrec = nullptr;     // parallel forward walk steps
    float *d_facc = nullptr;        // parallel forward accumulation buffer (slices fastest)
    int32_t *d_bsort = nullptr;     // parallel batch forward: sorted records, then key offsets
    int bsort_nb = 0;               // entries per batch sort pass
    float *d_ctr = nullptr;         // cone batches: the sinogram transposed [V][C][R]
    float *d_col = nullptr;         // column forward (translation scans): column sums [Nx][S]
    hipEvent_t fwd_done = nullptr;  // parallel: last forward on this handle, orders calls that share d_facc
    bpamd::Window *d_bwin = nullptr;       // back projection windows per (view, tile, chunk)
    bpamd::Window *d_fwin = nullptr;       // cone forward windows per (view, tile, chunk)
    bpamd::Window *d_fslab = nullptr;      // cone forward active slices per (view, tile, chunk)
    size_t table_bytes = 0;
};
