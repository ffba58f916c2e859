// Host-side launch plan and the launchers each kernel file exports.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "geom.h"

namespace bpamd {

// Everything a launch needs, fixed at creation from the shapes and the
// geometry alone (never from data).
struct Plan {
    Geo g;
    const ViewK *views = nullptr;   // device [V]
    const int32_t *idx = nullptr;   // device [V][Ny*Nx]
    const int32_t *rec = nullptr;   // parallel: device tap records [V][Ny*Nx][1 + ntap]
    const uint32_t *wrec = nullptr; // parallel: forward walk records [V + 1][regions][groups][2 + ntap][16]
    float *facc = nullptr;          // parallel: forward accumulation buffer [V][fwd_cb][fwd_s16]
    int fwd_cb = 0;                 // parallel: channels of facc (C plus ntap - 1 guards each side)
    int fwd_s16 = 0;                // parallel: slices of facc (S rounded up to 16 * fwd_spl)
    int fwd_spl = 1;                // parallel region walk: adjacent slices per lane (1 or 2)
    int rsx = 0, rsy = 0;           // parallel: forward region (pixels along x, y)
    int fwd_nbin = 0;               // parallel: bins of the walk-order sort (n_f span of a region + 2)
    int fwd_strategy = 1;           // parallel: 1 tile (region walk), 2 gather (per-view sorted walk)
    int gat_ng = 0;                 // gather: groups of 16 steps per view (all pixels, multiple of 4)
    int gat_segg = 0;               // gather: groups per segment (multiple of 4)
    int gat_nseg = 0;               // gather: segments per view
    const int4 *bwin = nullptr;     // back windows [V][tiles][chunks] (n0, nw, m0, nrw)
    const int4 *fwin = nullptr;     // cone forward windows [V][tiles][chunks]
    const int4 *fslab = nullptr;    // cone forward slabs [V][tiles][chunks] (first slice, passes, unit stride, 0)
    int ntap = 0;                   // parallel: taps per record
    int32_t *bsort = nullptr;       // parallel batch forward: sorted records [V][2 + ntap][bsort_nb] (null: atomics)
    int32_t *boff = nullptr;        // parallel batch forward: key offsets [V][fwd_cb + 1]
    int bsort_nb = 0;               // parallel batch forward: entries per sort pass
    float *ctr = nullptr;           // cone batches: the sinogram transposed, [V][C][R] (null: direct forms)
    int colmode = 0;                // parallel, every view at angle 0 (sin exactly 0): the column forms
    float *col = nullptr;           // column forward: the column sums [Nx][S]

    // back projection: lanes = pixels of a BT x BT tile, SL slices per lane
    int back_sl = 0;                // slices per chunk (accumulators per lane)
    int back_nwcap = 0;             // window channels capacity
    int back_nrcap = 0;             // window rows capacity (cone)
    int back_pc = 0;                // cone back LDS channel pitch: 33, 65, 129 or 257 (odd, compile-time in the kernel)
    size_t back_lds = 0;            // dynamic LDS bytes
    int back_ncg = 1;               // parallel back: 32-channel staging groups (1 or 2)

    // forward projection (parallel: FTX x FTY tiles; cone: CTX x CTY tiles)
    int fwd_sl = 0;
    int fwd_nwcap = 0;
    int fwd_nrcap = 0;
    size_t fwd_lds = 0;
    int fwd_vsplit = 1;             // view ranges per tile (grid z)
    int cone_stride = 1;            // cone forward: slices between the lanes of one instruction
    int cone_unit = 0;              // cone forward: some slab saves work (the slab-reading kernel)
    int cone_ty = 4;                // cone forward: tile rows (CTX x cone_ty pixels, 4 or 8)
    int cone_ncol = 1;              // cone forward: row-profile columns per wave (1, or cone_stride: interleaved slabs)
};

// Plan::fwd_strategy of the column forward (the public forward_strategy value
// that asks for it).
constexpr int kForwardColumn = 5;
constexpr int BT = 16;   // back tile edge (pixels), 256 threads
constexpr int FRW = 16;  // parallel forward waves per workgroup (four views each at a time)
constexpr int FRS = 48;  // parallel forward region edge (pixels): 48 * 48 voxels of 16 slices = 144 KiB of LDS
// the same with two slices per lane: 40 x 32 voxels of 32 slices fill the
// 160 KiB of LDS (fewer channel flushes per step than 32 x 32: 1.82 -> 1.70 ms
// at 512 x 512 x 64, 720 views)
constexpr int FRS2X = 40;
constexpr int FRS2Y = 32;

// Groups of 16 walk steps per (view, region): every pixel of the region, then
// zero steps up to a multiple of 5 groups (the walk rotates five record buffers).
inline int fwd_groups(int rsx, int rsy) { return ((rsx * rsy + 79) / 80) * 5; }
constexpr int CTX = 8;   // cone forward tile (pixels along x); 4 or 8 rows of them (Plan::cone_ty)
constexpr int CFW = 4;   // cone forward waves per workgroup (one view each at a time)
// LDS floats of one cone forward wave: its detector window [nwcap][nrp] and
// ncol row-profile columns [ncol][nrp] (rows of the window, the first
// projection step; with ncol = stride, lanes of one instruction add into
// column lane mod stride where a slab takes consecutive slices on rows
// closer than one apart)
__host__ __device__ inline int cone_fwd_wave_words(int nrp, int ncol) { return ncol * nrp; }

hipError_t launch_channel_index(const Geo &g, const ViewK *views, int32_t *idx, hipStream_t st);
hipError_t launch_par_taps(const Geo &g, const ViewK *views, int32_t *rec, int ntap, hipStream_t st);
hipError_t launch_par_region_records(const Geo &g, const int32_t *rec, uint32_t *out, int ntap, int rsx, int rsy,
                                    int nbin, int spl, hipStream_t st);
hipError_t launch_par_view_records(const Geo &g, const int32_t *rec, int32_t *order, uint32_t *out, int ntap,
                                  int ng, int segg, hipStream_t st);
hipError_t launch_fill_zero(float *buf, int64_t n, hipStream_t st);

// power 1: the adjoint of the forward; power 2: every tap weight squared
hipError_t launch_par_back(const Plan &p, const float *sino, float *recon, int power, hipStream_t st);
hipError_t launch_par_forward(const Plan &p, const float *recon, float *sino, hipStream_t st);
hipError_t par_forward_allow_lds(int ntap, int spl, size_t bytes);
// the slice-fastest accumulation buffer -> the sinogram (parallel beam)
hipError_t launch_par_unpack(const Plan &p, float *sino, hipStream_t st);
// buf [V][cb][s] (rows fastest, guard channels on each side) -> sino [V][R][C]
hipError_t launch_unpack_rows(const float *buf, float *sino, int nv, int nr, int nc, int cb, int s, int guard,
                              hipStream_t st);
// batches of voxel cylinders (entries outside [0, Ny*Nx) are inert padding)
// Entries per pass of the parallel batch forward's sort at most (4 per thread
// of its 1024-thread workgroup).
constexpr int kBatchPass = 4096;
// LDS bytes of the batch sort: a count per key (cb + 1) and the pass's sorted
// records (2 + ntap fields of nb entries).
inline size_t batch_sort_lds(int cb, int ntap, int nb) {
    return ((size_t)cb + 1 + (size_t)(2 + ntap) * nb) * sizeof(int);
}
hipError_t batch_sort_allow_lds(int ntap, size_t bytes);
// Whether the parallel batch back of n entries reads a slice-fastest copy of
// the sinogram (packed into facc first) rather than the sinogram itself.
bool back_pixels_packs(const Plan &p, int64_t n);
hipError_t launch_back_pixels(const Plan &p, const float *sino, const int32_t *pix, int n, float *cyl,
                              hipStream_t st);
hipError_t launch_forward_pixels(const Plan &p, const int32_t *pix, int n, const float *cyl, float *sino,
                                 hipStream_t st);
// Solver vector steps (csrc/solver.hip).  The elementwise steps:  d, a, b are vectors of n floats; `red` (when not
// null) receives one fp64 partial sum per block of the squared values noted.
enum VecOp : int {
    V_FILL = 0,      // d = value
    V_COPY,          // d = a
    V_RECIP,         // d = d > 0 ? 1/d : 0
    V_NORM,          // red += a^2
    V_SUB_NORM,      // d = a - b, red += d^2
    V_AXPY,          // d = d + c b, c = sign sc[num]/sc[den]; red += d^2 when asked
    V_XPBY,          // d = a + c d, c = sc[num]/sc[den]
    V_SIRT_RES,      // e = a - d (a = y, d = A x), red += e^2, d = b e (b = row weights)
    V_SIRT_UPD,      // d = d + value b a (b = column weights, a = back projection), clamped at 0 when flag
                     // (AXPY, XPBY and SIRT_UPD compute in fp64 and round once)
};

constexpr int kVecMaxBlocks = 1024;   // partial sums per reduction at most
// One vector step over n floats; when `red` is given, the per-block partial
// sums go there and, when sc_out >= 0, their total into sc_w[sc_out].
hipError_t launch_vec(int op, float *d, const float *a, const float *b, const double *sc, int num, int den,
                      double sign, double value, int flag, int64_t n, double *red, int sc_out, double *sc_w,
                      hipStream_t st);

hipError_t launch_cone_back(const Plan &p, const float *sino, float *recon, int power, hipStream_t st);
// transposed: sino is the handle's [V][C][R] buffer (then unpacked), else the
// caller's [V][R][C] sinogram; either must hold zeros
hipError_t launch_cone_forward(const Plan &p, const float *recon, float *sino, bool transposed, hipStream_t st);
hipError_t cone_forward_allow_lds(int radius, int stride, int ty, int rows, size_t bytes);

}  // namespace bpamd
