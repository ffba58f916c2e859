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
// Lanes are slices, 64 per chunk.  The per-(view, pixel) quantities are
// those of the full projectors: the parallel tap records evaluated with the
// creation pass's own fp64 code (the same bits as its table, without a
// scattered read of it per listed pixel), the cone's channel index from the
// table and then the same fp64 footprint.  The parallel forward sorts each
// view's entries by channel and writes whole sinogram rows; the parallel back
// and the cone kernels take one listed pixel per workgroup or wave.  These
// kernels serve batches, not whole volumes.
#include <algorithm>
#include <cmath>

#include "chan.h"
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

// Parallel back at the listed pixels: per view the pixel's tap record and
// NTAP detector cells of each slice's row.  A workgroup takes one listed pixel
// and 64 slices; its four waves take a quarter of the views each, and the
// four partial sums are added in a fixed order at the end.  In a wave the
// records of 64 views come in with one vector load per field (lane l: view vb
// + l, the next 64 views' meanwhile) and reach the wave by readlane, and the
// cells of the next PB_U views are loaded while the current ones are summed,
// so the wave waits on few round trips.  With PK the cells come from the
// slice-fastest copy of the sinogram (guard channels zero): a tap of 64
// slices is 256 consecutive bytes, where in the [V][R][C] sinogram it is 64
// rows apart.  A tap off the detector adds an exact zero in one form and is
// left out in the other, and the order of the sums is the same, so the two
// give the same bits.
constexpr int PB_U = 8;                           // views per load group of the batch back

template <int NTAP, bool PK>
__global__ __launch_bounds__(256) void par_back_pixels_kernel(const float *__restrict__ src,
                                                              const int32_t *__restrict__ pix, int n,
                                                              float *__restrict__ cyl,
                                                              const ViewK *__restrict__ views, Geo g, int cb,
                                                              int s16) {
    __shared__ float part[4][64];
    const int lane = (int)threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int i = (int)blockIdx.x;
    const int np = g.ny * g.nx;
    const int k = (int)blockIdx.y * 64 + lane;
    const int kc = min(k, g.ns - 1);                // lanes past the last slice load a valid cell, store nothing
    const int p = listed_pixel(pix, i, np);
    const int vper = (g.nv + 3) / 4;
    const int vbeg = wave * vper, vend = min(g.nv, vbeg + vper);
    float acc = 0.f;
    if (p >= 0 && vbeg < vend) {
        // tap records of views vb .. vb + 63 (lane l: view vb + l, clamped
        // into this wave's range), evaluated with the same fp64 operations as
        // the creation pass's table: the same bits, where reading the table
        // would fetch a cache line per view for 12 bytes
        const int pi = p / g.nx, pj = p % g.nx;
        auto load_recs = [&](int vb, int &rnf, int (&rw)[NTAP]) {
            float w[NTAP];
            rnf = par_tap_record(g, views[min(vb + lane, vend - 1)], pi, pj, NTAP, w);
#pragma unroll
            for (int t = 0; t < NTAP; ++t) rw[t] = __float_as_int(w[t]);
        };
        // cells and weights of views vb + j0 .. vb + j0 + PB_U - 1; a view
        // without a footprint here, or past the group, adds 0 x 0 (exact: the
        // sum is never -0).  With PK, lane l has formed view vb + l's column
        // address and weights (colp, cw), which the wave reads out per view.
        auto load_cells = [&](int vb, int cnt, int j0, int rnf, const int (&rw)[NTAP], uint64_t colp,
                              const float (&cw)[NTAP], float (&x)[PB_U][NTAP], float (&w)[PB_U][NTAP]) {
#pragma unroll
            for (int u = 0; u < PB_U; ++u) {
                const int j = min(j0 + u, cnt - 1);
                if (PK) {
                    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)colp, j);
                    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(colp >> 32), j);
                    // (a global address-space pointer: a generic one makes flat loads)
                    const __attribute__((address_space(1))) float *col =
                        reinterpret_cast<const __attribute__((address_space(1))) float *>(((uint64_t)hi << 32) | lo);
                    const bool in = j0 + u < cnt;
#pragma unroll
                    for (int t = 0; t < NTAP; ++t) {
                        const float val = col[(uint32_t)(kc + t * s16)];
                        x[u][t] = in ? val : 0.f;      // (a slot past the group reads a real cell)
                        w[u][t] = in ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cw[t]), j)) : 0.f;
                    }
                    continue;
                }
                const int nf = __builtin_amdgcn_readlane(rnf, j);
                const bool on = j0 + u < cnt && nf != INT32_MAX;
                const int v = vb + j;
                {
                    const float *row = src + ((int64_t)v * g.nr + kc) * g.nc;
#pragma unroll
                    for (int t = 0; t < NTAP; ++t) {
                        const int c = nf + t;
                        const bool in = on && c >= 0 && c < g.nc;
                        const float val = row[in ? c : 0];
                        x[u][t] = in ? val : 0.f;
                    }
                }
#pragma unroll
                for (int t = 0; t < NTAP; ++t) w[u][t] = on ? __int_as_float(__builtin_amdgcn_readlane(rw[t], j)) : 0.f;
            }
        };
        int rnf, rw[NTAP], nnf, nw[NTAP];
        load_recs(vbeg, rnf, rw);
        for (int vb = vbeg; vb < vend; vb += 64) {
            const int cnt = min(64, vend - vb);
            load_recs(vb + 64, nnf, nw);
            // PK: lane l's view vb + l, its tap column in the packed copy (the
            // zero guard column 0 where the view has no footprint or lies
            // past the range) and its weights (zero there)
            uint64_t colp = 0;
            float cw[NTAP];
            if (PK) {
                const bool on = vb + lane < vend && rnf != INT32_MAX;
                colp = reinterpret_cast<uint64_t>(
                    src + ((int64_t)min(vb + lane, vend - 1) * cb + (on ? rnf + NTAP - 1 : 0)) * s16);
#pragma unroll
                for (int t = 0; t < NTAP; ++t) cw[t] = on ? __int_as_float(rw[t]) : 0.f;
            }
            float x[PB_U][NTAP], w[PB_U][NTAP];
            load_cells(vb, cnt, 0, rnf, rw, colp, cw, x, w);
            for (int j0 = 0; j0 < cnt; j0 += PB_U) {
                float xn[PB_U][NTAP], wn[PB_U][NTAP];
                load_cells(vb, cnt, j0 + PB_U, rnf, rw, colp, cw, xn, wn);   // (past the group: clamped, adds nothing)
#pragma unroll
                for (int u = 0; u < PB_U; ++u)
#pragma unroll
                    for (int t = 0; t < NTAP; ++t) acc = fmaf(w[u][t], x[u][t], acc);
#pragma unroll
                for (int u = 0; u < PB_U; ++u)
#pragma unroll
                    for (int t = 0; t < NTAP; ++t) {
                        x[u][t] = xn[u][t];
                        w[u][t] = wn[u][t];
                    }
            }
            rnf = nnf;
#pragma unroll
            for (int t = 0; t < NTAP; ++t) rw[t] = nw[t];
        }
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && k < g.ns)
        cyl[(int64_t)i * g.ns + k] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
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

// Parallel forward of a batch without atomics, in two launches per pass of
// at most kBatchPass entries:
//   1. sort: per view, the pass's entries with a footprint in that view by
//      their first channel nf (a counting sort over the keys nf + NTAP - 1 in
//      LDS: counts, prefix sums, then each entry to its slot); it writes the
//      key offsets [V][cb + 1] and the sorted records field by field
//      [V][2 + NTAP][nbmax] (entry, key, the NTAP fp32 taps);
//   2. walk: a wave owns one view, one part of PB_CW detector channels and one
//      chunk of 64 slices (= rows: lane l is slice and row k0 + l).  The
//      entries whose taps reach the part are one run of the sorted records;
//      the wave adds them into NTAP ring accumulators (slot t holds channel lo
//      + t) and, as the walk passes a channel, writes it into an LDS tile
//      [64 rows][PB_CW channels], which it finally stores as whole sinogram
//      rows.  Every cell of the sinogram is written by exactly one wave, the
//      first pass overwriting and the others adding, so the forward needs no
//      zero fill, no atomics and no unpack.
// The sums over a channel run in sorted order, one rounding per add; the
// entries of one key are in the order their LDS increments landed, which can
// differ between calls (the reference's sum over voxels is in no particular
// order either).
constexpr int PB_SORT_THREADS = 1024;
constexpr int PB_EPT = kBatchPass / PB_SORT_THREADS;      // entries per sort thread
constexpr int PB_CW = 32;                                 // channels per walk part
constexpr int PB_D = 8;                                   // cylinder loads in flight ahead of their entry
static_assert(kBatchPass % PB_SORT_THREADS == 0, "whole entries per sort thread");

// Inclusive prefix sum of s over the threads of a PB_SORT_THREADS workgroup.
__device__ __forceinline__ int block_scan_incl(int s, int *wsum) {
    const int lane = (int)threadIdx.x & 63, wv = (int)threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(s, d, 64);
        if (lane >= d) s += t;
    }
    if (lane == 63) wsum[wv] = s;
    __syncthreads();
    if (wv == 0) {
        int t = lane < PB_SORT_THREADS / 64 ? wsum[lane] : 0;
#pragma unroll
        for (int d = 1; d < PB_SORT_THREADS / 64; d <<= 1) {
            const int u = __shfl_up(t, d, 64);
            if (lane >= d) t += u;
        }
        if (lane < PB_SORT_THREADS / 64) wsum[lane] = t;
    }
    __syncthreads();
    return s + (wv > 0 ? wsum[wv - 1] : 0);
}

template <int NTAP>
__global__ __launch_bounds__(PB_SORT_THREADS) void par_batch_sort_kernel(const int32_t *__restrict__ pix, int b0,
                                                                         int nb, const ViewK *__restrict__ views,
                                                                         Geo g, int cb, int32_t *__restrict__ srt,
                                                                         int32_t *__restrict__ off, int nbmax) {
    constexpr int RS = 2 + NTAP;
    extern __shared__ int hist[];                 // [cb + 1]: counts, then offsets; then the sorted records
    __shared__ int wsum[PB_SORT_THREADS / 64];
    const int v = (int)blockIdx.x, tid = (int)threadIdx.x;
    const int np = g.ny * g.nx;
    for (int c = tid; c <= cb; c += PB_SORT_THREADS) hist[c] = 0;
    __syncthreads();
    // the pixel ids (loads first, clamped so unconditional), then each
    // entry's tap record for this view, evaluated here with the same fp64
    // operations as the creation pass's table (the same bits, without a
    // scattered read of that table per entry)
    int pe[PB_EPT], key[PB_EPT];
    float wr[PB_EPT][NTAP];
#pragma unroll
    for (int u = 0; u < PB_EPT; ++u) pe[u] = pix[b0 + min(tid + u * PB_SORT_THREADS, nb - 1)];
    const ViewK vk = views[v];
#pragma unroll
    for (int u = 0; u < PB_EPT; ++u) {
        const bool in = tid + u * PB_SORT_THREADS < nb && pe[u] >= 0 && pe[u] < np;   // padding takes no slot
        const int q = in ? pe[u] : 0;
        const int nf = par_tap_record(g, vk, q / g.nx, q % g.nx, NTAP, wr[u]);
        key[u] = in && nf != INT32_MAX ? nf + (NTAP - 1) : -1;   // in [0, cb - NTAP + 1)
    }
#pragma unroll
    for (int u = 0; u < PB_EPT; ++u)
        if (key[u] >= 0) atomicAdd(&hist[key[u]], 1);
    __syncthreads();
    // exclusive prefix sums of the counts, each thread a run of consecutive keys
    const int per = (cb + PB_SORT_THREADS - 1) / PB_SORT_THREADS;
    const int c0 = min(tid * per, cb), c1 = min(c0 + per, cb);
    int s = 0;
    for (int c = c0; c < c1; ++c) s += hist[c];
    const int incl = block_scan_incl(s, wsum);
    int run = incl - s;
    for (int c = c0; c < c1; ++c) {
        const int t = hist[c];
        hist[c] = run;
        run += t;
    }
    if (tid == PB_SORT_THREADS - 1) hist[cb] = incl;
    __syncthreads();
    int32_t *ov = off + (int64_t)v * (cb + 1);
    for (int c = tid; c <= cb; c += PB_SORT_THREADS) ov[c] = hist[c];
    __syncthreads();
    // each entry to its slot of the sorted records, in LDS first ([RS][nbmax]
    // after the counts), then out to memory in whole rows: scattered 4-byte
    // stores straight to memory left partly written lines to be merged beyond
    // the cache
    int *lrec = hist + cb + 1;
    const int total = hist[cb];
    int pos[PB_EPT];
#pragma unroll
    for (int u = 0; u < PB_EPT; ++u) pos[u] = key[u] >= 0 ? atomicAdd(&hist[key[u]], 1) : 0;
#pragma unroll
    for (int u = 0; u < PB_EPT; ++u) {
        if (key[u] < 0) continue;
        lrec[pos[u]] = (tid + u * PB_SORT_THREADS) * g.ns;     // the entry's cylinder offset
        lrec[nbmax + pos[u]] = key[u];
#pragma unroll
        for (int t = 0; t < NTAP; ++t) lrec[(2 + t) * nbmax + pos[u]] = __float_as_int(wr[u][t]);
    }
    __syncthreads();
    int32_t *sv = srt + (int64_t)v * RS * nbmax;
#pragma unroll
    for (int f = 0; f < RS; ++f)
        for (int j = tid; j < total; j += PB_SORT_THREADS) sv[(int64_t)f * nbmax + j] = lrec[f * nbmax + j];
}

template <int NTAP>
__global__ __launch_bounds__(SW * 64) void par_batch_walk_kernel(const float *__restrict__ cyl, int b0,
                                                                 const int32_t *__restrict__ srt,
                                                                 const int32_t *__restrict__ off,
                                                                 float *__restrict__ sino, Geo g, int cb, int nbmax,
                                                                 int nparts, int nch, int accumulate) {
    constexpr int RS = 2 + NTAP, G = NTAP - 1;
    __shared__ float tiles[SW][64][PB_CW + 1];    // [row][channel], odd pitch
    const int lane = (int)threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int item = (int)blockIdx.x * SW + wave;
    if (item >= g.nv * nparts * nch) return;      // (no barrier in this kernel)
    const int chunk = item % nch, part = (item / nch) % nparts, v = item / (nch * nparts);
    const int ca = part * PB_CW, ce = min(g.nc, ca + PB_CW);   // this wave's channels [ca, ce)
    const int k0 = chunk * 64;
    const int kc = min(k0 + lane, g.ns - 1);      // lanes past the last slice load a valid voxel, store nothing
    float(*tile)[PB_CW + 1] = tiles[wave];
    // entries whose first channel lies in [ca - G, ce - 1]: keys [ca, ce + G)
    const int32_t *ov = off + (int64_t)v * (cb + 1);
    const int j0 = ov[ca], j1 = ov[ce + G];
    const int32_t *sv = srt + (int64_t)v * RS * nbmax;
    const float *cb0 = cyl + (int64_t)b0 * g.ns + kc;

    float acc[NTAP];
#pragma unroll
    for (int t = 0; t < NTAP; ++t) acc[t] = 0.f;
    int lo = ca - G;                              // channel of ring slot 0
    auto finish = [&]() {
        if (lo >= ca) tile[lane][lo - ca] = acc[0];
#pragma unroll
        for (int t = 0; t + 1 < NTAP; ++t) acc[t] = acc[t + 1];
        acc[NTAP - 1] = 0.f;
        ++lo;
    };
    if (j1 > j0) {
        // records of 64 entries, field f of entry jb + l in lane l (clamped
        // into the run: entries past its end are loaded but never added)
        auto load_recs = [&](int jb, int (&R)[RS]) {
            const int j = min(jb + lane, j1 - 1);
#pragma unroll
            for (int f = 0; f < RS; ++f) R[f] = sv[(int64_t)f * nbmax + j];
        };
        auto load_x = [&](int o) { return cb0[(uint32_t)o]; };
        float xq[PB_D];
        // one block of 64 entries from records R, with the next block's in N
        // (fetched meanwhile); the voxels of entry s + PB_D are loaded while
        // entry s is added
        // (unrolled by PB_D only, so that the buffer index is fixed; the
        // record lanes are uniform scalar indices)
        auto block = [&](int jb, int (&R)[RS], int (&N)[RS]) {
            load_recs(jb + 64, N);
#pragma unroll
            for (int s0 = 0; s0 < 64; s0 += PB_D) {
                const bool last = s0 + PB_D >= 64;
#pragma unroll
                for (int d = 0; d < PB_D; ++d) {
                    const int s = s0 + d;
                    const float x = xq[d];
                    const int o2 = last ? __builtin_amdgcn_readlane(N[0], s + PB_D - 64)
                                        : __builtin_amdgcn_readlane(R[0], s + PB_D);
                    xq[d] = load_x(o2);
                    if (jb + s < j1) {
                        const int nf = __builtin_amdgcn_readlane(R[1], s) - G;
                        while (lo < nf) finish();    // channels the walk has passed
#pragma unroll
                        for (int t = 0; t < NTAP; ++t)
                            acc[t] = fmaf(__int_as_float(__builtin_amdgcn_readlane(R[2 + t], s)), x, acc[t]);
                    }
                }
            }
        };
        int RA[RS], RB[RS];
        load_recs(j0, RA);
#pragma unroll
        for (int d = 0; d < PB_D; ++d) xq[d] = load_x(__builtin_amdgcn_readlane(RA[0], d));
        for (int jb = j0;;) {
            block(jb, RA, RB);
            if ((jb += 64) >= j1) break;
            block(jb, RB, RA);
            if ((jb += 64) >= j1) break;
        }
    }
    while (lo < ce) finish();
    // the tile's rows into the sinogram: half a wave per row (lanes of a row
    // on consecutive channels); LDS operations of a wave complete in order,
    // so the tile written above is what these reads see.  (Storing each
    // finished channel straight into its 64 rows instead, 64 scattered
    // 4-byte stores, took three times as long.)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int hc = lane & 31, hr = lane >> 5;
    const bool cok = ca + hc < ce;
    float *out = sino + ((int64_t)v * g.nr + k0) * g.nc + ca + hc;
    for (int r = hr; r < 64 && k0 + r < g.nr; r += 2) {
        if (cok) {
            float val = tile[r][hc];
            if (accumulate) val += out[(int64_t)r * g.nc];
            out[(int64_t)r * g.nc] = val;
        }
    }
}

// sino [V][R][C] (channels fastest) -> buf [V][cb][s16] (slices fastest, guard
// guard channels on each side, and slices past R, zero), through a 64 x 64
// LDS tile: the layout the batch back reads a tap's 64 slices from at once.
__global__ __launch_bounds__(256) void par_pack_kernel(const float *__restrict__ sino, float *__restrict__ buf,
                                                       int nr, int nc, int cb, int s16, int guard, int tn) {
    __shared__ float t[64][65];
    const int v = (int)(blockIdx.x / (unsigned)tn);
    const int n0 = (int)(blockIdx.x % (unsigned)tn) * 64;   // buffer channels
    const int r0 = (int)blockIdx.y * 64;
    const int a = (int)threadIdx.x & 63, b = (int)threadIdx.x >> 6;
    const int c = n0 + a - guard;                           // detector channel of lane a
    const bool cin = c >= 0 && c < nc;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int r = b + 4 * u;
        t[r][a] = (cin && r0 + r < nr) ? sino[((int64_t)v * nr + r0 + r) * nc + c] : 0.f;
    }
    __syncthreads();
    if (r0 + a < s16) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int n = b + 4 * u;
            if (n0 + n < cb) buf[((int64_t)v * cb + n0 + n) * s16 + r0 + a] = t[a][n];
        }
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

bool back_pixels_packs(const Plan &p, int64_t n) {
    const Geo &g = p.g;
    if (g.kind != 0 || !p.facc || n <= 0 || g.ns <= 0) return false;
    const double lanes = (double)std::min(64, g.ns);
    const double taps = (double)n * ((g.ns + 63) / 64) * g.nv * p.ntap;
    // cache lines: a tap read of 64 lanes touches one line per lane in the
    // sinogram, and lanes * 4 / 64 (+1 unaligned) in the packed copy, which
    // costs one read of the sinogram and one write of the copy
    const double direct = taps * lanes;
    const double packed = taps * (std::ceil(lanes * 4.0 / 64.0) + 1.0) +
                          ((double)g.nv * g.nr * g.nc + (double)g.nv * p.fwd_cb * p.fwd_s16) * 4.0 / 64.0;
    return packed < direct;
}

template <int NTAP>
static hipError_t par_back_pixels_n(const Plan &p, const float *sino, const int32_t *pix, int n, float *cyl,
                                    hipStream_t st) {
    const Geo &g = p.g;
    const dim3 grid((unsigned)n, (unsigned)((g.ns + 63) / 64));       // a listed pixel per workgroup
    if (back_pixels_packs(p, n)) {
        const int tn = (p.fwd_cb + 63) / 64;
        hipLaunchKernelGGL(par_pack_kernel, dim3((unsigned)(g.nv * tn), (unsigned)((p.fwd_s16 + 63) / 64)), dim3(256),
                           0, st, sino, p.facc, g.nr, g.nc, p.fwd_cb, p.fwd_s16, NTAP - 1, tn);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((par_back_pixels_kernel<NTAP, true>), grid, dim3(256), 0, st, p.facc, pix, n, cyl,
                           p.views, g, p.fwd_cb, p.fwd_s16);
    } else {
        hipLaunchKernelGGL((par_back_pixels_kernel<NTAP, false>), grid, dim3(256), 0, st, sino, pix, n, cyl,
                           p.views, g, p.fwd_cb, p.fwd_s16);
    }
    return hipGetLastError();
}

hipError_t launch_back_pixels(const Plan &p, const float *sino, const int32_t *pix, int n, float *cyl,
                              hipStream_t st) {
    const Geo &g = p.g;
    if (n == 0 || g.ns == 0) return hipSuccess;
    if (g.kind == 0) {
        switch (p.ntap) {
        case 2: return par_back_pixels_n<2>(p, sino, pix, n, cyl, st);
        case 3: return par_back_pixels_n<3>(p, sino, pix, n, cyl, st);
        case 4: return par_back_pixels_n<4>(p, sino, pix, n, cyl, st);
        case 5: return par_back_pixels_n<5>(p, sino, pix, n, cyl, st);
        case 6: return par_back_pixels_n<6>(p, sino, pix, n, cyl, st);
        case 7: return par_back_pixels_n<7>(p, sino, pix, n, cyl, st);
        default: return hipErrorInvalidValue;
        }
    }
    const dim3 grid((unsigned)((n + SW - 1) / SW), (unsigned)((g.ns + 63) / 64));
    BPAMD_SUBSET_R(cone_back_pixels_kernel, grid, dim3(SW * 64), 0, st, sino, pix, n, cyl, p.idx, p.views, g)
    return hipGetLastError();
}

// Sort and walk, one pass per bsort_nb entries (the first overwrites the
// sinogram, the others add to it).
template <int NTAP>
static hipError_t par_forward_pixels_n(const Plan &p, const int32_t *pix, int n, const float *cyl, float *sino,
                                       hipStream_t st) {
    const Geo &g = p.g;
    const int nparts = (g.nc + PB_CW - 1) / PB_CW, nch = (g.ns + 63) / 64;
    const int64_t items = (int64_t)g.nv * nparts * nch;
    const size_t lds = batch_sort_lds(p.fwd_cb, NTAP, p.bsort_nb);
    for (int b0 = 0; b0 < n; b0 += p.bsort_nb) {
        const int nb = std::min(p.bsort_nb, n - b0);
        hipLaunchKernelGGL((par_batch_sort_kernel<NTAP>), dim3((unsigned)g.nv), dim3(PB_SORT_THREADS), lds, st, pix, b0,
                           nb, p.views, g, p.fwd_cb, p.bsort, p.boff, p.bsort_nb);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((par_batch_walk_kernel<NTAP>), dim3((unsigned)((items + SW - 1) / SW)), dim3(SW * 64), 0,
                           st, cyl, b0, p.bsort, p.boff, sino, g, p.fwd_cb, p.bsort_nb, nparts, nch, b0 > 0 ? 1 : 0);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t batch_sort_allow_lds(int ntap, size_t bytes) {
    const void *f = nullptr;
    switch (ntap) {
    case 2: f = (const void *)par_batch_sort_kernel<2>; break;
    case 3: f = (const void *)par_batch_sort_kernel<3>; break;
    case 4: f = (const void *)par_batch_sort_kernel<4>; break;
    case 5: f = (const void *)par_batch_sort_kernel<5>; break;
    case 6: f = (const void *)par_batch_sort_kernel<6>; break;
    case 7: f = (const void *)par_batch_sort_kernel<7>; break;
    default: return hipErrorInvalidValue;
    }
    return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_forward_pixels(const Plan &p, const int32_t *pix, int n, const float *cyl, float *sino,
                                 hipStream_t st) {
    const Geo &g = p.g;
    if (g.kind == 0 && p.bsort && n > 0) {
        switch (p.ntap) {
        case 2: return par_forward_pixels_n<2>(p, pix, n, cyl, sino, st);
        case 3: return par_forward_pixels_n<3>(p, pix, n, cyl, sino, st);
        case 4: return par_forward_pixels_n<4>(p, pix, n, cyl, sino, st);
        case 5: return par_forward_pixels_n<5>(p, pix, n, cyl, sino, st);
        case 6: return par_forward_pixels_n<6>(p, pix, n, cyl, sino, st);
        case 7: return par_forward_pixels_n<7>(p, pix, n, cyl, sino, st);
        default: return hipErrorInvalidValue;
        }
    }
    if (g.kind == 0) {
        // detectors too wide for the sort's LDS counts: atomics into the
        // slice-fastest buffer, then the unpack
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
