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

// Cone back at the listed pixels: the footprint of each voxel-view in fp64
// with the full projectors' formulas (channel taps from the channel index,
// row placement product-then-sum, row taps, chord), split into its
// per-(view, pixel) part and its per-slice part.  A workgroup takes one listed
// pixel and 64 slices; its four waves take a quarter of the views each and
// their partial sums are added in a fixed order.  In a wave, lane l evaluates
// the per-(view, pixel) part for view vb + l (channel index, channel taps, row
// magnification, d^2 + a^2 and the chord factor),
// and the wave reads them out per view; lanes (slices) then place their row
// and gather.  A view without a footprint, a row off the detector or a tap
// cell off it adds an exact +0 (the sums are never -0), so the views run
// without branches, four at a time, their loads in flight together.  With PK
// the cells come from the sinogram transposed to [V][C][R]: the rows of one
// channel that 64 slices reach are then one run of memory instead of one
// cache line each.
constexpr int CB_U = 4;                           // views per group of the cone batch back

template <int R, bool PK>
__global__ __launch_bounds__(256) void cone_back_pixels_kernel(const float *__restrict__ sino,
                                                               const int32_t *__restrict__ pix, int n,
                                                               float *__restrict__ cyl,
                                                               const int32_t *__restrict__ idx,
                                                               const ViewK *__restrict__ views, Geo g) {
    constexpr int NTAP = 2 * R + 1;
    __shared__ float part[4][64];
    const int lane = (int)threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int i = (int)blockIdx.x;
    const int np = g.ny * g.nx;
    const int k = (int)blockIdx.y * 64 + lane;
    const int p = listed_pixel(pix, i, np);
    const int vper = (g.nv + 3) / 4;
    const int vbeg = wave * vper, vend = min(g.nv, vbeg + vper);
    float acc = 0.f;
    if (p >= 0 && vbeg < vend) {
        const double x = pix_x(g, p % g.nx), y = pix_y(g, p / g.nx);
        const double zk = slice_z(g, k);
        const int64_t vstride = (int64_t)g.nr * g.nc;
        auto rl_d = [](double d, int q) {         // lane q's double, as a wave-uniform value
            const long long b = __double_as_longlong(d);
            const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), q);
            const int hi = __builtin_amdgcn_readlane((int)(b >> 32), q);
            return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
        };
        auto rl_f = [](float f, int q) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), q)); };
        for (int vb = vbeg; vb < vend; vb += 64) {
            // lane l: the per-(view, pixel) part for view vb + l
            const int vl = min(vb + lane, vend - 1);
            const ViewK vk = views[vl];
            const int ncv = idx[(int64_t)vl * np + p];
            const bool on = vb + lane < vend && ncv >= -R && ncv <= g.nc - 1 + R;
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
            double hd[NTAP];
            tap_weights_d<R>(f, wch, hd);
            float hl[NTAP];
#pragma unroll
            for (int t = 0; t < NTAP; ++t) hl[t] = (float)hd[t];
            const double mrdv = mr * g.dv;
            const double r2 = d * d + a * a;              // the chord's (d^2 + a^2) + dz^2, summed in that order
            const float lsc = (float)(g.dv / mm);
            const uint64_t onm = __builtin_amdgcn_ballot_w64(on);
            const int cnt = min(64, vend - vb);
            for (int j0 = 0; j0 < cnt; j0 += CB_U) {
                float sv[CB_U];
#pragma unroll
                for (int u = 0; u < CB_U; ++u) {
                    const int j = min(j0 + u, cnt - 1);
                    const bool von = j0 + u < cnt && ((onm >> j) & 1u);
                    const int nc_j = __builtin_amdgcn_readlane(ncv, j);
                    const double mr_j = rl_d(mr, j), mrdv_j = rl_d(mrdv, j), r2_j = rl_d(r2, j);
                    const double zs_j = rl_d(vk.zsrc, j);
                    const float lsc_j = rl_f(lsc, j);
                    float h[NTAP];
#pragma unroll
                    for (int t = 0; t < NTAP; ++t) h[t] = rl_f(hl[t], j);
                    // this lane's slice: its row, row taps and chord
                    const double dz = zk - zs_j;
                    const double t0 = mr_j * dz;
                    const double wk = t0 + g.crow;
                    const double mkd = rint(wk);
                    const bool rok = von && !(mkd < -R || mkd > g.nr - 1 + R);
                    double gd[NTAP];
                    tap_weights_d<R>(wk - mkd, mrdv_j, gd);
                    const int mk = rok ? (int)mkd : 0;
                    const float lk = lsc_j * sqrtf((float)(r2_j + dz * dz));
                    const float *svv = sino + (int64_t)(vb + j) * vstride;
                    float s = 0.f;
#pragma unroll
                    for (int sg = 0; sg < NTAP; ++sg) {
                        const int m = mk - R + sg;
                        const bool mok = rok && m >= 0 && m < g.nr;
                        float rv = 0.f;
#pragma unroll
                        for (int t = 0; t < NTAP; ++t) {
                            const int c = nc_j - R + t;
                            const bool in = mok && c >= 0 && c < g.nc;
                            // (PK: the sinogram transposed, [V][C][R], so the
                            // 64 slices' rows of one channel are adjacent)
                            const float val = svv[in ? (PK ? (int64_t)c * g.nr + m : (int64_t)m * g.nc + c) : 0];
                            rv = fmaf(h[t], in ? val : 0.f, rv);
                        }
                        s = fmaf(lk * (float)gd[sg], rv, s);
                    }
                    sv[u] = rok ? s : 0.f;
                }
#pragma unroll
                for (int u = 0; u < CB_U; ++u) acc += sv[u];
            }
        }
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && k < g.ns)
        cyl[(int64_t)i * g.ns + k] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
}

// Cone forward of a batch: per view the wave first adds its slices' taps into
// an LDS band of the detector (the rows its 64 slices reach times the 2R + 1
// channel taps; a slice's row never decreases with the slice, so the rows in
// range form one band, from the first to the last lane in range), as plain
// read-modify-writes in `stride` passes, each taking the lanes whose slice is
// that pass's residue (the plan's stride puts the rows of one pass on distinct
// rows, as in the full cone forward; LDS float atomics cost tens of times
// more).  Then it adds the band, one global atomic per touched cell, to the
// sinogram transposed to [V][C][R] (the handle's; unpacked after), the lanes
// along the rows of one channel: a few 64-byte requests per channel, where the
// sinogram itself took one per row (about 66 per view at 256^3).  A band
// taller than the LDS holds (magnification far above one) takes the direct
// form, into the same transposed sinogram.
constexpr int CPB_CELLS = 1536;         // LDS band cells per wave (rows x taps)

template <int R>
__global__ __launch_bounds__(256) void cone_forward_pixels_kernel(const int32_t *__restrict__ pix, int n,
                                                                  const float *__restrict__ cyl,
                                                                  float *__restrict__ sino,
                                                                  const int32_t *__restrict__ idx,
                                                                  const ViewK *__restrict__ views, Geo g,
                                                                  int stride) {
    constexpr int NTAP = 2 * R + 1;
    constexpr int PROW = CPB_CELLS / NTAP;      // band rows at most
    __shared__ float band_all[4 * CPB_CELLS];
    const int lane = (int)threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int i = (int)blockIdx.x;                  // a listed pixel per workgroup, a quarter of the views per wave
    const int np = g.ny * g.nx;
    const int k = (int)blockIdx.y * 64 + lane;
    const int p = listed_pixel(pix, i, np);
    if (p < 0) return;                              // padding contributes nothing (no workgroup barrier below)
    const int vper = (g.nv + 3) / 4;
    const int vbeg = wave * vper, vend = min(g.nv, vbeg + vper);
    const bool kin = k < g.ns;
    const float xv = kin ? cyl[(int64_t)i * g.ns + k] : 0.f;
    const double x = pix_x(g, p % g.nx), y = pix_y(g, p / g.nx);
    const double zk = slice_z(g, k);
    float *band = band_all + wave * CPB_CELLS;
    for (int e = lane; e < CPB_CELLS; e += 64) band[e] = 0.f;
    auto rl_d = [](double d, int q) {             // lane q's double, as a wave-uniform value
        const long long b = __double_as_longlong(d);
        const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), q);
        const int hi = __builtin_amdgcn_readlane((int)(b >> 32), q);
        return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
    };
    auto rl_f = [](float f, int q) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), q)); };
    for (int vb = vbeg; vb < vend; vb += 64) {
        // lane l: the per-(view, pixel) part of the footprint for view vb + l
        // (the back's fp64 operations), read out by the wave per view
        const int vl = min(vb + lane, vend - 1);
        const ViewK vkl = views[vl];
        const int ncl = idx[(int64_t)vl * np + p];
        const bool onl = vb + lane < vend && ncl >= -R && ncl <= g.nc - 1 + R;
        double mrl, mrdvl, r2l;
        float hl[NTAP], lscl;
        {
            const double xc = x * vkl.c, ys = y * vkl.s, yc = y * vkl.c, xs = x * vkl.s;
            const double a = xc + ys;
            const double b = yc - xs;
            const double d = g.sid + b;
            const double drw = d * g.drow;
            mrl = g.sdd / drw;
            const double mc = g.sdd / (d * g.dch);
            const double f = (mc * a + g.cch + vkl.shift) - (double)ncl;
            const double mm = fmax(fabs(y + vkl.c * g.sid), fabs(vkl.s * g.sid - x));
            const double wch = mc * g.dv * mm / d;
            double hd[NTAP];
            tap_weights_d<R>(f, wch, hd);
#pragma unroll
            for (int t = 0; t < NTAP; ++t) hl[t] = (float)hd[t];
            mrdvl = mrl * g.dv;
            r2l = d * d + a * a;                        // the chord's (d^2 + a^2) + dz^2, summed in that order
            lscl = (float)(g.dv / mm);
        }
        const uint64_t onm = __builtin_amdgcn_ballot_w64(onl);
        const int cnt = min(64, vend - vb);
        for (int j = 0; j < cnt; ++j) {
            if (!((onm >> j) & 1u)) continue;          // uniform: no footprint in this view
            const int v = vb + j;
            const int ncv = __builtin_amdgcn_readlane(ncl, j);
            float h[NTAP];
#pragma unroll
            for (int t = 0; t < NTAP; ++t) h[t] = rl_f(hl[t], j);
            // this lane's slice: its row, row taps and chord
            const double dz = zk - rl_d(vkl.zsrc, j);
            const double t0 = rl_d(mrl, j) * dz;
            const double wk = t0 + g.crow;
            const double mkd = rint(wk);
            const bool ok = kin && !(mkd < -R || mkd > g.nr - 1 + R);
            double gd[NTAP];
            tap_weights_d<R>(wk - mkd, rl_d(mrdvl, j), gd);
            const int mk = ok ? (int)mkd : 0;
            const float lk = rl_f(lscl, j) * sqrtf((float)(rl_d(r2l, j) + dz * dz));
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
                                unsafeAtomicAdd(&sv[(int64_t)ch * g.nr + m], h[t] * c);
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
            const int rows = hi - lo + 1, cells = rows * NTAP;
            for (int e = lane; e < cells; e += 64) {
                // lanes along the rows of one channel, adjacent in the
                // transposed sinogram (a few 64-byte requests per channel
                // instead of one per row in the sinogram itself)
                const int mm = e % rows, t = e / rows;
                float *cell = band + mm * NTAP + t;
                const float val = *cell;
                *cell = 0.f;
                const int m = lo + mm, ch = ncv - R + t;
                if (val != 0.f && ch >= 0 && ch < g.nc)
                    unsafeAtomicAdd(&sv[(int64_t)ch * g.nr + m], val);
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }
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

#define BPAMD_SUBSET_R2(KERN, B, ...)                                                                         \
    switch (g.radius) {                                                                                       \
    case 1: hipLaunchKernelGGL((KERN<1, B>), __VA_ARGS__); break;                                             \
    case 2: hipLaunchKernelGGL((KERN<2, B>), __VA_ARGS__); break;                                             \
    case 3: hipLaunchKernelGGL((KERN<3, B>), __VA_ARGS__); break;                                             \
    case 4: hipLaunchKernelGGL((KERN<4, B>), __VA_ARGS__); break;                                             \
    default: return hipErrorInvalidValue;                                                                     \
    }

bool back_pixels_packs(const Plan &p, int64_t n) {
    const Geo &g = p.g;
    if (n <= 0 || g.ns <= 0) return false;
    if (g.kind == 0 ? !p.facc : !p.ctr) return false;
    const double lanes = (double)std::min(64, g.ns);
    // tap columns per (listed pixel, chunk, view): the parallel record's
    // channels; the cone's 2r + 1 channels (its 2r + 1 rows share their lines)
    const double cols = (double)n * ((g.ns + 63) / 64) * g.nv * (g.kind == 0 ? p.ntap : 2 * g.radius + 1);
    // cache lines: a column of 64 lanes touches one line per lane in the
    // sinogram, and lanes * 4 / 64 (+1 unaligned, +1 more for the cone's rows
    // beyond the slices) in the packed copy, which costs one read of the
    // sinogram and one write of the copy
    const double direct = cols * lanes;
    const double copy = g.kind == 0 ? (double)g.nv * p.fwd_cb * p.fwd_s16 : (double)g.nv * g.nr * g.nc;
    const double packed = cols * (std::ceil(lanes * 4.0 / 64.0) + (g.kind == 0 ? 1.0 : 2.0)) +
                          ((double)g.nv * g.nr * g.nc + copy) * 4.0 / 64.0;
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
    const dim3 grid((unsigned)n, (unsigned)((g.ns + 63) / 64));       // a listed pixel per workgroup
    if (back_pixels_packs(p, n)) {
        const int tn = (g.nc + 63) / 64;
        hipLaunchKernelGGL(par_pack_kernel, dim3((unsigned)(g.nv * tn), (unsigned)((g.nr + 63) / 64)), dim3(256), 0,
                           st, sino, p.ctr, g.nr, g.nc, g.nc, g.nr, 0, tn);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        BPAMD_SUBSET_R2(cone_back_pixels_kernel, true, grid, dim3(256), 0, st, p.ctr, pix, n, cyl, p.idx, p.views, g)
    } else {
        BPAMD_SUBSET_R2(cone_back_pixels_kernel, false, grid, dim3(256), 0, st, sino, pix, n, cyl, p.idx, p.views, g)
    }
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
    if (n == 0) return launch_fill_zero(sino, (int64_t)g.nv * g.nr * g.nc, st);
    if (!p.ctr) return hipErrorInvalidValue;      // (every cone handle with a sinogram keeps one)
    // into the handle's transposed sinogram, then unpacked
    const dim3 grid((unsigned)n, (unsigned)((g.ns + 63) / 64));       // a listed pixel per workgroup
    hipError_t e = launch_fill_zero(p.ctr, (int64_t)g.nv * g.nr * g.nc, st);
    if (e != hipSuccess) return e;
    BPAMD_SUBSET_R(cone_forward_pixels_kernel, grid, dim3(256), 0, st, pix, n, cyl, p.ctr, p.idx, p.views, g,
                   p.cone_stride)
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_unpack_rows(p.ctr, sino, g.nv, g.nr, g.nc, g.nc, g.nr, 0, st);
}

}  // namespace bpamd
