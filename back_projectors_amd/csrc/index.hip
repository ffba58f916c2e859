// The separate integer channel-index pass (MBIRJAX "Projector kernels" page,
// paragraph "Shared machinery, and the rounding defense": a small step of its
// own computes each voxel's channel and hands it to the projectors as data, so
// they never round a coordinate themselves).
//
// Every operation below is one IEEE fp64 operation rounded in the written
// order: this file is built with -ffp-contract=off and the pragma forbids
// fusing a product into a sum, and fp64 division on gfx950 is correctly
// rounded.  With the view cosines and sines taken from the host C library,
// n_c = rint(u) is therefore reproducible bit for bit, ties to even included.
#include "chan.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace bpamd {

__global__ __launch_bounds__(256) void channel_index_kernel(Geo g, const ViewK *__restrict__ views,
                                                            int32_t *__restrict__ idx) {
    const int np = g.ny * g.nx;
    const int64_t total = (int64_t)np * g.nv;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int v = (int)(e / np);
        const int p = (int)(e - (int64_t)v * np);
        const int i = p / g.nx;
        const int j = p - i * g.nx;
        const ViewK vk = views[v];
        idx[e] = (int32_t)rint(channel_coord_exact(g, vk, i, j));
    }
}

// Parallel-beam tap records, one per (view, pixel) (par_tap_record).
__global__ __launch_bounds__(256) void par_taps_kernel(Geo g, const ViewK *__restrict__ views,
                                                       int32_t *__restrict__ rec, int ntap) {
    const int np = g.ny * g.nx;
    const int64_t total = (int64_t)np * g.nv;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int v = (int)(e / np);
        const int p = (int)(e - (int64_t)v * np);
        const int i = p / g.nx;
        const int j = p - i * g.nx;
        float w[7];
        const int nf = par_tap_record(g, views[v], i, j, ntap, w);
        int32_t *r = rec + e * (1 + ntap);
        for (int t = 0; t < ntap; ++t) r[1 + t] = __float_as_int(w[t]);
        r[0] = nf;
    }
}

// The same records re-laid for the forward walk.  One workgroup per (view,
// region of RSX x RSY pixels): the region's pixels are ordered by their first
// tap channel n_f (ties by pixel index: a stable counting sort), so a walk in
// this order never returns to a channel it has passed.  The walk keeps NTAP
// accumulators as a ring: channel n lives in accumulator n mod NTAP, so a step
// touches every accumulator exactly once and nothing is ever moved between
// registers.  Steps are grouped by 16; per (view, region, group) the records
// are 2 + NTAP fields of 16 dwords, one dword per step:
//   field 0: LDS byte offset of the step's voxel row (pixel-in-region times
//            the bytes of one pixel's slices in the region copy, 64 or 128);
//   field 1: 0 when nothing is flushed after this step; else bits 0-6 = the
//            accumulators to flush, bits 7-13 = those among them below
//            n_f mod NTAP (their channel lies one ring turn up), bits 14-31 =
//            (n_f - (n_f mod NTAP)) / NTAP + 1, the ring turn of the step;
//   field 2 + r: the weight for accumulator r, i.e. the tap weight of channel
//            n_f + ((r - n_f) mod NTAP).
// Accumulator r thus holds channel NTAP * (turn - 1) + r, plus NTAP when its
// bit 7 + r is set.  It is flushed once its channel is below the next step's
// n_f (every channel finishes there, since the walk never comes back), and all
// of them after the last step that reaches the detector.  Steps of pixels that
// miss the detector (or lie outside the image) sort last, with zero weights
// and nothing to flush, and so do the steps that pad the walk to whole groups.
// Dynamic LDS: 2 * RSX * RSY + nbin + 1 ints.
__global__ __launch_bounds__(256) void par_region_records_kernel(Geo g, const int32_t *__restrict__ rec,
                                                                 uint32_t *__restrict__ out, int ntap, int rsx,
                                                                 int rsy, int nrx, int nreg, int ng, int nbin,
                                                                 uint32_t pxb) {
    extern __shared__ int sh[];
    const int rp = rsx * rsy;
    int *key = sh;                      // [rp] n_f - min n_f, or nbin - 1 for "no tap on the detector"
    int *perm = sh + rp;                // [rp] pixel at each walk position; later n_f at each position
    int *bin = sh + 2 * rp;             // [nbin + 1] counts, then running starts
    __shared__ int s_min, s_nvalid;
    const int64_t vr = blockIdx.x;
    const int region = (int)(vr % nreg);
    const int v = (int)(vr / nreg);
    const int i0 = (region / nrx) * rsy, j0 = (region % nrx) * rsx;
    const int np = g.ny * g.nx;
    const int nf_ = 2 + ntap;
    const int t = (int)threadIdx.x;
    auto nf_of = [&](int p) {
        const int i = i0 + p / rsx, j = j0 + p % rsx;
        if (i >= g.ny || j >= g.nx) return (int)INT32_MAX;
        return rec[((int64_t)v * np + i * g.nx + j) * (1 + ntap)];
    };
    if (t == 0) {
        s_min = INT32_MAX;
        s_nvalid = 0;
    }
    for (int e = t; e <= nbin; e += 256) bin[e] = 0;
    __syncthreads();
    for (int p = t; p < rp; p += 256) {
        const int nf = nf_of(p);
        if (nf != INT32_MAX) {
            atomicMin(&s_min, nf);
            atomicAdd(&s_nvalid, 1);
        }
    }
    __syncthreads();
    const int nfmin = s_min, nvalid = s_nvalid;
    for (int p = t; p < rp; p += 256) {
        const int nf = nf_of(p);
        const int k = nf == INT32_MAX ? nbin - 1 : min(nf - nfmin, nbin - 2);   // the plan bounds n_f - min < nbin - 1
        key[p] = k;
        atomicAdd(&bin[k], 1);
    }
    __syncthreads();
    if (t == 0) {                       // exclusive scan: bins are few
        int run = 0;
        for (int e = 0; e < nbin; ++e) {
            const int c = bin[e];
            bin[e] = run;
            run += c;
        }
    }
    __syncthreads();
    if (t < 64) {                       // stable scatter, 64 pixels at a time in pixel order
        for (int c0 = 0; c0 < rp; c0 += 64) {
            const int p = c0 + t;
            const int k = p < rp ? key[p] : -1;
            int below = 0;
            for (int l = 0; l < t; ++l) below += (c0 + l < rp && key[c0 + l] == k) ? 1 : 0;
            if (p < rp) perm[bin[k] + below] = p;
            // one wave, in lockstep: every lane reads its start before any lane adds
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            if (p < rp) atomicAdd(&bin[k], 1);
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        }
    }
    __syncthreads();
    // key[] now holds the n_f of each walk position
    for (int q = t; q < rp; q += 256) key[q] = q < nvalid ? nf_of(perm[q]) : INT32_MAX;
    __syncthreads();
    uint32_t *o = out + vr * (int64_t)ng * nf_ * 16;
    for (int q = t; q < ng * 16; q += 256) {
        uint32_t *oq = o + (q >> 4) * nf_ * 16 + (q & 15);     // field f of this step: oq[f * 16]
        const int p = q < rp ? perm[q] : 0;
        oq[0] = (uint32_t)p * pxb;                        // the pixel's voxel row in the region's LDS copy
        oq[16] = 0u;
        for (int r = 0; r < ntap; ++r) oq[(2 + r) * 16] = 0u;
        if (q >= nvalid) continue;
        const int nf = key[q];
        const int cm = ((nf % ntap) + ntap) % ntap;
        const int turn = (nf - cm) / ntap + 1;           // >= 0: n_f >= 1 - ntap
        // channels nf .. nf + fin - 1 are finished after this step
        const int fin = q + 1 < nvalid ? min(key[q + 1] - nf, ntap) : ntap;
        uint32_t mask = 0, up = 0;
        for (int d = 0; d < fin; ++d) {
            const int rr = (cm + d) % ntap;
            mask |= 1u << rr;
            if (rr < cm) up |= 1u << rr;
        }
        if (mask) oq[16] = mask | (up << 7) | ((uint32_t)turn << 14);
        const int i = i0 + p / rsx, j = j0 + p % rsx;
        const int32_t *rp_ = rec + ((int64_t)v * np + i * g.nx + j) * (1 + ntap);
        for (int rr = 0; rr < ntap; ++rr) oq[(2 + rr) * 16] = (uint32_t)rp_[1 + (rr - cm + ntap) % ntap];
    }
}

// Gather strategy: per view, every pixel ordered by its first tap channel
// (a counting sort, one workgroup per view; pixels of one channel keep an
// arbitrary order).  Keys are n_f + NTAP - 1 in [0, C + NTAP - 2]; pixels with
// no tap on the detector take key C + NTAP - 1 and sort last.  Dynamic LDS:
// nbin = C + NTAP ints.
__global__ __launch_bounds__(256) void par_view_sort_kernel(Geo g, const int32_t *__restrict__ rec,
                                                            int32_t *__restrict__ order, int ntap, int nbin) {
    extern __shared__ int bin[];
    const int v = (int)blockIdx.x;
    const int np = g.ny * g.nx;
    const int t = (int)threadIdx.x;
    auto key_of = [&](int p) {
        const int nf = rec[((int64_t)v * np + p) * (1 + ntap)];
        return nf == INT32_MAX ? nbin - 1 : nf + ntap - 1;
    };
    for (int e = t; e < nbin; e += 256) bin[e] = 0;
    __syncthreads();
    for (int p = t; p < np; p += 256) atomicAdd(&bin[key_of(p)], 1);
    __syncthreads();
    if (t == 0) {
        int run = 0;
        for (int e = 0; e < nbin; ++e) {
            const int c = bin[e];
            bin[e] = run;
            run += c;
        }
    }
    __syncthreads();
    int32_t *o = order + (int64_t)v * np;
    for (int p = t; p < np; p += 256) o[atomicAdd(&bin[key_of(p)], 1)] = p;
}

// The gather walk's records, in the region walk's format (see above) except
// that field 0 is the byte offset of the pixel's voxel cylinder in the
// volume, p * S * 4, a view's walk is all of its pixels, padded with zero
// steps to ng groups of 16, and is cut into segments of segg groups, each
// walked on its own: the last step of a segment flushes every accumulator.
// One thread per (view, step).
__global__ __launch_bounds__(256) void par_view_records_kernel(Geo g, const int32_t *__restrict__ rec,
                                                               const int32_t *__restrict__ order,
                                                               uint32_t *__restrict__ out, int ntap, int ng,
                                                               int segg) {
    const int np = g.ny * g.nx;
    const int nstep = ng * 16;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)g.nv * nstep) return;
    const int v = (int)(e / nstep);
    const int q = (int)(e - (int64_t)v * nstep);
    const int nf_ = 2 + ntap;
    uint32_t *oq = out + ((int64_t)v * ng + (q >> 4)) * nf_ * 16 + (q & 15);   // field f: oq[f * 16]
    const int32_t *ov = order + (int64_t)v * np;
    auto nf_at = [&](int s) { return s < np ? rec[((int64_t)v * np + ov[s]) * (1 + ntap)] : (int)INT32_MAX; };
    const int p = q < np ? ov[q] : 0;
    oq[0] = (uint32_t)((int64_t)p * g.ns * 4);
    oq[16] = 0u;
    for (int r = 0; r < ntap; ++r) oq[(2 + r) * 16] = 0u;
    const int nf = nf_at(q);
    if (nf == INT32_MAX) return;
    const int cm = ((nf % ntap) + ntap) % ntap;
    const int turn = (nf - cm) / ntap + 1;
    const int nx = nf_at(q + 1);
    // the walk's last step, and the last step of every segment, flush all
    const bool seg_end = (q + 1) % (segg * 16) == 0;
    const int fin = (nx != INT32_MAX && !seg_end) ? min(nx - nf, ntap) : ntap;
    uint32_t mask = 0, up = 0;
    for (int d = 0; d < fin; ++d) {
        const int rr = (cm + d) % ntap;
        mask |= 1u << rr;
        if (rr < cm) up |= 1u << rr;
    }
    if (mask) oq[16] = mask | (up << 7) | ((uint32_t)turn << 14);
    const int32_t *rp_ = rec + ((int64_t)v * np + p) * (1 + ntap);
    for (int rr = 0; rr < ntap; ++rr) oq[(2 + rr) * 16] = (uint32_t)rp_[1 + (rr - cm + ntap) % ntap];
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float4 *__restrict__ b4, float *__restrict__ tail,
                                                        int64_t n4, int ntail) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += stride)
        b4[e] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0.f;
}

hipError_t launch_channel_index(const Geo &g, const ViewK *views, int32_t *idx, hipStream_t st) {
    const int64_t total = (int64_t)g.ny * g.nx * g.nv;
    if (total == 0) return hipSuccess;
    const int64_t want = (total + 255) / 256;
    const int blocks = (int)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(channel_index_kernel, dim3(blocks), dim3(256), 0, st, g, views, idx);
    return hipGetLastError();
}

hipError_t launch_par_taps(const Geo &g, const ViewK *views, int32_t *rec, int ntap, hipStream_t st) {
    const int64_t total = (int64_t)g.ny * g.nx * g.nv;
    if (total == 0) return hipSuccess;
    const int64_t want = (total + 255) / 256;
    const int blocks = (int)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(par_taps_kernel, dim3(blocks), dim3(256), 0, st, g, views, rec, ntap);
    return hipGetLastError();
}

hipError_t launch_par_region_records(const Geo &g, const int32_t *rec, uint32_t *out, int ntap, int rsx, int rsy,
                                    int nbin, int spl, hipStream_t st) {
    const int nrx = (g.nx + rsx - 1) / rsx, nry = (g.ny + rsy - 1) / rsy;
    const int nreg = nrx * nry;
    const int ng = fwd_groups(rsx, rsy);
    const int64_t blocks = (int64_t)g.nv * nreg;
    if (blocks == 0) return hipSuccess;
    const size_t lds = (size_t)(2 * rsx * rsy + nbin + 1) * sizeof(int);
    hipLaunchKernelGGL(par_region_records_kernel, dim3((unsigned)blocks), dim3(256), lds, st, g, rec, out, ntap, rsx,
                       rsy, nrx, nreg, ng, nbin, (uint32_t)(64 * spl));
    return hipGetLastError();
}

hipError_t launch_par_view_records(const Geo &g, const int32_t *rec, int32_t *order, uint32_t *out, int ntap,
                                  int ng, int segg, hipStream_t st) {
    if (g.nv == 0) return hipSuccess;
    const int nbin = g.nc + ntap;
    hipLaunchKernelGGL(par_view_sort_kernel, dim3(g.nv), dim3(256), (size_t)nbin * sizeof(int), st, g, rec, order,
                       ntap, nbin);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = (int64_t)g.nv * ng * 16;
    hipLaunchKernelGGL(par_view_records_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, g, rec,
                       order, out, ntap, ng, segg);
    return hipGetLastError();
}

// Zero fill by kernel (not a memset node), so the path stays capturable.
hipError_t launch_fill_zero(float *buf, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    // align the vector part to 16 bytes
    int64_t head = (int64_t)(((16 - ((uintptr_t)buf & 15)) & 15) / 4);
    if (head > n) head = n;
    if (head > 0) {
        hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(256), 0, st, (float4 *)nullptr, buf, (int64_t)0,
                           (int)head);
    }
    const int64_t rest = n - head;
    const int64_t n4 = rest / 4;
    const int ntail = (int)(rest - n4 * 4);
    int64_t want = (n4 + 255) / 256;
    if (want < 1) want = 1;
    const int blocks = (int)(want < 8192 ? want : 8192);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, (float4 *)(buf + head),
                       buf + head + n4 * 4, n4, ntail);
    return hipGetLastError();
}

}  // namespace bpamd
