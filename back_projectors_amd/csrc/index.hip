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
#include "launch.h"

#pragma clang fp contract(off)

namespace bpamd {

__device__ __noinline__ double channel_coord_exact(const Geo &g, const ViewK &vk, int i, int j) {
    const double x = pix_x(g, j);
    const double y = pix_y(g, i);
    if (g.kind == 0) {
        const double xc = x * vk.c;
        const double ys = y * vk.s;
        const double t = xc + ys;
        const double tq = t / g.dch;
        const double u = tq + g.cch;
        return u + vk.shift;
    }
    const double xc = x * vk.c;
    const double ys = y * vk.s;
    const double yc = y * vk.c;
    const double xs = x * vk.s;
    const double a = xc + ys;
    const double b = yc - xs;
    const double d = g.sid + b;
    const double dc = d * g.dch;
    const double mc = g.sdd / dc;
    const double ma = mc * a;
    const double u = ma + g.cch;
    return u + vk.shift;
}

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
