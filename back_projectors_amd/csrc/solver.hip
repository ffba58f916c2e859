// Vector kernels of the CGLS and SIRT loops around the projector pair.
//
// The loops (diffct "Precision, training and reconstruction", section
// "Numerical solver API": stop rule ||y - A x|| <= atol + rtol ||y|| on every
// iterate, the first included; CGLS reading its two norms of an iteration
// together; SIRT reusing the last residual) live on the host; every vector
// step is one of the kernels here, so an iteration is a fixed sequence of
// launches on one stream with a single host read of the norms at its end.
//
// All of them stream HBM: one elementwise pass each, fused where a pass can
// carry a second job (the residual update also produces its squared norm,
// SIRT's residual is weighted in the same pass).  Scalars that depend on a
// reduction (alpha, beta) are read from device memory by the consumer, so no
// host round trip sits between the reduction and its use.  Norms accumulate
// in fp64; the reduction is two-pass with a fixed number of blocks and a fixed
// order, so it is deterministic.
#include "launch.h"

#pragma clang fp contract(off)

namespace bpamd {

namespace {

constexpr int VT = 256;         // threads per block
constexpr int VPER = 4;         // elements per thread per step (one float4 when aligned)

// coefficient sign * sc[num] / sc[den] (0 when the denominator is 0), kept in
// fp64: rounding the CGLS step length and direction weight to fp32 breaks the
// conjugacy of the directions far more than storing the vectors in fp32 does,
// so updates run in fp64 and round once, when stored
__device__ __forceinline__ double coef_of(const double *sc, int num, int den, double sign) {
    const double d = sc[den];
    return d != 0.0 ? sign * sc[num] / d : 0.0;
}

__device__ __forceinline__ double block_sum(double v) {
    __shared__ double part[VT / 64];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
    const int w = (int)threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) part[w] = v;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0)
        for (int i = 0; i < VT / 64; ++i) t += part[i];
    return t;   // valid in thread 0
}

}  // namespace

struct VecArgs {
    float *d;
    const float *a, *b;
    const double *sc;
    int num, den;
    double sign;
    double value;
    int flag;
};

template <int OP> constexpr bool reads_a() {
    return OP == V_COPY || OP == V_NORM || OP == V_SUB_NORM || OP == V_XPBY || OP == V_SIRT_RES || OP == V_SIRT_UPD;
}
template <int OP> constexpr bool reads_b() {
    return OP == V_SUB_NORM || OP == V_AXPY || OP == V_SIRT_RES || OP == V_SIRT_UPD;
}
template <int OP> constexpr bool reads_d() {
    return OP == V_RECIP || OP == V_AXPY || OP == V_XPBY || OP == V_SIRT_RES || OP == V_SIRT_UPD;
}

// One element: a, b, d are the element's values (those the op reads).
template <int OP>
__device__ __forceinline__ float vec_op(const VecArgs &v, double c, float a, float b, float d, double &acc) {
    float r = 0.f;
    if constexpr (OP == V_FILL) {
        r = (float)v.value;
    } else if constexpr (OP == V_COPY) {
        r = a;
    } else if constexpr (OP == V_RECIP) {
        r = d > 0.f ? 1.f / d : 0.f;
    } else if constexpr (OP == V_NORM) {
        acc += (double)a * (double)a;
    } else if constexpr (OP == V_SUB_NORM) {
        r = a - b;
        acc += (double)r * (double)r;
    } else if constexpr (OP == V_AXPY) {
        r = (float)((double)d + c * (double)b);
        acc += (double)r * (double)r;
    } else if constexpr (OP == V_XPBY) {
        r = (float)((double)a + c * (double)d);
    } else if constexpr (OP == V_SIRT_RES) {
        const float e = a - d;
        acc += (double)e * (double)e;
        r = b * e;
    } else if constexpr (OP == V_SIRT_UPD) {
        r = (float)((double)d + v.value * ((double)b * (double)a));
        if (v.flag) r = fmaxf(r, 0.f);
    }
    return r;
}

template <int OP>
__device__ __forceinline__ void vec_one(const VecArgs &v, double c, int64_t i, double &acc) {
    const float a = reads_a<OP>() ? v.a[i] : 0.f;
    const float b = reads_b<OP>() ? v.b[i] : 0.f;
    const float d = reads_d<OP>() ? v.d[i] : 0.f;
    const float r = vec_op<OP>(v, c, a, b, d, acc);
    if constexpr (OP != V_NORM) v.d[i] = r;
}

template <int OP>
__global__ __launch_bounds__(VT) void vec_kernel(VecArgs v, int64_t n, double *red) {
    double c = 0.0;
    if constexpr (OP == V_AXPY || OP == V_XPBY) c = coef_of(v.sc, v.num, v.den, v.sign);
    double acc = 0.0;
    const int64_t stride = (int64_t)gridDim.x * VT;
    for (int64_t i = (int64_t)blockIdx.x * VT + threadIdx.x; i < n; i += stride) vec_one<OP>(v, c, i, acc);
    if (red) {
        const double t = block_sum(acc);
        if (threadIdx.x == 0) red[blockIdx.x] = t;
    }
}

// The same with float4 accesses when every vector the op touches is 16-byte
// aligned; the tail of n % 4 elements runs in block 0.
template <int OP>
__global__ __launch_bounds__(VT) void vec4_kernel(VecArgs v, int64_t n, double *red) {
    double c = 0.0;
    if constexpr (OP == V_AXPY || OP == V_XPBY) c = coef_of(v.sc, v.num, v.den, v.sign);
    double acc = 0.0;
    const int64_t n4 = n / 4;
    const int64_t stride = (int64_t)gridDim.x * VT;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t q = (int64_t)blockIdx.x * VT + threadIdx.x; q < n4; q += stride) {
        const float4 a = reads_a<OP>() ? reinterpret_cast<const float4 *>(v.a)[q] : z;
        const float4 b = reads_b<OP>() ? reinterpret_cast<const float4 *>(v.b)[q] : z;
        const float4 d = reads_d<OP>() ? reinterpret_cast<const float4 *>(v.d)[q] : z;
        float4 r;
        r.x = vec_op<OP>(v, c, a.x, b.x, d.x, acc);
        r.y = vec_op<OP>(v, c, a.y, b.y, d.y, acc);
        r.z = vec_op<OP>(v, c, a.z, b.z, d.z, acc);
        r.w = vec_op<OP>(v, c, a.w, b.w, d.w, acc);
        if constexpr (OP != V_NORM) reinterpret_cast<float4 *>(v.d)[q] = r;
    }
    if (blockIdx.x == 0 && threadIdx.x < (unsigned)(n - 4 * n4)) vec_one<OP>(v, c, 4 * n4 + threadIdx.x, acc);
    if (red) {
        const double t = block_sum(acc);
        if (threadIdx.x == 0) red[blockIdx.x] = t;
    }
}

// sc[idx] = sum of red[0 .. nb) in a fixed order (one block).
__global__ __launch_bounds__(VT) void vec_reduce_final(const double *red, int nb, double *sc, int idx) {
    double acc = 0.0;
    for (int i = (int)threadIdx.x; i < nb; i += VT) acc += red[i];
    const double t = block_sum(acc);
    if (threadIdx.x == 0) sc[idx] = t;
}

int vec_blocks(int64_t n) {
    const int64_t per = (int64_t)VT * VPER * 4;   // about 16 elements per thread
    int64_t nb = (n + per - 1) / per;
    if (nb < 1) nb = 1;
    if (nb > kVecMaxBlocks) nb = kVecMaxBlocks;
    return (int)nb;
}

template <int OP>
static hipError_t vec_launch_t(const VecArgs &v, int64_t n, double *red, bool aligned, hipStream_t st) {
    const int nb = vec_blocks(n);
    if (aligned)
        hipLaunchKernelGGL(vec4_kernel<OP>, dim3(nb), dim3(VT), 0, st, v, n, red);
    else
        hipLaunchKernelGGL(vec_kernel<OP>, dim3(nb), dim3(VT), 0, st, v, n, red);
    return hipGetLastError();
}

static bool al16(const void *p) { return ((uintptr_t)p & 15) == 0; }

hipError_t launch_vec(int op, float *d, const float *a, const float *b, const double *sc, int num, int den,
                      double sign, double value, int flag, int64_t n, double *red, int sc_out, double *sc_w,
                      hipStream_t st) {
    if (n > 0) {
        VecArgs v{d, a, b, sc, num, den, sign, value, flag};
        const bool aligned = (!d || al16(d)) && (!a || al16(a)) && (!b || al16(b));
        hipError_t e;
        switch (op) {
        case V_FILL: e = vec_launch_t<V_FILL>(v, n, red, aligned, st); break;
        case V_COPY: e = vec_launch_t<V_COPY>(v, n, red, aligned, st); break;
        case V_RECIP: e = vec_launch_t<V_RECIP>(v, n, red, aligned, st); break;
        case V_NORM: e = vec_launch_t<V_NORM>(v, n, red, aligned, st); break;
        case V_SUB_NORM: e = vec_launch_t<V_SUB_NORM>(v, n, red, aligned, st); break;
        case V_AXPY: e = vec_launch_t<V_AXPY>(v, n, red, aligned, st); break;
        case V_XPBY: e = vec_launch_t<V_XPBY>(v, n, red, aligned, st); break;
        case V_SIRT_RES: e = vec_launch_t<V_SIRT_RES>(v, n, red, aligned, st); break;
        case V_SIRT_UPD: e = vec_launch_t<V_SIRT_UPD>(v, n, red, aligned, st); break;
        default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
    }
    if (red && sc_out >= 0) {
        hipLaunchKernelGGL(vec_reduce_final, dim3(1), dim3(VT), 0, st, red, n > 0 ? vec_blocks(n) : 0, sc_w,
                           sc_out);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace bpamd
