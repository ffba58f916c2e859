// Parallel-beam projector pair on gfx950.
//
// Detector row r sees slice r only (MBIRJAX "Projector kernels" page,
// paragraph "Geometry decides whether a slice can stream"), so every
// (view, pixel) pair has one set of channel taps shared by all slices of the
// voxel cylinder.  Those taps -- the first channel n_f and NTAP fp32 weights --
// come from the tap records the creation pass wrote in fp64; the projectors
// do no geometry arithmetic and never round a coordinate.
//
// Back (gather; paragraph "Forward scatters, back gathers"): a workgroup owns
// a BT x BT pixel tile and a chunk of SL slices; lanes are pixels, each with
// SL register accumulators.  Per view the sinogram cells the tile can reach
// (a channel window of SL rows) are staged in LDS, channel-major with slices
// fastest, by coalesced reads; each lane then reads each of its NTAP taps four
// slices at a time (one 16-byte LDS read, which gfx950 serves at about twice
// the bytes per clock of paired 4-byte reads) and accumulates.  Every voxel is
// written once and nothing collides.
//
// Forward (scatter with no colliding LDS or register updates): a workgroup
// holds a region of pixels (40 x 32, or 48 x 48 when the volume has 16 slices
// or fewer) and a chunk of 32 (16) slices in LDS and walks every view of its
// view range over it.  Each 16-lane row of a wave walks one view, its lanes
// holding two slices (16 apart) or one; the creation pass sorted the region's
// pixels by first tap channel per view (paragraph "Forward scatters, back
// gathers": the sort by channel, done once per geometry) and stored the walk
// as records that reach the lanes by DPP row broadcasts.  A view's NTAP
// current channels live in ring accumulators (channel n in accumulator n mod
// NTAP), so a step touches each exactly once; a channel the walk has passed is
// added once, with a global atomic of 16 slices per row, to a slice-fastest
// accumulation buffer, which a second kernel transposes into the sinogram.
// The gather strategy walks each view's list of all pixels the same way,
// reading the voxels from memory.  Float atomics in LDS are avoided on
// purpose: on gfx950 they cost tens of times a plain read-modify-write.
#include <type_traits>
#include <utility>

#include "launch.h"

namespace bpamd {

// Word 3 of a raw buffer resource on gfx950: 32-bit data format, no swizzle,
// no index stride (the loads below address bytes directly).
constexpr int kRawDwordRsrc = 0x00020000;
// A byte offset past the view's buffer range (one view of the sinogram, below
// 2^31 bytes): the range check makes its load a zero.
constexpr unsigned kOffRange = 0x80000000u;
// s_waitcnt immediate: vmcnt(n) and lgkmcnt(0) (expcnt at its maximum), and
// vmcnt(n) alone.
__host__ __device__ constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
__host__ __device__ constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Back projection.  Per view, the sinogram cells the tile can reach arrive in
// two steps, two views ahead of their use, with no registers held:
//   1. direct global-to-LDS loads copy the window's SL rows (RP = 32 or 64
//      channels each, the sinogram's own layout; cells off the detector or
//      past the last slice come in as zeros from the buffer range check) into
//      one of two raw buffers, wave w taking rows [w SL/4, (w + 1) SL/4);
//   2. each wave transposes the rows it loaded itself (its own load count is
//      all it waits for) into the slice-fastest window the gather reads, four
//      slices of one channel per 16-byte store.
// One barrier per view publishes the transposed window.  The barrier is the
// bare instruction behind compiler-only fences, with the waits written out:
// the workgroup fence of __syncthreads would wait for every load in flight,
// the next views' included.  The four buffers are separate LDS arrays and the
// view loop is unrolled by two, so that every access names its buffer and the
// compiler's own waits for the direct loads cover only the buffer they write;
// every load of a view is issued unconditionally (clamped indices past the
// last view), so that the wait counts are the same on every path.
template <int SL, int NTAP, int RP, int POW>
__global__ __launch_bounds__(BT *BT, 4) void par_back_kernel(const float *__restrict__ sino,
                                                              float *__restrict__ recon,
                                                              const int32_t *__restrict__ rec,
                                                              const int4 *__restrict__ wtab, Geo g, int nwcap) {
    // LDS pitch of one channel column: a multiple of four floats, so a lane
    // reads four slices of a tap with one 16-byte read; SLP / 4 is odd, so
    // 16 lanes on consecutive channels hit 16 distinct bank groups
    constexpr int SLP = SL + 4;
    static_assert(SL % 8 == 0 && (SLP / 4) % 2 == 1, "16-byte column reads need SL a multiple of 8");
    static_assert(RP == 32 || RP == 64, "raw rows of 32 or 64 channels");
    static_assert(RP == 32 || SL <= 32, "LDS: 64-channel windows take chunks of at most 32 slices");
    constexpr int NREC = 1 + NTAP;
    constexpr int R4 = SL / 4;            // raw rows per wave
    constexpr int RPI = 64 / RP;          // raw rows per load instruction
    constexpr int KD = R4 / RPI;          // load instructions per wave per view
    constexpr int G = R4 >= 4 ? 4 : 2;    // slices per transposed store
    constexpr int NU = RP * R4 / G;       // transposed stores per wave per view
    constexpr int UPL = (NU + 63) / 64;   // per lane
    __shared__ float raw0[SL * RP], raw1[SL * RP];      // [SL][RP]: rows as in the sinogram
    __shared__ float win0[RP * SLP], win1[RP * SLP];    // [nwcap <= RP][SLP]: slices fastest

    const int tiles_x = (g.nx + BT - 1) / BT;
    const int ntiles = tiles_x * ((g.ny + BT - 1) / BT);
    int tile, chunk;
    xcd_work_item((int)gridDim.x, (int)gridDim.y, tile, chunk);
    tile = __builtin_amdgcn_readfirstlane(tile);
    const int tj0 = (tile % tiles_x) * BT;
    const int ti0 = (tile / tiles_x) * BT;
    const int k0 = chunk * SL;
    const int nk = min(SL, g.ns - k0);

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = ti0 + tid / BT;
    const int j = tj0 + tid % BT;
    const bool valid = (i < g.ny) && (j < g.nx);
    const int np = g.ny * g.nx;
    const int p = valid ? i * g.nx + j : 0;
    const int64_t vfl = (int64_t)g.nr * g.nc;      // floats per view (bytes below 2^31, checked by the plan)
    const int vlast = g.nv - 1;

    // the window of view v (clamped), through a wave-uniform index: a scalar load
    auto window = [&](int v) { return wtab[(int64_t)__builtin_amdgcn_readfirstlane(min(v, vlast)) * ntiles + tile]; };
    // step 1 for view v (clamped: past the last view the loads are issued all
    // the same, into a buffer nothing reads again), window w, into raw buffer
    // rb: row r of the window is slice k0 + r, lane l of an instruction
    // channel w.x + l % RP of row l / RP
    auto dma_view = [&](int v, const int4 &w, float *rb) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(sino + (int64_t)min(v, vlast) * vfl), (short)0, (int)(vfl * 4), kRawDwordRsrc);
        const int c = lane % RP, n = w.x + c;
        const bool cok = c < w.y && (unsigned)n < (unsigned)g.nc;
        // (branch-free: a channel off the detector starts past the range; a
        // row past the last slice is a detector row past the last one, so its
        // offset is past the view's range anyway; the sums stay below 2^32)
        const unsigned base = cok ? (unsigned)(k0 * g.nc + n) * 4u : kOffRange;
#pragma unroll
        for (int u = 0; u < KD; ++u) {
            const int r0 = wave * R4 + u * RPI;          // first row of this instruction
            const int r = r0 + lane / RP;
            const unsigned off = base + (unsigned)(r * g.nc) * 4u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(rb + r0 * RP),
                                                     4, off, 0, 0, 0);
        }
    };
    // step 2: this wave's raw rows into the window: store unit u is channel
    // u % RP and G slices from row wave R4 + G (u / RP) (with RP = 32 the two
    // halves of a wave read rows 4 apart, in the same banks: a two-way
    // conflict on these few reads)
    auto transpose = [&](const float *rb, float *wb) {
#pragma unroll
        for (int e = 0; e < UPL; ++e) {
            const int u = lane + 64 * e;
            const int c = u % RP, r = wave * R4 + G * (u / RP);
            if (u < NU && c < nwcap) {
                float x[G];
#pragma unroll
                for (int t = 0; t < G; ++t) x[t] = rb[(r + t) * RP + c];
                float *dst = wb + c * SLP + r;
                if constexpr (G == 4)
                    *reinterpret_cast<float4 *>(dst) = make_float4(x[0], x[1], x[2], x[3]);
                else
                    *reinterpret_cast<float2 *>(dst) = make_float2(x[0], x[1]);
            }
        }
    };
    // the tap records of view v (clamped) for this lane's pixel (pixel 0 for
    // lanes outside the volume, whose records are never used)
    auto load_taps = [&](int v, int &nf, float (&w)[NTAP]) {
        const int32_t *r = rec + ((int64_t)min(v, vlast) * np + p) * NREC;
        nf = r[0];
#pragma unroll
        for (int t = 0; t < NTAP; ++t) {
            const float wt = __int_as_float(r[1 + t]);
            w[t] = POW == 2 ? wt * wt : wt;       // squared weights: the Hessian-diagonal back projection
        }
    };
    auto barrier = [&]() {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));   // this wave's LDS stores done
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    float acc[SL];
#pragma unroll
    for (int k = 0; k < SL; ++k) acc[k] = 0.f;
    if (g.nv == 0) return;

    // prologue: views 0 and 1 loaded, view 0 transposed.  The tap records
    // go to staging registers two views ahead (one set per view parity) and
    // reach the working set (nf, wt) after the wait that covers them, so the
    // gather never waits for a load
    int4 wa = window(0), wb = window(1);
    dma_view(0, wa, raw0);
    dma_view(1, wb, raw1);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    int nf, nfa, nfb;
    float wt[NTAP], wta[NTAP], wtb[NTAP];
    load_taps(0, nf, wt);
    load_taps(1, nfb, wtb);
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    transpose(raw0, win0);
    barrier();

    // one view: gather view v (working taps; window wv) from window buffer wc;
    // the loads of view v + 2 go out first (into rc, the raw buffer of view v,
    // transposed in the previous step), its tap records after the gather
    // (into the staging set sc of view v's parity); view v + 1's rows, loaded
    // one step earlier into rn, are transposed last, into wn, and its records
    // (staging set sn) become the working taps
    auto step = [&](int v, int4 &wv, int &nfc, float (&wtc)[NTAP], const int &nfn, const float (&wtn)[NTAP],
                    float *rc, const float *wc, const float *rn, float *wn) {
        const int4 w2 = window(v + 2);
        dma_view(v + 2, w2, rc);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (valid && nf != INT32_MAX && wv.y > 0) {
            const float4 *col = reinterpret_cast<const float4 *>(wc + (nf - wv.x) * SLP);
#pragma unroll
            for (int q = 0; q < SL / 4; ++q) {
                float4 c[NTAP];
#pragma unroll
                for (int t = 0; t < NTAP; ++t) c[t] = col[t * (SLP / 4) + q];
                float s0 = acc[4 * q], s1 = acc[4 * q + 1], s2 = acc[4 * q + 2], s3 = acc[4 * q + 3];
#pragma unroll
                for (int t = 0; t < NTAP; ++t) {
                    s0 = fmaf(wt[t], c[t].x, s0);
                    s1 = fmaf(wt[t], c[t].y, s1);
                    s2 = fmaf(wt[t], c[t].z, s2);
                    s3 = fmaf(wt[t], c[t].w, s3);
                }
                acc[4 * q] = s0;
                acc[4 * q + 1] = s1;
                acc[4 * q + 2] = s2;
                acc[4 * q + 3] = s3;
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        load_taps(v + 2, nfc, wtc);
        wv = w2;
        // issued after this wave's loads of view v + 1: its tap records, view
        // v + 2's KD rows and its records (the record loads are not counted,
        // however many instructions they take: all but the last KD loads
        // landed covers view v + 1, rows and records)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(wait_vm(KD));
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (v + 1 < g.nv) transpose(rn, wn);
        // the working taps, redefined by an empty statement: any wait for the
        // staged loads falls here, after the one above that covers them, and
        // not in front of the next gather
        nf = nfn;
        asm volatile("" : "+v"(nf));
#pragma unroll
        for (int t = 0; t < NTAP; ++t) {
            wt[t] = wtn[t];
            asm volatile("" : "+v"(wt[t]));
        }
        barrier();
    };
    for (int v = 0; v < g.nv; v += 2) {
        step(v, wa, nfa, wta, nfb, wtb, raw0, win0, raw1, win1);
        if (v + 1 >= g.nv) break;
        step(v + 1, wb, nfb, wtb, nfa, wta, raw1, win1, raw0, win0);
    }
    // (the loads issued for views past the last one land before the wave
    // ends; nothing reads them)
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    if (valid) {
        float *out = recon + (int64_t)p * g.ns + k0;
#pragma unroll
        for (int k = 0; k < SL; ++k)
            if (k < nk) out[k] = acc[k];
    }
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N - 1, unrolled at compile time.
template <class F, int... I>
__device__ __forceinline__ void static_for(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}

// Lane N of each 16-lane row, broadcast to its row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ uint32_t row_bcast(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + N, 0xf, 0xf, false);
}

// acc += w' * x, where w' is lane N of the row of w: one v_fmac with the
// broadcast folded into its DPP operand.  The s_nop gives the two wait states
// a DPP read needs after a VALU write of its source; the second product of a
// pair is covered by the first.
template <int N>
__device__ __forceinline__ void fmac_row_bcast(float &acc, uint32_t w, float x) {
    asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(w), "v"(x), "n"(N));
}
template <int N>
__device__ __forceinline__ void fmac2_row_bcast(float &a0, float &a1, uint32_t w0, uint32_t w1, float x) {
    asm("s_nop 1\n\tv_fmac_f32_dpp %0, %2, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
        : "+v"(a0), "+v"(a1)
        : "v"(w0), "v"(w1), "v"(x), "n"(N));
}

template <int N>
__device__ __forceinline__ void fmac4_row_bcast(float &a0, float &a1, float &b0, float &b1, uint32_t w0, uint32_t w1,
                                                float x, float y) {
    asm("s_nop 1\n\tv_fmac_f32_dpp %0, %4, %6 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %6 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %4, %7 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %5, %7 row_newbcast:%8 row_mask:0xf bank_mask:0xf"
        : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1)
        : "v"(w0), "v"(w1), "v"(x), "v"(y), "n"(N));
}

template <int N>
__device__ __forceinline__ void fmac2xy_row_bcast(float &a0, float &a1, uint32_t w, float x, float y) {
    asm("s_nop 1\n\tv_fmac_f32_dpp %0, %2, %3 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %2, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
        : "+v"(a0), "+v"(a1)
        : "v"(w), "v"(x), "v"(y), "n"(N));
}

// Lane N of each 16-lane row, broadcast to its row, without a prior value.
template <int N>
__device__ __forceinline__ uint32_t row_bcast_nb(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x150 + N, 0xf, 0xf, true);
}

template <int K, int SPL>
__global__ __launch_bounds__(FRW * 64) void par_forward_kernel(const float *__restrict__ recon,
                                                                float *__restrict__ facc,
                                                                const uint32_t *__restrict__ wrec, Geo g, int cb,
                                                                int s16, int rsx, int rsy, int nrx, int nreg, int ng,
                                                                int vsplit) {
    constexpr int NF = 2 + K;             // record fields per step
    constexpr int D = 4;                  // voxel reads in flight ahead of the step using them
    constexpr int CS = 16 * SPL;          // slices of a chunk: SPL per lane, 16 apart
    static_assert(SPL == 1 || SPL == 2, "one or two slices per lane");
    using XV = typename std::conditional<SPL == 2, float2, float>::type;   // a lane's voxels of one step
    extern __shared__ float xr[];         // the region's voxels, [pixel][CS slices]
    const int lane = (int)threadIdx.x & 63;
    const int row = lane >> 4, sl = lane & 15;
    // wave index, made visibly uniform so that per-view control stays scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    // Workgroup L of a view range is assumed to run on XCD L mod 8 (the
    // dispatch order): the slice chunks of one region get consecutive slots on
    // one XCD, so that they read the region's records through one L2.  Any
    // other placement is still correct, only slower.
    const int nch = (g.ns + CS - 1) / CS;
    const int per_range = 8 * ((nreg + 7) / 8) * nch;
    const int L = (int)(blockIdx.x % (unsigned)per_range);
    const int vrange = (int)(blockIdx.x / (unsigned)per_range);
    const int slot = L >> 3;
    const int region = (slot / nch) * 8 + (L & 7);
    if (region >= nreg) return;
    const int i0 = (region / nrx) * rsy, j0 = (region % nrx) * rsx;
    const int k0 = (slot % nch) * CS;
    const int rp = rsx * rsy;

    // a pixel's CS slices in LDS; with two slices per lane, slices k and
    // k + 16 side by side (k < 16), so that a lane's pair is one aligned
    // 8-byte read: two rows of a wave then share banks only when their pixels
    // have the same parity, where slices 16 apart shared them whenever that
    // held for any two of the four rows
    for (int e = (int)threadIdx.x; e < rp * CS; e += FRW * 64) {
        const int p = e / CS, k = e % CS;
        const int i = i0 + p / rsx, j = j0 + p % rsx;
        float val = 0.f;
        if (i < g.ny && j < g.nx && k0 + k < g.ns) val = recon[(int64_t)(i * g.nx + j) * g.ns + k0 + k];
        xr[SPL == 2 ? p * CS + (k % 16) * 2 + k / 16 : e] = val;
    }
    __syncthreads();

    const int vper = (g.nv + vsplit - 1) / vsplit;
    const int vbeg = vrange * vper;
    const int vend = min(g.nv, vbeg + vper);
    const char *xb = reinterpret_cast<const char *>(xr);
    char *fv = reinterpret_cast<char *>(facc + (int64_t)vbeg * cb * s16);
    // lane sl holds slices sl and sl + 16 of the chunk: one paired LDS read per
    // step, and a flush covers 16 consecutive slices (64 bytes) per atomic
    const uint32_t l4 = (uint32_t)sl * 4u;          // this lane's first slice, bytes
    const uint32_t s4 = (uint32_t)s16 * 4u;         // bytes between channels of the accumulation buffer
    const uint32_t ks = (uint32_t)K * s4;           // bytes per ring turn
    const int64_t gstride = (int64_t)NF * 16;       // dwords per group of 16 steps
    constexpr int PD = 4;                           // groups of records in flight ahead of their use

    // each row of a wave walks its own view; views past the range walk the
    // all-zero records of view nv (no weights, no flushes)
    for (int q0 = vbeg + wave * 4; q0 < vend; q0 += FRW * 4) {
        const int vrow = q0 + row < vend ? q0 + row : g.nv;
        const uint32_t *rb = wrec + ((int64_t)vrow * nreg + region) * ng * gstride + sl;
        // byte offset from fv (this workgroup's first view) of ring turn 0,
        // accumulator r, for this lane's first slice: turn T, accumulator r is
        // at vb[r] + T * ks (modulo 2^32; the sum itself stays below 2^31)
        uint32_t vb[K];
#pragma unroll
        for (int r = 0; r < K; ++r)
            vb[r] = (uint32_t)(((min(vrow, g.nv - 1) - vbeg) * cb + (K - 1)) * s16 + k0) * 4u + l4 + r * s4 - ks;
        float acc[SPL][K];
#pragma unroll
        for (int s = 0; s < SPL; ++s)
#pragma unroll
            for (int r = 0; r < K; ++r) acc[s][r] = 0.f;

        auto load_group = [&](int gi, uint32_t (&R)[NF]) {
            const uint32_t *b = rb + (int64_t)gi * gstride;
#pragma unroll
            for (int f = 0; f < NF; ++f) R[f] = b[f * 16];
        };
        // one group of 16 steps from R; the group PD turns later is fetched
        // into P meanwhile (always issued, for a static wait count)
        auto walk_group = [&](int gi, uint32_t (&R)[NF], uint32_t (&P)[NF]) {
            load_group(min(gi + PD, ng - 1), P);
            uint64_t m = __builtin_amdgcn_ballot_w64(R[1] != 0u);
            m |= m >> 32;
            m |= m >> 16;
            const uint32_t fl = (uint32_t)m & 0xffffu;      // steps after which some row flushes
            XV xq[16];
            auto read_x = [&](auto SC) {
                constexpr int S = decltype(SC)::value;
                if constexpr (SPL == 2)
                    xq[S] = *reinterpret_cast<const float2 *>(xb + (row_bcast<S>(R[0]) + 2u * l4));
                else
                    xq[S] = *reinterpret_cast<const float *>(xb + (row_bcast<S>(R[0]) + l4));
            };
            static_for(read_x, std::make_integer_sequence<int, D>{});
            static_for(
                [&](auto SC) {
                    constexpr int S = decltype(SC)::value;
                    if constexpr (S + D < 16) read_x(std::integral_constant<int, S + D>{});
                    if constexpr (SPL == 2) {
#pragma unroll
                        for (int r = 0; r < K; r += 2) {
                            if (r + 1 < K)
                                fmac4_row_bcast<S>(acc[0][r], acc[0][r + 1 < K ? r + 1 : r], acc[SPL - 1][r],
                                                   acc[SPL - 1][r + 1 < K ? r + 1 : r], R[2 + r],
                                                   R[r + 1 < K ? 3 + r : 2 + r], xq[S].x, xq[S].y);
                            else
                                fmac2xy_row_bcast<S>(acc[0][r], acc[SPL - 1][r], R[2 + r], xq[S].x, xq[S].y);
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < K; r += 2) {
                            if (r + 1 < K)
                                fmac2_row_bcast<S>(acc[0][r], acc[0][r + 1 < K ? r + 1 : r], R[2 + r],
                                                   R[r + 1 < K ? 3 + r : 2 + r], xq[S]);
                            else
                                fmac_row_bcast<S>(acc[0][r], R[2 + r], xq[S]);
                        }
                    }
                    if (__builtin_expect((fl >> S) & 1u, 0)) {       // out of line: most steps flush nothing
                        const uint32_t f = row_bcast_nb<S>(R[1]);     // this row's flush word
                        const uint32_t t = f >> 14;
#pragma unroll
                        for (int r = 0; r < K; ++r) {
                            if (f & (1u << r)) {
                                const uint32_t turn = t + ((f >> (7 + r)) & 1u);
                                float *dst = reinterpret_cast<float *>(fv + (__umul24(turn, ks) + vb[r]));
#pragma unroll
                                for (int s = 0; s < SPL; ++s) {
                                    unsafeAtomicAdd(dst + 16 * s, acc[s][r]);
                                    acc[s][r] = 0.f;
                                }
                            }
                        }
                    }
                },
                std::make_integer_sequence<int, 16>{});
        };

        // PD + 1 record buffers in rotation (no copies, so no early waits)
        uint32_t RB0[NF], RB1[NF], RB2[NF], RB3[NF], RB4[NF];
        // issued in order (no reordering across the barriers), so that the
        // wait for a buffer never covers the loads of later ones
        load_group(0, RB0);
        __builtin_amdgcn_sched_barrier(0);
        load_group(1, RB1);
        __builtin_amdgcn_sched_barrier(0);
        load_group(2, RB2);
        __builtin_amdgcn_sched_barrier(0);
        load_group(3, RB3);
        __builtin_amdgcn_sched_barrier(0);
        for (int gi = 0; gi < ng; gi += 5) {          // ng is a multiple of 5 (zero groups pad it)
            walk_group(gi, RB0, RB4);
            walk_group(gi + 1, RB1, RB0);
            walk_group(gi + 2, RB2, RB1);
            walk_group(gi + 3, RB3, RB2);
            walk_group(gi + 4, RB4, RB3);
        }
    }
}

// Gather strategy walk.  Same lanes (16 slices x 4 rows, a view per row),
// ring accumulators, records and flushes as the region walk, but a row walks
// one segment of its view's sorted pixel list (all pixels of the image), and
// reads each step's voxels from the volume with a vector load (64 bytes per
// row, cached).  A workgroup takes 64 consecutive views at one (segment, slice
// chunk): their segments cover nearly the same pixels, which then come from
// the cache.  The last step of every segment flushes all accumulators, so a
// channel split between two segments is added once by each.
// The voxels of group g + 1 are loaded while group g is summed, the
// records three groups ahead; two voxel buffers and four record buffers rotate
// without copies (the walk is unrolled by four groups).
template <int K>
__global__ __launch_bounds__(FRW * 64) void par_gather_kernel(const float *__restrict__ recon,
                                                               float *__restrict__ facc,
                                                               const uint32_t *__restrict__ wrec, Geo g, int cb,
                                                               int s16, int ng, int segg, int nseg) {
    constexpr int NF = 2 + K;
    constexpr int PD = 3;                 // record groups in flight ahead of their use
    const int lane = (int)threadIdx.x & 63;
    const int row = lane >> 4, sl = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int nvb = (g.nv + 63) / 64;
    const int vb = (int)(blockIdx.x % (unsigned)nvb) * 64;
    const int rest = (int)(blockIdx.x / (unsigned)nvb);
    const int seg = rest % nseg, chunk = rest / nseg;
    const int k0 = chunk * 16;
    const int g0 = seg * segg, g1 = min(ng, g0 + segg);    // both multiples of 4
    const int q0 = vb + wave * 4;
    if (q0 >= g.nv) return;
    // each row walks its own view; views past the end walk the zero records of view nv
    const int vrow = q0 + row < g.nv ? q0 + row : g.nv;
    const uint32_t *rb = wrec + (int64_t)vrow * ng * NF * 16 + sl;
    // lanes past the last slice read slice k0 (a valid address) and drop it:
    // the loads stay unpredicated, so every lane is active for the DPP
    // broadcasts that form their addresses (a DPP read from an inactive lane
    // returns nothing)
    const bool kin = k0 + sl < g.ns;
    const char *xb = reinterpret_cast<const char *>(recon);
    const uint32_t xl = (uint32_t)(k0 + (kin ? sl : 0)) * 4u;     // + p * S * 4 from the records
    const uint32_t s4 = (uint32_t)s16 * 4u;
    const uint32_t ks = (uint32_t)K * s4;
    char *fv = reinterpret_cast<char *>(facc + (int64_t)vb * cb * s16);
    uint32_t vbo[K];
#pragma unroll
    for (int r = 0; r < K; ++r)
        vbo[r] = (uint32_t)(((min(vrow, g.nv - 1) - vb) * cb + (K - 1)) * s16 + k0) * 4u + (uint32_t)sl * 4u + r * s4 - ks;
    float acc[K];
#pragma unroll
    for (int r = 0; r < K; ++r) acc[r] = 0.f;

    auto load_group = [&](int gi, uint32_t (&R)[NF]) {
        const uint32_t *b = rb + (int64_t)gi * NF * 16;
#pragma unroll
        for (int f = 0; f < NF; ++f) R[f] = b[f * 16];
    };
    auto load_x = [&](const uint32_t (&R)[NF], float (&X)[16]) {
        static_for(
            [&](auto SC) {
                constexpr int S = decltype(SC)::value;
                const float xv = *reinterpret_cast<const float *>(xb + (row_bcast<S>(R[0]) + xl));
                X[S] = kin ? xv : 0.f;
            },
            std::make_integer_sequence<int, 16>{});
    };
    // one group: fetch the records PD groups ahead into P and the voxels of the
    // next group (records RN) into XN, then sum this group (records R, voxels X)
    auto walk_group = [&](int gi, const uint32_t (&R)[NF], const uint32_t (&RN)[NF], uint32_t (&P)[NF],
                          const float (&X)[16], float (&XN)[16]) {
        load_group(min(gi + PD, g1 - 1), P);
        load_x(RN, XN);
        uint64_t m = __builtin_amdgcn_ballot_w64(R[1] != 0u);
        m |= m >> 32;
        m |= m >> 16;
        const uint32_t fl = (uint32_t)m & 0xffffu;
        static_for(
            [&](auto SC) {
                constexpr int S = decltype(SC)::value;
#pragma unroll
                for (int r = 0; r < K; r += 2) {
                    if (r + 1 < K)
                        fmac2_row_bcast<S>(acc[r], acc[r + 1 < K ? r + 1 : r], R[2 + r], R[r + 1 < K ? 3 + r : 2 + r],
                                           X[S]);
                    else
                        fmac_row_bcast<S>(acc[r], R[2 + r], X[S]);
                }
                if (__builtin_expect((fl >> S) & 1u, 0)) {
                    const uint32_t f = row_bcast_nb<S>(R[1]);
                    const uint32_t t = f >> 14;
#pragma unroll
                    for (int r = 0; r < K; ++r) {
                        if (f & (1u << r)) {
                            const uint32_t turn = t + ((f >> (7 + r)) & 1u);
                            unsafeAtomicAdd(reinterpret_cast<float *>(fv + (__umul24(turn, ks) + vbo[r])), acc[r]);
                            acc[r] = 0.f;
                        }
                    }
                }
            },
            std::make_integer_sequence<int, 16>{});
    };

    uint32_t R0[NF], R1[NF], R2[NF], R3[NF];
    float XA[16], XB[16];
    load_group(g0, R0);
    __builtin_amdgcn_sched_barrier(0);
    load_group(min(g0 + 1, g1 - 1), R1);
    __builtin_amdgcn_sched_barrier(0);
    load_group(min(g0 + 2, g1 - 1), R2);
    __builtin_amdgcn_sched_barrier(0);
    load_x(R0, XA);
    for (int gi = g0; gi < g1; gi += 4) {
        walk_group(gi, R0, R1, R3, XA, XB);
        walk_group(gi + 1, R1, R2, R0, XB, XA);
        walk_group(gi + 2, R2, R3, R1, XA, XB);
        walk_group(gi + 3, R3, R0, R2, XB, XA);
    }
    // every segment's last step flushes all accumulators (the records say so)
}

// Translation scans (every view at angle 0, the detector shifted per view):
// the channel coordinate of a pixel centre, (x cos + y sin) / dch + ... with
// sin = 0 exactly, does not depend on the pixel's row, so every pixel of a
// column j has the same tap record in every view (the creation pass's records
// of row 0 serve for all rows, bit for bit).  The operator then factors
// through the column sums: sino[v][k][n] = sum over j of w_{n - nf(v,j)}(v, j)
// times the sum over rows i of x[i][j][k], and the back projection is one
// value per (column, slice), the same in every row.

// cs[j][k] = sum over rows i of x[i][j][k]: a workgroup takes 64 consecutive
// (column, slice) cells, each wave a quarter of the rows (16 rows' loads in
// flight), and adds the four partial sums in a fixed order.
__global__ __launch_bounds__(256) void par_colsum_kernel(const float *__restrict__ x, float *__restrict__ cs, int ny,
                                                         int tot) {
    __shared__ float part[4][64];
    const int lane = (int)threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int e = (int)blockIdx.x * 64 + lane;            // j * S + k
    const float *px = x + min(e, tot - 1);
    const int rper = (ny + 3) / 4, r0 = wave * rper, r1 = min(ny, r0 + rper);
    float s = 0.f;
    int i = r0;
    for (; i + 16 <= r1; i += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = px[(int64_t)(i + u) * tot];
#pragma unroll
        for (int u = 0; u < 16; ++u) s += v[u];
    }
    for (; i < r1; ++i) s += px[(int64_t)i * tot];
    part[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && e < tot) cs[e] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
}

// The forward from the column sums: a wave owns view v, a block of 64
// channels and a chunk of 64 slices, and adds into an LDS tile [channel][slice]
// every column whose taps reach the block (columns in order; the records of 64
// columns per vector load, read out by readlane; the column sums of eight
// columns loaded together), then stores the tile as sinogram rows.  Each lane
// adds only into its own slice of the tile.
template <int NTAP, int POW>
__global__ __launch_bounds__(64) void par_colfwd_kernel(const float *__restrict__ cs, const int32_t *__restrict__ rec,
                                                        float *__restrict__ sino, Geo g, int nblk, int nchk) {
    __shared__ float tile[64][65];
    const int lane = (int)threadIdx.x;
    const int item = (int)blockIdx.x;
    const int chunk = item % nchk, blk = (item / nchk) % nblk, v = item / (nchk * nblk);
    const int n0 = blk * 64, k0 = chunk * 64;
    const int kc = min(k0 + lane, g.ns - 1);               // lanes past the last slice add, but store nothing
    const int np = g.ny * g.nx;
    const int32_t *rv = rec + (int64_t)v * np * (1 + NTAP);   // row 0 of view v
#pragma unroll 8
    for (int c = 0; c < 64; ++c) tile[c][lane] = 0.f;
    for (int j0 = 0; j0 < g.nx; j0 += 64) {
        const int32_t *r = rv + (int64_t)min(j0 + lane, g.nx - 1) * (1 + NTAP);
        const int rnf = r[0];
        int rw[NTAP];
#pragma unroll
        for (int t = 0; t < NTAP; ++t) rw[t] = r[1 + t];
        // the columns of this group whose taps reach the block, in order,
        // eight at a time: their column sums are loaded together, then added
        uint64_t m = __builtin_amdgcn_ballot_w64(j0 + lane < g.nx && rnf != INT32_MAX && rnf <= n0 + 63 &&
                                                 rnf + NTAP - 1 >= n0);
        while (m) {
            int js[8];
            float xs[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                js[u] = m ? (int)__builtin_ctzll(m) : -1;
                m &= m - 1;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) xs[u] = cs[(int64_t)(j0 + max(js[u], 0)) * g.ns + kc];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (js[u] < 0) break;                 // uniform
                const int nf = __builtin_amdgcn_readlane(rnf, js[u]);
#pragma unroll
                for (int t = 0; t < NTAP; ++t) {
                    const int c = nf + t - n0;
                    float w = __int_as_float(__builtin_amdgcn_readlane(rw[t], js[u]));
                    if (POW == 2) w = w * w;
                    if (c >= 0 && c < 64) tile[c][lane] = fmaf(w, xs[u], tile[c][lane]);
                }
            }
        }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);    // (LDS operations of a wave complete in order)
    const int n = n0 + lane;
    if (n < g.nc)
        for (int r = 0; r < 64 && k0 + r < g.nr; ++r) sino[((int64_t)v * g.nr + k0 + r) * g.nc + n] = tile[lane][r];
}

// The back of a translation scan: lane e of the grid is the (column, slice)
// cell j * S + k; it sums over views, taps in order, exactly as the back
// kernel does for any pixel of column j (the same bits), eight views' loads
// in flight, then stores the value into every row, the cells of a wave
// contiguous in each.
template <int NTAP, int POW>
__global__ __launch_bounds__(64) void par_colback_kernel(const float *__restrict__ sino,
                                                         const int32_t *__restrict__ rec, float *__restrict__ recon,
                                                         Geo g) {
    constexpr int U = 8;
    const int tot = g.nx * g.ns;
    const int e = (int)blockIdx.x * 64 + (int)threadIdx.x;
    const int ec = min(e, tot - 1);
    const int j = ec / g.ns, k = ec - j * g.ns;
    const int np = g.ny * g.nx;
    float acc = 0.f;
    for (int v0 = 0; v0 < g.nv; v0 += U) {
        int nf[U];
        float w[U][NTAP], y[U][NTAP];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = min(v0 + u, g.nv - 1);
            const int32_t *r = rec + ((int64_t)v * np + j) * (1 + NTAP);
            nf[u] = v0 + u < g.nv ? r[0] : INT32_MAX;
#pragma unroll
            for (int t = 0; t < NTAP; ++t) {
                const float wt = __int_as_float(r[1 + t]);
                w[u][t] = POW == 2 ? wt * wt : wt;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float *row = sino + ((int64_t)min(v0 + u, g.nv - 1) * g.nr + k) * g.nc;
#pragma unroll
            for (int t = 0; t < NTAP; ++t) {
                const int c = nf[u] + t;
                const bool in = nf[u] != INT32_MAX && c >= 0 && c < g.nc;
                const float val = row[in ? c : 0];
                y[u][t] = in ? val : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (nf[u] != INT32_MAX)                  // a view without a footprint here is left out, as in the back
#pragma unroll
                for (int t = 0; t < NTAP; ++t) acc = fmaf(w[u][t], y[u][t], acc);
    }
    if (e < tot)
        for (int i = 0; i < g.ny; ++i) recon[(int64_t)i * tot + e] = acc;
}

// facc [V][cb][s16] (slices fastest, K - 1 guard channels each side) ->
// sino [V][R][C] (channels fastest), through a 64 x 64 LDS tile.  (The cone
// batches use it too, on the sinogram transposed, with no guard channels.)
__global__ __launch_bounds__(256) void par_unpack_kernel(const float *__restrict__ facc, float *__restrict__ sino,
                                                         int nr, int nc, int cb, int s64, int guard, int tn) {
    __shared__ float t[64][65];
    const int v = (int)(blockIdx.x / (unsigned)tn);
    const int n0 = (int)(blockIdx.x % (unsigned)tn) * 64;
    const int r0 = (int)blockIdx.y * 64;
    const int a = (int)threadIdx.x & 63, b = (int)threadIdx.x >> 6;
    const float *src = facc + ((int64_t)v * cb + guard + n0) * s64 + r0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int n = b + 4 * u;
        t[n][a] = (n0 + n < nc && r0 + a < nr) ? src[(int64_t)n * s64 + a] : 0.f;
    }
    __syncthreads();
    float *dst = sino + ((int64_t)v * nr + r0) * nc + n0;
    if (n0 + a < nc) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int r = b + 4 * u;
            if (r0 + r < nr) dst[(int64_t)r * nc + a] = t[a][r];
        }
    }
}

template <int SL, int NTAP, int POW>
static hipError_t par_back_t(const Plan &p, const float *sino, float *recon, hipStream_t st) {
    const Geo &g = p.g;
    const int tiles = ((g.nx + BT - 1) / BT) * ((g.ny + BT - 1) / BT);
    const int chunks = (g.ns + SL - 1) / SL;
    // (LDS is static in the kernel: raw and transposed windows of 32 or 64 channels)
    if (p.back_ncg == 1) {
        hipLaunchKernelGGL((par_back_kernel<SL, NTAP, 32, POW>), dim3(tiles, chunks), dim3(BT * BT), 0, st,
                           sino, recon, p.rec, p.bwin, g, p.back_nwcap);
    } else {
        if constexpr (SL <= 32)
            hipLaunchKernelGGL((par_back_kernel<SL, NTAP, 64, POW>), dim3(tiles, chunks), dim3(BT * BT), 0, st,
                               sino, recon, p.rec, p.bwin, g, p.back_nwcap);
        else
            return hipErrorInvalidValue;   // the plan takes chunks of at most 32 slices for 64-channel windows
    }
    return hipGetLastError();
}

template <int K, int SPL>
static hipError_t par_fwd_s(const Plan &p, const float *recon, hipStream_t st) {
    const Geo &g = p.g;
    const int nrx = (g.nx + p.rsx - 1) / p.rsx, nry = (g.ny + p.rsy - 1) / p.rsy;
    const int ng = fwd_groups(p.rsx, p.rsy);
    const int64_t per_range = 8 * (int64_t)((nrx * nry + 7) / 8) * ((g.ns + 16 * SPL - 1) / (16 * SPL));
    hipLaunchKernelGGL((par_forward_kernel<K, SPL>), dim3((unsigned)(per_range * p.fwd_vsplit)), dim3(FRW * 64),
                       p.fwd_lds, st, recon, p.facc, p.wrec, g, p.fwd_cb, p.fwd_s16, p.rsx, p.rsy, nrx, nrx * nry, ng,
                       p.fwd_vsplit);
    return hipGetLastError();
}

template <int K>
static hipError_t par_fwd_t(const Plan &p, const float *recon, hipStream_t st) {
    return p.fwd_spl == 2 ? par_fwd_s<K, 2>(p, recon, st) : par_fwd_s<K, 1>(p, recon, st);
}

template <int SL, int POW>
static hipError_t par_back_sl(const Plan &p, const float *sino, float *recon, hipStream_t st) {
    switch (p.ntap) {
    case 2: return par_back_t<SL, 2, POW>(p, sino, recon, st);
    case 3: return par_back_t<SL, 3, POW>(p, sino, recon, st);
    case 4: return par_back_t<SL, 4, POW>(p, sino, recon, st);
    case 5: return par_back_t<SL, 5, POW>(p, sino, recon, st);
    case 6: return par_back_t<SL, 6, POW>(p, sino, recon, st);
    case 7: return par_back_t<SL, 7, POW>(p, sino, recon, st);
    default: return hipErrorInvalidValue;
    }
}

template <int POW>
static hipError_t par_back_pow(const Plan &p, const float *sino, float *recon, hipStream_t st) {
    switch (p.back_sl) {
    case 8: return par_back_sl<8, POW>(p, sino, recon, st);
    case 16: return par_back_sl<16, POW>(p, sino, recon, st);
    case 32: return par_back_sl<32, POW>(p, sino, recon, st);
    case 64: return par_back_sl<64, POW>(p, sino, recon, st);
    default: return hipErrorInvalidValue;
    }
}

template <int POW>
static hipError_t par_colback_pow(const Plan &p, const float *sino, float *recon, hipStream_t st) {
    const Geo &g = p.g;
    const int64_t tot = (int64_t)g.nx * g.ns;
    const dim3 grid((unsigned)((tot + 63) / 64));
    switch (p.ntap) {
    case 2: hipLaunchKernelGGL((par_colback_kernel<2, POW>), grid, dim3(64), 0, st, sino, p.rec, recon, g); break;
    case 3: hipLaunchKernelGGL((par_colback_kernel<3, POW>), grid, dim3(64), 0, st, sino, p.rec, recon, g); break;
    case 4: hipLaunchKernelGGL((par_colback_kernel<4, POW>), grid, dim3(64), 0, st, sino, p.rec, recon, g); break;
    case 5: hipLaunchKernelGGL((par_colback_kernel<5, POW>), grid, dim3(64), 0, st, sino, p.rec, recon, g); break;
    case 6: hipLaunchKernelGGL((par_colback_kernel<6, POW>), grid, dim3(64), 0, st, sino, p.rec, recon, g); break;
    case 7: hipLaunchKernelGGL((par_colback_kernel<7, POW>), grid, dim3(64), 0, st, sino, p.rec, recon, g); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_par_back(const Plan &p, const float *sino, float *recon, int power, hipStream_t st) {
    if (p.colmode) return power == 2 ? par_colback_pow<2>(p, sino, recon, st) : par_colback_pow<1>(p, sino, recon, st);
    return power == 2 ? par_back_pow<2>(p, sino, recon, st) : par_back_pow<1>(p, sino, recon, st);
}

// The forward of a translation scan: column sums, then the channel gather.
static hipError_t par_colfwd(const Plan &p, const float *recon, float *sino, hipStream_t st) {
    const Geo &g = p.g;
    const int tot = g.nx * g.ns;
    hipLaunchKernelGGL(par_colsum_kernel, dim3((unsigned)((tot + 63) / 64)), dim3(256), 0, st, recon, p.col, g.ny, tot);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nblk = (g.nc + 63) / 64, nchk = (g.ns + 63) / 64;
    const dim3 grid((unsigned)((int64_t)g.nv * nblk * nchk));
    switch (p.ntap) {
    case 2: hipLaunchKernelGGL((par_colfwd_kernel<2, 1>), grid, dim3(64), 0, st, p.col, p.rec, sino, g, nblk, nchk); break;
    case 3: hipLaunchKernelGGL((par_colfwd_kernel<3, 1>), grid, dim3(64), 0, st, p.col, p.rec, sino, g, nblk, nchk); break;
    case 4: hipLaunchKernelGGL((par_colfwd_kernel<4, 1>), grid, dim3(64), 0, st, p.col, p.rec, sino, g, nblk, nchk); break;
    case 5: hipLaunchKernelGGL((par_colfwd_kernel<5, 1>), grid, dim3(64), 0, st, p.col, p.rec, sino, g, nblk, nchk); break;
    case 6: hipLaunchKernelGGL((par_colfwd_kernel<6, 1>), grid, dim3(64), 0, st, p.col, p.rec, sino, g, nblk, nchk); break;
    case 7: hipLaunchKernelGGL((par_colfwd_kernel<7, 1>), grid, dim3(64), 0, st, p.col, p.rec, sino, g, nblk, nchk); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int K>
static hipError_t par_gather_t(const Plan &p, const float *recon, hipStream_t st) {
    const Geo &g = p.g;
    const int nvb = (g.nv + 63) / 64;
    const int64_t blocks = (int64_t)nvb * p.gat_nseg * ((g.ns + 15) / 16);
    hipLaunchKernelGGL((par_gather_kernel<K>), dim3((unsigned)blocks), dim3(FRW * 64), 0, st, recon, p.facc, p.wrec, g,
                       p.fwd_cb, p.fwd_s16, p.gat_ng, p.gat_segg, p.gat_nseg);
    return hipGetLastError();
}

// Zero the accumulation buffer, walk, then unpack into the sinogram (which the
// unpack writes in full, so the sinogram needs no fill of its own).
hipError_t launch_par_forward(const Plan &p, const float *recon, float *sino, hipStream_t st) {
    const Geo &g = p.g;
    if (p.fwd_strategy == kForwardColumn) return par_colfwd(p, recon, sino, st);
    hipError_t e = launch_fill_zero(p.facc, (int64_t)g.nv * p.fwd_cb * p.fwd_s16, st);
    if (e != hipSuccess) return e;
    if (p.fwd_strategy == 2) {
        switch (p.ntap) {
        case 2: e = par_gather_t<2>(p, recon, st); break;
        case 3: e = par_gather_t<3>(p, recon, st); break;
        case 4: e = par_gather_t<4>(p, recon, st); break;
        case 5: e = par_gather_t<5>(p, recon, st); break;
        case 6: e = par_gather_t<6>(p, recon, st); break;
        case 7: e = par_gather_t<7>(p, recon, st); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (p.ntap) {
        case 2: e = par_fwd_t<2>(p, recon, st); break;
        case 3: e = par_fwd_t<3>(p, recon, st); break;
        case 4: e = par_fwd_t<4>(p, recon, st); break;
        case 5: e = par_fwd_t<5>(p, recon, st); break;
        case 6: e = par_fwd_t<6>(p, recon, st); break;
        case 7: e = par_fwd_t<7>(p, recon, st); break;
        default: return hipErrorInvalidValue;
        }
    }
    if (e != hipSuccess) return e;
    return launch_par_unpack(p, sino, st);
}

hipError_t launch_unpack_rows(const float *buf, float *sino, int nv, int nr, int nc, int cb, int s, int guard,
                              hipStream_t st) {
    const int tn = (nc + 63) / 64;
    if (nv == 0 || tn == 0 || nr == 0) return hipSuccess;
    hipLaunchKernelGGL(par_unpack_kernel, dim3((unsigned)(nv * tn), (nr + 63) / 64), dim3(256), 0, st, buf, sino, nr,
                       nc, cb, s, guard, tn);
    return hipGetLastError();
}

hipError_t launch_par_unpack(const Plan &p, float *sino, hipStream_t st) {
    return launch_unpack_rows(p.facc, sino, p.g.nv, p.g.nr, p.g.nc, p.fwd_cb, p.fwd_s16, p.ntap - 1, st);
}

// The region walk holds its voxels in more LDS than the default limit.
hipError_t par_forward_allow_lds(int ntap, int spl, size_t bytes) {
    const void *f = nullptr;
#define BPAMD_PF(KK)                                                                                          \
    case KK: f = spl == 2 ? (const void *)par_forward_kernel<KK, 2> : (const void *)par_forward_kernel<KK, 1>; break;
    switch (ntap) {
    BPAMD_PF(2) BPAMD_PF(3) BPAMD_PF(4) BPAMD_PF(5) BPAMD_PF(6) BPAMD_PF(7)
    default: return hipErrorInvalidValue;
    }
#undef BPAMD_PF
    return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace bpamd
