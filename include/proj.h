/*
 * proj.h -- C ABI of the matched voxel-driven projector pair for MI355X (gfx950).
 *
 * The operator pair (MBIRJAX "Projector kernels" page):
 *   - the forward projector maps a voxel-cylinder volume to a sinogram: every
 *     voxel is mapped to a detector channel and its trapezoid footprint taps
 *     are added into that channel and its neighbours (section "The XLA
 *     kernels", paragraph "Forward scatters, back gathers");
 *   - the back projector is its exact adjoint and gathers the same taps from
 *     the sinogram into the voxels (same paragraph; "How the kernels work",
 *     closing remark that both directions take their weights from the same
 *     geometry code, so they stay a matched pair);
 *   - the integer channel of every (view, pixel) is computed by a separate
 *     step and handed to the projectors as data, so no projector rounds a
 *     coordinate to a channel itself (paragraph "Shared machinery, and the
 *     rounding defense");
 *   - parallel beam: detector row r sees only slice r (paragraph "Geometry
 *     decides whether a slice can stream"); cone beam with a flat detector:
 *     one slice spreads over a band of rows given by an affine function of
 *     the slice index, with a 3x3 tap block ("The cone back kernel: a fused
 *     vertical fan").
 * The footprint model, per (view, pixel): channel coordinate u (parallel:
 * (x cos t + y sin t)/dch + centre + shift; flat cone: SDD a/(d dch) + centre +
 * shift), n_c = rint(u), and tap n in [n_c - r, n_c + r] weighted by
 * L * |[n - 1/2, n + 1/2] ∩ [u - W/2, u + W/2]| with W = dv max(|cos|,|sin|)/dch
 * and L = dv / max(|cos|,|sin|) (the cone adds the fan obliquity and a row
 * factor of the same form); the fp64 CPU reference under oracle/ writes it out.
 *
 * Layouts (all C order, float32, device memory, caller-owned):
 *   recon  [Ny][Nx][S]  slices fastest: one contiguous voxel cylinder per
 *                       pixel p = i*Nx + j (MBIRJAX "Sharding overview" page,
 *                       section "The two shardings");
 *   sino   [V][R][C]    channels fastest, one [R][C] block per view;
 *   index  [V][Ny*Nx]   int32 channel index n_c = rint(u) of every view and
 *                       pixel (round half to even).
 *
 * Threading / streams: calls are asynchronous on the HIP stream passed in
 * (NULL = the default stream).  They allocate nothing, copy nothing between
 * host and device and never synchronise.  A handle is immutable after
 * proj_create; concurrent calls on different streams are allowed when their
 * output buffers are distinct.
 *
 * Errors: every check runs before anything is written or launched, so an
 * error return leaves all outputs untouched.  No C++ exception crosses this
 * boundary.  proj_last_error() gives a human-readable reason for the last
 * failure on the calling thread.
 */
#ifndef BPAMD_PROJ_H
#define BPAMD_PROJ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct proj_handle_s *proj_handle; /* opaque; owned by the library */

typedef enum {
    PROJ_OK = 0,
    PROJ_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad shape, non-finite or inconsistent geometry */
    PROJ_ERR_UNSUPPORTED = -2,      /* valid request the kernels cannot serve (size limits) */
    PROJ_ERR_ALIAS = -3,            /* input and output buffers overlap */
    PROJ_ERR_OUT_OF_MEMORY = -4,    /* device allocation failed in proj_create */
    PROJ_ERR_DEVICE = -5            /* a HIP call or kernel launch failed */
} proj_status;

typedef enum {
    PROJ_PARALLEL = 0,  /* parallel beam; row r of the detector sees slice r only */
    PROJ_CONE_FLAT = 1  /* point source, flat detector; circular or helical orbit */
} proj_kind;

/*
 * Acquisition geometry.  Lengths are in the same unit as delta_voxel.
 * Pixel (i, j) of slice k has its centre at
 *     x = (j - (Nx-1)/2) dv,  y = (i - (Ny-1)/2) dv,  z = (k - (S-1)/2) dv.
 * View v looks along angle theta_v: a parallel ray hits detector coordinate
 * t = x cos(theta) + y sin(theta); for cone beam the source sits at distance
 * source_iso on the far side, at height source_z[v], and the flat detector is
 * source_detector away from the source, perpendicular to the central ray.
 * Channel n (row m) has its centre at n = (C-1)/2 + det_channel_offset + t/dch
 * (m = (R-1)/2 + det_row_offset + ...).  The arrays are copied by proj_create.
 */
typedef struct {
    int32_t kind;                /* proj_kind */
    int32_t num_views;           /* V; must equal sino_shape[0] */
    const double *angles;        /* [V] radians; required when V > 0 */
    const double *channel_shift; /* [V] lateral detector shift in channels, or NULL (all 0) */
    const double *source_z;      /* [V] source height (cone only; helical orbits), or NULL */
    double delta_voxel;          /* dv > 0 */
    double delta_channel;        /* dch > 0 */
    double delta_row;            /* drow > 0; parallel beam requires drow == dv */
    double source_iso;           /* cone: source to rotation axis, > in-plane radius of the volume */
    double source_detector;      /* cone: source to detector plane, > source_iso */
    double det_channel_offset;   /* detector centre offset, channels (usually 0) */
    double det_row_offset;       /* detector centre offset, rows (usually 0) */
    int32_t psf_radius;          /* taps on each side of the centre channel (and row), 1..4 */
    int32_t forward_strategy;    /* PROJ_FORWARD_AUTO (0): chosen from the shapes; parallel beam:
                                    PROJ_FORWARD_TILE (1), PROJ_FORWARD_GATHER (2) or
                                    PROJ_FORWARD_COLUMN (5); cone beam:
                                    PROJ_FORWARD_CONE_TILE_8X4 (3) or _8X8 (4) */
} proj_geometry;

/*
 * Parallel-beam forward strategies (MBIRJAX "Projector kernels" page,
 * "Forward scatters, back gathers": a per-voxel scatter, or a reduction over
 * voxels sorted by channel).  Both walk voxels in the order of their first tap
 * channel, so every channel is finished in registers before it is added out:
 *   TILE   -- a region of pixels is held on chip and walked for every view;
 *             each finished channel is added once per (view, region).
 *   GATHER -- per view every pixel, sorted by channel at creation; walks read
 *             the voxels from memory, each channel is added about once per view.
 *   COLUMN -- only where every view angle has a sine of exactly 0 (a
 *             translation scan at angle 0): a pixel's channel coordinate then
 *             does not depend on its row, so each column of the volume is
 *             summed over its rows once and each view adds the column sums
 *             through the columns' taps.  (The back projection of such a scan
 *             likewise computes one value per column and slice and writes it
 *             to every row, whatever the forward strategy; it gives the same
 *             bits as the general back projection.)
 * AUTO takes the choice from the shapes alone (COLUMN wherever it applies);
 * all give the same sinogram up to the order of fp32 additions.
 * Cone-beam forward tiles: a workgroup holds 8 x 4 or 8 x 8 pixels and adds
 * a detector window per view to the sinogram with one global atomic per
 * cell; larger tiles flush fewer cells per voxel, smaller ones skip more
 * slices that miss the detector.  AUTO estimates both from the windows and
 * takes the faster; CONE_TILE_8X4 / _8X8 force one.  The sinogram is the
 * same up to the order of fp32 additions.
 */
enum {
    PROJ_FORWARD_AUTO = 0,
    PROJ_FORWARD_TILE = 1,
    PROJ_FORWARD_GATHER = 2,
    PROJ_FORWARD_CONE_TILE_8X4 = 3,
    PROJ_FORWARD_CONE_TILE_8X8 = 4,
    PROJ_FORWARD_COLUMN = 5
};

/*
 * proj_create: validate the geometry, copy it to the device, run the fp64
 * channel-index pass and fix the launch plan from the shapes alone.
 *   g            geometry (read only, copied)
 *   recon_shape  {Ny, Nx, S}, each >= 0
 *   sino_shape   {V, R, C}, each >= 0; parallel beam requires R == S
 *   hip_device   HIP device ordinal the handle lives on
 *   out          receives the handle (NULL on error)
 * Limits: V*Ny*Nx, Ny*Nx*S and V*R*C below 2^31 elements.  Geometries the
 * kernels cannot hold return PROJ_ERR_UNSUPPORTED, the reason in
 * proj_last_error(): more than 7 channel taps per voxel, a detector window
 * too large for the on-chip staging (channels or rows far finer than the
 * voxels), or, for the cone, a row magnification below 1/3 anywhere in the
 * scan (rows more than three voxel pitches apart, so that three slices can
 * share a row).
 * Synchronises the device once (creation is not on the hot path).
 */
proj_status proj_create(const proj_geometry *g, const int64_t recon_shape[3],
                        const int64_t sino_shape[3], int hip_device, proj_handle *out);

/*
 * proj_forward: sino = A recon.  recon_dev [Ny][Nx][S] is read, sino_dev
 * [V][R][C] is overwritten (entries no tap reaches become exactly 0).
 * The two buffers must not overlap.  Asynchronous on hip_stream.
 *
 * Graph capture: proj_forward, proj_back, proj_back_squared,
 * proj_forward_pixels and proj_back_pixels allocate, copy and synchronise
 * nothing and use no memset, so they can be captured into a HIP graph.  Outside
 * a capture, forwards on one handle (proj_forward and proj_forward_pixels,
 * both geometries) and batch back projections large enough to pack the
 * sinogram (proj_back_pixels) are ordered on the GPU (they share the handle's
 * accumulation, sort or transposed-sinogram buffer); inside a capture that
 * ordering is the graph's.  So two such captured calls on one handle must not run
 * concurrently, and a replayed graph holding one must be ordered by the caller
 * against every other such call of the same handle on another stream (an
 * event after the replay, a stream wait before the next one).  The solvers
 * (proj_cgls, proj_sirt) synchronise and cannot be captured.
 */
proj_status proj_forward(proj_handle h, const float *recon_dev, float *sino_dev, void *hip_stream);

/*
 * proj_forward_noalloc: proj_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops, harnesses that forbid
 * allocation).  Same operation, layouts, overlap rule and errors as
 * proj_forward, and the same kernels; it allocates nothing.  Parallel beam
 * adds its partial sums into a fixed device array of the library, at most
 * 144 MiB (one copy per GPU, held until the process ends), instead of the
 * handle's accumulation buffer; the buffer needs V * (C + 2 (taps - 1)) *
 * (S rounded up to 16 or 32) * 4 bytes (142 MB for 512x512x64 at 720 views),
 * and a handle that needs more returns PROJ_ERR_UNSUPPORTED before any
 * write.  Cone beam needs no scratch: its kernels add straight into sino_dev
 * (one 64-byte request per detector row of a window column, where
 * proj_forward adds into the handle's transposed sinogram, whole lines at a
 * time, and unpacks it), so the cone forward runs slower here.
 * Every call on one GPU shares that array: two calls that can overlap in time
 * on one GPU (other streams, a replayed graph beside an eager call, any
 * handles) race and must be ordered by the caller.  Calls of proj_forward on
 * the same handle do not touch the array.  The first call on each GPU looks
 * up the array's device address; make it outside a graph capture.
 * Asynchronous on hip_stream.
 */
proj_status proj_forward_noalloc(proj_handle h, const float *recon_dev, float *sino_dev, void *hip_stream);

/*
 * proj_back: recon = A^T sino, the exact adjoint of proj_forward.  sino_dev is
 * read, recon_dev is overwritten.  The two buffers must not overlap.
 * Asynchronous on hip_stream.
 */
proj_status proj_back(proj_handle h, const float *sino_dev, float *recon_dev, void *hip_stream);

/*
 * proj_back_squared: recon[p][k] = sum over views and taps of w^2 *
 * sino[v][row][n] -- the back projection with every tap weight squared, the
 * one the diagonal of A^T A (a least-squares Hessian) needs.  The MBIRJAX
 * "Projector kernels" page, "Gradient and Hessian can take different paths",
 * calls the same kernels with the weights unchanged for the gradient and with
 * coefficient power 2 for the Hessian diagonal.  Layouts, ownership, overlap
 * rule and errors as proj_back; with sino = 1 everywhere it writes
 * sum_i A_ij^2.  Asynchronous on hip_stream.
 */
proj_status proj_back_squared(proj_handle h, const float *sino_dev, float *recon_dev, void *hip_stream);

/*
 * Projection of a batch of voxel cylinders (a cylinder is the S voxels of one
 * recon pixel, all slices).  The MBIRJAX "Sharding Overview" page, section
 * "Why cone beam projects whole cylinders", has the owner of a group of views
 * collect the full cylinders of a batch of pixels and project them; the same
 * page asks that the zeros that pad a batch to a fixed size stay exactly
 * inert.
 *
 *   pixels_dev   device int32 [n]: flat recon pixel ids p = i*Nx + j.  An id
 *                outside [0, Ny*Nx) marks a padding entry.  Ids may repeat.
 *   n            batch size, n >= 0, n*S below 2^31.
 *   cyl_dev      device float [n][S], slices fastest: entry i is the cylinder
 *                of pixel pixels_dev[i].
 *   sino_dev     device float [V][R][C].
 *
 * proj_forward_pixels: sino = A x, where x is zero except that pixel
 * pixels_dev[i] holds cylinder i (a repeated id adds its cylinders).  A
 * padding entry adds nothing whatever its cylinder holds (NaN included).  sino
 * is overwritten.
 *
 * proj_back_pixels: cylinder i = row pixels_dev[i] of A^T sino (the pixel's
 * column of proj_back's output); a padding entry's cylinder is written as
 * zeros.
 *
 * Both are exact adjoints of each other on the listed pixels.  No buffer may
 * overlap another.  Asynchronous on hip_stream.  These serve batches: their
 * cost grows with n*S*V, not with the volume, plus one pass over the sinogram
 * (the forward writes all of it; a back of a large batch first packs it into
 * a layout with its columns contiguous).  A cone-beam handle keeps a
 * transposed copy of the sinogram's size for this.  A parallel forward sorts each view's entries by channel
 * in passes of up to 4096 entries and writes every sinogram cell from one
 * wave, without atomics; the entries of one channel are summed in the order
 * the sort placed them, which may differ between calls (results then differ
 * by rounding only).
 */
proj_status proj_forward_pixels(proj_handle h, const int32_t *pixels_dev, int64_t n, const float *cyl_dev,
                                float *sino_dev, void *hip_stream);
proj_status proj_back_pixels(proj_handle h, const float *sino_dev, const int32_t *pixels_dev, int64_t n,
                             float *cyl_dev, void *hip_stream);

/*
 * Iterative reconstruction around the pair: CGLS and SIRT.  What they return
 * and when they stop follows the diffct page "Precision, training and
 * reconstruction", section "Numerical solver API":
 *   - stop when ||y - A x|| <= atol + rtol ||y||, tested on the initial
 *     iterate too (then no iteration runs);
 *   - the residual history holds ||y - A x0|| and then one value per
 *     completed iteration;
 *   - SIRT has a relaxation factor and a nonnegativity switch, and feeds the
 *     last residual into the next update (one forward and one back projection
 *     per iteration);
 *   - CGLS reads its two norms of an iteration (the residual and A^T of it)
 *     together.
 * The iterations themselves are the textbook ones, in fp32 vectors with fp64
 * norms:
 *   CGLS (Bjorck's least-squares arrangement of conjugate gradients):
 *     r = y - A x, s = A^T r, p = s, gamma = ||s||^2; per iteration
 *     q = A p, alpha = gamma/||q||^2, x += alpha p, r -= alpha q,
 *     s = A^T r, p = s + (||s||^2/gamma) p;
 *   SIRT: x += relaxation * C A^T R (y - A x), R = 1/(row sums of A),
 *     C = 1/(column sums of A), 0 where a sum is 0, then x = max(x, 0) when
 *     nonnegative.  R and C are computed at the start of each call (one
 *     forward and one back projection of ones).
 *
 *   sino_dev      device float [V][R][C], the data y (read only).
 *   x0_dev        device float [Ny][Nx][S] initial iterate, or NULL for 0;
 *                 it may be recon_dev itself (a warm start in place), else it
 *                 must not overlap any other buffer and is left unchanged.
 *   recon_dev     device float [Ny][Nx][S], receives the last iterate.
 *   work_dev      device workspace, 256-byte aligned, at least
 *                 proj_solver_workspace_size() bytes (two sinogram-sized and
 *                 two volume-sized fp32 vectors and a few KiB of fp64
 *                 scalars); its contents on entry do not matter.
 *   iterations    most iterations to run, >= 0.
 *   atol, rtol    finite, >= 0.
 *   relaxation    SIRT only: finite, > 0 (1 is the usual choice).
 *   residual_history  host double [iterations + 1] or NULL; entries past
 *                 info->iterations + 1 are not written.
 *   info          host, receives iterations, converged and the stop reason.
 * The calls block: they synchronise hip_stream once per iteration to read
 * the residual norm, and return with the last iterate written.  They allocate
 * nothing.  No buffer may overlap another (except x0_dev == recon_dev).
 */
typedef enum {
    PROJ_STOP_CONVERGED = 0,   /* the stop rule held */
    PROJ_STOP_ITERATIONS = 1,  /* the iteration limit was reached */
    PROJ_STOP_STATIONARY = 2,  /* CGLS: A^T r is exactly 0 (the least-squares equations hold) */
    PROJ_STOP_BREAKDOWN = 3    /* CGLS: A p is exactly 0 */
} proj_stop_reason;

typedef struct {
    int32_t iterations;  /* completed iterations */
    int32_t converged;   /* 1 when the stop rule held */
    int32_t reason;      /* proj_stop_reason */
    int32_t reserved;
} proj_solver_info;

proj_status proj_solver_workspace_size(proj_handle h, int64_t *bytes);
proj_status proj_cgls(proj_handle h, const float *sino_dev, const float *x0_dev, float *recon_dev,
                      void *work_dev, int64_t work_bytes, int32_t iterations, double atol, double rtol,
                      double *residual_history, proj_solver_info *info, void *hip_stream);
proj_status proj_sirt(proj_handle h, const float *sino_dev, const float *x0_dev, float *recon_dev,
                      void *work_dev, int64_t work_bytes, int32_t iterations, double atol, double rtol,
                      double relaxation, int32_t nonnegative, double *residual_history, proj_solver_info *info,
                      void *hip_stream);

/*
 * proj_channel_index: copy the handle's channel-index table n_c[V][Ny*Nx]
 * (int32, round half to even of the fp64 channel coordinate) into index_dev.
 * Asynchronous on hip_stream.
 */
proj_status proj_channel_index(proj_handle h, int32_t *index_dev, void *hip_stream);

/*
 * proj_plan_query: run every check of proj_create and choose the launch plan
 * without touching any GPU; write the plan's one-line description into buf
 * (at most len bytes, may be NULL).  Returns what proj_create would return
 * for the same arguments before it allocates.
 */
proj_status proj_plan_query(const proj_geometry *g, const int64_t recon_shape[3],
                            const int64_t sino_shape[3], char *buf, int len);

/* proj_destroy: free the handle's device tables.  NULL is ignored. */
void proj_destroy(proj_handle h);

/* proj_status_string: static name of a status code. */
const char *proj_status_string(proj_status s);

/* proj_last_error: reason for the last failed call on this thread ("" if none). */
const char *proj_last_error(void);

/*
 * proj_describe: write a one-line, NUL-terminated description of the launch
 * plan (kernels, tile sizes, table bytes) into buf (at most len bytes).
 * Returns the length it needed.
 */
int proj_describe(proj_handle h, char *buf, int len);

#ifdef __cplusplus
}
#endif

#endif /* BPAMD_PROJ_H */
