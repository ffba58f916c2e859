/*
 * Plain, slow, fp64 CPU reference of the matched voxel-driven projector pair.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no source with the HIP library.
 *
 * What it computes (readings of the MBIRJAX "Projector kernels" page unless
 * another page is named):
 *   - forward projection scatters each voxel's trapezoid detector taps into
 *     the channels it lands on; back projection gathers the same taps, so the
 *     two are an exact adjoint pair ("Forward scatters, back gathers"; "How the
 *     kernels work", closing remark on the matched pair);
 *   - the tap arithmetic is shared by all geometries and a geometry supplies
 *     only its coordinate math and weight scale, while the integer channel is
 *     a separate, exported step ("Shared machinery, and the rounding defense");
 *   - the taps form a partition of unity ("Gradient and Hessian can take
 *     different paths");
 *   - parallel beam: detector row r sees only slice r ("Geometry decides
 *     whether a slice can stream"; "Sharding Overview" page, "Why cone beam
 *     projects whole cylinders");
 *   - cone beam: a 3x3 tap block, and the detector row of a voxel is an exact
 *     affine function of its slice index ("The cone back kernel: a fused
 *     vertical fan");
 *   - CPU keeps the plain voxel-driven scatter loop ("Forward scatters, back
 *     gathers").
 * The footprint is an equal-area, equal-FWHM box of the pixel's shadow
 * convolved with the detector cell, in the spirit of the separable-footprint
 * projector of Long, Fessler and Balter (IEEE TMI 2010); the formulas below
 * are this file's own statement of that model.
 *
 * Arithmetic is IEEE fp64 with no contraction (build with -ffp-contract=off),
 * every product and sum rounded in the written order, so the channel index
 * rint(u) is reproducible bit for bit.  Loop orders are fixed, so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#pragma STDC FP_CONTRACT OFF

typedef struct {
    int32_t kind;            /* 0 parallel, 1 flat-detector cone (circular or helical) */
    int32_t nviews;          /* V */
    const double *angles;    /* [V] view angle theta_v, radians */
    const double *shift;     /* [V] lateral detector shift in channels, or NULL */
    const double *zsrc;      /* [V] source height in voxel units (cone), or NULL */
    double dv, dch, drow;    /* voxel, channel and row pitch */
    double sid, sdd;         /* source-iso and source-detector distance (cone) */
    double ch_off, row_off;  /* detector centre offsets, channels / rows */
    int32_t radius;          /* taps on each side of the centre channel (and row) */
    int32_t ny, nx, ns;      /* recon (Ny, Nx, S), slices fastest */
    int32_t nr, nc;          /* sinogram rows R and channels C, per view */
} orc_geom;

/* Per (view, pixel) quantities. */
typedef struct {
    double u;        /* continuous channel coordinate of the voxel centre */
    int32_t nc;      /* rint(u), ties to even */
    double w;        /* channel footprint width W (channel units) */
    double len;      /* in-plane chord scale L */
    /* cone only */
    double mr;       /* row magnification over row pitch */
    double rho;      /* in-plane source to voxel distance */
    double wrow;     /* row footprint width */
} orc_vp;

/* Overlap length of the unit cell centred at d with the centred interval
 * [-a/2, a/2].  As a function of d it is a trapezoid, and summed over all
 * integer shifts of d it equals a. */
static double ov(double d, double a)
{
    double hi = fmin(d + 0.5, a / 2.0);
    double lo = fmax(d - 0.5, -a / 2.0);
    double r = hi - lo;
    return r > 0.0 ? r : 0.0;
}

static double centre(int32_t n) { return ((double)n - 1.0) / 2.0; }

/* Pixel centre coordinates: x follows the column j, y the row i. */
static double pix_x(const orc_geom *g, int32_t j) { return ((double)j - centre(g->nx)) * g->dv; }
static double pix_y(const orc_geom *g, int32_t i) { return ((double)i - centre(g->ny)) * g->dv; }
static double slice_z(const orc_geom *g, int32_t k) { return ((double)k - centre(g->ns)) * g->dv; }

static void vp_geometry(const orc_geom *g, double c, double s, int32_t v, int32_t i, int32_t j, orc_vp *o)
{
    double x = pix_x(g, j), y = pix_y(g, i);
    double shift = g->shift ? g->shift[v] : 0.0;
    double cch = centre(g->nc) + g->ch_off;
    memset(o, 0, sizeof(*o));
    if (g->kind == 0) {
        /* parallel: detector coordinate t = x cos(theta) + y sin(theta) */
        double xc = x * c;
        double ys = y * s;
        double t = xc + ys;
        double tq = t / g->dch;
        double u = tq + cch;
        u = u + shift;
        double m = fmax(fabs(c), fabs(s));
        o->u = u;
        o->w = g->dv * m / g->dch;
        o->len = g->dv / m;
    } else {
        /* flat-detector cone: a along the detector, b towards the detector;
         * the source sits at b = -SID, the detector plane at b = SDD - SID. */
        double xc = x * c, ys = y * s, yc = y * c, xs = x * s;
        double a = xc + ys;
        double b = yc - xs;
        double d = g->sid + b;
        double dc = d * g->dch;
        double drw = d * g->drow;
        double mc = g->sdd / dc;
        double mr = g->sdd / drw;
        double ma = mc * a;
        double u = ma + cch;
        u = u + shift;
        double gam = atan2(a, d);
        double alpha = g->angles[v] - gam;     /* in-plane ray direction, parallel convention */
        double m = fmax(fabs(cos(alpha)), fabs(sin(alpha)));
        o->u = u;
        o->w = mc * g->dv * m / cos(gam);
        o->len = g->dv / m;
        o->mr = mr;
        o->rho = hypot(d, a);
        o->wrow = mr * g->dv;
    }
    o->nc = (int32_t)rint(o->u);
}

/* Cone per-slice row data: continuous row w_k, its rounded row m_c(k) and
 * the chord scale L_k including the vertical obliquity. */
static void cone_row(const orc_geom *g, const orc_vp *o, int32_t v, int32_t k,
                     double *wk, int32_t *mck, double *lk)
{
    double zs = g->zsrc ? g->zsrc[v] : 0.0;
    double dz = slice_z(g, k) - zs;
    double crow = centre(g->nr) + g->row_off;
    double t = o->mr * dz;
    *wk = t + crow;
    *mck = (int32_t)rint(*wk);
    double q = dz / o->rho;
    *lk = o->len * sqrt(1.0 + q * q);
}

/* The views' cos/sin, once per view, from the C library in fp64. */
static void view_trig(const orc_geom *g, int32_t v, double *c, double *s)
{
    *c = cos(g->angles[v]);
    *s = sin(g->angles[v]);
}

/* --------------------------------------------------------------------------
 * Exported entry points.
 * ------------------------------------------------------------------------ */

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* n_c[v, p] = rint(u(v, p)), p = i*Nx + j. */
void orc_channel_index(const orc_geom *g, int32_t *out)
{
    const int64_t np = (int64_t)g->ny * g->nx;
#pragma omp parallel for schedule(static)
    for (int32_t v = 0; v < g->nviews; ++v) {
        double c, s;
        view_trig(g, v, &c, &s);
        for (int32_t i = 0; i < g->ny; ++i)
            for (int32_t j = 0; j < g->nx; ++j) {
                orc_vp o;
                vp_geometry(g, c, s, v, i, j, &o);
                out[(int64_t)v * np + (int64_t)i * g->nx + j] = o.nc;
            }
    }
}

/* Continuous channel coordinates u[v, p] (fp64), for tests of the model. */
void orc_channel_coord(const orc_geom *g, double *out)
{
    const int64_t np = (int64_t)g->ny * g->nx;
    for (int32_t v = 0; v < g->nviews; ++v) {
        double c, s;
        view_trig(g, v, &c, &s);
        for (int32_t i = 0; i < g->ny; ++i)
            for (int32_t j = 0; j < g->nx; ++j) {
                orc_vp o;
                vp_geometry(g, c, s, v, i, j, &o);
                out[(int64_t)v * np + (int64_t)i * g->nx + j] = o.u;
            }
    }
}

/* Forward projection of one view into yv[R, C] (overwritten), with the
 * absolute sums av[R, C] = sum |w * x| when av is not NULL.  Loop order: pixels
 * ascending, then slices, then row taps, then channel taps. */
static void forward_view(const orc_geom *g, const float *x, const double *xd, int32_t v, double *yv, double *av)
{
    const int64_t nrc = (int64_t)g->nr * g->nc;
    const int r = g->radius;
    double c, s;
    memset(yv, 0, sizeof(double) * nrc);
    if (av) memset(av, 0, sizeof(double) * nrc);
    view_trig(g, v, &c, &s);
    for (int32_t i = 0; i < g->ny; ++i)
        for (int32_t j = 0; j < g->nx; ++j) {
            orc_vp o;
            vp_geometry(g, c, s, v, i, j, &o);
            const int64_t xo = ((int64_t)i * g->nx + j) * g->ns;
            for (int32_t k = 0; k < g->ns; ++k) {
                double val = xd ? xd[xo + k] : (double)x[xo + k];
                if (g->kind == 0) {
                    for (int tau = -r; tau <= r; ++tau) {
                        int32_t n = o.nc + tau;
                        if (n < 0 || n >= g->nc) continue;
                        double w = o.len * ov((double)n - o.u, o.w);
                        int64_t at = (int64_t)k * g->nc + n;
                        yv[at] += w * val;
                        if (av) av[at] += fabs(w * val);
                    }
                } else {
                    double wk, lk;
                    int32_t mck;
                    cone_row(g, &o, v, k, &wk, &mck, &lk);
                    for (int sg = -r; sg <= r; ++sg) {
                        int32_t m = mck + sg;
                        if (m < 0 || m >= g->nr) continue;
                        double gw = ov((double)m - wk, o.wrow);
                        for (int tau = -r; tau <= r; ++tau) {
                            int32_t n = o.nc + tau;
                            if (n < 0 || n >= g->nc) continue;
                            double h = ov((double)n - o.u, o.w);
                            double w = lk * h * gw;
                            int64_t at = (int64_t)m * g->nc + n;
                            yv[at] += w * val;
                            if (av) av[at] += fabs(w * val);
                        }
                    }
                }
            }
        }
}

/* Back projection into one pixel's cylinder xp[S] (overwritten); views
 * ascending, then slices, then row taps, then channel taps.  With power 2
 * every tap weight is squared: the back projection the Hessian diagonal of a
 * least-squares fit uses ("Gradient and Hessian can take different paths",
 * coefficient power 2). */
static void back_pixel(const orc_geom *g, const float *y, const double *yd, int power, int32_t i, int32_t j,
                       double *xp, double *ap)
{
    const int64_t nrc = (int64_t)g->nr * g->nc;
    const int r = g->radius;
    memset(xp, 0, sizeof(double) * g->ns);
    if (ap) memset(ap, 0, sizeof(double) * g->ns);
    for (int32_t v = 0; v < g->nviews; ++v) {
        double c, s;
        orc_vp o;
        view_trig(g, v, &c, &s);
        vp_geometry(g, c, s, v, i, j, &o);
        const int64_t yo = (int64_t)v * nrc;
        for (int32_t k = 0; k < g->ns; ++k) {
            if (g->kind == 0) {
                for (int tau = -r; tau <= r; ++tau) {
                    int32_t n = o.nc + tau;
                    if (n < 0 || n >= g->nc) continue;
                    double w = o.len * ov((double)n - o.u, o.w);
                    if (power == 2) w = w * w;
                    const int64_t at = yo + (int64_t)k * g->nc + n;
                    double t = w * (yd ? yd[at] : (double)y[at]);
                    xp[k] += t;
                    if (ap) ap[k] += fabs(t);
                }
            } else {
                double wk, lk;
                int32_t mck;
                cone_row(g, &o, v, k, &wk, &mck, &lk);
                for (int sg = -r; sg <= r; ++sg) {
                    int32_t m = mck + sg;
                    if (m < 0 || m >= g->nr) continue;
                    double gw = ov((double)m - wk, o.wrow);
                    for (int tau = -r; tau <= r; ++tau) {
                        int32_t n = o.nc + tau;
                        if (n < 0 || n >= g->nc) continue;
                        double h = ov((double)n - o.u, o.w);
                        double w = lk * h * gw;
                        if (power == 2) w = w * w;
                        const int64_t at = yo + (int64_t)m * g->nc + n;
                        double t = w * (yd ? yd[at] : (double)y[at]);
                        xp[k] += t;
                        if (ap) ap[k] += fabs(t);
                    }
                }
            }
        }
    }
}

/* Full forward: y[V, R, C] (fp64, overwritten); threads split views. */
void orc_forward(const orc_geom *g, const float *x, double *y, double *ay)
{
    const int64_t nrc = (int64_t)g->nr * g->nc;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t v = 0; v < g->nviews; ++v)
        forward_view(g, x, NULL, v, y + v * nrc, ay ? ay + v * nrc : NULL);
}

/* Forward of selected views only: y[nsel, R, C]. */
void orc_forward_views(const orc_geom *g, const float *x, int32_t nsel, const int32_t *views,
                       double *y, double *ay)
{
    const int64_t nrc = (int64_t)g->nr * g->nc;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t q = 0; q < nsel; ++q)
        forward_view(g, x, NULL, views[q], y + q * nrc, ay ? ay + q * nrc : NULL);
}

/* Full back projection: x[Ny, Nx, S] (fp64, overwritten); threads split
 * pixels.  power is 1 (the adjoint) or 2 (every weight squared). */
void orc_back_power(const orc_geom *g, const float *y, int power, double *x, double *ax)
{
    const int64_t np = (int64_t)g->ny * g->nx;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < np; ++p) {
        int32_t i = (int32_t)(p / g->nx), j = (int32_t)(p % g->nx);
        back_pixel(g, y, NULL, power, i, j, x + p * g->ns, ax ? ax + p * g->ns : NULL);
    }
}

void orc_back(const orc_geom *g, const float *y, double *x, double *ax) { orc_back_power(g, y, 1, x, ax); }

/* The same forward and back with fp64 inputs, for iterates that are not fp32
 * data (the reference solvers): the arithmetic is the one above, only the
 * input is read without a rounding to fp32. */
void orc_forward_f64(const orc_geom *g, const double *x, double *y)
{
    const int64_t nrc = (int64_t)g->nr * g->nc;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t v = 0; v < g->nviews; ++v) forward_view(g, NULL, x, v, y + v * nrc, NULL);
}

void orc_back_f64(const orc_geom *g, const double *y, double *x)
{
    const int64_t np = (int64_t)g->ny * g->nx;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < np; ++p) {
        int32_t i = (int32_t)(p / g->nx), j = (int32_t)(p % g->nx);
        back_pixel(g, NULL, y, 1, i, j, x + p * g->ns, NULL);
    }
}

/* Back projection of selected pixels only: x[nsel, S]. */
void orc_back_pixels_power(const orc_geom *g, const float *y, int power, int32_t nsel, const int64_t *pix,
                           double *x, double *ax)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t q = 0; q < nsel; ++q) {
        int64_t p = pix[q];
        int32_t i = (int32_t)(p / g->nx), j = (int32_t)(p % g->nx);
        back_pixel(g, y, NULL, power, i, j, x + (int64_t)q * g->ns, ax ? ax + (int64_t)q * g->ns : NULL);
    }
}

void orc_back_pixels(const orc_geom *g, const float *y, int32_t nsel, const int64_t *pix, double *x, double *ax)
{
    orc_back_pixels_power(g, y, 1, nsel, pix, x, ax);
}

/* Every nonzero tap of one voxel (v, i, j, k): channel, row and weight.
 * Returns the number written (at most (2r+1)^2), for tests of the footprint. */
int orc_voxel_taps(const orc_geom *g, int32_t v, int32_t i, int32_t j, int32_t k,
                   int32_t *rows, int32_t *chans, double *w, int cap)
{
    const int r = g->radius;
    double c, s;
    orc_vp o;
    int cnt = 0;
    view_trig(g, v, &c, &s);
    vp_geometry(g, c, s, v, i, j, &o);
    if (g->kind == 0) {
        for (int tau = -r; tau <= r; ++tau) {
            int32_t n = o.nc + tau;
            if (n < 0 || n >= g->nc) continue;
            double wt = o.len * ov((double)n - o.u, o.w);
            if (wt == 0.0 || cnt >= cap) continue;
            rows[cnt] = k; chans[cnt] = n; w[cnt] = wt; ++cnt;
        }
    } else {
        double wk, lk;
        int32_t mck;
        cone_row(g, &o, v, k, &wk, &mck, &lk);
        for (int sg = -r; sg <= r; ++sg) {
            int32_t m = mck + sg;
            if (m < 0 || m >= g->nr) continue;
            double gw = ov((double)m - wk, o.wrow);
            for (int tau = -r; tau <= r; ++tau) {
                int32_t n = o.nc + tau;
                if (n < 0 || n >= g->nc) continue;
                double h = ov((double)n - o.u, o.w);
                double wt = lk * h * gw;
                if (wt == 0.0 || cnt >= cap) continue;
                rows[cnt] = m; chans[cnt] = n; w[cnt] = wt; ++cnt;
            }
        }
    }
    return cnt;
}

/* The per-(view, pixel) footprint parameters, for tests:
 * out = {u, nc, W, L, Mr, rho, Wrow}. */
void orc_vp_params(const orc_geom *g, int32_t v, int32_t i, int32_t j, double *out)
{
    double c, s;
    orc_vp o;
    view_trig(g, v, &c, &s);
    vp_geometry(g, c, s, v, i, j, &o);
    out[0] = o.u; out[1] = (double)o.nc; out[2] = o.w; out[3] = o.len;
    out[4] = o.mr; out[5] = o.rho; out[6] = o.wrow;
}

/* Overlap helper exported for the quadrature test. */
double orc_ov(double d, double a) { return ov(d, a); }
