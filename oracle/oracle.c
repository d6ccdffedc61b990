/*
 * oracle.c -- plain, slow CPU oracle for tile-based 2D-Gaussian rasterization.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library: every quantity here is written out from its definition.
 *
 * What it computes (sources are the pages' text, cited by page title and
 * section; the pages print no formulas, so each definition below is the
 * plainest reading that their text supports):
 *
 *  - "GaussianImage" (Overview): an image is a set of 2D Gaussians with 8
 *    parameters each (position, covariance, colour) and it is rendered by
 *    accumulated summation.  Here params[n] = (mux, muy, l11, l21, l22,
 *    cr, cg, cb) with the covariance Sigma = L L^T, L = [[l11,0],[l21,l22]]
 *    (the Cholesky form of the "gaussianimage_cholesky" scripts), and
 *      I_k(p) = sum_n c_{n,k} exp(-q_n(p)/2),  q = d^T Sigma^-1 d, d = p - mu,
 *    over the Gaussians whose 3-sigma cutoff admits pixel p.  Pixel (row i,
 *    col j) samples the point (j+0.5, i+0.5).
 *  - "Drawing with Gaussians" (Overview, 2D fitting): the variant in which the
 *    Gaussians are alpha-composited over a trainable background:
 *      alpha_n = o_n w_n, C = sum_n c_n alpha_n T_n + T_final bg,
 *      T_1 = 1, T_{n+1} = T_n (1 - alpha_n), in Gaussian index order, stopping
 *    after the first Gaussian that drives T below 1e-4.
 *    o_n = sigmoid(min(lambda_n, ln 999)).
 *  - "FlashImgs" (Commands, train --loss l2): the L2 (mean squared error)
 *    fitting loss, and the Adam optimiser named by the fvdb page
 *    (GaussianSplatOptimizer) with textbook defaults.
 *  - fvdb page (GaussianSplatReconstructionConfig, tile_size): 16x16 tiles;
 *    (eps_2d): a small pixel pad on the screen-space bounding box.
 *
 * The cutoff decision is made in fp32 (the kernel's precision) by the exact
 * operation sequence stated in cutoff_setup()/cutoff_in(); every value
 * (weights, images, gradients) is computed in fp64 from the definitions
 * above, using the 2x2 adjugate for Sigma^-1 and matrix calculus for the
 * derivatives.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_TILE 16
#define LOG2E_D 1.44269504088896340736

/* ------------------------------------------------------------------------ */
/* fp32 cutoff decision (the one place where floating point decides an      */
/* integer: whether a pair is summed, and which tiles a Gaussian lands in). */
/* ------------------------------------------------------------------------ */

typedef struct {
    int ok;            /* 0: culled (non-finite or singular), contributes nothing */
    float mx, my;      /* mean, fp32 */
    float a, b, c;     /* rows of L^-1 scaled by sqrt(log2(e)/2): e = (a dx)^2 + (b dx + c dy)^2 */
    int j0, j1, i0, i1;/* inclusive pixel box of the 3-sigma cutoff (j: column, i: row); empty if j0 > j1 */
} cutoff32;

/* fp32 constants, each the fp32 value nearest its definition. */
static float c_scale(void) { return (float)sqrt(0.5 * LOG2E_D); }  /* sqrt(log2(e)/2) */
static float c_e9(void)    { return (float)(4.5 * LOG2E_D); }      /* 9 * log2(e)/2   */
static float c_lmax(void)  { return (float)log(999.0); }           /* logit(0.999)    */

static cutoff32 cutoff_setup(const double *pd, const double *logit, int W, int H)
{
    cutoff32 s;
    memset(&s, 0, sizeof s);
    float p[8];
    for (int k = 0; k < 8; ++k) {
        p[k] = (float)pd[k];
        if (!isfinite(p[k])) return s;
    }
    if (logit && !isfinite((float)*logit)) return s;
    const float l11 = p[2], l21 = p[3], l22 = p[4];
    if (l11 == 0.0f || l22 == 0.0f) return s;
    float i11 = 1.0f / l11;      /* built with -ffp-contract=off: each fp32 rounding as written */
    float i22 = 1.0f / l22;
    float t = l21 * i11;
    float k = -(t * i22);
    if (!isfinite(i11) || !isfinite(i22) || !isfinite(k)) return s;
    const float S = c_scale();
    float a = i11 * S, b = k * S, c = i22 * S;
    s.a = a; s.b = b; s.c = c;
    s.mx = p[0]; s.my = p[1];
    /* 3-sigma half-extents of the ellipse q <= 9 plus a 1/256 px pad */
    float sx = 3.0f * fabsf(l11);
    float rx = sx + 0.00390625f;
    float l22sq = l22 * l22;
    float syy = fmaf(l21, l21, l22sq);
    float sy = 3.0f * sqrtf(syy);
    float ry = sy + 0.00390625f;
    float cx = s.mx - 0.5f, cy = s.my - 0.5f;
    float fj0 = ceilf(cx - rx), fj1 = floorf(cx + rx);
    float fi0 = ceilf(cy - ry), fi1 = floorf(cy + ry);
    fj0 = fmaxf(fj0, 0.0f); fi0 = fmaxf(fi0, 0.0f);
    fj1 = fminf(fj1, (float)(W - 1)); fi1 = fminf(fi1, (float)(H - 1));
    s.ok = 1;
    if (!(fj0 <= fj1) || !(fi0 <= fi1)) { s.j0 = 1; s.j1 = 0; s.i0 = 1; s.i1 = 0; return s; }
    s.j0 = (int)fj0; s.j1 = (int)fj1; s.i0 = (int)fi0; s.i1 = (int)fi1;
    return s;
}

/* The fp32 decision for pixel (i, j): returns 1 iff the pair is summed. */
static int cutoff_in(const cutoff32 *s, int i, int j)
{
    if (!s->ok) return 0;
    float px = (float)j + 0.5f, py = (float)i + 0.5f;
    float dx = px - s->mx, dy = py - s->my;
    float u = s->a * dx;
    float t = s->b * dx;
    float v = fmaf(s->c, dy, t);
    float uu = u * u;
    float e = fmaf(v, v, uu);
    return e <= c_e9();
}

/* Exposed for the pins: the fp32 exponent e at pixel (i, j) and the setup. */
float oracle_cutoff_exponent(const double *param, int i, int j, float *abc_out /*[5]: mx,my,a,b,c*/)
{
    cutoff32 s = cutoff_setup(param, NULL, 1 << 20, 1 << 20);
    if (abc_out) { abc_out[0] = s.mx; abc_out[1] = s.my; abc_out[2] = s.a; abc_out[3] = s.b; abc_out[4] = s.c; }
    if (!s.ok) return NAN;
    float px = (float)j + 0.5f, py = (float)i + 0.5f;
    float dx = px - s.mx, dy = py - s.my;
    float u = s.a * dx;
    float t = s.b * dx;
    float v = fmaf(s.c, dy, t);
    float uu = u * u;
    return fmaf(v, v, uu);
}

float oracle_const(int which)
{
    switch (which) {
    case 0: return c_scale();
    case 1: return c_e9();
    case 2: return c_lmax();
    default: return NAN;
    }
}

/* ------------------------------------------------------------------------ */
/* fp64 values                                                              */
/* ------------------------------------------------------------------------ */

typedef struct {
    double mx, my, l11, l21, l22, c[3];
    double sxx, sxy, syy, det;     /* Sigma = L L^T and its determinant */
    double pxx, pxy, pyy;          /* Sigma^-1 by the adjugate */
    double o;                      /* opacity (alpha variant) */
    int clamped;                   /* lambda >= ln 999: o held at its clamp */
} gauss64;

static gauss64 gauss_setup(const double *p, const double *logit)
{
    gauss64 g;
    g.mx = p[0]; g.my = p[1]; g.l11 = p[2]; g.l21 = p[3]; g.l22 = p[4];
    g.c[0] = p[5]; g.c[1] = p[6]; g.c[2] = p[7];
    g.sxx = g.l11 * g.l11;
    g.sxy = g.l11 * g.l21;
    g.syy = g.l21 * g.l21 + g.l22 * g.l22;
    g.det = (g.l11 * g.l22) * (g.l11 * g.l22);   /* det(L L^T) = det(L)^2 */
    g.pxx = g.syy / g.det;
    g.pxy = -g.sxy / g.det;
    g.pyy = g.sxx / g.det;
    g.o = 1.0; g.clamped = 0;
    if (logit) {
        double lam = *logit;
        double lmax = (double)c_lmax();
        if (lam >= lmax) { lam = lmax; g.clamped = 1; }
        g.o = 1.0 / (1.0 + exp(-lam));
    }
    return g;
}

/* q = d^T Sigma^-1 d at the pixel centre */
static double gauss_q(const gauss64 *g, int i, int j, double *dx_out, double *dy_out)
{
    double dx = (j + 0.5) - g->mx, dy = (i + 0.5) - g->my;
    if (dx_out) *dx_out = dx;
    if (dy_out) *dy_out = dy;
    return g->pxx * dx * dx + 2.0 * g->pxy * dx * dy + g->pyy * dy * dy;
}

/* Derivatives of q w.r.t. (mux, muy, l11, l21, l22), by matrix calculus:
 *   dq/dmu = -2 Sigma^-1 d,
 *   dq/dL  = -2 Sigma^-1 d d^T Sigma^-1 L  (lower-triangular entries). */
/* The same derivatives with every inner sum replaced by the sum of the absolute
 * values of its terms (a running-error scale for fp32 evaluations of dq). */
static void gauss_dq_abs(const gauss64 *g, double dx, double dy, double dqa[5])
{
    double zx = fabs(g->pxx * dx) + fabs(g->pxy * dy);
    double zy = fabs(g->pxy * dx) + fabs(g->pyy * dy);
    dqa[0] = 2.0 * zx;
    dqa[1] = 2.0 * zy;
    double zl0 = zx * fabs(g->l11) + zy * fabs(g->l21);
    double zl1 = zy * fabs(g->l22);
    dqa[2] = 2.0 * zx * zl0;
    dqa[3] = 2.0 * zy * zl0;
    dqa[4] = 2.0 * zy * zl1;
}

static void gauss_dq(const gauss64 *g, double dx, double dy, double dq[5])
{
    double zx = g->pxx * dx + g->pxy * dy;   /* z = Sigma^-1 d */
    double zy = g->pxy * dx + g->pyy * dy;
    dq[0] = -2.0 * zx;
    dq[1] = -2.0 * zy;
    /* (z z^T L)_{r,c} = z_r * (z^T L)_c ; (z^T L) = (zx l11 + zy l21, zy l22) */
    double zl0 = zx * g->l11 + zy * g->l21;
    double zl1 = zy * g->l22;
    dq[2] = -2.0 * zx * zl0;   /* entry (0,0): l11 */
    dq[3] = -2.0 * zy * zl0;   /* entry (1,0): l21 */
    dq[4] = -2.0 * zy * zl1;   /* entry (1,1): l22 */
}

/* ------------------------------------------------------------------------ */
/* Binning by definition                                                    */
/* ------------------------------------------------------------------------ */

/* Per-Gaussian inclusive pixel box (j0,i0,j1,i1; -1s when culled or empty)
 * and tile count.  Returns the number of culled Gaussians. */
int64_t oracle_footprint(int W, int H, int64_t n, const double *params, const double *logit,
                         int32_t *pix_box, uint32_t *counts)
{
    int64_t culled = 0;
    for (int64_t g = 0; g < n; ++g) {
        cutoff32 s = cutoff_setup(params + 8 * g, logit ? logit + g : NULL, W, H);
        if (!s.ok) ++culled;
        if (!s.ok || s.j0 > s.j1 || s.i0 > s.i1) {
            if (pix_box) { pix_box[4*g+0] = -1; pix_box[4*g+1] = -1; pix_box[4*g+2] = -1; pix_box[4*g+3] = -1; }
            counts[g] = 0;
            continue;
        }
        if (pix_box) { pix_box[4*g+0] = s.j0; pix_box[4*g+1] = s.i0; pix_box[4*g+2] = s.j1; pix_box[4*g+3] = s.i1; }
        int tx0 = s.j0 / ORACLE_TILE, tx1 = s.j1 / ORACLE_TILE;
        int ty0 = s.i0 / ORACLE_TILE, ty1 = s.i1 / ORACLE_TILE;
        counts[g] = (uint32_t)((tx1 - tx0 + 1) * (ty1 - ty0 + 1));
    }
    return culled;
}

/* Tile lists by definition: tile t's list is every Gaussian whose tile box
 * holds t, in ascending index order; the lists are concatenated in tile order.
 * offsets[n] = instances emitted by Gaussians before n (offsets[N] = M).
 * Returns M, or -(M) - 1 when M exceeds cap (nothing written to keys/vals). */
int64_t oracle_bin(int W, int H, int64_t n, const double *params, const double *logit,
                   uint32_t *offsets, uint32_t *keys, uint32_t *vals, uint32_t *ranges, int64_t cap)
{
    const int tx = (W + ORACLE_TILE - 1) / ORACLE_TILE, ty = (H + ORACLE_TILE - 1) / ORACLE_TILE;
    const int64_t T = (int64_t)tx * ty;
    int32_t *box = (int32_t *)malloc(sizeof(int32_t) * 4 * (n > 0 ? n : 1));
    uint32_t *cnt = (uint32_t *)malloc(sizeof(uint32_t) * (n > 0 ? n : 1));
    oracle_footprint(W, H, n, params, logit, box, cnt);
    int64_t M = 0;
    for (int64_t g = 0; g < n; ++g) { offsets[g] = (uint32_t)M; M += cnt[g]; }
    offsets[n] = (uint32_t)M;
    if (M > cap) { free(box); free(cnt); return -M - 1; }
    int64_t pos = 0;
    for (int64_t t = 0; t < T; ++t) {
        int ttx = (int)(t % tx), tty = (int)(t / tx);
        ranges[2*t] = (uint32_t)pos;
        for (int64_t g = 0; g < n; ++g) {
            if (cnt[g] == 0) continue;
            int tx0 = box[4*g+0] / ORACLE_TILE, ty0 = box[4*g+1] / ORACLE_TILE;
            int tx1 = box[4*g+2] / ORACLE_TILE, ty1 = box[4*g+3] / ORACLE_TILE;
            if (ttx >= tx0 && ttx <= tx1 && tty >= ty0 && tty <= ty1) {
                keys[pos] = (uint32_t)t; vals[pos] = (uint32_t)g; ++pos;
            }
        }
        ranges[2*t+1] = (uint32_t)pos;
        if (ranges[2*t] == ranges[2*t+1]) { ranges[2*t] = 0; ranges[2*t+1] = 0; }
    }
    free(box); free(cnt);
    return M;
}

/* Counts pairs whose fp32 cutoff admits the pixel although the pixel lies
 * outside the Gaussian's pixel box (a non-conservative box).  Brute force. */
int64_t oracle_box_leaks(int W, int H, int64_t n, const double *params)
{
    int64_t leaks = 0;
    #pragma omp parallel for reduction(+:leaks) schedule(dynamic, 64)
    for (int64_t g = 0; g < n; ++g) {
        cutoff32 s = cutoff_setup(params + 8 * g, NULL, W, H);
        if (!s.ok) continue;
        for (int i = 0; i < H; ++i)
            for (int j = 0; j < W; ++j)
                if (cutoff_in(&s, i, j) && !(j >= s.j0 && j <= s.j1 && i >= s.i0 && i <= s.i1)) ++leaks;
    }
    return leaks;
}

/* Smallest |e - E9| over all pairs (how far every decision is from flipping). */
double oracle_cutoff_margin(int W, int H, int64_t n, const double *params)
{
    double m = INFINITY;
    const double e9 = (double)c_e9();
    for (int64_t g = 0; g < n; ++g) {
        cutoff32 s = cutoff_setup(params + 8 * g, NULL, W, H);
        if (!s.ok) continue;
        for (int i = 0; i < H; ++i)
            for (int j = 0; j < W; ++j) {
                float e = oracle_cutoff_exponent(params + 8 * g, i, j, NULL);
                double d = fabs((double)e - e9);
                if (d < m) m = d;
            }
    }
    return m;
}

/* ------------------------------------------------------------------------ */
/* Renders                                                                  */
/* ------------------------------------------------------------------------ */

static void pixel_of(const int32_t *pix, int64_t p, int W, int *i, int *j)
{
    if (pix) { *i = pix[2*p]; *j = pix[2*p+1]; }
    else { *i = (int)(p / W); *j = (int)(p % W); }
}

/* Accumulated-sum image at npix pixels (pix = NULL: every pixel, row-major).
 * out[k*npix + p] = I_k(p); sabs[k*npix + p] = sum_n |c_{n,k}| w_n(p).
 * cutoff = 0 sums every Gaussian at every pixel (test-only: no 3-sigma cut). */
void oracle_render_sum(int W, int H, int64_t n, const double *params, const int32_t *pix, int64_t npix,
                       int cutoff, double *out, double *sabs)
{
    cutoff32 *cs = (cutoff32 *)malloc(sizeof(cutoff32) * (n > 0 ? n : 1));
    gauss64 *gs = (gauss64 *)malloc(sizeof(gauss64) * (n > 0 ? n : 1));
    for (int64_t g = 0; g < n; ++g) { cs[g] = cutoff_setup(params + 8*g, NULL, W, H); gs[g] = gauss_setup(params + 8*g, NULL); }
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npix; ++p) {
        int i, j; pixel_of(pix, p, W, &i, &j);
        double acc[3] = {0, 0, 0}, aab[3] = {0, 0, 0};
        for (int64_t g = 0; g < n; ++g) {
            if (!cs[g].ok) continue;
            if (cutoff && !cutoff_in(&cs[g], i, j)) continue;
            double w = exp(-0.5 * gauss_q(&gs[g], i, j, NULL, NULL));
            for (int k = 0; k < 3; ++k) { acc[k] += gs[g].c[k] * w; aab[k] += fabs(gs[g].c[k]) * w; }
        }
        for (int k = 0; k < 3; ++k) { out[k*npix + p] = acc[k]; if (sabs) sabs[k*npix + p] = aab[k]; }
    }
    free(cs); free(gs);
}

/* Gradient of L = sum_{k,p} G_k(p) I_k(p) for the sum image (G = dL/dI at
 * every pixel, [3,H,W]).  dparams[n,8] and, if given, the per-entry sum of
 * |per-pair contribution| aabs[n,8] and the running-error scale acond[n,8]:
 * the same sum with every inner sum of a contribution (g.c, Sigma^-1 d, ...)
 * taken over absolute values. */
void oracle_grad_sum(int W, int H, int64_t n, const double *params, const double *G, int cutoff,
                     double *dparams, double *aabs, double *acond)
{
    const int nt = omp_get_max_threads();
    cutoff32 *cs = (cutoff32 *)malloc(sizeof(cutoff32) * (n > 0 ? n : 1));
    gauss64 *gs = (gauss64 *)malloc(sizeof(gauss64) * (n > 0 ? n : 1));
    for (int64_t g = 0; g < n; ++g) { cs[g] = cutoff_setup(params + 8*g, NULL, W, H); gs[g] = gauss_setup(params + 8*g, NULL); }
    double *part = (double *)calloc((size_t)nt * 24 * (n > 0 ? n : 1), sizeof(double));
    const int64_t HW = (int64_t)H * W;
    #pragma omp parallel
    {
        double *mine = part + (size_t)omp_get_thread_num() * 24 * (n > 0 ? n : 1);
        #pragma omp for schedule(dynamic, 4)
        for (int i = 0; i < H; ++i)
            for (int j = 0; j < W; ++j) {
                const double gk[3] = {G[(int64_t)i*W + j], G[HW + (int64_t)i*W + j], G[2*HW + (int64_t)i*W + j]};
                if (gk[0] == 0.0 && gk[1] == 0.0 && gk[2] == 0.0) continue;   /* contributes exactly 0 */
                for (int64_t g = 0; g < n; ++g) {
                    if (!cs[g].ok) continue;
                    if (cutoff && !cutoff_in(&cs[g], i, j)) continue;
                    double dx, dy;
                    double q = gauss_q(&gs[g], i, j, &dx, &dy);
                    double w = exp(-0.5 * q);
                    double gc = gk[0]*gs[g].c[0] + gk[1]*gs[g].c[1] + gk[2]*gs[g].c[2];
                    double dq[5];
                    gauss_dq(&gs[g], dx, dy, dq);
                    double dqa[5];
                    gauss_dq_abs(&gs[g], dx, dy, dqa);
                    double gca = fabs(gk[0]*gs[g].c[0]) + fabs(gk[1]*gs[g].c[1]) + fabs(gk[2]*gs[g].c[2]);
                    double contrib[8], cond[8];
                    for (int t = 0; t < 5; ++t) { contrib[t] = gc * w * (-0.5) * dq[t]; cond[t] = gca * w * 0.5 * dqa[t]; }
                    for (int k = 0; k < 3; ++k) { contrib[5+k] = gk[k] * w; cond[5+k] = fabs(contrib[5+k]); }
                    for (int t = 0; t < 8; ++t) {
                        mine[24*g + t] += contrib[t];
                        mine[24*g + 8 + t] += fabs(contrib[t]);
                        mine[24*g + 16 + t] += cond[t];
                    }
                }
            }
    }
    for (int64_t g = 0; g < n; ++g)
        for (int t = 0; t < 8; ++t) {
            double s = 0, a = 0, c = 0;
            for (int th = 0; th < nt; ++th) {
                s += part[(size_t)th*24*n + 24*g + t];
                a += part[(size_t)th*24*n + 24*g + 8 + t];
                c += part[(size_t)th*24*n + 24*g + 16 + t];
            }
            dparams[8*g + t] = s;
            if (aabs) aabs[8*g + t] = a;
            if (acond) acond[8*g + t] = c;
        }
    free(part); free(cs); free(gs);
}

/* Alpha-composited image.  For each pixel the Gaussians are visited in index
 * order; a Gaussian whose cutoff admits the pixel has alpha = o w and adds
 * c alpha T; then T <- T (1 - alpha); after the first Gaussian that leaves
 * T < 1e-4 the pixel stops.  C += T bg.
 *  out[3,npix], t_final[npix], last[npix] = index of the last Gaussian
 *  composited (-1 if none), ambiguous[npix] = 1 when some transmittance met
 *  by the stop test lies within 1e-3 (relative) of 1e-4, so fp32 rounding may
 *  move the stop by one Gaussian.  force_last (may be NULL): per pixel,
 *  stop after this Gaussian index instead of testing T (>= n: never stop,
 *  -1: composite nothing).  sabs (may be NULL): per channel
 *  sum_n |c_n| alpha_n T_n + T |bg|, the scale of the error metric. */
void oracle_render_alpha(int W, int H, int64_t n, const double *params, const double *logit, const double *bg,
                         const int32_t *pix, int64_t npix, const int64_t *force_last,
                         double *out, double *t_final, int64_t *last, int32_t *ambiguous, double *sabs)
{
    cutoff32 *cs = (cutoff32 *)malloc(sizeof(cutoff32) * (n > 0 ? n : 1));
    gauss64 *gs = (gauss64 *)malloc(sizeof(gauss64) * (n > 0 ? n : 1));
    for (int64_t g = 0; g < n; ++g) { cs[g] = cutoff_setup(params + 8*g, logit + g, W, H); gs[g] = gauss_setup(params + 8*g, logit + g); }
    const double thr = 1e-4, band = 1e-3;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npix; ++p) {
        int i, j; pixel_of(pix, p, W, &i, &j);
        double C[3] = {0, 0, 0}, A[3] = {0, 0, 0}, T = 1.0;
        int64_t lst = -1; int amb = 0;
        int64_t fl = force_last ? force_last[p] : 0;
        if (!(force_last && fl < 0)) {
            for (int64_t g = 0; g < n; ++g) {
                if (!cs[g].ok || !cutoff_in(&cs[g], i, j)) continue;
                double w = exp(-0.5 * gauss_q(&gs[g], i, j, NULL, NULL));
                double al = gs[g].o * w;
                for (int k = 0; k < 3; ++k) { C[k] += gs[g].c[k] * al * T; A[k] += fabs(gs[g].c[k]) * al * T; }
                T *= (1.0 - al);
                lst = g;
                if (force_last) { if (g >= fl) break; continue; }
                if (fabs(T - thr) <= band * thr) amb = 1;
                if (T < thr) break;
            }
        }
        for (int k = 0; k < 3; ++k) {
            out[k*npix + p] = C[k] + T * bg[k];
            if (sabs) sabs[k*npix + p] = A[k] + T * fabs(bg[k]);
        }
        if (t_final) t_final[p] = T;
        if (last) last[p] = lst;
        if (ambiguous) ambiguous[p] = amb;
    }
    free(cs); free(gs);
}

/* Gradient of L = sum G_k(p) C_k(p) for the alpha image at every pixel, with
 * each pixel's stopping point held fixed (force_last as above, or the oracle's
 * own stop when NULL).  dparams[n,8], dlogit[n], dbg[3]; aabs[n,9] (8 params +
 * logit) is the per-entry sum of |per-pair contribution| and acond[n,9] the
 * running-error scale (inner sums over absolute values, as in oracle_grad_sum).
 * The suffix sums are formed directly from the stored contributors (no division). */
void oracle_grad_alpha(int W, int H, int64_t n, const double *params, const double *logit, const double *bg,
                       const double *G, const int64_t *force_last,
                       double *dparams, double *dlogit, double *dbg, double *aabs, double *acond)
{
    const int nt = omp_get_max_threads();
    cutoff32 *cs = (cutoff32 *)malloc(sizeof(cutoff32) * (n > 0 ? n : 1));
    gauss64 *gs = (gauss64 *)malloc(sizeof(gauss64) * (n > 0 ? n : 1));
    for (int64_t g = 0; g < n; ++g) { cs[g] = cutoff_setup(params + 8*g, logit + g, W, H); gs[g] = gauss_setup(params + 8*g, logit + g); }
    const size_t stride = 28;   /* 9 sums + 9 abs sums + 9 running-error scales + pad */
    double *part = (double *)calloc((size_t)nt * stride * (n > 0 ? n : 1), sizeof(double));
    double *pbg = (double *)calloc((size_t)nt * 3, sizeof(double));
    const int64_t HW = (int64_t)H * W;
    const double thr = 1e-4;
    #pragma omp parallel
    {
        const int th = omp_get_thread_num();
        double *mine = part + (size_t)th * stride * (n > 0 ? n : 1);
        int64_t cap = 64;
        int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * cap);
        double *wv = (double *)malloc(sizeof(double) * cap);
        double *Tv = (double *)malloc(sizeof(double) * cap);
        #pragma omp for schedule(dynamic, 4)
        for (int64_t p = 0; p < HW; ++p) {
            int i = (int)(p / W), j = (int)(p % W);
            const double gk[3] = {G[p], G[HW + p], G[2*HW + p]};
            if (gk[0] == 0.0 && gk[1] == 0.0 && gk[2] == 0.0) continue;   /* contributes exactly 0 */
            /* forward: collect contributors */
            int64_t K = 0; double T = 1.0;
            int64_t fl = force_last ? force_last[p] : 0;
            if (!(force_last && fl < 0)) {
                for (int64_t g = 0; g < n; ++g) {
                    if (!cs[g].ok || !cutoff_in(&cs[g], i, j)) continue;
                    double w = exp(-0.5 * gauss_q(&gs[g], i, j, NULL, NULL));
                    if (K == cap) {
                        cap *= 2;
                        idx = (int64_t *)realloc(idx, sizeof(int64_t) * cap);
                        wv = (double *)realloc(wv, sizeof(double) * cap);
                        Tv = (double *)realloc(Tv, sizeof(double) * cap);
                    }
                    idx[K] = g; wv[K] = w; Tv[K] = T; ++K;
                    T *= (1.0 - gs[g].o * w);
                    if (force_last) { if (g >= fl) break; continue; }
                    if (T < thr) break;
                }
            }
            /* dC/dbg = T_final */
            for (int k = 0; k < 3; ++k) pbg[3*th + k] += gk[k] * T;
            /* backward: S_m = sum_{r>m} c_r alpha_r T_r + T_final bg, per channel */
            double S[3] = {T * bg[0], T * bg[1], T * bg[2]};
            double Sa[3] = {T * fabs(bg[0]), T * fabs(bg[1]), T * fabs(bg[2])};
            for (int64_t m = K - 1; m >= 0; --m) {
                const gauss64 *gg = &gs[idx[m]];
                double w = wv[m], Tm = Tv[m], al = gg->o * w;
                double dC_dal = 0.0, dC_dal_a = 0.0;   /* sum_k G_k dC_k/dalpha, and over |terms| */
                for (int k = 0; k < 3; ++k) {
                    dC_dal += gk[k] * (Tm * gg->c[k] - S[k] / (1.0 - al));
                    dC_dal_a += fabs(gk[k]) * (Tm * fabs(gg->c[k]) + Sa[k] / (1.0 - al));
                }
                double contrib[9], cond[9];
                double dx, dy;
                gauss_q(gg, i, j, &dx, &dy);
                double dq[5], dqa[5];
                gauss_dq(gg, dx, dy, dq);
                gauss_dq_abs(gg, dx, dy, dqa);
                /* alpha = o w, w = exp(-q/2) */
                for (int t = 0; t < 5; ++t) {
                    contrib[t] = dC_dal * gg->o * w * (-0.5) * dq[t];
                    cond[t] = dC_dal_a * gg->o * w * 0.5 * dqa[t];
                }
                for (int k = 0; k < 3; ++k) { contrib[5+k] = gk[k] * al * Tm; cond[5+k] = fabs(contrib[5+k]); }
                contrib[8] = gg->clamped ? 0.0 : dC_dal * w * gg->o * (1.0 - gg->o);
                cond[8] = gg->clamped ? 0.0 : dC_dal_a * w * gg->o * (1.0 - gg->o);
                double *dst = mine + stride * idx[m];
                for (int t = 0; t < 9; ++t) { dst[t] += contrib[t]; dst[9 + t] += fabs(contrib[t]); dst[18 + t] += cond[t]; }
                for (int k = 0; k < 3; ++k) { S[k] += gg->c[k] * al * Tm; Sa[k] += fabs(gg->c[k]) * al * Tm; }
            }
        }
        free(idx); free(wv); free(Tv);
    }
    for (int64_t g = 0; g < n; ++g) {
        for (int t = 0; t < 9; ++t) {
            double s = 0, a = 0, c = 0;
            for (int th = 0; th < nt; ++th) {
                s += part[(size_t)th*stride*n + stride*g + t];
                a += part[(size_t)th*stride*n + stride*g + 9 + t];
                c += part[(size_t)th*stride*n + stride*g + 18 + t];
            }
            if (t < 8) dparams[8*g + t] = s; else dlogit[g] = s;
            if (aabs) aabs[9*g + t] = a;
            if (acond) acond[9*g + t] = c;
        }
    }
    for (int k = 0; k < 3; ++k) { double s = 0; for (int th = 0; th < nt; ++th) s += pbg[3*th + k]; dbg[k] = s; }
    free(part); free(pbg); free(cs); free(gs);
}

/* ------------------------------------------------------------------------ */
/* Loss and optimiser                                                       */
/* ------------------------------------------------------------------------ */

/* L = mean (I - T)^2 over all m entries; grad (may be NULL) = dL/dI. */
double oracle_loss_l2(int64_t m, const double *img, const double *tgt, double *grad)
{
    double s = 0.0;
    for (int64_t e = 0; e < m; ++e) {
        double d = img[e] - tgt[e];
        s += d * d;
        if (grad) grad[e] = 2.0 * d / (double)m;
    }
    return m > 0 ? s / (double)m : 0.0;
}

/* One Adam step (bias-corrected, no weight decay) on rows x row_len entries,
 * lr per slot of the row; step t >= 1. */
void oracle_adam(int64_t rows, int row_len, double *p, const double *g, double *m, double *v,
                 const double *lr, double b1, double b2, double eps, int step)
{
    const double bc1 = 1.0 - pow(b1, step), bc2 = 1.0 - pow(b2, step);
    for (int64_t r = 0; r < rows; ++r)
        for (int s = 0; s < row_len; ++s) {
            int64_t e = r * row_len + s;
            m[e] = b1 * m[e] + (1.0 - b1) * g[e];
            v[e] = b2 * v[e] + (1.0 - b2) * g[e] * g[e];
            double mh = m[e] / bc1, vh = v[e] / bc2;
            p[e] -= lr[s] * mh / (sqrt(vh) + eps);
        }
}

int oracle_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* Rotation-scale Gaussians and rendering at another resolution             */
/* ------------------------------------------------------------------------ */
/* "GaussianImage" (Overview and its training scripts): besides the Cholesky
 * factor, a Gaussian's covariance may be given by a rotation angle and two
 * scales ("gaussianimage_rs").  "FlashImgs" (Library API) keeps the tensors
 * xy, scale, rot, feat and renders a trained set at any output size.
 * Here prs[n] = (mux, muy, sx, sy, theta, cr, cg, cb), theta in radians:
 *   Sigma = R diag(sx^2, sy^2) R^T,  R = [[cos, -sin], [sin, cos]],
 * so with r = R^T d (d = p - mu, coordinates along the Gaussian's axes)
 *   q = (r1/sx)^2 + (r2/sy)^2,  r1 = cos dx + sin dy,  r2 = -sin dx + cos dy.
 * Rendering at scale (fx, fy) maps the image plane by D = diag(fx, fy): mean
 * D mu and covariance D Sigma D, i.e. the new image's pixel centre p is the
 * point D^-1 p of the original frame.  The cutoff is q <= 9 in fp64; a pair
 * whose q lies within 1e-4 (relative) of 9 is "ambiguous": an fp32 pipeline
 * that forms the covariance by other (rounded) steps may decide it either
 * way, so the magnitude of its contribution is reported separately. */

typedef struct { int ok; double mx, my, sx, sy, cs, sn, c[3]; } rsg;

static rsg rs_setup(const double *p)
{
    rsg g;
    memset(&g, 0, sizeof g);
    for (int k = 0; k < 8; ++k)
        if (!isfinite(p[k])) return g;
    if (p[2] == 0.0 || p[3] == 0.0) return g;
    g.mx = p[0]; g.my = p[1]; g.sx = p[2]; g.sy = p[3];
    g.cs = cos(p[4]); g.sn = sin(p[4]);
    g.c[0] = p[5]; g.c[1] = p[6]; g.c[2] = p[7];
    g.ok = 1;
    return g;
}

#define RS_AMBIG 1e-4

/* 0: outside the cutoff, 1: inside, 2: inside or outside within the ambiguity band */
static int rs_class(double q, int cutoff)
{
    if (!cutoff) return 1;
    if (fabs(q - 9.0) <= 9.0 * RS_AMBIG) return 2;
    return q <= 9.0 ? 1 : 0;
}

/* Sum image of rotation-scale Gaussians rendered at scale (fx, fy), at npix
 * pixels (pix = NULL: every pixel of the W x H output, row-major).
 * out[3,npix]; sabs[3,npix] = sum |c| w; amb[3,npix] = sum |c| w over the
 * ambiguous pairs (those are included in out when q <= 9). */
void oracle_render_sum_rs(int W, int H, int64_t n, const double *prs, double fx, double fy, const int32_t *pix,
                          int64_t npix, int cutoff, double *out, double *sabs, double *amb)
{
    rsg *gs = (rsg *)malloc(sizeof(rsg) * (n > 0 ? n : 1));
    for (int64_t g = 0; g < n; ++g) gs[g] = rs_setup(prs + 8 * g);
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npix; ++p) {
        int i, j; pixel_of(pix, p, W, &i, &j);
        const double x = (j + 0.5) / fx, y = (i + 0.5) / fy;
        double acc[3] = {0, 0, 0}, aab[3] = {0, 0, 0}, am[3] = {0, 0, 0};
        for (int64_t g = 0; g < n; ++g) {
            if (!gs[g].ok) continue;
            const double dx = x - gs[g].mx, dy = y - gs[g].my;
            const double r1 = gs[g].cs * dx + gs[g].sn * dy, r2 = -gs[g].sn * dx + gs[g].cs * dy;
            const double q = (r1 / gs[g].sx) * (r1 / gs[g].sx) + (r2 / gs[g].sy) * (r2 / gs[g].sy);
            const int cl = rs_class(q, cutoff);
            if (cl == 0) continue;
            const double w = exp(-0.5 * q);
            for (int k = 0; k < 3; ++k) {
                if (cl == 2) am[k] += fabs(gs[g].c[k]) * w;
                if (cl == 2 && q > 9.0) continue;
                acc[k] += gs[g].c[k] * w;
                aab[k] += fabs(gs[g].c[k]) * w;
            }
        }
        for (int k = 0; k < 3; ++k) {
            out[k*npix + p] = acc[k];
            if (sabs) sabs[k*npix + p] = aab[k];
            if (amb) amb[k*npix + p] = am[k];
        }
    }
    free(gs);
}

/* Gradient of L = sum_{k,p} G_k(p) I_k(p) (G [3,H,W] over the output image)
 * with respect to the rotation-scale parameters prs[n,8] of the image
 * rendered at scale (fx, fy).  With h = dL/dq = -w/2 (g . c):
 *   dq/dmu    = -2 (r1/sx^2 R[:,0] + r2/sy^2 R[:,1]),  R[:,0] = (cos, sin), R[:,1] = (-sin, cos)
 *   dq/dsx    = -2 r1^2 / sx^3,   dq/dsy = -2 r2^2 / sy^3,
 *   dq/dtheta = 2 r1 r2 (1/sx^2 - 1/sy^2)   (dr1/dtheta = r2, dr2/dtheta = -r1),
 *   dL/dc_k   = sum_p G_k w.
 * acond[n,8]: running-error scale (every inner sum over absolute values);
 * amb[n,8]: sum of |contribution| over the ambiguous pairs. */
void oracle_grad_sum_rs(int W, int H, int64_t n, const double *prs, double fx, double fy, const double *G,
                        int cutoff, double *dparams, double *acond, double *amb)
{
    const int nt = omp_get_max_threads();
    const size_t nn = (size_t)(n > 0 ? n : 1);
    rsg *gs = (rsg *)malloc(sizeof(rsg) * nn);
    for (int64_t g = 0; g < n; ++g) gs[g] = rs_setup(prs + 8 * g);
    double *part = (double *)calloc((size_t)nt * 24 * nn, sizeof(double));
    const int64_t HW = (int64_t)H * W;
    #pragma omp parallel
    {
        double *mine = part + (size_t)omp_get_thread_num() * 24 * nn;
        #pragma omp for schedule(dynamic, 4)
        for (int i = 0; i < H; ++i)
            for (int j = 0; j < W; ++j) {
                const double gk[3] = {G[(int64_t)i*W + j], G[HW + (int64_t)i*W + j], G[2*HW + (int64_t)i*W + j]};
                if (gk[0] == 0.0 && gk[1] == 0.0 && gk[2] == 0.0) continue;   /* contributes exactly 0 */
                const double x = (j + 0.5) / fx, y = (i + 0.5) / fy;
                for (int64_t g = 0; g < n; ++g) {
                    const rsg *s = &gs[g];
                    if (!s->ok) continue;
                    const double dx = x - s->mx, dy = y - s->my;
                    const double r1 = s->cs * dx + s->sn * dy, r2 = -s->sn * dx + s->cs * dy;
                    const double ix2 = 1.0 / (s->sx * s->sx), iy2 = 1.0 / (s->sy * s->sy);
                    const double q = r1 * r1 * ix2 + r2 * r2 * iy2;
                    const int cl = rs_class(q, cutoff);
                    if (cl == 0 || (cl == 2 && q > 9.0 && !amb)) continue;
                    const double w = exp(-0.5 * q);
                    const double gc = gk[0]*s->c[0] + gk[1]*s->c[1] + gk[2]*s->c[2];
                    const double gca = fabs(gk[0]*s->c[0]) + fabs(gk[1]*s->c[1]) + fabs(gk[2]*s->c[2]);
                    const double h = -0.5 * w * gc, ha = 0.5 * w * gca;
                    const double a1 = fabs(s->cs * dx) + fabs(s->sn * dy), a2 = fabs(s->sn * dx) + fabs(s->cs * dy);
                    double dq[5], dqa[5];
                    dq[0] = -2.0 * (r1 * ix2 * s->cs - r2 * iy2 * s->sn);
                    dq[1] = -2.0 * (r1 * ix2 * s->sn + r2 * iy2 * s->cs);
                    dq[2] = -2.0 * r1 * r1 * ix2 / s->sx;
                    dq[3] = -2.0 * r2 * r2 * iy2 / s->sy;
                    dq[4] = 2.0 * r1 * r2 * (ix2 - iy2);
                    dqa[0] = 2.0 * (a1 * ix2 * fabs(s->cs) + a2 * iy2 * fabs(s->sn));
                    dqa[1] = 2.0 * (a1 * ix2 * fabs(s->sn) + a2 * iy2 * fabs(s->cs));
                    dqa[2] = 2.0 * a1 * a1 * ix2 / fabs(s->sx);
                    dqa[3] = 2.0 * a2 * a2 * iy2 / fabs(s->sy);
                    dqa[4] = 2.0 * a1 * a2 * (ix2 + iy2);
                    double contrib[8], cond[8];
                    for (int t = 0; t < 5; ++t) { contrib[t] = h * dq[t]; cond[t] = ha * dqa[t]; }
                    for (int k = 0; k < 3; ++k) { contrib[5+k] = gk[k] * w; cond[5+k] = fabs(contrib[5+k]); }
                    const int inside = !(cl == 2 && q > 9.0);
                    for (int t = 0; t < 8; ++t) {
                        if (inside) { mine[24*g + t] += contrib[t]; mine[24*g + 8 + t] += cond[t]; }
                        if (cl == 2) mine[24*g + 16 + t] += fabs(contrib[t]);
                    }
                }
            }
    }
    for (int64_t g = 0; g < n; ++g) {
        for (int t = 0; t < 8; ++t) {
            double s = 0, c = 0, a = 0;
            for (int th = 0; th < nt; ++th) {
                s += part[(size_t)th*24*nn + 24*g + t];
                c += part[(size_t)th*24*nn + 24*g + 8 + t];
                a += part[(size_t)th*24*nn + 24*g + 16 + t];
            }
            dparams[8*g + t] = s;
            if (acond) acond[8*g + t] = c;
            if (amb) amb[8*g + t] = a;
        }
    }
    free(part); free(gs);
}

/* The chain rule of the conversion to the Cholesky form at scale (fx, fy): given the gradient
 * dout[n,8] w.r.t. (D mu, L', c) with L' = D chol(Sigma), out[n,8] = J^T dout w.r.t. the
 * rotation-scale params, J = d(D mu, L', c)/d(mu, sx, sy, theta, c), and scale[n,8] = |J|^T |dout|
 * (the size of the terms the sum adds).  The factor of Sigma = R diag(sx^2, sy^2) R^T:
 *   l11 = sqrt(A), l21 = B/l11, l22 = P/l11,
 *   A = (cos ax)^2 + (sin ay)^2, B = cos sin (ax^2 - ay^2), P = ax ay, ax = |sx|, ay = |sy|,
 * differentiated by hand (then l' = (fx l11, fy l21, fy l22)).  A zero scale gives zeros. */
void oracle_rs_cholesky_grad(int64_t n, const double *prs, double fx, double fy, const double *dout, double *out,
                             double *scale)
{
    for (int64_t g = 0; g < n; ++g) {
        const double *p = prs + 8 * g, *d = dout + 8 * g;
        double *o = out + 8 * g, *sc = scale + 8 * g;
        for (int t = 0; t < 8; ++t) { o[t] = 0.0; sc[t] = 0.0; }
        const rsg r = rs_setup(p);
        if (!r.ok) continue;
        const double cs = r.cs, sn = r.sn, ax = fabs(r.sx), ay = fabs(r.sy);
        const double A = cs * cs * ax * ax + sn * sn * ay * ay, B = cs * sn * (ax * ax - ay * ay), P = ax * ay;
        const double l11 = sqrt(A), l21 = B / l11, l22 = P / l11;
        const double dA[3] = {2 * cs * cs * ax, 2 * sn * sn * ay, -2 * B};
        const double dB[3] = {2 * cs * sn * ax, -2 * cs * sn * ay, (cs * cs - sn * sn) * (ax * ax - ay * ay)};
        const double dP[3] = {ay, ax, 0.0};
        const double sg[3] = {r.sx < 0 ? -1.0 : 1.0, r.sy < 0 ? -1.0 : 1.0, 1.0};
        o[0] = fx * d[0]; sc[0] = fabs(o[0]);
        o[1] = fy * d[1]; sc[1] = fabs(o[1]);
        for (int k = 0; k < 3; ++k) {
            const double d11 = dA[k] / (2 * l11);
            const double j[3] = {fx * sg[k] * d11, fy * sg[k] * (dB[k] - l21 * d11) / l11,
                                 fy * sg[k] * (dP[k] - l22 * d11) / l11};
            o[2 + k] = j[0] * d[2] + j[1] * d[3] + j[2] * d[4];
            sc[2 + k] = fabs(j[0] * d[2]) + fabs(j[1] * d[3]) + fabs(j[2] * d[4]);
        }
        for (int t = 5; t < 8; ++t) { o[t] = d[t]; sc[t] = fabs(d[t]); }
    }
}

/* ------------------------------------------------------------------------ */
/* SSIM pixel loss                                                          */
/* ------------------------------------------------------------------------ */
/* "Drawing with Gaussians" (2D fitting): the pixel loss (1 - w) L1 +
 * w (1 - SSIM), w = 0.2; "FlashImgs" (Commands, --loss l2 / l1 / l2+ssim /
 * l1+ssim; parse_loss gives the (l1, l2, ssim) ratios); fvdb (ssim_lambda).
 * The pages print no SSIM formula; the reading is the usual structural
 * similarity index: per channel, local statistics under an 11x11 Gaussian
 * window (sigma 1.5, weights normalised to sum 1), pixels outside the image
 * count as 0 (the map has the image's size), and
 *   SSIM(p) = (2 mx my + C1)(2 sxy + C2) / ((mx^2 + my^2 + C1)(sxx + syy + C2)),
 *   mx = sum_q G(q-p) x(q), sxx = sum_q G(q-p) x(q)^2 - mx^2,
 *   sxy = sum_q G(q-p) x(q) y(q) - mx my,  C1 = 0.01^2, C2 = 0.03^2,
 * x = the rendered image, y = the target; SSIM = the mean of the map over
 * the 3HW entries.  The loss:
 *   L = w1 mean|x - y| + w2 mean (x - y)^2 + ws (1 - SSIM).
 * Its gradient with respect to x, with f = SSIM(p) a function of the window
 * moments (mx, my, Exx, Eyy, Exy) at p:
 *   dSSIM/dx(q) = (1/3HW) sum_p G(q-p) [df/dmx(p) + 2 x(q) df/dExx(p)
 *                                     + y(q) df/dExy(p)],
 *   df/dmx  = f (2my/n1 - 2my/n2 - 2mx/d1 + 2mx/d2),
 *   df/dExx = -f / d2,   df/dExy = 2 f / n2,
 * n1 = 2 mx my + C1, n2 = 2 sxy + C2, d1 = mx^2 + my^2 + C1, d2 = sxx + syy + C2.
 * d|x - y|/dx = sign(x - y) (0 at 0). */

static void ssim_window(double g[11])
{
    double s = 0.0;
    for (int k = 0; k < 11; ++k) { g[k] = exp(-((k - 5) * (k - 5)) / (2.0 * 1.5 * 1.5)); s += g[k]; }
    for (int k = 0; k < 11; ++k) g[k] /= s;
}

/* The five window moments at every pixel of one channel (zero outside). */
static void ssim_moments(int W, int H, const double *x, const double *y, double *m /*[5][H*W]*/)
{
    double g[11];
    ssim_window(g);
    const int64_t HW = (int64_t)H * W;
    #pragma omp parallel for schedule(static)
    for (int i = 0; i < H; ++i)
        for (int j = 0; j < W; ++j) {
            double s[5] = {0, 0, 0, 0, 0};
            for (int a = -5; a <= 5; ++a)
                for (int b = -5; b <= 5; ++b) {
                    int ii = i + a, jj = j + b;
                    if (ii < 0 || ii >= H || jj < 0 || jj >= W) continue;
                    double wgt = g[a + 5] * g[b + 5];
                    double xv = x[(int64_t)ii * W + jj], yv = y[(int64_t)ii * W + jj];
                    s[0] += wgt * xv; s[1] += wgt * yv;
                    s[2] += wgt * xv * xv; s[3] += wgt * yv * yv; s[4] += wgt * xv * yv;
                }
            for (int k = 0; k < 5; ++k) m[k * HW + (int64_t)i * W + j] = s[k];
        }
}

/* Loss value and (if dx != NULL) dL/dx [3,H,W]; ssim_map (may be NULL) [3,H,W];
 * dscale (may be NULL) [3,H,W]: a running-error scale of dL/dx (every sum
 * and every inner sum taken over absolute values).  Returns L; *ssim_out =
 * the mean SSIM. */
double oracle_loss_ssim(int W, int H, const double *x, const double *y, double w1, double w2, double ws,
                        double *dx, double *ssim_map, double *dscale, double *ssim_out)
{
    const double C1 = 0.0001, C2 = 0.0009;
    const int64_t HW = (int64_t)H * W, N = 3 * HW;
    double g[11];
    ssim_window(g);
    double *m = (double *)malloc(sizeof(double) * 5 * HW);
    double *D = (double *)malloc(sizeof(double) * 6 * HW);     /* df/dmx, df/dExx, df/dExy and their abs scales */
    double l1 = 0.0, l2 = 0.0, ss = 0.0;
    for (int k = 0; k < 3; ++k) {
        const double *xk = x + k * HW, *yk = y + k * HW;
        ssim_moments(W, H, xk, yk, m);
        for (int64_t p = 0; p < HW; ++p) {
            const double mx = m[p], my = m[HW + p];
            const double sxx = m[2*HW + p] - mx * mx, syy = m[3*HW + p] - my * my, sxy = m[4*HW + p] - mx * my;
            const double n1 = 2 * mx * my + C1, n2 = 2 * sxy + C2, d1 = mx * mx + my * my + C1, d2 = sxx + syy + C2;
            const double f = (n1 * n2) / (d1 * d2);
            ss += f;
            if (ssim_map) ssim_map[k * HW + p] = f;
            D[p] = f * (2 * my / n1 - 2 * my / n2 - 2 * mx / d1 + 2 * mx / d2);
            D[HW + p] = -f / d2;
            D[2*HW + p] = 2 * f / n2;
            D[3*HW + p] = fabs(f) * (2 * fabs(my) / fabs(n1) + 2 * fabs(my) / fabs(n2) + 2 * fabs(mx) / fabs(d1) +
                                     2 * fabs(mx) / fabs(d2));
            D[4*HW + p] = fabs(D[HW + p]);
            D[5*HW + p] = fabs(D[2*HW + p]);
            const double e = xk[p] - yk[p];
            l1 += fabs(e);
            l2 += e * e;
        }
        if (!dx) continue;
        #pragma omp parallel for schedule(static)
        for (int i = 0; i < H; ++i)
            for (int j = 0; j < W; ++j) {
                double s0 = 0, s1 = 0, s2 = 0, a0 = 0, a1 = 0, a2 = 0;
                for (int a = -5; a <= 5; ++a)
                    for (int b = -5; b <= 5; ++b) {
                        int ii = i + a, jj = j + b;
                        if (ii < 0 || ii >= H || jj < 0 || jj >= W) continue;
                        double wgt = g[a + 5] * g[b + 5];
                        int64_t pp = (int64_t)ii * W + jj;
                        s0 += wgt * D[pp]; s1 += wgt * D[HW + pp]; s2 += wgt * D[2*HW + pp];
                        a0 += wgt * D[3*HW + pp]; a1 += wgt * D[4*HW + pp]; a2 += wgt * D[5*HW + pp];
                    }
                const int64_t q = (int64_t)i * W + j;
                const double xv = xk[q], yv = yk[q], e = xv - yv;
                const double dssim = (s0 + 2 * xv * s1 + yv * s2) / (double)N;
                const double sg = e > 0 ? 1.0 : (e < 0 ? -1.0 : 0.0);
                dx[k * HW + q] = w1 * sg / (double)N + w2 * 2 * e / (double)N - ws * dssim;
                if (dscale)
                    dscale[k * HW + q] = fabs(w1) / (double)N + fabs(w2) * 2 * (fabs(xv) + fabs(yv)) / (double)N +
                                         fabs(ws) * (a0 + 2 * fabs(xv) * a1 + fabs(yv) * a2) / (double)N;
            }
    }
    free(m); free(D);
    if (ssim_out) *ssim_out = ss / (double)N;
    return w1 * l1 / (double)N + w2 * l2 / (double)N + ws * (1.0 - ss / (double)N);
}

/* ------------------------------------------------------------------------ */
/* Moment-matching merge                                                    */
/* ------------------------------------------------------------------------ */
/* "FlashImgs" (Commands, merge: an overcomplete set merged down, 80K -> 50K,
 * by moment matching; Library API: merge_gaussians).  The pages give no
 * formula; the reading: a Gaussian n of the sum image is the function
 * c_n exp(-q_n/2), whose integral per channel is 2 pi |det L_n| c_{n,k}.  Two
 * Gaussians (i, j) merge into the one whose mean and covariance are those of
 * the mixture weighted by the masses w = |det L| sum_k |c_k|:
 *   W = w_i + w_j,  mu = (w_i mu_i + w_j mu_j) / W,
 *   Sigma = sum_{n=i,j} (w_n / W) (Sigma_n + (mu_n - mu)(mu_n - mu)^T),
 * L = chol(Sigma) (positive diagonal), and whose colour keeps each channel's
 * integral:  c_k = (|det L_i| c_{i,k} + |det L_j| c_{j,k}) / |det L|.
 * W = 0 (no mass) takes equal weights.  Sigma_n = L_n L_n^T as elsewhere. */
/* The merged Gaussian of a and b (Cholesky-form rows of 8) into o (moment matching, above). */
static void merge_two(const double *a, const double *b, double *o)
{
    const double *pp[2] = {a, b};
    double det[2], w[2], S[2][3];
    for (int s = 0; s < 2; ++s) {
        const double *p = pp[s];
        det[s] = fabs(p[2] * p[4]);
        w[s] = det[s] * (fabs(p[5]) + fabs(p[6]) + fabs(p[7]));
        S[s][0] = p[2] * p[2];                 /* Sigma11 */
        S[s][1] = p[2] * p[3];                 /* Sigma21 */
        S[s][2] = p[3] * p[3] + p[4] * p[4];   /* Sigma22 */
    }
    double W = w[0] + w[1];
    double f0 = W > 0 ? w[0] / W : 0.5, f1 = W > 0 ? w[1] / W : 0.5;
    const double mx = f0 * a[0] + f1 * b[0], my = f0 * a[1] + f1 * b[1];
    double s11 = 0, s21 = 0, s22 = 0;
    for (int s = 0; s < 2; ++s) {
        const double f = s ? f1 : f0;
        const double dx = pp[s][0] - mx, dy = pp[s][1] - my;
        s11 += f * (S[s][0] + dx * dx);
        s21 += f * (S[s][1] + dx * dy);
        s22 += f * (S[s][2] + dy * dy);
    }
    const double l11 = sqrt(s11), l21 = s21 / l11, l22 = sqrt(s22 - l21 * l21);
    const double dn = l11 * l22;
    o[0] = mx; o[1] = my; o[2] = l11; o[3] = l21; o[4] = l22;
    for (int k = 0; k < 3; ++k) o[5 + k] = (det[0] * a[5 + k] + det[1] * b[5 + k]) / dn;
}

void oracle_merge_pairs(int64_t np, const double *params, const int64_t *pairs, double *out)
{
    for (int64_t t = 0; t < np; ++t)
        merge_two(params + 8 * pairs[2*t], params + 8 * pairs[2*t + 1], out + 8 * t);
}

/* ------------------------------------------------------------------------ */
/* Merging a set down to a target count ("FlashImgs", merge: train an       */
/* overcomplete set, merge similar Gaussians down by moment matching, 80K   */
/* -> 50K, finetune).  The pages name neither the similarity nor the pair   */
/* rule; the reading here:                                                  */
/*  - cost of merging i and j: the bound on the increase of the            */
/*    Kullback-Leibler divergence when two components of a mixture are     */
/*    replaced by their moment-matched merge (Runnalls, "Kullback-Leibler   */
/*    approach to Gaussian mixture reduction", IEEE Trans. AES 2007):       */
/*      B = 1/2 [ W log det Sigma_m - w_i log det Sigma_i - w_j log det Sigma_j ], */
/*    with the masses w and the merged covariance Sigma_m of merge_two      */
/*    (W = w_i + w_j; B = 0 when W = 0), evaluated with the smaller index   */
/*    first, and B = +inf when det Sigma_m is not positive;                 */
/*  - candidates: the other mergeable Gaussians whose mean lies in the same */
/*    or a neighbouring 16 x 16 cell (cell = floor(mu / 16) per axis,       */
/*    clamped to the image's tiles); mergeable = all 8 params finite and    */
/*    l11, l22 nonzero;                                                     */
/*  - one round: every Gaussian picks its cheapest candidate (ties: the     */
/*    smaller index); pairs that pick each other are merged, all of them,   */
/*    or, when that is more than the count still to remove, the cheapest   */
/*    ones by (fp32 rounding of B, smaller index);                          */
/*  - the merged Gaussian takes the smaller index's place; the set keeps    */
/*    index order otherwise; rounds repeat until the target is reached or   */
/*    no pair picks each other.                                             */
/* The cost's fp64 operations are done in the order written (no FMA).      */
/* ------------------------------------------------------------------------ */

static int mergeable(const double *p)
{
    for (int k = 0; k < 8; ++k)
        if (!isfinite(p[k])) return 0;
    return p[2] != 0.0 && p[4] != 0.0;
}

/* Merge cost of a and b (a: the smaller index). */
static double merge_cost(const double *a, const double *b)
{
    const double da = fabs(a[2] * a[4]), db = fabs(b[2] * b[4]);
    const double wa = da * ((fabs(a[5]) + fabs(a[6])) + fabs(a[7]));
    const double wb = db * ((fabs(b[5]) + fabs(b[6])) + fabs(b[7]));
    const double W = wa + wb;
    const double fa = W > 0 ? wa / W : 0.5, fb = W > 0 ? wb / W : 0.5;
    const double mx = fa * a[0] + fb * b[0], my = fa * a[1] + fb * b[1];
    const double ax = a[0] - mx, ay = a[1] - my, bx = b[0] - mx, by = b[1] - my;
    const double s11 = fa * (a[2] * a[2] + ax * ax) + fb * (b[2] * b[2] + bx * bx);
    const double s21 = fa * (a[2] * a[3] + ax * ay) + fb * (b[2] * b[3] + bx * by);
    const double s22 = fa * ((a[3] * a[3] + a[4] * a[4]) + ay * ay) + fb * ((b[3] * b[3] + b[4] * b[4]) + by * by);
    const double dm = s11 * s22 - s21 * s21;
    if (!(dm > 0.0)) return INFINITY;
    if (W == 0.0) return 0.0;
    return 0.5 * (W * log(dm) - wa * log(da * da) - wb * log(db * db));
}

double oracle_merge_cost(const double *a, const double *b) { return merge_cost(a, b); }

static void merge_cell(const double *p, int tx, int ty, int *cx, int *cy)
{
    double x = floor(p[0] / ORACLE_TILE), y = floor(p[1] / ORACLE_TILE);
    x = x < 0 ? 0 : (x > tx - 1 ? tx - 1 : x);
    y = y < 0 ? 0 : (y > ty - 1 ? ty - 1 : y);
    *cx = (int)x;
    *cy = (int)y;
}

/* One round on params[n,8] (image W x H): the pairs merged, (i, j) with i < j, in ascending i,
 * written to pairs[2 * count]; at most max_pairs.  best[n] (may be NULL): each Gaussian's pick
 * (-1: none). */
int64_t oracle_merge_round(int W, int H, int64_t n, const double *params, int64_t max_pairs, int64_t *pairs,
                           int64_t *best)
{
    const int tx = (W + ORACLE_TILE - 1) / ORACLE_TILE, ty = (H + ORACLE_TILE - 1) / ORACLE_TILE;
    int *cx = (int *)malloc(sizeof(int) * (n > 0 ? n : 1)), *cy = (int *)malloc(sizeof(int) * (n > 0 ? n : 1));
    int64_t *pick = (int64_t *)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
    double *pc = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
    char *ok = (char *)malloc(n > 0 ? n : 1);
    for (int64_t i = 0; i < n; ++i) {
        ok[i] = (char)mergeable(params + 8 * i);
        if (ok[i]) merge_cell(params + 8 * i, tx, ty, &cx[i], &cy[i]);
    }
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < n; ++i) {
        pick[i] = -1;
        pc[i] = INFINITY;
        if (!ok[i]) continue;
        for (int64_t j = 0; j < n; ++j) {
            if (j == i || !ok[j]) continue;
            if (abs(cx[i] - cx[j]) > 1 || abs(cy[i] - cy[j]) > 1) continue;
            const double c = i < j ? merge_cost(params + 8 * i, params + 8 * j)
                                   : merge_cost(params + 8 * j, params + 8 * i);
            if (pick[i] < 0 || c < pc[i] || (c == pc[i] && j < pick[i])) { pick[i] = j; pc[i] = c; }
        }
    }
    /* mutual picks, ascending smaller index */
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t j = pick[i];
        if (j > i && pick[j] == i && isfinite(pc[i])) { pairs[2 * m] = i; pairs[2 * m + 1] = j; ++m; }
    }
    if (m > max_pairs) {            /* keep the cheapest max_pairs by (fp32 cost, smaller index) */
        float *key = (float *)malloc(sizeof(float) * m);
        for (int64_t t = 0; t < m; ++t) key[t] = (float)pc[pairs[2 * t]];
        char *keep = (char *)calloc(m, 1);
        for (int64_t k = 0; k < max_pairs; ++k) {            /* selection, smallest first */
            int64_t b = -1;
            for (int64_t t = 0; t < m; ++t)
                if (!keep[t] && (b < 0 || key[t] < key[b])) b = t;   /* ascending t breaks ties */
            keep[b] = 1;
        }
        int64_t o = 0;
        for (int64_t t = 0; t < m; ++t)
            if (keep[t]) { pairs[2 * o] = pairs[2 * t]; pairs[2 * o + 1] = pairs[2 * t + 1]; ++o; }
        m = o;
        free(key); free(keep);
    }
    if (best)
        for (int64_t i = 0; i < n; ++i) best[i] = pick[i];
    free(cx); free(cy); free(pick); free(pc); free(ok);
    return m;
}

/* The set after merging the pairs (ascending smaller index, disjoint): out[n - npairs, 8]. */
int64_t oracle_merge_apply(int64_t n, const double *params, int64_t npairs, const int64_t *pairs, double *out)
{
    int64_t *partner = (int64_t *)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) partner[i] = -1;
    for (int64_t t = 0; t < npairs; ++t) { partner[pairs[2*t]] = pairs[2*t + 1]; partner[pairs[2*t + 1]] = pairs[2*t]; }
    int64_t o = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (partner[i] < 0) memcpy(out + 8 * o++, params + 8 * i, 8 * sizeof(double));
        else if (partner[i] > i) merge_two(params + 8 * i, params + 8 * partner[i], out + 8 * o++);
    }
    free(partner);
    return o;
}

/* Rounds until n_out == target or no pair is found: out[n, 8] (the first n_out rows used).  The
 * set is a set of fp32 parameters (the form every other call takes them in): after each round the
 * merged rows are rounded to fp32, and the next round starts from those values. */
int64_t oracle_merge_to(int W, int H, int64_t n, const double *params, int64_t target, double *out,
                        int64_t *rounds)
{
    double *cur = (double *)malloc(sizeof(double) * 8 * (n > 0 ? n : 1));
    int64_t *pairs = (int64_t *)malloc(sizeof(int64_t) * (n > 0 ? n : 2));
    memcpy(cur, params, sizeof(double) * 8 * n);
    int64_t m = n, r = 0;
    while (m > target) {
        const int64_t np = oracle_merge_round(W, H, m, cur, m - target, pairs, NULL);
        if (np == 0) break;
        m = oracle_merge_apply(m, cur, np, pairs, out);
        for (int64_t k = 0; k < 8 * m; ++k) cur[k] = (double)(float)out[k];
        ++r;
    }
    memcpy(out, cur, sizeof(double) * 8 * m);
    if (rounds) *rounds = r;
    free(cur); free(pairs);
    return m;
}
/* ------------------------------------------------------------------------ */
/* Adaptive density control ("FlashImgs", Training features: every 300      */
/* steps from step 150, dead, out-of-bounds and bloated Gaussians are       */
/* relocated to high-error pixels).  The pages give no thresholds; the      */
/* reading here:                                                            */
/*  - dead: some parameter non-finite, l11 or l22 zero, or every colour     */
/*    below one 8-bit level in size (max_k |c_k| < 1/255);                  */
/*  - out of bounds: the mean outside [0, W) x [0, H);                      */
/*  - bloated: the larger eigenvalue of Sigma above (max(W, H)/16)^2, i.e.  */
/*    the longer axis' standard deviation above 1/16 of the image;          */
/*  - error of pixel p: e = sum_k r_k^2 with r = target - image, in fp32 as */
/*    fma(r_b, r_b, fma(r_g, r_g, r_r * r_r)), a NaN error counting as 0;   */
/*  - the K = min(#flagged, W H) pixels of largest e (ties: smaller pixel   */
/*    index) taken in ascending pixel index go, one each, to the flagged    */
/*    Gaussians in ascending index: mean = the pixel centre, L = s0 I (s0   */
/*    the caller's initial size), colour = r at that pixel (the Gaussian    */
/*    then fills the residual at its centre).                               */
/* The flag decisions are fp64 comparisons of quantities formed in the     */
/* order written; bloated <=> not (s11 <= t and s22 <= t and                */
/* (t - s11)(t - s22) >= s21^2), t = (max(W,H)/16)^2, Sigma from L.         */
/* ------------------------------------------------------------------------ */

/* 1: dead, 2: out of bounds, 4: bloated (0: kept). */
static int adc_flag(const float *p, int W, int H)
{
    int f = 0;
    for (int k = 0; k < 8; ++k)
        if (!isfinite(p[k])) return 1;
    if (p[2] == 0.0f || p[4] == 0.0f) return 1;
    const double cm = fmax(fabs((double)p[5]), fmax(fabs((double)p[6]), fabs((double)p[7])));
    if (cm < 1.0 / 255.0) f |= 1;
    if (!(p[0] >= 0.0f && p[0] < (float)W && p[1] >= 0.0f && p[1] < (float)H)) f |= 2;
    const double l11 = p[2], l21 = p[3], l22 = p[4];
    const double s11 = l11 * l11, s21 = l11 * l21, s22 = l21 * l21 + l22 * l22;
    const double side = (double)(W > H ? W : H) / 16.0, t = side * side;
    if (!(s11 <= t && s22 <= t && (t - s11) * (t - s22) >= s21 * s21)) f |= 4;
    return f;
}

/* params[n,8] fp32 (updated in place), image / target [3,H,W] fp32; flags[n] out (may be NULL).
 * Returns the number of Gaussians relocated. */
int64_t oracle_adc(int W, int H, int64_t n, float *params, const float *image, const float *target, float s0,
                   int32_t *flags)
{
    const int64_t np = (int64_t)W * H;
    int64_t nf = 0;
    int *fl = (int *)malloc(sizeof(int) * (n > 0 ? n : 1));
    for (int64_t g = 0; g < n; ++g) {
        fl[g] = adc_flag(params + 8 * g, W, H);
        if (flags) flags[g] = fl[g];
        nf += fl[g] != 0;
    }
    const int64_t K = nf < np ? nf : np;
    if (K == 0) { free(fl); return 0; }
    float *e = (float *)malloc(sizeof(float) * np);
    for (int64_t p = 0; p < np; ++p) {
        const float r0 = target[p] - image[p], r1 = target[np + p] - image[np + p];
        const float r2 = target[2 * np + p] - image[2 * np + p];
        e[p] = fmaf(r2, r2, fmaf(r1, r1, r0 * r0));
        if (!(e[p] >= 0.0f)) e[p] = 0.0f;                 /* a NaN error counts as none */
    }
    /* the K-th largest error (ties: smaller index first) by sorting pixel indices */
    int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * np);
    for (int64_t p = 0; p < np; ++p) idx[p] = p;
    /* insertion into a max-ordered prefix would be O(np K); a full sort is plain enough */
    for (int64_t w = 1; w < np; w *= 2) {                 /* bottom-up merge sort, stable */
        int64_t *tmp = (int64_t *)malloc(sizeof(int64_t) * np);
        for (int64_t lo = 0; lo < np; lo += 2 * w) {
            int64_t a = lo, am = lo + w < np ? lo + w : np, b = am, bm = lo + 2 * w < np ? lo + 2 * w : np, o = lo;
            while (a < am && b < bm) tmp[o++] = (e[idx[b]] > e[idx[a]]) ? idx[b++] : idx[a++];
            while (a < am) tmp[o++] = idx[a++];
            while (b < bm) tmp[o++] = idx[b++];
        }
        memcpy(idx, tmp, sizeof(int64_t) * np);
        free(tmp);
    }
    char *sel = (char *)calloc(np, 1);
    for (int64_t k = 0; k < K; ++k) sel[idx[k]] = 1;
    int64_t g = 0, moved = 0;
    for (int64_t p = 0; p < np && moved < K; ++p) {
        if (!sel[p]) continue;
        while (fl[g] == 0) ++g;                             /* the next flagged Gaussian */
        float *q = params + 8 * g;
        q[0] = (float)(p % W) + 0.5f;
        q[1] = (float)(p / W) + 0.5f;
        q[2] = s0; q[3] = 0.0f; q[4] = s0;
        q[5] = target[p] - image[p];
        q[6] = target[np + p] - image[np + p];
        q[7] = target[2 * np + p] - image[2 * np + p];
        ++g;
        ++moved;
    }
    free(e); free(idx); free(sel); free(fl);
    return moved;
}
