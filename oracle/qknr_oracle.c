/*
 * qknr_oracle.c -- plain fp64 CPU oracle for per-head QK-Norm followed by RoPE.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or constant generator with
 * the HIP library, and it does not include the library's header.
 *
 * What it computes, per row (one token, one head; a row is a head_dim vector x):
 *
 *   RMSNorm with a static weight and a per-row inverse-RMS scalar.  The
 *   decomposition "static affine weight times one dynamic inverse-RMS scalar per
 *   token and head group" is the one stated in the abstract of "QK-Normed MLA:
 *   QK normalization without full key caching".  It is applied per head, as in
 *   the "per-head QK normalization" of the QG-MIL abstract and the "grouped-query
 *   attention with per-head QK-normalization" of the HobbyLM abstract:
 *       ms  = (1/D) * sum_j x_j^2
 *       r   = 1 / sqrt(ms + eps)
 *       n_j = w_j * x_j * r
 *
 *   then rotary position embedding (RoPE, as named in the abstract of "Rope to
 *   Nope and Back Again: A New Hybrid Attention Strategy") on the first R
 *   channels only ("Fractional Rotation, Full Potential? Investigating
 *   Performance and Convergence of Partial RoPE", abstract: rotation applied to
 *   a subset of the hidden dimensions).  With h = R/2 and the half-split pairing
 *   (i, i+h):
 *       theta_i = theta^(-2i/R)                       (fp64)
 *       phi_i   = pos * theta_i                       (fp64)
 *       c_i     = fp32(cos(phi_i)), s_i = fp32(sin(phi_i))
 *       y_i     = n_i c_i - n_{i+h} s_i
 *       y_{i+h} = n_{i+h} c_i + n_i s_i
 *       y_j     = n_j                                 for R <= j < D
 *
 *   The norm-then-RoPE order is the one in which the fused "QK-RoPE" prologue of
 *   "Chronicals: A High-Performance Framework for LLM Fine-Tuning with 3.51x
 *   Speedup over Unsloth" (abstract, contribution (1)) sits: the normalised
 *   query/key vectors are what gets rotated.
 *
 * Backward: the gradient of  L = <dy, y>  with respect to x and w:
 *       g_i     = dy_i c_i + dy_{i+h} s_i ;  g_{i+h} = dy_{i+h} c_i - dy_i s_i
 *       g_j     = dy_j                                for j >= R
 *       xh_j    = x_j r ;  u_j = w_j g_j
 *       dx_j    = r * (u_j - xh_j * (1/D) sum_k u_k xh_k)
 *       dw_j   += g_j * xh_j                          (sum over every row)
 *
 * Variants (flags and optional arguments of oracle_fwd_ex / oracle_bwd_ex):
 *   ORACLE_INTERLEAVED    pairs (2i, 2i+1) instead of (i, i+h):
 *                           y_2i = n_2i c_i - n_2i+1 s_i ; y_2i+1 = n_2i+1 c_i + n_2i s_i
 *   ORACLE_FREQ_HEAD_DIM  theta_i = theta^(-2i/D) instead of theta^(-2i/R)
 *   ORACLE_LAYERNORM      QK-LayerNorm ("Nyonic Technical Report", abstract: RoPE
 *                         with QK-LayerNorm): the row mean m is subtracted first,
 *                           m = (1/D) sum_j x_j ; r = 1/sqrt((1/D) sum_j (x_j - m)^2 + eps)
 *                           n_j = w_j (x_j - m) r
 *                         backward: xh = (x - m) r ; u = w g ;
 *                           dx = r (u - mean(u) - xh * mean(u xh))
 *   bias b ([D], optional) n_j += b_j before the rotation; db += g (summed over rows)
 *   frequency table       theta_i given by the caller (RoPE "extensions" change the
 *                         per-pair frequencies: Rope to Nope and Back Again,
 *                         abstract), and an attention factor a multiplying cos and
 *                         sin before their fp32 rounding: c_i = fp32(a cos phi_i)
 * A weight-free norm (parameter-free QK norm) is the weight vector of ones,
 * which the caller passes.
 *
 * Norm groups and per-head weights (oracle_fwd_gen / oracle_bwd_gen):
 *   g consecutive heads of one token share the statistics: the mean and the
 *   inverse RMS run over the g*D values of the group (QK-Normed MLA abstract:
 *   one dynamic inverse-RMS scalar per token and head group; SwiftQK abstract:
 *   layerwise QK-Norm, normalised over the full hidden vector, is the group of
 *   every head).  g = 1 is the per-head norm above.  With ORACLE_HEAD_WEIGHTS
 *   the weights (and biases, and their gradients) are [H, D], one vector per
 *   head, instead of one [D] vector shared by the heads.  The backward of a
 *   group is the per-row formula with its means taken over the group:
 *       dx = r (u - mean_grp(u) [LayerNorm only] - xh * mean_grp(u xh))
 *   RoPE still rotates each head's first R channels on its own.
 *
 * Everything is fp64 scalar loops, one row at a time, in the order written
 * above.  Build with -O2 -ffp-contract=off and no fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAX_D 1024
#define ORACLE_INTERLEAVED 1
#define ORACLE_FREQ_HEAD_DIM 2
#define ORACLE_LAYERNORM 4
#define ORACLE_HEAD_WEIGHTS 8

/* theta_i = theta^(-2i/denom), fp64.  RoPE frequencies (Rope to Nope and
 * Back Again, abstract: RoPE of Su et al.); the exponent's denominator is the
 * rotated width R for partial rotation (Fractional Rotation ... Partial RoPE,
 * abstract), or D with ORACLE_FREQ_HEAD_DIM. */
static double oracle_inv_freq(double theta, int i, int denom)
{
    return pow(theta, -2.0 * (double)i / (double)denom);
}

/* a*cos and a*sin of pos*theta_i, i < R/2, computed in fp64 and rounded to
 * fp32; theta_i from the table `freq` when given, else from the formula. */
void oracle_rope_cos_sin_gen(int64_t pos, double theta, int R, int denom, const double *freq,
                             double attn, double *c, double *s)
{
    int h = R / 2;
    for (int i = 0; i < h; ++i) {
        double f = freq ? freq[i] : oracle_inv_freq(theta, i, denom);
        double phi = (double)pos * f;
        c[i] = (double)(float)(attn * cos(phi));
        s[i] = (double)(float)(attn * sin(phi));
    }
}

void oracle_rope_cos_sin_ex(int64_t pos, double theta, int R, int denom, double *c, double *s)
{
    oracle_rope_cos_sin_gen(pos, theta, R, denom, 0, 1.0, c, s);
}

void oracle_rope_cos_sin(int64_t pos, double theta, int R, double *c, double *s)
{
    oracle_rope_cos_sin_ex(pos, theta, R, R, c, s);
}

/* Rotation of the first R channels by +phi_i: half-split pairs (i, i+h). */
static void oracle_rotate_half_split(const double *n, const double *c, const double *s, int R,
                                     double *y)
{
    int h = R / 2;
    for (int i = 0; i < h; ++i) {
        y[i] = n[i] * c[i] - n[i + h] * s[i];
        y[i + h] = n[i + h] * c[i] + n[i] * s[i];
    }
}

/* Rotation of the first R channels by +phi_i: interleaved pairs (2i, 2i+1). */
static void oracle_rotate_interleaved(const double *n, const double *c, const double *s, int R,
                                      double *y)
{
    int h = R / 2;
    for (int i = 0; i < h; ++i) {
        y[2 * i] = n[2 * i] * c[i] - n[2 * i + 1] * s[i];
        y[2 * i + 1] = n[2 * i + 1] * c[i] + n[2 * i] * s[i];
    }
}

/* Transposes of the two rotations (rotation by -phi_i), for the backward.
 * The rotation is orthogonal up to the fp32 rounding of c, s. */
static void oracle_rotate_half_split_t(const double *dy, const double *c, const double *s, int R,
                                       double *g)
{
    int h = R / 2;
    for (int i = 0; i < h; ++i) {
        g[i] = dy[i] * c[i] + dy[i + h] * s[i];
        g[i + h] = dy[i + h] * c[i] - dy[i] * s[i];
    }
}

static void oracle_rotate_interleaved_t(const double *dy, const double *c, const double *s, int R,
                                        double *g)
{
    int h = R / 2;
    for (int i = 0; i < h; ++i) {
        g[2 * i] = dy[2 * i] * c[i] + dy[2 * i + 1] * s[i];
        g[2 * i + 1] = dy[2 * i + 1] * c[i] - dy[2 * i] * s[i];
    }
}

/* Statistics of one row: the centre m (0 for RMSNorm, the row mean for
 * LayerNorm) and the inverse scale r = 1/sqrt(mean((x - m)^2) + eps) (QK-Normed
 * MLA abstract: one dynamic inverse-RMS scalar per row). */
static double oracle_row_stats(const double *x, int D, double eps, int flags, double *m_out)
{
    double m = 0.0;
    if (flags & ORACLE_LAYERNORM) {
        double sx = 0.0;
        for (int j = 0; j < D; ++j)
            sx += x[j];
        m = sx / (double)D;
    }
    double ss = 0.0;
    for (int j = 0; j < D; ++j)
        ss += (x[j] - m) * (x[j] - m);
    double ms = ss / (double)D;
    *m_out = m;
    return 1.0 / sqrt(ms + eps);
}

static void oracle_fwd_row(const double *x, const double *w, const double *b, const double *c,
                           const double *s, int D, int R, double eps, int flags, double *y)
{
    double n[ORACLE_MAX_D];
    double m;
    double r = oracle_row_stats(x, D, eps, flags, &m);
    for (int j = 0; j < D; ++j)
        n[j] = w[j] * (x[j] - m) * r;
    if (b)
        for (int j = 0; j < D; ++j)
            n[j] += b[j];
    if (flags & ORACLE_INTERLEAVED)
        oracle_rotate_interleaved(n, c, s, R, y);
    else
        oracle_rotate_half_split(n, c, s, R, y);
    for (int j = R; j < D; ++j)
        y[j] = n[j];
}

static void oracle_bwd_row(const double *x, const double *w, const double *dy,
                           const double *c, const double *s, int D, int R,
                           double eps, int flags, double *dx, double *dw, double *db)
{
    double g[ORACLE_MAX_D], xh[ORACLE_MAX_D], u[ORACLE_MAX_D];
    double m;
    double r = oracle_row_stats(x, D, eps, flags, &m);
    /* g = R^T dy */
    if (flags & ORACLE_INTERLEAVED)
        oracle_rotate_interleaved_t(dy, c, s, R, g);
    else
        oracle_rotate_half_split_t(dy, c, s, R, g);
    for (int j = R; j < D; ++j)
        g[j] = dy[j];
    double dot = 0.0, su = 0.0;
    for (int j = 0; j < D; ++j) {
        xh[j] = (x[j] - m) * r;
        u[j] = w[j] * g[j];
        dot += u[j] * xh[j];
        su += u[j];
    }
    double mean = dot / (double)D;
    /* LayerNorm: the centring adds the -mean(u) term */
    double mu = (flags & ORACLE_LAYERNORM) ? su / (double)D : 0.0;
    for (int j = 0; j < D; ++j) {
        dx[j] = r * (u[j] - mu - xh[j] * mean);
        dw[j] += g[j] * xh[j];
    }
    if (db)
        for (int j = 0; j < D; ++j)
            db[j] += g[j];
}

static int oracle_check(int D, int R, int64_t tokens, int hq, int hkv)
{
    if (D <= 0 || D > ORACLE_MAX_D || R < 0 || R > D || (R % 2) != 0)
        return 1;
    if (tokens < 0 || hq < 0 || hkv < 0)
        return 1;
    return 0;
}

/*
 * Forward over a token range.  q: [tokens, hq, D], k: [tokens, hkv, D], row
 * major; wq, wk: [D]; bq, bk: [D] or NULL; pos: [tokens]; flags: ORACLE_*
 * above; freq: R/2 frequencies or NULL; attn: factor on cos and sin (1 = none).
 * Outputs have the shapes of q and k.  Returns 0 on success, 1 on bad sizes.
 */
int oracle_fwd_ex(const double *q, const double *k, const double *wq,
                  const double *wk, const double *bq, const double *bk,
                  const int32_t *pos, int64_t tokens, int hq, int hkv, int D, int R,
                  double eps, double theta, int flags, const double *freq, double attn,
                  double *yq, double *yk)
{
    if (oracle_check(D, R, tokens, hq, hkv))
        return 1;
    int denom = (flags & ORACLE_FREQ_HEAD_DIM) ? D : R;
    double c[ORACLE_MAX_D / 2 + 1], s[ORACLE_MAX_D / 2 + 1];
    for (int64_t t = 0; t < tokens; ++t) {
        oracle_rope_cos_sin_gen(pos[t], theta, R, denom, freq, attn, c, s);
        for (int hd = 0; hd < hq; ++hd) {
            int64_t off = (t * hq + hd) * (int64_t)D;
            oracle_fwd_row(q + off, wq, bq, c, s, D, R, eps, flags, yq + off);
        }
        for (int hd = 0; hd < hkv; ++hd) {
            int64_t off = (t * hkv + hd) * (int64_t)D;
            oracle_fwd_row(k + off, wk, bk, c, s, D, R, eps, flags, yk + off);
        }
    }
    return 0;
}

int oracle_fwd(const double *q, const double *k, const double *wq,
               const double *wk, const int32_t *pos, int64_t tokens, int hq,
               int hkv, int D, int R, double eps, double theta, double *yq,
               double *yk)
{
    return oracle_fwd_ex(q, k, wq, wk, 0, 0, pos, tokens, hq, hkv, D, R, eps, theta, 0, 0, 1.0,
                         yq, yk);
}

/*
 * Backward over a token range.  dyq/dyk are the upstream gradients of the
 * forward outputs.  dwq/dwk ([D] each) and, when not NULL, dbq/dbk are
 * ACCUMULATED into (the caller zeroes them), so that a caller may split the
 * rows into ranges and add the ranges' sums.  The biases do not enter dq, dk.
 */
int oracle_bwd_ex(const double *q, const double *k, const double *wq,
                  const double *wk, const int32_t *pos, int64_t tokens, int hq,
                  int hkv, int D, int R, double eps, double theta, int flags,
                  const double *freq, double attn, const double *dyq, const double *dyk,
                  double *dq, double *dk, double *dwq, double *dwk, double *dbq, double *dbk)
{
    if (oracle_check(D, R, tokens, hq, hkv))
        return 1;
    int denom = (flags & ORACLE_FREQ_HEAD_DIM) ? D : R;
    double c[ORACLE_MAX_D / 2 + 1], s[ORACLE_MAX_D / 2 + 1];
    for (int64_t t = 0; t < tokens; ++t) {
        oracle_rope_cos_sin_gen(pos[t], theta, R, denom, freq, attn, c, s);
        for (int hd = 0; hd < hq; ++hd) {
            int64_t off = (t * hq + hd) * (int64_t)D;
            oracle_bwd_row(q + off, wq, dyq + off, c, s, D, R, eps, flags, dq + off, dwq, dbq);
        }
        for (int hd = 0; hd < hkv; ++hd) {
            int64_t off = (t * hkv + hd) * (int64_t)D;
            oracle_bwd_row(k + off, wk, dyk + off, c, s, D, R, eps, flags, dk + off, dwk, dbk);
        }
    }
    return 0;
}

int oracle_bwd(const double *q, const double *k, const double *wq,
               const double *wk, const int32_t *pos, int64_t tokens, int hq,
               int hkv, int D, int R, double eps, double theta,
               const double *dyq, const double *dyk, double *dq, double *dk,
               double *dwq, double *dwk)
{
    return oracle_bwd_ex(q, k, wq, wk, pos, tokens, hq, hkv, D, R, eps, theta, 0, 0, 1.0, dyq,
                         dyk, dq, dk, dwq, dwk, 0, 0);
}

/* ---- norm groups and per-head weights --------------------------------------- */

/* Forward of one norm group: g heads of one token, x holding their g*D values.
 * w and b point at the weight / bias of the group's first head; wstride is 0
 * (one [D] vector for every head) or D (per-head [H, D] vectors).  n is
 * scratch of g*D values. */
static void oracle_fwd_group(const double *x, const double *w, const double *b, int wstride,
                             const double *c, const double *s, int g, int D, int R, double eps,
                             int flags, double *n, double *y)
{
    double m;
    double r = oracle_row_stats(x, g * D, eps, flags, &m);
    for (int hd = 0; hd < g; ++hd)
        for (int j = 0; j < D; ++j) {
            double v = w[hd * wstride + j] * (x[hd * D + j] - m) * r;
            if (b)
                v += b[hd * wstride + j];
            n[hd * D + j] = v;
        }
    for (int hd = 0; hd < g; ++hd) {
        const double *nh = n + hd * D;
        double *yh = y + hd * D;
        if (flags & ORACLE_INTERLEAVED)
            oracle_rotate_interleaved(nh, c, s, R, yh);
        else
            oracle_rotate_half_split(nh, c, s, R, yh);
        for (int j = R; j < D; ++j)
            yh[j] = nh[j];
    }
}

/* Backward of one norm group; dw / db (NULL: not wanted) point at the
 * gradient vector of the group's first head, strided like w.  gg, xh, u are
 * scratch of g*D values. */
static void oracle_bwd_group(const double *x, const double *w, int wstride, const double *dy,
                             const double *c, const double *s, int g, int D, int R, double eps,
                             int flags, double *gg, double *xh, double *u, double *dx,
                             double *dw, double *db)
{
    int L = g * D;
    double m;
    double r = oracle_row_stats(x, L, eps, flags, &m);
    for (int hd = 0; hd < g; ++hd) {
        const double *dyh = dy + hd * D;
        double *gh = gg + hd * D;
        if (flags & ORACLE_INTERLEAVED)
            oracle_rotate_interleaved_t(dyh, c, s, R, gh);
        else
            oracle_rotate_half_split_t(dyh, c, s, R, gh);
        for (int j = R; j < D; ++j)
            gh[j] = dyh[j];
    }
    double dot = 0.0, su = 0.0;
    for (int hd = 0; hd < g; ++hd)
        for (int j = 0; j < D; ++j) {
            int e = hd * D + j;
            xh[e] = (x[e] - m) * r;
            u[e] = w[hd * wstride + j] * gg[e];
            dot += u[e] * xh[e];
            su += u[e];
        }
    double mean = dot / (double)L;
    double mu = (flags & ORACLE_LAYERNORM) ? su / (double)L : 0.0;
    for (int e = 0; e < L; ++e)
        dx[e] = r * (u[e] - mu - xh[e] * mean);
    for (int hd = 0; hd < g; ++hd)
        for (int j = 0; j < D; ++j) {
            int e = hd * D + j;
            if (dw)
                dw[hd * wstride + j] += gg[e] * xh[e];
            if (db)
                db[hd * wstride + j] += gg[e];
        }
}

static int oracle_check_groups(int hq, int hkv, int gq, int gk)
{
    return gq < 1 || gk < 1 || (hq > 0 && hq % gq != 0) || (hkv > 0 && hkv % gk != 0);
}

/*
 * Forward with norm groups: gq heads of q (gk of k) share one inverse RMS;
 * with ORACLE_HEAD_WEIGHTS in flags wq, bq are [hq, D] and wk, bk [hkv, D],
 * else [D].  Other arguments as oracle_fwd_ex.  Returns 0, or 1 on bad sizes
 * (including a group size that does not divide the head count) or when the
 * scratch cannot be allocated.
 */
int oracle_fwd_gen(const double *q, const double *k, const double *wq,
                   const double *wk, const double *bq, const double *bk,
                   const int32_t *pos, int64_t tokens, int hq, int hkv, int D, int R,
                   double eps, double theta, int flags, const double *freq, double attn,
                   int gq, int gk, double *yq, double *yk)
{
    if (oracle_check(D, R, tokens, hq, hkv) || oracle_check_groups(hq, hkv, gq, gk))
        return 1;
    int denom = (flags & ORACLE_FREQ_HEAD_DIM) ? D : R;
    int ws = (flags & ORACLE_HEAD_WEIGHTS) ? D : 0;
    int gmax = gq > gk ? gq : gk;
    double *n = (double *)malloc(sizeof(double) * (size_t)gmax * (size_t)D);
    if (!n)
        return 1;
    double c[ORACLE_MAX_D / 2 + 1], s[ORACLE_MAX_D / 2 + 1];
    for (int64_t t = 0; t < tokens; ++t) {
        oracle_rope_cos_sin_gen(pos[t], theta, R, denom, freq, attn, c, s);
        for (int h0 = 0; h0 < hq; h0 += gq) {
            int64_t off = (t * hq + h0) * (int64_t)D;
            oracle_fwd_group(q + off, wq + h0 * ws, bq ? bq + h0 * ws : 0, ws, c, s, gq, D, R, eps,
                             flags, n, yq + off);
        }
        for (int h0 = 0; h0 < hkv; h0 += gk) {
            int64_t off = (t * hkv + h0) * (int64_t)D;
            oracle_fwd_group(k + off, wk + h0 * ws, bk ? bk + h0 * ws : 0, ws, c, s, gk, D, R, eps,
                             flags, n, yk + off);
        }
    }
    free(n);
    return 0;
}

/*
 * Backward with norm groups; dwq/dwk (and dbq/dbk when not NULL) have the
 * weights' shapes and are ACCUMULATED into, as in oracle_bwd_ex.
 */
int oracle_bwd_gen(const double *q, const double *k, const double *wq,
                   const double *wk, const int32_t *pos, int64_t tokens, int hq,
                   int hkv, int D, int R, double eps, double theta, int flags,
                   const double *freq, double attn, int gq, int gk, const double *dyq,
                   const double *dyk, double *dq, double *dk, double *dwq, double *dwk,
                   double *dbq, double *dbk)
{
    if (oracle_check(D, R, tokens, hq, hkv) || oracle_check_groups(hq, hkv, gq, gk))
        return 1;
    int denom = (flags & ORACLE_FREQ_HEAD_DIM) ? D : R;
    int ws = (flags & ORACLE_HEAD_WEIGHTS) ? D : 0;
    int gmax = gq > gk ? gq : gk;
    size_t L = (size_t)gmax * (size_t)D;
    double *scratch = (double *)malloc(sizeof(double) * 3 * L);
    if (!scratch)
        return 1;
    double c[ORACLE_MAX_D / 2 + 1], s[ORACLE_MAX_D / 2 + 1];
    for (int64_t t = 0; t < tokens; ++t) {
        oracle_rope_cos_sin_gen(pos[t], theta, R, denom, freq, attn, c, s);
        for (int h0 = 0; h0 < hq; h0 += gq) {
            int64_t off = (t * hq + h0) * (int64_t)D;
            oracle_bwd_group(q + off, wq + h0 * ws, ws, dyq + off, c, s, gq, D, R, eps, flags,
                             scratch, scratch + L, scratch + 2 * L, dq + off, dwq + h0 * ws,
                             dbq ? dbq + h0 * ws : 0);
        }
        for (int h0 = 0; h0 < hkv; h0 += gk) {
            int64_t off = (t * hkv + h0) * (int64_t)D;
            oracle_bwd_group(k + off, wk + h0 * ws, ws, dyk + off, c, s, gk, D, R, eps, flags,
                             scratch, scratch + L, scratch + 2 * L, dk + off, dwk + h0 * ws,
                             dbk ? dbk + h0 * ws : 0);
        }
    }
    free(scratch);
    return 0;
}

/*
 * Round fp64 values to bfloat16 (1 sign, 8 exponent, 7 stored significand
 * bits) in ONE step, round-to-nearest with ties to even, and return the bit
 * patterns.  bf16 has the exponent range of fp32 and 8 significand bits, so a
 * finite value is rounded to a multiple of its quantum 2^(e-7) (e = floor(log2
 * |v|), clamped below at -126 for subnormals); values that round to 2^128 or
 * beyond become infinity.  NaN maps to the quiet NaN 0x7fc0 with the input's
 * sign.
 */
void oracle_round_bf16(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        double x = v[i];
        uint16_t sign = signbit(x) ? 0x8000u : 0u;
        if (isnan(x)) {
            out[i] = (uint16_t)(sign | 0x7fc0u);
            continue;
        }
        double a = fabs(x);
        if (isinf(a)) {
            out[i] = (uint16_t)(sign | 0x7f80u);
            continue;
        }
        if (a == 0.0) {
            out[i] = sign;
            continue;
        }
        int e;
        (void)frexp(a, &e);       /* a = m * 2^e, m in [0.5, 1) */
        int ex = e - 1;           /* a in [2^ex, 2^(ex+1)) */
        if (ex < -126)
            ex = -126;            /* subnormal range: fixed quantum 2^-133 */
        double quantum = ldexp(1.0, ex - 7);
        double m = nearbyint(a / quantum); /* a/quantum is exact: power of two */
        double r = m * quantum;
        if (r >= ldexp(1.0, 128)) {
            out[i] = (uint16_t)(sign | 0x7f80u);
            continue;
        }
        /* r is a bf16 value; it is exactly representable in fp32. */
        float f = (float)r;
        uint32_t bits;
        memcpy(&bits, &f, sizeof bits);
        out[i] = (uint16_t)(sign | (bits >> 16));
    }
}

/* ---- Best-Fit-Decreasing sequence packing ----------------------------------
 *
 * Packing of documents into buffers of `capacity` tokens with Best-Fit
 * Decreasing ("Chronicals: A High-Performance Framework for LLM Fine-Tuning
 * with 3.51x Speedup over Unsloth", abstract, contribution (4): BFD sequence
 * packing removes padding).  The pages fix no tie-breaks; this oracle takes:
 *   - documents in order of length, longest first, equal lengths in input
 *     order (a stable sort);
 *   - each document goes into the open bin with the smallest remaining
 *     capacity among those it fits in, the lowest bin index among equals;
 *     otherwise it opens a new bin (bins are numbered in opening order);
 *   - bin b occupies tokens [b * capacity, (b + 1) * capacity) of the packed
 *     buffers; its documents follow each other in placement order, and the
 *     rest of the bin, if any, is one filler segment;
 *   - position ids count 0, 1, ... from the start of every segment (document
 *     or filler); cu_seqlens lists the start of every segment in token order,
 *     then the end of the last bin.
 * Returns 0, 1 when more than max_bins bins would be needed (outputs then
 * undefined), 2 when a length lies outside [1, capacity].
 * doc_start[i] is document i's first token; counts = {bins, segments}.
 */
int oracle_bfd_pack(const int32_t *len, int n, int capacity, int max_bins, int32_t *doc_start,
                    int32_t *pos, int32_t *cu, int32_t *counts)
{
    for (int i = 0; i < n; ++i)
        if (len[i] < 1 || len[i] > capacity)
            return 2;
    int *order = (int *)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    int *fill = (int *)calloc((size_t)(max_bins > 0 ? max_bins : 1), sizeof(int));
    int *ndoc = (int *)calloc((size_t)(max_bins > 0 ? max_bins : 1), sizeof(int));
    int *rank = (int *)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    if (!order || !fill || !ndoc || !rank) {
        free(order); free(fill); free(ndoc); free(rank);
        return 1;
    }
    /* stable insertion sort by length, longest first */
    for (int i = 0; i < n; ++i) {
        int j = i;
        while (j > 0 && len[order[j - 1]] < len[i]) {
            order[j] = order[j - 1];
            --j;
        }
        order[j] = i;
    }
    int nb = 0, st = 0;
    for (int r = 0; r < n && st == 0; ++r) {
        int i = order[r], L = len[i], best = -1;
        for (int b = 0; b < nb; ++b)
            if (capacity - fill[b] >= L && (best < 0 || fill[b] > fill[best]))
                best = b;  /* most filled = smallest remaining; strict > keeps the lowest index */
        if (best < 0) {
            if (nb == max_bins) {
                st = 1;
                break;
            }
            best = nb++;
        }
        doc_start[i] = best * capacity + fill[best];
        rank[i] = ndoc[best]++;
        fill[best] += L;
    }
    if (st == 0) {
        /* segment index of the first segment of each bin */
        int seg = 0;
        for (int b = 0; b < nb; ++b) {
            int first = seg;
            seg += ndoc[b] + (fill[b] < capacity ? 1 : 0);
            ndoc[b] = first;  /* reused: first segment of bin b */
        }
        for (int i = 0; i < n; ++i) {
            int b = doc_start[i] / capacity;
            cu[ndoc[b] + rank[i]] = doc_start[i];
            for (int t = 0; t < len[i]; ++t)
                pos[doc_start[i] + t] = t;
        }
        for (int b = 0; b < nb; ++b)
            if (fill[b] < capacity) {
                int nd = 0;
                for (int i = 0; i < n; ++i)
                    if (doc_start[i] / capacity == b)
                        ++nd;
                cu[ndoc[b] + nd] = b * capacity + fill[b];
                for (int t = 0; t < capacity - fill[b]; ++t)
                    pos[b * capacity + fill[b] + t] = t;
            }
        cu[seg] = nb * capacity;
        counts[0] = nb;
        counts[1] = seg;
    }
    free(order); free(fill); free(ndoc); free(rank);
    return st;
}
