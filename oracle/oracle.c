/*
 * oracle.c -- plain fp64 CPU reference for fused RMSNorm / LayerNorm
 * (forward and backward) and interleaved RoPE (forward and inverse).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the package's smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code, header, table or
 * constant with the HIP library.
 *
 * What it computes: the plain definitions, in IEEE double, with sums taken
 * left to right in index order.  The pages this follows claim that their
 * fused kernels change memory traffic, not the mathematics (Helios
 * 性能优化全解析, 内核一 FlashNorm: the row is read once instead of three
 * times; 内核二 FlashRoPE: no intermediate tensors; both kernel files carry a
 * consistency test so that the speed-up does not change results).  So the
 * reference is the definition, not the fused algorithm.
 *
 * Readings taken where the pages are silent:
 *   - eps sits inside the square root, 1/sqrt(ms + eps) and 1/sqrt(var + eps)
 *     (LLM层的优化算子, 编写定制融合算子: the LayerNorm example divides by
 *     sqrt(var + eps));
 *   - divisors are the true row length n; the variance is biased (/n)
 *     (same example);
 *   - the cached per-row statistic is the reciprocal square root;
 *   - a missing weight means 1, a missing bias means 0; the Gemma variant
 *     scales by (1 + w);
 *   - RoPE pairs are interleaved (2i, 2i+1) = (real, imag); the inverse is
 *     the same rotation with sin negated (内核二 FlashRoPE);
 *   - RoPE angles: 1-D, pos * theta^(-2i/D); 3-D, the D/2 pairs are split
 *     into consecutive t / h / w blocks of P_t, P_h, P_w pairs, and pair j of
 *     axis a's block uses pos_a * theta^(-2j/(2 P_a)); tokens are ordered
 *     frame-major, then height, then width;
 *   - the tanh-approximated GeLU uses c = sqrt(2/pi), printed as 0.79788456
 *     in 编写定制融合算子 (the two differ by 1e-9 relative).
 *
 * Inputs are read through a dtype tag (fp64, fp32, bf16 or fp16 bit patterns) and
 * widened exactly to double, so the oracle sees the very bytes the GPU saw.
 * Outputs are always double and are never rounded to the storage dtype.
 *
 * Parallelism: rows are independent, so row loops may run under OpenMP; no
 * sum is split or reordered.  Column sums (dw, dgamma, dbeta) run serially in
 * row order.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F64 0
#define OR_F32 1
#define OR_BF16 2
#define OR_F16 3

/* IEEE binary16 -> double, exactly: 1 sign bit, 5 exponent bits (bias 15),
 * 10 fraction bits; exponent 0 is the subnormal range (fraction * 2^-24),
 * exponent 31 is infinity or NaN. */
static double half_to_double(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

static double ld(const void *p, int dt, int64_t i)
{
    if (dt == OR_F64)
        return ((const double *)p)[i];
    if (dt == OR_F32)
        return (double)((const float *)p)[i];
    if (dt == OR_F16)
        return half_to_double(((const uint16_t *)p)[i]);
    /* bf16: the 16 stored bits are the top half of an IEEE single */
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* The widening above, exposed so that it can be checked on its own. */
void oracle_widen(const void *p, int dt, int64_t count, double *out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = ld(p, dt, i);
}

/* weight as used by the scaling step: w, or 1 + w for the Gemma variant,
 * or 1 when there is no weight */
static double weight(const void *w, int wdt, int gemma, int64_t j)
{
    if (!w)
        return 1.0;
    return gemma ? 1.0 + ld(w, wdt, j) : ld(w, wdt, j);
}

/* ------------------------------------------------------------------ */
/* D1  RMSNorm forward                                                 */
/*   ms_i = (1/n) sum_j x_ij^2 ;  r_i = 1/sqrt(ms_i + eps)              */
/*   y_ij = (x_ij r_i) w'_j ;     inv_rms_i = r_i                      */
/* Helios 性能优化全解析, 内核一 FlashNorm (sum of squares, inverse      */
/* root, multiply by the weight; Gemma offset of 1.0 on the weight).   */
/* ------------------------------------------------------------------ */
void oracle_rmsnorm_fwd(const void *x, int xdt, const void *w, int wdt,
                        int gemma, int64_t rows, int64_t n, double eps,
                        double *y, double *inv_rms)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        double ss = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double v = ld(x, xdt, i * n + j);
            ss += v * v;
        }
        double ms = ss / (double)n;
        double r = 1.0 / sqrt(ms + eps);
        if (inv_rms)
            inv_rms[i] = r;
        if (y)
            for (int64_t j = 0; j < n; ++j) {
                double xhat = ld(x, xdt, i * n + j) * r;
                y[i * n + j] = xhat * weight(w, wdt, gemma, j);
            }
    }
}

/* ------------------------------------------------------------------ */
/* D2  RMSNorm backward (calculus of D1; the pages only say that the   */
/* backward reuses the forward's cached per-row statistic).            */
/*   g_ij = dy_ij w'_j ;  xhat_ij = x_ij r_i                            */
/*   c_i  = (1/n) sum_j g_ij xhat_ij                                    */
/*   dx_ij = r_i (g_ij - xhat_ij c_i)                                   */
/*   dw_j  = sum_i dy_ij xhat_ij      (same with the Gemma offset)      */
/* r_i is recomputed here from x; the GPU's cache is never read.       */
/* ------------------------------------------------------------------ */
void oracle_rmsnorm_bwd(const void *dy, const void *x, int dt, const void *w,
                        int wdt, int gemma, int64_t rows, int64_t n,
                        double eps, double *dx, double *dw)
{
    double *r = (double *)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1));
    oracle_rmsnorm_fwd(x, dt, NULL, 0, 0, rows, n, eps, NULL, r);
    if (dx) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            double c = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                double g = ld(dy, dt, i * n + j) * weight(w, wdt, gemma, j);
                double xhat = ld(x, dt, i * n + j) * r[i];
                c += g * xhat;
            }
            c /= (double)n;
            for (int64_t j = 0; j < n; ++j) {
                double g = ld(dy, dt, i * n + j) * weight(w, wdt, gemma, j);
                double xhat = ld(x, dt, i * n + j) * r[i];
                dx[i * n + j] = r[i] * (g - xhat * c);
            }
        }
    }
    if (dw) {
        for (int64_t j = 0; j < n; ++j)
            dw[j] = 0.0;
        for (int64_t i = 0; i < rows; ++i)
            for (int64_t j = 0; j < n; ++j)
                dw[j] += ld(dy, dt, i * n + j) * (ld(x, dt, i * n + j) * r[i]);
    }
    free(r);
}

/* ------------------------------------------------------------------ */
/* D3  LayerNorm forward                                               */
/*   mu_i = (1/n) sum_j x_ij ;  var_i = (1/n) sum_j (x_ij - mu_i)^2      */
/*   r_i = 1/sqrt(var_i + eps) ;  xhat = (x - mu) r ;  y = xhat g + b    */
/* Helios 性能优化全解析, 内核一 FlashNorm (mean, variance, scale);      */
/* LLM层的优化算子, 编写定制融合算子 (biased variance, eps in the root,  */
/* then weight and bias).                                              */
/* ------------------------------------------------------------------ */
void oracle_layernorm_fwd(const void *x, int xdt, const void *gamma,
                          const void *beta, int wdt, int64_t rows, int64_t n,
                          double eps, double *y, double *mean, double *rstd)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < n; ++j)
            s += ld(x, xdt, i * n + j);
        double mu = s / (double)n;
        double q = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double d = ld(x, xdt, i * n + j) - mu;
            q += d * d;
        }
        double var = q / (double)n;
        double r = 1.0 / sqrt(var + eps);
        if (mean)
            mean[i] = mu;
        if (rstd)
            rstd[i] = r;
        if (y)
            for (int64_t j = 0; j < n; ++j) {
                double xhat = (ld(x, xdt, i * n + j) - mu) * r;
                double g = gamma ? ld(gamma, wdt, j) : 1.0;
                double b = beta ? ld(beta, wdt, j) : 0.0;
                y[i * n + j] = xhat * g + b;
            }
    }
}

/* ------------------------------------------------------------------ */
/* D4  LayerNorm backward (calculus of D3)                             */
/*   g = dy gamma ; a_i = (1/n) sum_j g ; b_i = (1/n) sum_j g xhat       */
/*   dx = r (g - a - xhat b) ; dgamma_j = sum_i dy xhat ;               */
/*   dbeta_j = sum_i dy                                                 */
/* ------------------------------------------------------------------ */
void oracle_layernorm_bwd(const void *dy, const void *x, int dt,
                          const void *gamma, int wdt, int64_t rows, int64_t n,
                          double eps, double *dx, double *dgamma,
                          double *dbeta)
{
    size_t m = (size_t)(rows > 0 ? rows : 1);
    double *mu = (double *)malloc(sizeof(double) * m);
    double *r = (double *)malloc(sizeof(double) * m);
    oracle_layernorm_fwd(x, dt, NULL, NULL, 0, rows, n, eps, NULL, mu, r);
    if (dx) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            double sa = 0.0, sb = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                double g = ld(dy, dt, i * n + j) * (gamma ? ld(gamma, wdt, j) : 1.0);
                double xhat = (ld(x, dt, i * n + j) - mu[i]) * r[i];
                sa += g;
                sb += g * xhat;
            }
            double a = sa / (double)n, b = sb / (double)n;
            for (int64_t j = 0; j < n; ++j) {
                double g = ld(dy, dt, i * n + j) * (gamma ? ld(gamma, wdt, j) : 1.0);
                double xhat = (ld(x, dt, i * n + j) - mu[i]) * r[i];
                dx[i * n + j] = r[i] * (g - a - xhat * b);
            }
        }
    }
    if (dgamma || dbeta) {
        for (int64_t j = 0; j < n; ++j) {
            if (dgamma)
                dgamma[j] = 0.0;
            if (dbeta)
                dbeta[j] = 0.0;
        }
        for (int64_t i = 0; i < rows; ++i)
            for (int64_t j = 0; j < n; ++j) {
                double d = ld(dy, dt, i * n + j);
                if (dgamma)
                    dgamma[j] += d * ((ld(x, dt, i * n + j) - mu[i]) * r[i]);
                if (dbeta)
                    dbeta[j] += d;
            }
    }
    free(mu);
    free(r);
}

/* ------------------------------------------------------------------ */
/* D5  RoPE angles, one row of D/2 angles per token.                   */
/* The pages give no frequency formula; the readings are in the file   */
/* header.  1-D: phi(s, i) = (pos0 + s) * theta^(-2i/D).               */
/* ------------------------------------------------------------------ */
void oracle_rope_angles_1d(int64_t tokens, int64_t head_dim, int64_t pos0,
                           double theta, double *angle /* [tokens][D/2] */)
{
    int64_t half = head_dim / 2;
    for (int64_t s = 0; s < tokens; ++s)
        for (int64_t i = 0; i < half; ++i) {
            double omega = pow(theta, -2.0 * (double)i / (double)head_dim);
            angle[s * half + i] = (double)(pos0 + s) * omega;
        }
}

/* 3-D: token s = (f * H + h) * W + w.  Pairs [0, Pt) follow the frame
 * index f, [Pt, Pt+Ph) the row h, [Pt+Ph, Pt+Ph+Pw) the column w; pair j of
 * an axis with P pairs has frequency theta^(-2j / (2P)). */
void oracle_rope_angles_3d(int64_t frames, int64_t height, int64_t width,
                           int64_t pt, int64_t ph, int64_t pw, double theta,
                           double *angle /* [F*H*W][pt+ph+pw] */)
{
    int64_t half = pt + ph + pw;
    for (int64_t f = 0; f < frames; ++f)
        for (int64_t h = 0; h < height; ++h)
            for (int64_t w = 0; w < width; ++w) {
                int64_t s = (f * height + h) * width + w;
                double *a = angle + s * half;
                for (int64_t j = 0; j < pt; ++j)
                    a[j] = (double)f * pow(theta, -2.0 * (double)j / (double)(2 * pt));
                for (int64_t j = 0; j < ph; ++j)
                    a[pt + j] = (double)h * pow(theta, -2.0 * (double)j / (double)(2 * ph));
                for (int64_t j = 0; j < pw; ++j)
                    a[pt + ph + j] = (double)w * pow(theta, -2.0 * (double)j / (double)(2 * pw));
            }
}

/* ------------------------------------------------------------------ */
/* D6  interleaved RoPE, forward or inverse.                           */
/* Helios 性能优化全解析, 内核二 FlashRoPE: the real part sits at 2i, the */
/* imaginary part at 2i+1, the pair is rotated by the token's angle,   */
/* and the inverse is the same rotation with sin negated.              */
/*   a' = a cos(phi) - b (sigma sin(phi))                              */
/*   b' = a (sigma sin(phi)) + b cos(phi),  sigma = +1 / -1 (inverse)   */
/* x is contiguous [batch][tokens][heads][head_dim]; out likewise.     */
/* ------------------------------------------------------------------ */
void oracle_rope_apply(const void *x, int xdt, int64_t batch, int64_t tokens,
                       int64_t heads, int64_t head_dim,
                       const double *angle /* [tokens][D/2] */, int inverse,
                       double *out)
{
    int64_t half = head_dim / 2;
    double sigma = inverse ? -1.0 : 1.0;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bb = 0; bb < batch; ++bb)
        for (int64_t s = 0; s < tokens; ++s)
            for (int64_t h = 0; h < heads; ++h) {
                int64_t base = ((bb * tokens + s) * heads + h) * head_dim;
                for (int64_t i = 0; i < half; ++i) {
                    double phi = angle[s * half + i];
                    double c = cos(phi), sn = sigma * sin(phi);
                    double a = ld(x, xdt, base + 2 * i);
                    double b = ld(x, xdt, base + 2 * i + 1);
                    out[base + 2 * i] = a * c - b * sn;
                    out[base + 2 * i + 1] = a * sn + b * c;
                }
            }
}

/* ------------------------------------------------------------------ */
/* D7  LayerNorm followed by the tanh-approximated GeLU.               */
/* LLM层的优化算子, 编写定制融合算子: the fused example normalises the  */
/* row, applies weight and bias, then                                  */
/*   gelu(v) = 0.5 v (1 + tanh(c (v + 0.044715 v^3))),                  */
/* with c = sqrt(2/pi) (printed there as 0.79788456).                  */
/* Backward (calculus): with the pre-activation a = xhat gamma + beta  */
/* recomputed from x, dy = dout gelu'(a), then D4 with dy:             */
/*   gelu'(v) = 0.5 (1 + t) + 0.5 v (1 - t^2) c (1 + 3 0.044715 v^2),    */
/*   t = tanh(c (v + 0.044715 v^3)).                                    */
/* ------------------------------------------------------------------ */
static const double GELU_A = 0.044715;

static double gelu_c(void)
{
    const double pi = 3.14159265358979323846;
    return sqrt(2.0 / pi);
}

double oracle_gelu_tanh(double v)
{
    return 0.5 * v * (1.0 + tanh(gelu_c() * (v + GELU_A * v * v * v)));
}

double oracle_gelu_tanh_grad(double v)
{
    double c = gelu_c();
    double t = tanh(c * (v + GELU_A * v * v * v));
    return 0.5 * (1.0 + t) + 0.5 * v * (1.0 - t * t) * c * (1.0 + 3.0 * GELU_A * v * v);
}

void oracle_layernorm_gelu_fwd(const void *x, int xdt, const void *gamma,
                               const void *beta, int wdt, int64_t rows,
                               int64_t n, double eps, double *y,
                               double *mean, double *rstd)
{
    oracle_layernorm_fwd(x, xdt, gamma, beta, wdt, rows, n, eps, y, mean, rstd);
    if (y) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < rows; ++i)
            for (int64_t j = 0; j < n; ++j)
                y[i * n + j] = oracle_gelu_tanh(y[i * n + j]);
    }
}

void oracle_layernorm_gelu_bwd(const void *dout, const void *x, int dt,
                               const void *gamma, const void *beta, int wdt,
                               int64_t rows, int64_t n, double eps,
                               double *dx, double *dgamma, double *dbeta)
{
    size_t m = (size_t)(rows > 0 ? rows : 1);
    double *mu = (double *)malloc(sizeof(double) * m);
    double *r = (double *)malloc(sizeof(double) * m);
    double *dy = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * m);
    oracle_layernorm_fwd(x, dt, NULL, NULL, 0, rows, n, eps, NULL, mu, r);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double xhat = (ld(x, dt, i * n + j) - mu[i]) * r[i];
            double a = xhat * (gamma ? ld(gamma, wdt, j) : 1.0) + (beta ? ld(beta, wdt, j) : 0.0);
            dy[i * n + j] = ld(dout, dt, i * n + j) * oracle_gelu_tanh_grad(a);
        }
    if (dx) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            double sa = 0.0, sb = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                double g = dy[i * n + j] * (gamma ? ld(gamma, wdt, j) : 1.0);
                double xhat = (ld(x, dt, i * n + j) - mu[i]) * r[i];
                sa += g;
                sb += g * xhat;
            }
            double a = sa / (double)n, b = sb / (double)n;
            for (int64_t j = 0; j < n; ++j) {
                double g = dy[i * n + j] * (gamma ? ld(gamma, wdt, j) : 1.0);
                double xhat = (ld(x, dt, i * n + j) - mu[i]) * r[i];
                dx[i * n + j] = r[i] * (g - a - xhat * b);
            }
        }
    }
    if (dgamma || dbeta) {
        for (int64_t j = 0; j < n; ++j) {
            if (dgamma)
                dgamma[j] = 0.0;
            if (dbeta)
                dbeta[j] = 0.0;
        }
        for (int64_t i = 0; i < rows; ++i)
            for (int64_t j = 0; j < n; ++j) {
                double d = dy[i * n + j];
                if (dgamma)
                    dgamma[j] += d * ((ld(x, dt, i * n + j) - mu[i]) * r[i]);
                if (dbeta)
                    dbeta[j] += d;
            }
    }
    free(mu);
    free(r);
    free(dy);
}

/* Threads the OpenMP loops above use (reported with the CPU timing). */
int oracle_max_threads(void) { return omp_get_max_threads(); }
