/*
 * oracle.c -- plain, slow CPU oracle for the resident image-VAE decoder's
 * conv path. TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the HIP library never does, and the
 * two share no code.
 *
 * Everything is float64, NCHW, direct loops. Each function is the plain
 * definition of one step of the decoder as the source pages state it:
 *
 *   page "cortiq-engine 0.8.3, src/gpu_wgpu/qi21_vae.rs" (the resident
 *   decoder): module doc (NHWC implicit-GEMM convs, nearest-2x folded into
 *   the gather, f16 conv inputs, f32 accumulation), the RMSN_SRC kernel
 *   (RMS_norm), the `guard` function (range-guarded casts);
 *
 *   page "cortiq-engine 0.7.6, src/vae.rs" (the CPU NCHW decoder):
 *   `Conv2d::apply` (stride 1, pad k/2), `upsample2x`, `silu`.
 *
 * The only place f16 appears is `orc_f16_round`, which the caller applies at
 * the sites where the path stores f16.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------
 * IEEE-754 binary16 rounding, round-to-nearest-even, written from the
 * format's definition: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits; normal numbers (1.f) * 2^e with e in [-14, 15], subnormals
 * (0.f) * 2^-14; largest finite 65504. The pages store f16 through
 * `pack2x16float` (RMSN_SRC, CAST_SRC) without naming a rounding mode; the
 * reading taken is the IEEE default, round to nearest with ties to even.
 * Overflow gives +-inf (the pages report NaN images when the unguarded
 * stream passes the f16 range, see `guard`).
 * ------------------------------------------------------------------------ */
static double rne_integer(double t) /* t >= 0, |t| < 2^52 */
{
    double r = floor(t);
    double d = t - r; /* exact */
    if (d > 0.5) return r + 1.0;
    if (d < 0.5) return r;
    /* a tie: keep the even neighbour */
    return (fmod(r, 2.0) == 0.0) ? r : r + 1.0;
}

double orc_f16_round(double v)
{
    if (isnan(v)) return v;
    if (isinf(v)) return v;
    if (v == 0.0) return v; /* keeps the sign of zero */
    double a = fabs(v);
    int e2;
    frexp(a, &e2);      /* a = m * 2^e2, m in [0.5, 1) */
    int e = e2 - 1;     /* a in [2^e, 2^(e+1)) */
    if (e < -14) e = -14; /* subnormal range shares the quantum 2^-24 */
    double q = ldexp(1.0, e - 10); /* spacing of binary16 values here */
    double r = rne_integer(a / q) * q; /* a / q is exact (power of two) */
    if (r > 65504.0) r = INFINITY;
    return (v < 0) ? -r : r;
}

void orc_f16_round_n(const double *x, double *y, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = orc_f16_round(x[i]);
}

/* ------------------------------------------------------------------------
 * 2-D convolution, stride 1, zero padding k/2, square k x k kernel
 * (page vae.rs, `Conv2d::apply`: out[o][y][x] = b[o] +
 * sum_{i,ky,kx} w[o][i][ky][kx] * x[i][y+ky-k/2][x+kx-k/2], zero outside).
 * x: [ci][h][w], wt: [co][ci][k][k], bias: [co] or NULL, y: [co][h][w].
 * The bias is added after the weighted sum.
 * ------------------------------------------------------------------------ */
void orc_conv2d(const double *x, int ci, int h, int w, const double *wt, int co, int k,
                const double *bias, double *y)
{
    const int pad = k / 2;
#pragma omp parallel for collapse(2) schedule(static)
    for (int o = 0; o < co; ++o) {
        for (int r = 0; r < h; ++r) {
            double *yr = y + ((int64_t)o * h + r) * w;
            for (int c = 0; c < w; ++c) yr[c] = 0.0;
            for (int i = 0; i < ci; ++i) {
                for (int ky = 0; ky < k; ++ky) {
                    const int sy = r + ky - pad;
                    if (sy < 0 || sy >= h) continue;
                    const double *xr = x + ((int64_t)i * h + sy) * w;
                    for (int kx = 0; kx < k; ++kx) {
                        const double wv = wt[(((int64_t)o * ci + i) * k + ky) * k + kx];
                        const int dx = kx - pad;
                        const int c0 = dx < 0 ? -dx : 0;
                        const int c1 = dx > 0 ? w - dx : w;
                        for (int c = c0; c < c1; ++c) yr[c] += wv * xr[c + dx];
                    }
                }
            }
            if (bias)
                for (int c = 0; c < w; ++c) yr[c] += bias[o];
        }
    }
}

/* ------------------------------------------------------------------------
 * Nearest-neighbour 2x upsample (page vae.rs, `upsample2x`):
 * dst[c][y][x] = src[c][y/2][x/2]. x: [c][h][w] -> y: [c][2h][2w].
 * ------------------------------------------------------------------------ */
void orc_upsample2x(const double *x, int c, int h, int w, double *y)
{
#pragma omp parallel for schedule(static)
    for (int ch = 0; ch < c; ++ch)
        for (int r = 0; r < 2 * h; ++r)
            for (int q = 0; q < 2 * w; ++q)
                y[((int64_t)ch * 2 * h + r) * 2 * w + q] = x[((int64_t)ch * h + r / 2) * w + q / 2];
}

/* ------------------------------------------------------------------------
 * The 3x3 conv of the nearest-2x upsampled image with the upsample folded
 * into the gather (page qi21_vae.rs, module doc: the upsample is folded
 * into the A-tile gather; `Rec::conv_s` with `up`). Output [co][2h][2w];
 * tap (ky,kx) at output (r,c) reads x[i][(r+ky-1)/2][(c+kx-1)/2] when
 * 0 <= r+ky-1 < 2h and 0 <= c+kx-1 < 2w, else 0: the zero padding lies in
 * upsampled coordinates, as "upsample, then conv" (page vae.rs,
 * `VaeDecoder::decode`) implies. Summation order equals orc_conv2d run on
 * orc_upsample2x's output, so the two agree bit for bit.
 * ------------------------------------------------------------------------ */
void orc_conv2d_up2(const double *x, int ci, int h, int w, const double *wt, int co,
                    const double *bias, double *y)
{
    const int H2 = 2 * h, W2 = 2 * w;
#pragma omp parallel for collapse(2) schedule(static)
    for (int o = 0; o < co; ++o) {
        for (int r = 0; r < H2; ++r) {
            double *yr = y + ((int64_t)o * H2 + r) * W2;
            for (int c = 0; c < W2; ++c) yr[c] = 0.0;
            for (int i = 0; i < ci; ++i) {
                for (int ky = 0; ky < 3; ++ky) {
                    const int uy = r + ky - 1;
                    if (uy < 0 || uy >= H2) continue;
                    const double *xr = x + ((int64_t)i * h + uy / 2) * w;
                    for (int kx = 0; kx < 3; ++kx) {
                        const double wv = wt[(((int64_t)o * ci + i) * 3 + ky) * 3 + kx];
                        const int dx = kx - 1;
                        const int c0 = dx < 0 ? -dx : 0;
                        const int c1 = dx > 0 ? W2 - dx : W2;
                        for (int c = c0; c < c1; ++c) yr[c] += wv * xr[(c + dx) / 2];
                    }
                }
            }
            if (bias)
                for (int c = 0; c < W2; ++c) yr[c] += bias[o];
        }
    }
}

/* ------------------------------------------------------------------------
 * The same convolutions at chosen output pixels only, for outputs too large
 * to compute whole. pix[j] = r * W_out + c in output coordinates; up2 = 1
 * selects the folded-upsample gather (then W_out = 2w). y: [npix][co].
 * Each value is the definition above written out for one output element.
 * ------------------------------------------------------------------------ */
void orc_conv2d_at(const double *x, int ci, int h, int w, const double *wt, int co, int k,
                   int up2, const double *bias, const int64_t *pix, int64_t npix, double *y)
{
    const int pad = k / 2;
    const int Hout = up2 ? 2 * h : h, Wout = up2 ? 2 * w : w;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t j = 0; j < npix; ++j) {
        for (int o = 0; o < co; ++o) {
            const int r = (int)(pix[j] / Wout), c = (int)(pix[j] % Wout);
            double acc = 0.0;
            for (int i = 0; i < ci; ++i)
                for (int ky = 0; ky < k; ++ky)
                    for (int kx = 0; kx < k; ++kx) {
                        int sy = r + ky - pad, sx = c + kx - pad;
                        if (sy < 0 || sy >= Hout || sx < 0 || sx >= Wout) continue;
                        if (up2) { sy /= 2; sx /= 2; }
                        acc += wt[(((int64_t)o * ci + i) * k + ky) * k + kx] *
                               x[((int64_t)i * h + sy) * w + sx];
                    }
            if (bias) acc += bias[o];
            y[j * co + o] = acc;
        }
    }
}

/* ------------------------------------------------------------------------
 * Per-pixel RMS_norm over the channels (page qi21_vae.rs, RMSN_SRC and
 * `Rec::rmsn`): v = x + b (bias optional, added on read);
 * y_c = v_c * sqrt(C) / max(||v||_2, eps) * gamma_c, with C the real channel
 * count and the sum over the real channels; optional SiLU y / (1 + e^-y)
 * (page vae.rs, `silu`). x, y: NCHW [c][p] (p = pixels).
 * ------------------------------------------------------------------------ */
void orc_rmsnorm(const double *x, int c, int64_t p, const double *bias, const double *gamma,
                 int silu, double eps, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < p; ++q) {
        double ss = 0.0;
        for (int ch = 0; ch < c; ++ch) {
            const double v = x[(int64_t)ch * p + q] + (bias ? bias[ch] : 0.0);
            ss += v * v;
        }
        const double n = sqrt(ss);
        const double inv = sqrt((double)c) / (n > eps ? n : eps);
        for (int ch = 0; ch < c; ++ch) {
            const double v = x[(int64_t)ch * p + q] + (bias ? bias[ch] : 0.0);
            double t = v * inv * gamma[ch];
            if (silu) t = t / (1.0 + exp(-t));
            y[(int64_t)ch * p + q] = t;
        }
    }
}
