/*
 * qdg_oracle.c -- the CPU oracle of the Q8_0 decode GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * statement of what the GPU library computes.  Only the test-suite, the smoke
 * check and the CPU-baseline leg of the benchmark load it; the product path never
 * does.  It shares no source, header, table or helper with the GPU library.
 *
 * Built with `gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math`: every float
 * operation below is one IEEE binary32 (or binary64) operation rounded to nearest
 * even, and the only fused multiply-adds are the explicit fmaf() calls where the
 * method prescribes one rounding.
 *
 * Sources (page title, then the section / symbol on that page):
 *   [P1] "logicaffeine_compile/codegen_cuda/lane/kernels.rs" -- module doc
 *        (numerics contract), PRELUDE (lk_two_scale, lk_two_words, lk_quant_lane,
 *        lk_q8_term, lk_q8_acc, lk_q8_sum4, lk_q8_block_dot, lk_q8_round,
 *        lk_q8_rows_dot), QUANT (lk_quant), GEMV_Q8 (lk_gemv_q8), lk_w.
 *   [P2] "QWEN38_EXTRA_KERNELS" -- "SPLIT-K FOR THE NARROW PROJECTIONS"
 *        (gk_gemv_hl_sk, gk_sk_combine).
 *   [P3] "model-as-a-kernel mak_cuda/megakernel.cu" -- amax_key, ph_argmax_part,
 *        ph_argmax_fin (first index among equal maxima).
 *   The producers of the quantized activation: [P1] RMSNORM (lk_rmsnorm_row),
 *   lk_act, GLU; [P2] gk_add_rmsnorm_q8f, gk_silu_had_q8.
 *
 * Modes: 0 Dequant (f32 activation, f64 sums), 1 Int8Act, 2 TwoPassInt8 ([P1]
 * mode()).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_QK 32

/* IEEE binary16 -> binary32, exact widening, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 holds
 * zero and the subnormals (fraction * 2^-24), exponent 31 holds inf / NaN. */
static float orc_half(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 31;
    const int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return (float)(sign ? -v : v);
}

float orc_half_to_float(uint16_t h) { return orc_half(h); }

/* Round to the nearest integer, ties to even ([P1] __float2int_rn).  nearbyintf
 * rounds in the current mode, which is round-to-nearest-even by default. */
static int orc_rn(float v)
{
    if (isnan(v)) return 0; /* outside the contract; only keeps the oracle defined */
    float r = nearbyintf(v);
    if (r > 2147483520.0f) return 2147483647;
    if (r < -2147483648.0f) return -2147483647 - 1;
    return (int)r;
}

static int orc_clamp8(int v) { return v > 127 ? 127 : (v < -128 ? -128 : v); }

/*
 * quantize_act -- [P1] module doc (the activation quantizer: 32 values per
 * scale), lk_quant_lane, lk_two_scale, lk_two_words; [P2] section on two-pass
 * int8 activations.
 *
 * Per row t and 32-block g:  a = max |x|.
 *   Int8Act:  s = a > 0 ? a/127 : 1;       h = rn(x/s)
 *   TwoPass:  s = max(a, 1e-30)/127;       h = clamp(rn(x/s));
 *             r = fma(-h, s, x)  (one rounding);
 *             l = clamp(rn(r / (s*2^-7)))
 * xs[t][g] = s.  The Int8Act word is not clamped on the page; |h| <= 127 holds
 * for every block whose scale is a normal float, and outside that (a below
 * ~1.5e-36) the oracle saturates to int8 so that it stays defined.
 */
int orc_quantize(int mode, const float *x, int64_t B, int64_t K,
                 int8_t *xq, int8_t *xl, float *xs)
{
    if ((mode != 1 && mode != 2) || K % ORC_QK) return -1;
    const int64_t nb = K / ORC_QK;
    for (int64_t t = 0; t < B; ++t) {
        for (int64_t g = 0; g < nb; ++g) {
            const float *v = x + t * K + g * ORC_QK;
            float a = 0.0f;
            for (int i = 0; i < ORC_QK; ++i) {
                float m = fabsf(v[i]);
                if (m > a) a = m;
            }
            float s;
            if (mode == 1)
                s = a > 0.0f ? a / 127.0f : 1.0f;
            else
                s = (a > 1e-30f ? a : 1e-30f) / 127.0f;
            xs[t * nb + g] = s;
            for (int i = 0; i < ORC_QK; ++i) {
                const int64_t k = t * K + g * ORC_QK + i;
                if (mode == 1) {
                    xq[k] = (int8_t)orc_clamp8(orc_rn(v[i] / s));
                } else {
                    const int h = orc_clamp8(orc_rn(v[i] / s));
                    const float r = fmaf(-(float)h, s, v[i]);
                    const float lsc = s * 0.0078125f;
                    const int l = orc_clamp8(orc_rn(r / lsc));
                    xq[k] = (int8_t)h;
                    xl[k] = (int8_t)l;
                }
            }
        }
    }
    return 0;
}

/* The exact int32 dot of one 32-value block of a weight row and an activation
 * row ([P1] lk_q8_block_dot: exact in integers). */
static int32_t orc_block_dot(const int8_t *w, const int8_t *a)
{
    int64_t d = 0;
    for (int i = 0; i < ORC_QK; ++i) d += (int64_t)w[i] * (int64_t)a[i];
    return (int32_t)d;
}

/* dh[t][o][g] = sum w*h and, for TwoPass, dl[t][o][g] = sum w*l. */
int orc_block_dots(int mode, const int8_t *wq, int64_t N, int64_t K,
                   const int8_t *xq, const int8_t *xl, int64_t B,
                   int32_t *dh, int32_t *dl)
{
    if ((mode != 1 && mode != 2) || K % ORC_QK) return -1;
    const int64_t nb = K / ORC_QK;
    for (int64_t t = 0; t < B; ++t)
        for (int64_t o = 0; o < N; ++o)
            for (int64_t g = 0; g < nb; ++g) {
                const int8_t *w = wq + o * K + g * ORC_QK;
                dh[(t * N + o) * nb + g] = orc_block_dot(w, xq + t * K + g * ORC_QK);
                if (mode == 2)
                    dl[(t * N + o) * nb + g] = orc_block_dot(w, xl + t * K + g * ORC_QK);
            }
    return 0;
}

/*
 * One quantized row dot over blocks [g0, g1) -- [P1] lk_q8_term, lk_q8_acc,
 * lk_q8_sum4, lk_q8_rows_dot (module doc: quantized sums are f32, in one fixed
 * order).
 *
 * Block g's step is p <- fma(alpha, beta, p) with
 *   Int8Act:  alpha = fl(sigma * s),  beta = (float)D
 *   TwoPass:  alpha = sigma,          beta = fma(s, (float)D, fl(fl(s*2^-7) * (float)E))
 * (sigma the block's weight scale, s its activation scale, D / E the exact
 * int32 dots with the high / low words).  Step g goes into partial g mod 4, each
 * partial taking its blocks in ascending order from +0, and the row's value is
 * (P0 + P2) + (P1 + P3).
 */
static float orc_row_quant(int mode, const int8_t *w, const uint16_t *wsr,
                           const int8_t *h, const int8_t *l, const float *s,
                           int64_t g0, int64_t g1)
{
    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t g = g0; g < g1; ++g) {
        const float sigma = orc_half(wsr[g]);
        const float d = (float)orc_block_dot(w + g * ORC_QK, h + g * ORC_QK);
        float alpha, beta;
        if (mode == 1) {
            alpha = sigma * s[g];
            beta = d;
        } else {
            const float e = (float)orc_block_dot(w + g * ORC_QK, l + g * ORC_QK);
            const float lo = (s[g] * 0.0078125f) * e;
            alpha = sigma;
            beta = fmaf(s[g], d, lo);
        }
        p[g % 4] = fmaf(alpha, beta, p[g % 4]);
    }
    return (p[0] + p[2]) + (p[1] + p[3]);
}

/*
 * The plain Dequant row: y = fl( sum_k sigma_{k/32} * w_k * x_k ) with every
 * product and sum in binary64 ([P1] module doc on the Dequant mode, lk_acc<0>,
 * accumulator()).  Each product sigma*w*x is exact in binary64
 * (11 + 8 + 24 significant bits); the sum runs in ascending k from +0 and is
 * rounded once to binary32.
 */
static float orc_row_dequant(const int8_t *w, const uint16_t *wsr, const float *x, int64_t K)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const double sw = (double)orc_half(wsr[k / ORC_QK]) * (double)w[k];
        acc += sw * (double)x[k];
    }
    return (float)acc;
}

static void orc_set_threads(int nthreads)
{
#ifdef _OPENMP
    omp_set_num_threads(nthreads > 0 ? nthreads : 1);
#else
    (void)nthreads;
#endif
}

/*
 * y[t][o] over the whole row ([P1] lk_gemv_q8: Y[t,o] = sum_k X[t,k] W[o,k]).
 * Dequant reads x; Int8Act reads xq, xs; TwoPass reads xq, xl, xs.  Rows are
 * independent, so the row loop may run on several threads without changing any
 * row's arithmetic.
 */
int orc_gemv(int mode, const int8_t *wq, const uint16_t *ws, int64_t N, int64_t K,
             const float *x, const int8_t *xq, const int8_t *xl, const float *xs,
             int64_t B, float *y, int nthreads)
{
    if (mode < 0 || mode > 2 || K % ORC_QK) return -1;
    const int64_t nb = K / ORC_QK;
    orc_set_threads(nthreads);
    for (int64_t t = 0; t < B; ++t) {
#pragma omp parallel for schedule(static)
        for (int64_t o = 0; o < N; ++o) {
            const int8_t *w = wq + o * K;
            const uint16_t *wsr = ws + o * nb;
            if (mode == 0)
                y[t * N + o] = orc_row_dequant(w, wsr, x + t * K, K);
            else
                y[t * N + o] = orc_row_quant(mode, w, wsr, xq + t * K,
                                             mode == 2 ? xl + t * K : NULL,
                                             xs + t * nb, 0, nb);
        }
    }
    return 0;
}

/*
 * Split-K chunk boundaries -- [P2] gk_gemv_hl_sk: K runs in 512-value
 * superblocks, nq = K/512 of them, per = ceil(nq/S); chunk s takes superblocks
 * [s*per, min((s+1)*per, nq)), and the K mod 512 tail goes to the last chunk.
 * Written as block boundaries: chunk s is blocks [first[s], first[s+1]).
 */
int orc_split_bounds(int64_t K, int S, int32_t *first)
{
    if (S < 1 || K % ORC_QK) return -1;
    const int64_t nq = K / 512, nb = K / ORC_QK;
    const int64_t per = (nq + S - 1) / S;
    for (int s = 0; s < S; ++s) {
        int64_t q0 = (int64_t)s * per;
        if (q0 > nq) q0 = nq;
        first[s] = (int32_t)(q0 * 16);
    }
    first[S] = (int32_t)nb;
    return 0;
}

/* part[s][t][o]: the quantized row dot restricted to chunk s (same steps and
 * order as the whole row, over the chunk's blocks). */
int orc_gemv_split(int mode, const int8_t *wq, const uint16_t *ws, int64_t N, int64_t K,
                   const int8_t *xq, const int8_t *xl, const float *xs, int64_t B,
                   int S, float *part, int nthreads)
{
    if ((mode != 1 && mode != 2) || S < 1 || S > 64 || K % ORC_QK) return -1;
    int32_t first[65];
    orc_split_bounds(K, S, first);
    const int64_t nb = K / ORC_QK;
    orc_set_threads(nthreads);
    for (int s = 0; s < S; ++s)
        for (int64_t t = 0; t < B; ++t) {
#pragma omp parallel for schedule(static)
            for (int64_t o = 0; o < N; ++o)
                part[((int64_t)s * B + t) * N + o] =
                    orc_row_quant(mode, wq + o * K, ws + o * nb, xq + t * K,
                                  mode == 2 ? xl + t * K : NULL, xs + t * nb,
                                  first[s], first[s + 1]);
        }
    return 0;
}

/* [P2] gk_sk_combine: y = sum of the partials in ascending chunk order from 0. */
int orc_combine(const float *part, int S, int64_t B, int64_t N, float *y)
{
    if (S < 1) return -1;
    for (int64_t i = 0; i < B * N; ++i) {
        float a = 0.0f;
        for (int s = 0; s < S; ++s) a = a + part[(int64_t)s * B * N + i];
        y[i] = a;
    }
    return 0;
}

/* The first index among equal maxima ([P1] module doc; [P3] ph_argmax_*: lowest
 * index on ties).  Strict '>' keeps the earlier of equal values, and IEEE '>'
 * treats -0 and +0 as equal. */
int orc_argmax(const float *y, int64_t B, int64_t N, int32_t *idx)
{
    if (N < 1) return -1;
    for (int64_t t = 0; t < B; ++t) {
        const float *r = y + t * N;
        int64_t bi = 0;
        float bv = r[0];
        for (int64_t i = 1; i < N; ++i)
            if (r[i] > bv) { bv = r[i]; bi = i; }
        idx[t] = (int32_t)bi;
    }
    return 0;
}

/*
 * The binary64 anchor of the tolerance test.  Quantized modes: the value the
 * encoded operands stand for, Y = sum_g sigma_g * s_g * (D_g + E_g/128) (E = 0
 * for Int8Act), each block term and the running sum in binary64 (D + E/128 is
 * exact there; the product with sigma*s rounds once, some 2^-53 relative);
 * Dequant: the binary64 sum of the exact products sigma*w*x.  tnorm is the
 * Euclidean norm of the row's block terms, the scale below which a relative
 * comparison means nothing.
 */
int orc_reference_f64(int mode, const int8_t *wq, const uint16_t *ws, int64_t N, int64_t K,
                      const float *x, const int8_t *xq, const int8_t *xl, const float *xs,
                      int64_t B, double *Y, double *tnorm, int nthreads)
{
    if (mode < 0 || mode > 2 || K % ORC_QK) return -1;
    const int64_t nb = K / ORC_QK;
    orc_set_threads(nthreads);
    for (int64_t t = 0; t < B; ++t) {
#pragma omp parallel for schedule(static)
        for (int64_t o = 0; o < N; ++o) {
            double acc = 0.0, sq = 0.0;
            for (int64_t g = 0; g < nb; ++g) {
                const double sigma = (double)orc_half(ws[o * nb + g]);
                const int8_t *w = wq + o * K + g * ORC_QK;
                double term;
                if (mode == 0) {
                    double inner = 0.0;
                    for (int i = 0; i < ORC_QK; ++i)
                        inner += sigma * (double)w[i] * (double)x[t * K + g * ORC_QK + i];
                    term = inner;
                } else {
                    const double d = (double)orc_block_dot(w, xq + t * K + g * ORC_QK);
                    const double e = mode == 2 ? (double)orc_block_dot(w, xl + t * K + g * ORC_QK) : 0.0;
                    term = sigma * (double)xs[t * nb + g] * (d + e / 128.0);
                }
                acc += term;
                sq += term * term;
            }
            Y[t * N + o] = acc;
            tnorm[t * N + o] = sqrt(sq);
        }
    }
    return 0;
}

/*
 * rmsnorm -- [P1] RMSNORM (the doc of lk_rmsnorm and lk_rmsnorm_row: per row,
 * v = x (+ r), y = v / sqrt(mean(v^2) + eps) * w, the sum v written out as the
 * next residual stream when asked); [P2] gk_add_rmsnorm_q8f (the residual add
 * folded into the norm that follows it, its result stored back).
 *
 * Readings: the residual sum is one binary32 addition, v = fl32(x + r), and is
 * the value stored to s.  The norm is then evaluated in binary64 from those
 * binary32 values -- the squares are exact there, the sum runs in ascending
 * index order, then mean + eps, sqrt, (v / den) * w in that order -- and y is
 * rounded once to binary32.  w NULL means no weight (y = v / den).  K need not
 * be a multiple of 32 here.
 */
int orc_rmsnorm(const float *x, const float *r, const float *w, float eps, int64_t B, int64_t K,
                float *s, float *y)
{
    if (K < 1 || B < 0) return -1;
    for (int64_t t = 0; t < B; ++t) {
        const float *xr = x + t * K;
        double sum = 0.0;
        for (int64_t i = 0; i < K; ++i) {
            float v = xr[i];
            if (r) v = v + r[t * K + i];
            if (s) s[t * K + i] = v;
            sum += (double)v * (double)v;
        }
        const double den = sqrt(sum / (double)K + (double)eps);
        for (int64_t i = 0; i < K; ++i) {
            float v = xr[i];
            if (r) v = v + r[t * K + i];
            double o = (double)v / den;
            if (w) o = o * (double)w[i];
            y[t * K + i] = (float)o;
        }
    }
    return 0;
}

/*
 * swiglu -- [P1] lk_act (silu is g / (1 + e^-g)) and GLU (the gated product
 * act(g) * u that feeds the next quantized GEMV); [P2] gk_silu_had_q8 (silu(g)
 * times u, then the 32-value block quantizer).
 *
 * Reading: h = (g / (1 + exp(-g))) * u in that order, evaluated in binary64 from
 * the binary32 inputs and rounded once to binary32.  exp(-g) overflows to +inf
 * for g below about -709, where g / inf is a signed zero, which is the limit.
 */
int orc_swiglu(const float *g, const float *u, int64_t n, float *h)
{
    if (n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) {
        const double gv = (double)g[i];
        const double silu = gv / (1.0 + exp(-gv));
        h[i] = (float)(silu * (double)u[i]);
    }
    return 0;
}

int orc_version(void) { return 1; }
