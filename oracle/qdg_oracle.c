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
 *   The other block formats: [P1] module doc, BLOCKS (lk_sub and its helpers),
 *   lk_row_dot, lk_sub_dot.
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

/*
 * glu -- [P1] lk_act (the activation numbers: 0 silu g / (1 + e^-g), 1 sigmoid
 * 1 / (1 + e^-g), 2 the GELU in ggml's tanh form g / (1 + e^-2z) with
 * z = sqrt(2/pi) * (g + 0.044715 g^3)) and GLU / lk_gemv_glu (the gated value
 * u * act(g) that feeds the next quantized GEMV); [P3] the gelu-gated MLP of the
 * megakernel page (gelu_tanh(gate) times up).
 *
 * Reading: h = act(g) * u, each step below evaluated in binary64 from the
 * binary32 g and u in the order written and rounded once to binary32, as for
 * silu above (act 0 is the same computation as orc_swiglu).  The two constants
 * of the GELU are the binary64 values of sqrt(2/pi) and 0.044715 (the page
 * writes them as binary32 literals of those numbers); g^3 is (g * g) * g.
 * exp overflows to +inf for large negative arguments, where the quotients are
 * signed zeros, their limits.  act outside 0..2: -1.
 */
int orc_glu(int act, const float *g, const float *u, int64_t n, float *h)
{
    static const double c1 = 0.79788456080286535588, c2 = 0.044715;
    if (n < 0 || act < 0 || act > 2) return -1;
    for (int64_t i = 0; i < n; ++i) {
        const double gv = (double)g[i];
        double a;
        if (act == 0) {
            a = gv / (1.0 + exp(-gv));
        } else if (act == 1) {
            a = 1.0 / (1.0 + exp(-gv));
        } else {
            const double z = c1 * (gv + c2 * ((gv * gv) * gv));
            a = gv / (1.0 + exp(-2.0 * z));
        }
        h[i] = (float)(a * (double)u[i]);
    }
    return 0;
}

/*
 * Block formats other than the split Q8_0 -- [P1] module doc (a matrix in any
 * other GGUF format keeps its blocks as stored; a 32-weight sub-block decodes to
 * int8 levels with a scale d and an offset c per half of 16, weight = d*level +
 * c) and BLOCKS (which formats, and what each block's fields mean).  Format ids
 * are the GGUF type numbers.  Each decoder below is written from the GGUF block
 * layout itself, every field located by its byte or bit position in the block.
 *
 * Geometry: values per block (32, or 256 for a super-block) and bytes per block.
 */
enum {
    ORC_Q4_0 = 2, ORC_Q4_1 = 3, ORC_Q5_0 = 6, ORC_Q5_1 = 7, ORC_Q2_K = 10, ORC_Q3_K = 11,
    ORC_Q4_K = 12, ORC_Q5_K = 13, ORC_Q6_K = 14, ORC_IQ4_NL = 20, ORC_IQ4_XS = 23, ORC_MXFP4 = 39
};

int orc_fmt_geometry(int fmt, int *values, int *bytes)
{
    int v = 32, b;
    switch (fmt) {
    case ORC_Q4_0: b = 18; break;
    case ORC_Q4_1: b = 20; break;
    case ORC_Q5_0: b = 22; break;
    case ORC_Q5_1: b = 24; break;
    case ORC_IQ4_NL: b = 18; break;
    case ORC_MXFP4: b = 17; break;
    case ORC_Q2_K: v = 256; b = 84; break;
    case ORC_Q3_K: v = 256; b = 110; break;
    case ORC_Q4_K: v = 256; b = 144; break;
    case ORC_Q5_K: v = 256; b = 176; break;
    case ORC_Q6_K: v = 256; b = 210; break;
    case ORC_IQ4_XS: v = 256; b = 136; break;
    default: return -1;
    }
    *values = v;
    *bytes = b;
    return 0;
}

/* A little-endian binary16 at p, as a float (exact widening). */
static float orc_h16(const uint8_t *p) { return orc_half((uint16_t)(p[0] | (p[1] << 8))); }

/* [P1] lk_e8m0_half: the E8M0 scale 2^(e-127), halved because the E2M1 level
 * table below is doubled (so its levels are integers): 2^(e-128). */
static float orc_e8m0_half(uint8_t e) { return ldexpf(1.0f, (int)e - 128); }

/* Bits [pos, pos + width) of the block at p, read as one little-endian bit
 * string (bit pos is bit pos mod 8 of byte pos / 8), lowest bit first. */
static unsigned orc_bits(const uint8_t *p, int pos, int width)
{
    unsigned v = 0;
    for (int i = 0; i < width; ++i) v |= (unsigned)((p[(pos + i) >> 3] >> ((pos + i) & 7)) & 1u) << i;
    return v;
}

/* The 12-byte (96-bit) scale field of a Q4_K / Q5_K super-block holds eight
 * six-bit scales and eight six-bit mins, one pair per 32-weight sub-block j:
 *   j < 4:  scale = bits 8j .. 8j+5,            min = bits 32+8j .. 32+8j+5;
 *   j >= 4 (i = j - 4): the low four bits of scale are bits 64+8i .. 64+8i+3 and
 *           of min bits 64+8i+4 .. 64+8i+7; their high two bits are the spare
 *           top bits of the first two groups, bits 8i+6, 8i+7 (scale) and
 *           32+8i+6, 32+8i+7 (min). */
static int orc_k4_field(const uint8_t *s12, int j, int is_min)
{
    const int base = is_min ? 32 : 0;
    if (j < 4) return (int)orc_bits(s12, base + 8 * j, 6);
    const int i = j - 4;
    return (int)(orc_bits(s12, 64 + 8 * i + (is_min ? 4 : 0), 4) | (orc_bits(s12, base + 8 * i + 6, 2) << 4));
}

/* [P1] lk_iq4_level: the sixteen non-linear IQ4 levels. */
static const int8_t ORC_IQ4[16] = {-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113};
/* [P1] the doubled E2M1 values of MXFP4, by nibble. */
static const int8_t ORC_E2M1X2[16] = {0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12};

/* Sub-block sb (32 weights) of a row: levels v[32], and per half h (weights
 * 16h .. 16h+15) the scale d[h] and offset c[h] (binary32). */
static int orc_decode_sub(int fmt, const uint8_t *row, int64_t sb, int8_t *v, float *d, float *c)
{
    c[0] = c[1] = 0.0f;
    if (fmt == ORC_Q4_0 || fmt == ORC_Q4_1 || fmt == ORC_IQ4_NL) {
        const int bytes = fmt == ORC_Q4_1 ? 20 : 18;
        const uint8_t *b = row + sb * bytes;
        d[0] = d[1] = orc_h16(b);
        if (fmt == ORC_Q4_1) c[0] = c[1] = orc_h16(b + 2);
        const uint8_t *qs = b + (fmt == ORC_Q4_1 ? 4 : 2);
        for (int i = 0; i < 16; ++i) {
            const int lo = qs[i] & 15, hi = qs[i] >> 4;
            if (fmt == ORC_IQ4_NL) {
                v[i] = ORC_IQ4[lo];
                v[i + 16] = ORC_IQ4[hi];
            } else {
                v[i] = (int8_t)(lo - (fmt == ORC_Q4_0 ? 8 : 0));
                v[i + 16] = (int8_t)(hi - (fmt == ORC_Q4_0 ? 8 : 0));
            }
        }
    } else if (fmt == ORC_Q5_0 || fmt == ORC_Q5_1) {
        const int bytes = fmt == ORC_Q5_1 ? 24 : 22;
        const uint8_t *b = row + sb * bytes;
        d[0] = d[1] = orc_h16(b);
        if (fmt == ORC_Q5_1) c[0] = c[1] = orc_h16(b + 2);
        const uint8_t *hb = b + (fmt == ORC_Q5_1 ? 4 : 2);
        const uint32_t qh = (uint32_t)hb[0] | ((uint32_t)hb[1] << 8) | ((uint32_t)hb[2] << 16) | ((uint32_t)hb[3] << 24);
        const uint8_t *qs = hb + 4;
        const int off = fmt == ORC_Q5_0 ? 16 : 0;
        for (int i = 0; i < 16; ++i) {
            /* bit i of qh is the fifth bit of weight i, bit i + 16 that of weight i + 16 */
            v[i] = (int8_t)(((qs[i] & 15) | (((qh >> i) & 1) << 4)) - off);
            v[i + 16] = (int8_t)(((qs[i] >> 4) | (((qh >> (i + 16)) & 1) << 4)) - off);
        }
    } else if (fmt == ORC_MXFP4) {
        const uint8_t *b = row + sb * 17;
        d[0] = d[1] = orc_e8m0_half(b[0]);
        for (int i = 0; i < 16; ++i) {
            v[i] = ORC_E2M1X2[b[1 + i] & 15];
            v[i + 16] = ORC_E2M1X2[b[1 + i] >> 4];
        }
    } else if (fmt == ORC_Q4_K || fmt == ORC_Q5_K) {
        /* Q4_K, 144 bytes: d (binary16, bytes 0-1), dmin (binary16, bytes 2-3),
         * the scale field (bytes 4-15), 128 bytes of four-bit levels (from byte 16).
         * Q5_K, 176 bytes: the same head, then 32 bytes of fifth bits (bytes
         * 16-47), then the four-bit levels (from byte 48).  Weight l (0..31) of
         * sub-block j: its four bits are bits 4*(j mod 2) .. +3 of level byte
         * 32*(j/2) + l (two sub-blocks share 32 bytes, the even one in the low
         * nibbles); under Q5_K its fifth bit (worth 16) is bit j of fifth-bit
         * byte l.  weight = d*scale_j*level - dmin*min_j. */
        const int q5 = fmt == ORC_Q5_K;
        const uint8_t *b = row + (sb >> 3) * (q5 ? 176 : 144);
        const int j = (int)(sb & 7);
        const int lev0 = q5 ? 48 : 16;
        d[0] = d[1] = orc_h16(b) * (float)orc_k4_field(b + 4, j, 0);
        c[0] = c[1] = -(orc_h16(b + 2) * (float)orc_k4_field(b + 4, j, 1));
        for (int l = 0; l < 32; ++l) {
            unsigned lv = orc_bits(b, 8 * (lev0 + 32 * (j / 2) + l) + 4 * (j % 2), 4);
            if (q5) lv |= orc_bits(b, 8 * (16 + l) + j, 1) << 4;
            v[l] = (int8_t)lv;
        }
    } else if (fmt == ORC_Q2_K) {
        /* Q2_K, 84 bytes: sixteen scale bytes (one per 16-weight group g: scale in
         * bits 0-3, min in bits 4-7), 64 bytes of two-bit levels (bytes 16-79),
         * d (binary16, bytes 80-81), dmin (binary16, bytes 82-83).  Weight w
         * (0..255) of the super-block: with h = w / 128, k = (w mod 128) / 32 and
         * l = w mod 32, its level is bits 2k, 2k+1 of level byte 32h + l.
         * weight = d*scale_g*level - dmin*min_g with g = w / 16. */
        const uint8_t *b = row + (sb >> 3) * 84;
        const float dd = orc_h16(b + 80), dm = orc_h16(b + 82);
        for (int l = 0; l < 32; ++l) {
            const int w = 32 * (int)(sb & 7) + l;
            v[l] = (int8_t)orc_bits(b, 8 * (16 + 32 * (w / 128) + w % 32) + 2 * ((w % 128) / 32), 2);
        }
        for (int h = 0; h < 2; ++h) {
            const int g = 2 * (int)(sb & 7) + h;
            d[h] = dd * (float)orc_bits(b, 8 * g, 4);
            c[h] = -(dm * (float)orc_bits(b, 8 * g + 4, 4));
        }
    } else if (fmt == ORC_Q3_K) {
        const uint8_t *b = row + (sb >> 3) * 110;
        const int j = (int)(sb & 7), half = j >> 2, k = j & 3;
        const uint8_t *q = b + 32 + 32 * half;  /* two-bit low parts */
        const uint8_t *hm = b;                  /* 32 bytes of high-bit masks */
        const uint8_t *sp = b + 96;             /* 12 bytes: 16 six-bit scales */
        const float dd = orc_h16(b + 108);
        const int mbit = 4 * half + k;
        for (int l = 0; l < 32; ++l) {
            const int low = (q[l] >> (2 * k)) & 3;
            v[l] = (int8_t)(low - (((hm[l] >> mbit) & 1) ? 0 : 4));
        }
        for (int h = 0; h < 2; ++h) {
            /* six-bit scale i (0..15): its low 4 bits are nibble i / 8 of byte
             * i mod 8, its high 2 bits are bits 2*(i / 4) of byte 8 + i mod 4 */
            const int i = 8 * half + 2 * k + h;
            const int lo4 = (sp[i & 7] >> (4 * (i >> 3))) & 15;
            const int hi2 = (sp[8 + (i & 3)] >> (2 * (i >> 2))) & 3;
            d[h] = dd * (float)((lo4 | (hi2 << 4)) - 32);
        }
    } else if (fmt == ORC_Q6_K) {
        const uint8_t *b = row + (sb >> 3) * 210;
        const int j = (int)(sb & 7), half = j >> 2, k = j & 3;
        const uint8_t *ql = b + 64 * half;
        const uint8_t *qh = b + 128 + 32 * half;
        const int8_t *sc = (const int8_t *)(b + 192 + 8 * half);
        const float dd = orc_h16(b + 208);
        for (int l = 0; l < 32; ++l) {
            int lo = (k & 1) ? ql[l + 32] : ql[l];
            lo = (k & 2) ? lo >> 4 : lo & 15;
            v[l] = (int8_t)((lo | (((qh[l] >> (2 * k)) & 3) << 4)) - 32);
        }
        d[0] = dd * (float)sc[2 * k];
        d[1] = dd * (float)sc[2 * k + 1];
    } else if (fmt == ORC_IQ4_XS) {
        /* IQ4_XS, 136 bytes: d (binary16, bytes 0-1); the high two bits of the
         * eight six-bit sub-block scales (bits 16 + 2j, 16 + 2j + 1: bytes 2-3);
         * their low four bits (bits 32 + 4j .. 32 + 4j + 3: bytes 4-7); 128 bytes
         * of four-bit indices (from byte 8).  Sub-block j's scale is
         * d * (six-bit value - 32); weight l (0..31) of it is the IQ4 level of
         * bits 4*(l / 16) .. +3 of index byte 16j + l mod 16. */
        const uint8_t *b = row + (sb >> 3) * 136;
        const int j = (int)(sb & 7);
        const int ls = (int)(orc_bits(b, 32 + 4 * j, 4) | (orc_bits(b, 16 + 2 * j, 2) << 4));
        d[0] = d[1] = orc_h16(b) * (float)(ls - 32);
        for (int l = 0; l < 32; ++l) v[l] = ORC_IQ4[orc_bits(b, 8 * (8 + 16 * j + l % 16) + 4 * (l / 16), 4)];
    } else {
        return -1;
    }
    return 0;
}

/* Row bytes of a K-value row in format fmt (0 if K does not fit the format). */
int64_t orc_fmt_row_bytes(int fmt, int64_t K)
{
    int v, b;
    if (orc_fmt_geometry(fmt, &v, &b) || K % v) return 0;
    return K / v * b;
}

/* Every sub-block of N rows: levels [N][K], d and c [N][K/16] (one per half). */
int orc_fmt_decode(int fmt, const uint8_t *w, int64_t N, int64_t K, int8_t *levels, float *d, float *c)
{
    const int64_t rb = orc_fmt_row_bytes(fmt, K);
    if (!rb) return -1;
    for (int64_t o = 0; o < N; ++o)
        for (int64_t sb = 0; sb < K / 32; ++sb)
            if (orc_decode_sub(fmt, w + o * rb, sb, levels + o * K + 32 * sb, d + o * (K / 16) + 2 * sb,
                               c + o * (K / 16) + 2 * sb))
                return -1;
    return 0;
}

/*
 * The GEMV of a block-format matrix, batch 1 -- [P1] lk_row_dot, lk_sub_dot.
 *  Dequant: each weight is fl(fl(d*level) + c) as the CPU dequantizer rounds
 *    it; the products with x and their sum are binary64 (ascending k), rounded
 *    once to binary32.
 *  Int8Act / TwoPass: per sub-block g, the exact int32 dots of each half with
 *    the activation words, dh_h = sum level*h and sh_h = sum h (and dl, sl with
 *    the low words); part = ((d0*dh0 + c0*sh0) + d1*dh1) + c1*sh1, every product
 *    and sum one binary32 rounding, left to right; TwoPass adds
 *    fl(2^-7 * (the same with dl, sl)).  The row is the Q8_0 row's structure:
 *    step p <- fma(s_g, part, p) into partial g mod 4 in ascending g from +0,
 *    then (P0 + P2) + (P1 + P3).
 */
/* The quantized row dot of one row over sub-blocks [g0, g1) (the steps below). */
static float orc_fmt_row_quant(int fmt, int mode, const uint8_t *row, int64_t g0, int64_t g1,
                               const int8_t *xq, const int8_t *xl, const float *xs, int *bad)
{
    int8_t v[32];
    float d[2], c[2];
    float P[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t g = g0; g < g1; ++g) {
        if (orc_decode_sub(fmt, row, g, v, d, c)) { *bad = 1; return 0.0f; }
        int32_t dh[2] = {0, 0}, sh[2] = {0, 0}, dl[2] = {0, 0}, sl[2] = {0, 0};
        for (int i = 0; i < 32; ++i) {
            const int h = i >> 4;
            dh[h] += (int32_t)v[i] * xq[32 * g + i];
            sh[h] += xq[32 * g + i];
            if (mode == 2) {
                dl[h] += (int32_t)v[i] * xl[32 * g + i];
                sl[h] += xl[32 * g + i];
            }
        }
        float part = d[0] * (float)dh[0];
        part = part + c[0] * (float)sh[0];
        part = part + d[1] * (float)dh[1];
        part = part + c[1] * (float)sh[1];
        if (mode == 2) {
            float lo = d[0] * (float)dl[0];
            lo = lo + c[0] * (float)sl[0];
            lo = lo + d[1] * (float)dl[1];
            lo = lo + c[1] * (float)sl[1];
            part = part + 0.0078125f * lo;
        }
        P[g & 3] = fmaf(xs[g], part, P[g & 3]);
    }
    return (P[0] + P[2]) + (P[1] + P[3]);
}

/* The Dequant sum of one row over sub-blocks [g0, g1), binary64, ascending k. */
static double orc_fmt_row_dequant(int fmt, const uint8_t *row, int64_t g0, int64_t g1, const float *x, int *bad)
{
    int8_t v[32];
    float d[2], c[2];
    double acc = 0.0;
    for (int64_t g = g0; g < g1; ++g) {
        if (orc_decode_sub(fmt, row, g, v, d, c)) { *bad = 1; return 0.0; }
        for (int i = 0; i < 32; ++i) {
            const float wv = (d[i >> 4] * (float)v[i]) + c[i >> 4];
            acc += (double)wv * (double)x[32 * g + i];
        }
    }
    return acc;
}

/*
 * splits == 1: the row as above.  splits > 1: the QWEN38 page's chunk rule in
 * sub-blocks (orc_split_bounds: 512-value superblocks), each chunk's partial
 * summed as a whole row is over the chunk's sub-blocks, then added in
 * ascending chunk order from 0 (gk_sk_combine) -- binary32 under the quantized
 * modes, binary64 under Dequant with one final rounding.
 */
int orc_gemv_fmt(int fmt, int mode, const uint8_t *w, int64_t N, int64_t K, const float *x,
                 const int8_t *xq, const int8_t *xl, const float *xs, int splits, float *y, int nthreads)
{
    const int64_t rb = orc_fmt_row_bytes(fmt, K);
    if (!rb || mode < 0 || mode > 2 || splits < 1 || splits > 64) return -1;
    const int64_t nb = K / 32;
    int32_t first[65];
    if (orc_split_bounds(K, splits, first)) return -1;
    orc_set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t o = 0; o < N; ++o) {
        const uint8_t *row = w + o * rb;
        if (splits == 1) {
            y[o] = mode == 0 ? (float)orc_fmt_row_dequant(fmt, row, 0, nb, x, &bad)
                             : orc_fmt_row_quant(fmt, mode, row, 0, nb, xq, xl, xs, &bad);
            continue;
        }
        if (mode == 0) {
            double a = 0.0;
            for (int s = 0; s < splits; ++s) a += orc_fmt_row_dequant(fmt, row, first[s], first[s + 1], x, &bad);
            y[o] = (float)a;
        } else {
            float a = 0.0f;
            for (int s = 0; s < splits; ++s)
                a = a + orc_fmt_row_quant(fmt, mode, row, first[s], first[s + 1], xq, xl, xs, &bad);
            y[o] = a;
        }
    }
    return bad ? -1 : 0;
}

int orc_version(void) { return 1; }
