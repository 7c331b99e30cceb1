/*
 * qdg.h -- C ABI of the MI355X (gfx950) Q8_0 decode GEMV library, libqdg.so.
 *
 * The library computes the memory-bound matrix-vector product of LLM decode
 * against a Q8_0 weight matrix, as the lane kernel library page
 * ("logicaffeine_compile/codegen_cuda/lane/kernels.rs") defines it, with the
 * split-K and combine of the "QWEN38_EXTRA_KERNELS" page and the first-index
 * arg-max of the "model-as-a-kernel mak_cuda/megakernel.cu" page.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named as device pointers are HIP device memory the caller owns.
 *    The library allocates no device memory per call and keeps no pointer to a
 *    caller's buffer after it returns.  Its state: the thread-local error code
 *    of qdg_last_hip_error() and event binding of qdg_time_next_launch(), the
 *    process-wide tuning knobs (qdg_set_tuning), and, once
 *    qdg_gemv_q8_argmax_noalloc has run on a GPU, that GPU's 1 MiB key array.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 *    runs asynchronously; nothing synchronises.
 *  - Every argument is checked before anything is enqueued.  A negative status
 *    means nothing was enqueued, except QDG_EHIP, which reports that the HIP
 *    runtime refused a launch (qdg_last_hip_error() holds its hipError_t).
 *  - The same inputs give the same output bits on every call: every sum runs in
 *    a fixed order, no result depends on workgroup scheduling, and no floating
 *    point atomics are used.
 *  - Layouts are row-major and dense.  K is a multiple of 32.  wq, xq, xl and x
 *    must be 16-byte aligned; ws 2-byte; xs, y, out, partials and idx 4-byte;
 *    the arg-max workspace 8-byte.
 *
 * Data (lane kernel library page: module doc, lk_w; QWEN38 page: split-K)
 *   wq  int8     [N][K]        weight values
 *   ws  binary16 [N][K/32]     one weight scale per 32 values (bit patterns)
 *   x   float    [B][K]        activation (Dequant mode)
 *   xq  int8     [B][K]        activation words (high words under TwoPass)
 *   xl  int8     [B][K]        TwoPass low words
 *   xs  float    [B][K/32]     activation scale per 32 values
 *   y   float    [B][N]        output
 *   partials float [S][B][N]   split-K partial sums, chunk-major
 */
#ifndef QDG_H
#define QDG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QDG_ABI_VERSION 1

/* Numerics modes (lane kernel library page, mode()). */
enum {
    QDG_DEQUANT = 0, /* f32 activation, weight scaled in the kernel, binary64 sums  */
    QDG_INT8ACT = 1, /* activation quantized per 32-block, int8 dots, f32 sums      */
    QDG_TWOPASS = 2  /* high and low int8 words of the activation, f32 sums         */
};

/* Status codes.  0 is success; every failure is negative. */
enum {
    QDG_OK = 0,
    QDG_EINVAL = -1,     /* NULL where a pointer is required, or an unknown mode     */
    QDG_ESHAPE = -2,     /* K not a positive multiple of 32, N or B out of range     */
    QDG_EALIGN = -3,     /* a pointer breaks the alignment rule above               */
    QDG_EMODE = -4,      /* the mode does not support this B / splits combination   */
    QDG_EWORKSPACE = -5, /* a workspace is smaller than its *_workspace_bytes() size  */
    QDG_EHIP = -6        /* the HIP runtime refused a launch                        */
};

/* Limits. */
#define QDG_MAX_B 64        /* activation rows per call (above 16: K % 256 == 0,     */
                            /* ws 16-byte aligned)                                     */
#define QDG_MAX_SPLITS 64   /* split-K chunks                                        */

typedef void *qdg_stream; /* a hipStream_t */

/* One weight matrix of a multi-matrix call (qdg_gemv_q8_parts): device
 * pointers wq int8 [N][K], ws binary16 bits [N][K/32], y f32 [N]. */
#define QDG_MAX_PARTS 6
typedef struct qdg_part {
  const int8_t *wq;
  const uint16_t *ws;
  int64_t N;
  float *y;
} qdg_part;

/* QDG_ABI_VERSION of the built library. */
int qdg_abi_version(void);

/* A static, human-readable name of a status code (never NULL). */
const char *qdg_status_str(int status);

/* The hipError_t behind the calling thread's last QDG_EHIP (0 if none). */
int qdg_last_hip_error(void);

/*
 * Quantize B activation rows of K values (lane kernel library page: module doc
 * on the activation quantizer, lk_quant_lane, lk_two_scale, lk_two_words, kernel
 * lk_quant).  Per 32-value block with a = max|x|:
 *   QDG_INT8ACT: s = a > 0 ? a/127 : 1; xq = round(x/s)
 *   QDG_TWOPASS: s = max(a, 1e-30)/127; xq = clamp(round(x/s)); r = fma(-xq, s, x)
 *                (one rounding); xl = clamp(round(r / (s/128)))
 * round is to nearest, ties to even; division is IEEE; clamps are to [-128, 127]
 * (the Int8Act word never reaches them for a block whose scale is a normal
 * float).  xs[t][g] = s.  xl must be NULL for QDG_INT8ACT.  Inputs: device
 * x [B][K]; outputs: device xq, xl [B][K], xs [B][K/32].  B >= 1 (rows are
 * independent), K >= 32 and a multiple of 32, B*K < 2^62.  Values outside the
 * contract (NaN, Inf, blocks with 0 < a < 1e-30 under Int8Act) give unspecified
 * words but never fault.
 */
int qdg_quantize_act(int mode, const float *x, int64_t B, int64_t K,
                     int8_t *xq, int8_t *xl, float *xs, qdg_stream stream);

/*
 * Y[t][o] = sum_k X[t][k] * W[o][k] for a Q8_0 matrix W of N rows of K values
 * (lane kernel library page: lk_gemv_q8, lk_q8_rows_dot, lk_q8_term, lk_q8_sum4;
 * QWEN38 page: gk_gemv_hl_sk for splits > 1).
 *
 *  QDG_DEQUANT  reads x (xq, xl, xs must be NULL); every product and sum in
 *               binary64, rounded once to binary32.  B == 1, splits == 1.
 *  QDG_INT8ACT  reads xq, xs.  TwoPass reads xq, xl, xs.  Block g's step is
 *  QDG_TWOPASS  p <- fma(a, b, p) with a = fl(sigma*s), b = D (Int8Act) or
 *               a = sigma, b = fma(s, D, fl(fl(s/128)*E)) (TwoPass), D and E the
 *               exact int32 block dots; step g goes into partial g mod 4, each
 *               partial takes its blocks in ascending order from +0, and the
 *               result is (P0 + P2) + (P1 + P3).  1 <= B <= QDG_MAX_B (B > 1
 *               runs on int8 MFMA and sums every row exactly as B == 1 does;
 *               B > 16, a prefill chunk, needs K a multiple of 256 and ws
 *               16-byte aligned, else QDG_EMODE).
 *
 * splits == 1: out is y [B][N].  splits > 1 (quantized modes): out is
 * partials [splits][B][N]; chunk s covers the blocks the QWEN38 page's chunk
 * rule gives (qdg_split_bounds) and sums them in the same order as a whole row;
 * reduce with qdg_sk_combine.  1 <= splits <= QDG_MAX_SPLITS.
 * All array arguments are device pointers; N >= 1, K >= 32 and a multiple of 32,
 * N*K < 2^62.
 */
int qdg_gemv_q8(int mode, const int8_t *wq, const uint16_t *ws, int64_t N, int64_t K,
                const float *x, const int8_t *xq, const int8_t *xl, const float *xs,
                int64_t B, int splits, float *out, qdg_stream stream);

/*
 * y[t][o] = sum over s = 0..splits-1, ascending, starting from 0.0f, of
 * partials[s][t][o] (QWEN38 page, gk_sk_combine): one binary32 addition per
 * chunk, no atomics.  Device pointers; partials [splits][B][N], y [B][N].
 */
int qdg_sk_combine(const float *partials, int splits, int64_t B, int64_t N, float *y,
                   qdg_stream stream);

/* Host only: 1 when qdg_gemv_q8_sk combines the chunks of (mode, K, splits)
 * inside a workgroup (in LDS, workspace untouched), 0 when it goes through the
 * workspace, negative status on bad arguments.  shape (host, 2 entries, or
 * NULL) receives the in-workgroup launch's rows and waves per workgroup (0, 0
 * for the workspace path). */
int qdg_gemv_sk_combines_in_workgroup(int mode, int64_t K, int splits, int32_t *shape);

/* Bytes of device workspace qdg_gemv_q8_sk and qdg_gemv_q8_fused need (0 for an
 * unsupported shape): tickets, then room for S x N binary64 partials. */
size_t qdg_gemv_sk_workspace_bytes(int64_t B, int64_t N, int splits);

/*
 * The split-K GEMV and its combine in one launch (QDG_INT8ACT, QDG_TWOPASS;
 * B == 1): the chunks of the QWEN38 page's chunk rule run as in qdg_gemv_q8,
 * and each row's chunk partials are added in ascending chunk order from 0, in
 * place of the QWEN38 page's separate combine kernel.  Two placements, with the
 * same bits:
 *   - 2 <= splits <= 16 with at least two non-empty chunks, when the activation
 *     row and the workgroup's weight scales fit in 79 KiB of LDS (K/32 x (36 or
 *     68 + 8 x row groups) bytes; for QDG_TWOPASS K up to 28128 at splits 5,
 *     34048 at splits 13 to 16, more for QDG_INT8ACT): a row tile's chunks are
 *     the waves of one workgroup and meet in LDS; the workspace is not touched;
 *   - otherwise the last workgroup of each 16-row tile to finish (an atomic
 *     ticket per tile; the lane kernel library page's last-arriving-block
 *     pattern) sums the tile's partials through the workspace.
 * y [1][N] is bit-identical to qdg_gemv_q8(splits) + qdg_sk_combine: which
 * chunk finishes last changes nothing.  Inputs as
 * qdg_gemv_q8 (xq, xl, xs from qdg_quantize_act); workspace: device memory of at
 * least qdg_gemv_sk_workspace_bytes(1, N, splits) bytes, 256-byte aligned and
 * zero-filled before its first use; every call that completes leaves all of it
 * zero again (the tickets and the partial slots, which the last arriver reads
 * until it finds them published, then clears), so it needs no clearing between
 * calls.  Calls that share a workspace must not overlap in time (one stream, or
 * events between them).
 */
int qdg_gemv_q8_sk(int mode, const int8_t *wq, const uint16_t *ws, int64_t N, int64_t K,
                   const int8_t *xq, const int8_t *xl, const float *xs, int64_t B, int splits,
                   float *y, void *workspace, size_t workspace_bytes, qdg_stream stream);

/*
 * One decode projection in one launch (B == 1): qdg_quantize_act, qdg_gemv_q8 with
 * `splits` chunks and qdg_sk_combine fused.  Every workgroup quantizes the
 * activation blocks of its own chunk into LDS with the quantizer's arithmetic,
 * runs the split-K GEMV on them, and the last workgroup of each 16-row tile to
 * finish sums the tile's partials in ascending chunk order (as qdg_gemv_q8_sk).
 * y [1][N] is bit-identical to the three calls.  QDG_DEQUANT (no quantizer)
 * splits K the same way with binary64 chunk partials, which the last workgroup
 * adds from +0 in ascending order in binary64 and rounds once to binary32: the
 * plain definition within the Dequant tolerance, not the bits of splits == 1.
 * Inputs:
 * device x float [1][K] (16-byte aligned); device workspace as for
 * qdg_gemv_q8_sk (at least qdg_gemv_sk_workspace_bytes(1, N, splits) bytes,
 * 256-byte aligned, zero-filled before its first use, left zeroed by every call
 * that completes; NULL allowed when splits == 1).  Calls that share a workspace
 * must not overlap in time.  The quantized words are not written out.
 */
int qdg_gemv_q8_fused(int mode, const int8_t *wq, const uint16_t *ws, int64_t N, int64_t K,
                      const float *x, int splits, float *y, void *workspace,
                      size_t workspace_bytes, qdg_stream stream);

/* Bytes of device workspace qdg_argmax needs for B rows of N values. */
size_t qdg_argmax_workspace_bytes(int64_t B, int64_t N);

/*
 * idx[t] = the smallest i with y[t][i] equal to the row's maximum (lane kernel
 * library page, module doc: first of equal maxima; megakernel page: amax_key,
 * ph_argmax_part, ph_argmax_fin).  Values compare as IEEE floats (-0 equals +0);
 * NaN is outside the contract.  Device pointers: y [B][N], idx int32 [B],
 * workspace of at least qdg_argmax_workspace_bytes(B, N) bytes (contents on
 * entry ignored, on return unspecified).  1 <= B, 1 <= N < 2^31.
 */
int qdg_argmax(const float *y, int64_t B, int64_t N, int32_t *idx,
               void *workspace, size_t workspace_bytes, qdg_stream stream);

/* Bytes of device workspace qdg_gemv_q8_argmax needs for N output rows (0 if N is out of range). */
size_t qdg_gemv_argmax_workspace_bytes(int64_t N);

/*
 * The LM-head tail in two launches (B == 1, splits == 1): the GEMV of
 * qdg_gemv_q8 writes the logits y [1][N] and, from each workgroup of 16 rows,
 * the arg-max key of its largest logit (megakernel page: amax_key and the
 * per-block arg-max partials of ph_argmax_part, here in the GEMV's epilogue);
 * a final pass over the keys writes idx[0] = the smallest i with y[i] equal to
 * the maximum (lane kernel library page, module doc: first of equal maxima;
 * IEEE comparison, -0 equals +0, NaN outside the contract).  y is the same as
 * qdg_gemv_q8's and idx the same as qdg_argmax's over it.  Arguments as
 * qdg_gemv_q8 (x for QDG_DEQUANT, else xq/xs, and xl for QDG_TWOPASS), plus
 * device idx int32 [1] and a device workspace of at least
 * qdg_gemv_argmax_workspace_bytes(N) bytes, 8-byte aligned (contents on entry
 * ignored).  N < 2^31.
 */
int qdg_gemv_q8_argmax(int mode, const int8_t *wq, const uint16_t *ws, int64_t N, int64_t K,
                       const float *x, const int8_t *xq, const int8_t *xl, const float *xs,
                       float *y, int32_t *idx, void *workspace, size_t workspace_bytes,
                       qdg_stream stream);

/*
 * qdg_gemv_q8_argmax without a caller's workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same launches, logits and index as
 * qdg_gemv_q8_argmax, with the per-tile arg-max keys in a 1 MiB array that the
 * library holds on each GPU it runs on (taken at the first call on a device,
 * kept until the process ends; nothing is allocated per call).  N up to
 * 2,097,152 rows (131072 keys); larger N returns QDG_EWORKSPACE before anything
 * is enqueued.  Every call on a GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (two streams, or two threads) race on it: order
 * them.  The array needs no clearing: each call writes every key it reads.  The
 * stream must belong to the current device.  Other arguments, checks and
 * statuses as qdg_gemv_q8_argmax.
 */
int qdg_gemv_q8_argmax_noalloc(int mode, const int8_t *wq, const uint16_t *ws, int64_t N, int64_t K,
                               const float *x, const int8_t *xq, const int8_t *xl, const float *xs,
                               float *y, int32_t *idx, qdg_stream stream);

/*
 * The residual add and RMSNorm, then the activation quantizer, in one launch:
 * the producer of the words a quantized GEMV reads (lane kernel library page,
 * RMSNORM: v = x + r, y = v / sqrt(mean(v^2) + eps) * w, the sum written out
 * as the next residual stream; QWEN38 page, gk_add_rmsnorm_q8f).  Per row t:
 *   v = x[t] + r[t]   one binary32 addition per value (v = x[t] when r is NULL);
 *                     s[t] = v when s is given (s needs r);
 *   y = v / sqrt(mean(v^2) + eps) * w   evaluated in binary64 from the binary32
 *                     v and w, rounded once to binary32 (no w when w is NULL);
 *                     written to y when y is given;
 *   xq, xl, xs        y quantized as qdg_quantize_act quantizes it.
 * The binary32 y is within one unit in the last place of the exactly rounded
 * value, and is the same on every run.  QDG_DEQUANT writes only y (required;
 * xq, xl and xs must be NULL), for the Dequant GEMV that reads f32 activations.
 * QDG_INT8ACT needs xq and xs (xl NULL), QDG_TWOPASS all three.
 * Device pointers: x, r, s, y [B][K] (16-byte aligned); w [K] (16-byte
 * aligned); xq, xl [B][K] (16-byte aligned); xs [B][K/32].  s and y may be x
 * itself (an in-place residual update); no other buffers may overlap.
 * 1 <= B < 2^31, K a multiple of 32 with 32 <= K <= qdg_rmsnorm_max_k();
 * eps >= 0 and finite.  A row of zeros with eps == 0 gives NaN (0/0) as the
 * formula does; its words are then unspecified.
 */
int qdg_rmsnorm_quantize(int mode, const float *x, const float *r, float *s, const float *w,
                         float eps, int64_t B, int64_t K, float *y, int8_t *xq, int8_t *xl,
                         float *xs, qdg_stream stream);

/* The largest K qdg_rmsnorm_quantize accepts (one workgroup holds a row). */
int64_t qdg_rmsnorm_max_k(void);

/* Bytes of device workspace qdg_gemv_q8_rmsnorm needs for N output rows (0 if N
 * is out of its range): one word a row, in whole 256-byte lines. */
size_t qdg_gemv_rmsnorm_workspace_bytes(int64_t N);

/* The largest N qdg_gemv_q8_rmsnorm accepts: the last workgroup holds the row's
 * N binary32 values in its LDS between the norm's two passes. */
int64_t qdg_gemv_rmsnorm_max_n(void);

/*
 * A projection with the residual add, the RMSNorm and the quantizer of the next
 * projection's activation in its epilogue, in one launch (lane kernel library
 * page, GEMV_Q8_NORM, lk_gemv_q8_norm: the blocks write their rows, and one
 * block then norms the row they make up).  Here every workgroup publishes its
 * rows to the workspace's slots, and one more workgroup gathers them as they
 * fill and runs the norm and the quantizer.  One activation row (B == 1).  Its
 * outputs are bit-identical to
 *   qdg_gemv_q8_sk(mode, wq, ws, N, K, xq, xl, xs, 1, splits, y, ...)
 *   qdg_rmsnorm_quantize(qmode, y, r, s, w, eps, 1, N, yn, hq, hl, hs, ...)
 * run one after the other: y [N] is the projection, s = y + r the next residual
 * stream, yn the normed row and (hq, hl, hs) its words in mode qmode, ready for
 * the next projection's qdg_gemv_q8_sk.
 *   mode   QDG_INT8ACT or QDG_TWOPASS (QDG_DEQUANT: QDG_EMODE), with xq, xl, xs
 *          as qdg_gemv_q8_sk takes them;
 *   splits one that qdg_gemv_sk_combines_in_workgroup accepts for (mode, K),
 *          else QDG_EMODE: the chunks of every row meet inside a workgroup;
 *   qmode  QDG_DEQUANT (writes only yn, required; hq, hl, hs NULL),
 *          QDG_INT8ACT (hq, hs; hl NULL) or QDG_TWOPASS (hq, hl, hs), as
 *          qdg_rmsnorm_quantize's mode;
 *   y, yn  f32 [N] or NULL each; r, s [N], r or NULL, s only with r; w [N] or
 *          NULL; eps >= 0 and finite.
 * Device pointers; wq, ws, xq, xl, xs aligned as qdg_gemv_q8_sk asks; y 4-byte
 * aligned; r, s, w, yn, hq, hl 16-byte aligned, hs 4-byte aligned.  N a
 * multiple of 32 with 32 <= N <= qdg_gemv_rmsnorm_max_n(); K >= 32, a multiple
 * of 32.  s may be r (an in-place residual update); no other buffers overlap.
 * workspace: at least qdg_gemv_rmsnorm_workspace_bytes(N) bytes, 256-byte
 * aligned, zero-filled before its first use and left zeroed by every call that
 * completes; calls that share a workspace must not overlap in time.
 */
int qdg_gemv_q8_rmsnorm(int mode, const int8_t *wq, const uint16_t *ws, int64_t N, int64_t K,
                        const int8_t *xq, const int8_t *xl, const float *xs, int splits, float *y,
                        const float *r, float *s, const float *w, float eps, int qmode, float *yn,
                        int8_t *hq, int8_t *hl, float *hs, void *workspace, size_t workspace_bytes,
                        qdg_stream stream);

/*
 * SwiGLU, then the activation quantizer, in one launch (lane kernel library
 * page, lk_act and GLU: silu(g) = g / (1 + e^-g), times u; QWEN38 page,
 * gk_silu_had_q8): h = (g / (1 + exp(-g))) * u per value, evaluated in binary64
 * from the binary32 g and u and rounded once to binary32 (within one unit in
 * the last place of the exactly rounded value); written to h when h is given;
 * then quantized as qdg_quantize_act quantizes it.  QDG_DEQUANT writes only h
 * (required; xq, xl, xs NULL).  Device pointers: g, u, h [B][K] (16-byte
 * aligned; h may be g or u); xq, xl [B][K] (16-byte aligned), xs [B][K/32].
 * B >= 1, K >= 32 and a multiple of 32, B*K < 2^62.
 */
int qdg_swiglu_quantize(int mode, const float *g, const float *u, int64_t B, int64_t K,
                        float *h, int8_t *xq, int8_t *xl, float *xs, qdg_stream stream);

/* The activations of the gated product (lane kernel library page, lk_act's ACT numbers). */
enum {
  QDG_ACT_SILU = 0,      /* g / (1 + e^-g): SwiGLU                                       */
  QDG_ACT_SIGMOID = 1,   /* 1 / (1 + e^-g)                                               */
  QDG_ACT_GELU_TANH = 2  /* g / (1 + e^-2z), z = sqrt(2/pi) * (g + 0.044715 g^3): GeGLU  */
};

/*
 * The same with any of lk_act's activations (lane kernel library page, lk_act
 * and GLU / lk_gemv_glu: u * act(g); the megakernel page's gelu-gated MLP):
 * h = act(g) * u per value, each step in binary64 from the binary32 g and u in
 * the order written -- g^3 as (g*g)*g, the GELU's constants the binary64 values
 * of sqrt(2/pi) and 0.044715 -- and rounded once to binary32 (within one unit in
 * the last place of the exactly rounded value); then quantized as
 * qdg_quantize_act quantizes it.  act QDG_ACT_SILU is qdg_swiglu_quantize, bit
 * for bit.  An act outside the three: QDG_EINVAL.  Arguments otherwise as
 * qdg_swiglu_quantize.
 */
int qdg_glu_quantize(int act, int mode, const float *g, const float *u, int64_t B, int64_t K,
                     float *h, int8_t *xq, int8_t *xl, float *xs, qdg_stream stream);

/*
 * Up to QDG_MAX_PARTS weight matrices over one activation row in one launch:
 * q, k and v, or gate and up, side by side (lane kernel library page,
 * GEMV_PARTS, lk_parts, lk_part_y).  parts (host array of nparts) gives each
 * matrix and its output; all share K and the activation.  Every part's y is
 * bit-identical to the single-matrix call with the same splits:
 *   QDG_INT8ACT, QDG_TWOPASS: qdg_gemv_q8_sk with (xq, xl, xs) -- splits must
 *     be one it combines inside a workgroup (qdg_gemv_sk_combines_in_workgroup
 *     == 1), else QDG_EMODE;
 *   QDG_DEQUANT: qdg_gemv_q8_fused with x (splits at most 16 non-empty chunks,
 *     else QDG_EMODE).
 * Needs no workspace.  Alignment as the single-matrix calls; 1 <= nparts <=
 * QDG_MAX_PARTS, every N >= 1, K >= 32 and a multiple of 32.
 */
int qdg_gemv_q8_parts(int mode, const qdg_part *parts, int nparts, int64_t K, const float *x,
                      const int8_t *xq, const int8_t *xl, const float *xs, int splits,
                      qdg_stream stream);

/*
 * The gate and up projections of one activation row with the SwiGLU and the
 * quantizer as the epilogue, in one launch (lane kernel library page, GLU,
 * lk_gemv_glu with a quantized output; lk_act): g = Wg x and u = Wu x as
 * qdg_gemv_q8 computes them (splits 1), h = silu(g) * u as qdg_swiglu_quantize
 * computes it, and (hq, hl, hs) = h quantized in the same mode -- the words the
 * down projection reads.  Bit-identical to those three calls; g and u never
 * reach memory.  QDG_INT8ACT or QDG_TWOPASS (hl exactly under TwoPass).
 * Device pointers: wg, wu int8 [F][K] (16-byte aligned); sg, su binary16 bits
 * [F][K/32]; xq, xl [K], xs [K/32] (from qdg_quantize_act or a producer); h f32
 * [F] or NULL (16-byte aligned); hq, hl [F]; hs [F/32].  F a positive multiple
 * of 32 (one quantized block per 32 outputs); K a multiple of 32 whose
 * activation row and 64 rows of scales fit the LDS budget (K up to 13184 for
 * QDG_TWOPASS, 15776 for QDG_INT8ACT), else QDG_EMODE.
 */
int qdg_gemv_glu_q8(int mode, const int8_t *wg, const uint16_t *sg, const int8_t *wu,
                    const uint16_t *su, int64_t F, int64_t K, const int8_t *xq, const int8_t *xl,
                    const float *xs, float *h, int8_t *hq, int8_t *hl, float *hs, qdg_stream stream);

/* The same with any of lk_act's activations (h = act(g) * u as qdg_glu_quantize
 * computes it; lane kernel library page, lk_gemv_glu's ACT): bit-identical to two
 * qdg_gemv_q8 calls and qdg_glu_quantize.  act QDG_ACT_SILU is qdg_gemv_glu_q8;
 * an act outside the three: QDG_EINVAL.  Arguments otherwise as qdg_gemv_glu_q8. */
int qdg_gemv_glu_act_q8(int act, int mode, const int8_t *wg, const uint16_t *sg, const int8_t *wu,
                        const uint16_t *su, int64_t F, int64_t K, const int8_t *xq, const int8_t *xl,
                        const float *xs, float *h, int8_t *hq, int8_t *hl, float *hs, qdg_stream stream);

/*
 * The gate and up projections under the Dequant numerics with the gated product
 * as the epilogue, in one launch (lane kernel library page, GLU: lk_gemv_glu
 * with the Dequant accumulator and a binary32 output; lk_act): g = Wg x and
 * u = Wu x as qdg_gemv_q8 computes them under QDG_DEQUANT (splits 1: the same
 * chunk count for F rows and the same order), h = act(g) * u as
 * qdg_glu_quantize computes it.  Bit-identical to those three calls (the
 * producer under QDG_DEQUANT, h only) while QDG_TUNE_DQ_SEG keeps its default;
 * g and u never reach memory.  h is the input of the down projection under
 * QDG_DEQUANT.
 * Device pointers: wg, wu int8 [F][K] (16-byte aligned); sg, su binary16 bits
 * [F][K/32] (2-byte aligned); x f32 [K] (16-byte aligned); h f32 [F] (4-byte
 * aligned), which must not overlap x, the weights or the scales (QDG_EINVAL).
 * act one of QDG_ACT_*, else QDG_EINVAL.  F >= 1 (any F: h is not quantized)
 * with F/4 < 2^31, K >= 32 a multiple of 32 up to 2^31, else QDG_ESHAPE.
 */
int qdg_gemv_glu_dequant(int act, const int8_t *wg, const uint16_t *sg, const int8_t *wu,
                         const uint16_t *su, int64_t F, int64_t K, const float *x, float *h,
                         qdg_stream stream);

/* GGUF type numbers of the other block formats (qdg_gemv_fmt). */
enum {
  QDG_FMT_Q4_0 = 2, QDG_FMT_Q4_1 = 3, QDG_FMT_Q5_0 = 6, QDG_FMT_Q5_1 = 7,
  QDG_FMT_Q2_K = 10, QDG_FMT_Q3_K = 11, QDG_FMT_Q4_K = 12, QDG_FMT_Q5_K = 13,
  QDG_FMT_Q6_K = 14, QDG_FMT_IQ4_NL = 20, QDG_FMT_IQ4_XS = 23, QDG_FMT_MXFP4 = 39
};

/* Host only: bytes of one K-value row in block format fmt (K/32 blocks of 17-24
 * bytes, or K/256 super-blocks of 84-210 bytes); 0 for an unknown format or a K
 * that is not a whole number of its blocks. */
int64_t qdg_fmt_row_bytes(int fmt, int64_t K);

/*
 * y[o] = sum_k W[o][k] x[k] for a matrix kept in another GGUF block format, its
 * blocks as the checkpoint stores them, row o at w + o*qdg_fmt_row_bytes(fmt, K)
 * (lane kernel library page: module doc on the other formats; BLOCKS / lk_sub
 * for the layouts; lk_row_dot, lk_sub_dot for the sums).  A 32-weight sub-block
 * decodes to int8 levels with a scale d and an offset c per half of 16,
 * weight = d*level + c.
 *  QDG_DEQUANT  reads x; each weight fl(fl(d*level) + c), products and sums in
 *               binary64, rounded once.
 *  QDG_INT8ACT  reads xq, xs (xq, xl, xs under QDG_TWOPASS); per sub-block g the
 *  QDG_TWOPASS  exact dots dh = sum level*h and sh = sum h of each half, part =
 *               ((d0*dh0 + c0*sh0) + d1*dh1) + c1*sh1 with one rounding per
 *               operation, TwoPass adding fl(2^-7 * the same with the low
 *               words); p <- fma(xs[g], part, p) into partial g mod 4 in
 *               ascending g, then (P0 + P2) + (P1 + P3).
 * splits: the row is cut into the chunks of the QWEN38 page's split-K rule
 * (gk_gemv_hl_sk: 512-value groups, ceil(groups / splits) a chunk, the K mod 512
 * tail in the last), each chunk summed as above from +0 and the chunk partials
 * added in ascending chunk order from +0 (gk_sk_combine) -- in binary32 for the
 * quantized modes, binary64 before the one rounding for QDG_DEQUANT.  splits == 1
 * is the unsplit row.  The chunks are summed by the waves of one workgroup,
 * several chunks a wave in turn where that lets every workgroup be resident at
 * once.
 * Batch 1.  w 16-byte aligned; x, xq, xl 16-byte aligned; y [N].  N >= 1 and K
 * a positive whole number of the format's blocks; 1 <= splits <= QDG_MAX_SPLITS
 * (QDG_EINVAL otherwise).
 */
int qdg_gemv_fmt(int fmt, int mode, const uint8_t *w, int64_t N, int64_t K, const float *x,
                 const int8_t *xq, const int8_t *xl, const float *xs, int splits, float *y,
                 qdg_stream stream);

/* Host only; asks the current device (its compute-unit count, the kernel's
 * occupancy): the chunk waves a workgroup's rows get in qdg_gemv_fmt for this
 * shape, W >= 1 -- each wave sums the non-empty chunks w, w + W, ... of the
 * split rule in turn; W equal to the chunk count is a wave a chunk.  The result
 * never changes the output bits.  Negative status on bad arguments (those
 * qdg_gemv_fmt rejects without touching memory). */
int qdg_gemv_fmt_chunk_waves(int fmt, int mode, int64_t N, int64_t K, int splits);

/* Host only, the same for the Dequant chunk-wave kernel of qdg_gemv_q8_fused and
 * qdg_gemv_q8_parts on one matrix of N rows: QDG_EMODE where that kernel does
 * not serve (K, splits). */
int qdg_gemv_dq_chunk_waves(int64_t N, int64_t K, int splits);

/*
 * Test hook: the exact int32 per-block dots the GEMV forms (lane kernel library
 * page, lk_q8_block_dot), dh[t][o][g] = sum_{k in block g} wq[o][k]*xq[t][k] and,
 * under QDG_TWOPASS, dl[t][o][g] with xl (dl must be NULL for QDG_INT8ACT).
 * Device pointers; dh, dl int32 [B][N][K/32]; B in [1, QDG_MAX_B].
 */
int qdg_block_dots(int mode, const int8_t *wq, int64_t N, int64_t K,
                   const int8_t *xq, const int8_t *xl, int64_t B,
                   int32_t *dh, int32_t *dl, qdg_stream stream);

/*
 * Measurement hook: reads `bytes` bytes of device memory at `buf` once, as fast
 * as the library knows how (contiguous 64 KiB slabs per workgroup, 16-byte
 * nontemporal loads), and does nothing else, so its time is the practical
 * ceiling of a GEMV launch that moves the same bytes.  `sink` is a device array
 * of 256 uint32 that is written only in the practically impossible case that
 * the folded data hits one fixed value (it keeps the loads from being dead).
 * bytes >= 16 and a multiple of 16; buf 16-byte aligned.
 */
int qdg_stream_read(const void *buf, int64_t bytes, uint32_t *sink, qdg_stream stream);

/*
 * Row-tiled weights (megakernel page, the GEMV's tiled-weights option: weight
 * tiles of consecutive rows stored together, so the loads that one group of
 * rows issues at once form one contiguous stream; only addresses change).  The
 * tile here is four rows by 256 values, the bytes of one 64-lane request of the
 * split-K GEMV: wt byte ((t*(K/256) + s)*4 + r)*256 + c holds wq row 4t + r,
 * column 256s + c.  wq [N][K] and wt [N*K] are device arrays, 16-byte aligned,
 * not overlapping (QDG_EINVAL if they do); N a positive multiple of 4, K a
 * positive multiple of 256 (else QDG_ESHAPE).  The weight scales keep their
 * plain [N][K/32] layout.  The caller owns both arrays.
 */
int qdg_q8_tile_rows(const int8_t *wq, int64_t N, int64_t K, int8_t *wt, qdg_stream stream);

/*
 * qdg_gemv_q8_sk's in-workgroup placement over row-tiled weights wt (from
 * qdg_q8_tile_rows): the same terms in the same order, so y [1][N] is
 * bit-identical to qdg_gemv_q8_sk over the plain weights with the same splits.
 * QDG_INT8ACT or QDG_TWOPASS (xl as qdg_gemv_q8_sk); splits must be one that
 * qdg_gemv_sk_combines_in_workgroup accepts for (mode, K), else QDG_EMODE; N a
 * multiple of 4 and K of 256 (else QDG_ESHAPE).  Alignment as qdg_gemv_q8_sk
 * (wt 16 bytes).  Needs no workspace.
 */
int qdg_gemv_q8_sk_tiled(int mode, const int8_t *wt, const uint16_t *ws, int64_t N, int64_t K,
                         const int8_t *xq, const int8_t *xl, const float *xs, int splits, float *y,
                         qdg_stream stream);

/*
 * MFMA-tiled weights for the batched GEMV (megakernel page, the GEMV's
 * tiled-weights option: only the addresses of the weights change).  One record
 * per (64-row group q, 8-block step s, residue r in 0..3), in that row-major
 * order, holds what one wave of qdg_gemv_q8_mma_tiled consumes in one step:
 *   - bytes 0..4095: byte 1024*m + 16*l + 8*h + j (tile m in 0..3, lane l in
 *     0..63, c = l mod 16, u = l / 16, h in 0..1) is byte 8*u + j of block
 *     8*s + r + 4*h of row 64*q + 16*m + c -- a lane's 16 bytes are the int8
 *     MFMA's B operands of the step's two blocks;
 *   - bytes 4096..4351: 16-bit word 8*c + 2*m + h is the binary16 scale (bits)
 *     of that row and block.
 * Rows past N are zero.  qdg_q8_tile_mma_bytes gives the size,
 * ceil(N/64) * (K/256) * 4 * 4352, or 0 when the shape is not served: K a
 * positive multiple of 256 below 2^30, N >= 1 (and the record count below
 * 2^31).  wq [N][K] (16-byte aligned), ws [N][K/32] (2-byte aligned) and wt
 * (16-byte aligned) are device arrays; wt must not overlap wq or ws
 * (QDG_EINVAL).  The caller owns all three.
 */
int64_t qdg_q8_tile_mma_bytes(int64_t N, int64_t K);
int qdg_q8_tile_mma(const int8_t *wq, const uint16_t *ws, int64_t N, int64_t K, uint8_t *wt,
                    qdg_stream stream);

/*
 * qdg_quantize_act for 1 <= B <= QDG_MAX_B rows, with the words and scales
 * written in the MFMA order that qdg_gemv_q8_mma_tiled reads, in T activation
 * tiles of 16 rows (T = 1, 2 or 4 for B <= 16, <= 32, <= 64; rows 16*a .. 16*a + 15
 * form tile a).  Tile a holds, for step s (8 blocks) and residue r in 0..3, a
 * record (s, r) of 1024 word bytes -- byte 16*l + 8*h + j (lane l, t = l mod 16,
 * u = l / 16) being word 8*u + j of block 8*s + r + 4*h of row 16*a + t -- and 32
 * scales, scale 16*h + t of the record being that block's scale of row 16*a + t.
 * Records run (s, r) in row-major order within a tile, tiles one after the
 * other: xq (and xl under QDG_TWOPASS) hold 16*T*K bytes, xs 16*T*K/32 floats.
 * The words and scales of rows t < B are qdg_quantize_act's on the same x, bit
 * for bit; rows B..16*T-1 are those of a zero row.  x [B][K] (16-byte aligned);
 * xq, xl 16-byte aligned; xs 4-byte.  K as qdg_q8_tile_mma (else QDG_ESHAPE).
 */
int qdg_quantize_act_mma(int mode, const float *x, int64_t B, int64_t K, int8_t *xq, int8_t *xl,
                         float *xs, qdg_stream stream);

/*
 * qdg_gemv_q8 for 1 <= B <= QDG_MAX_B activation rows over MFMA-tiled weights
 * wt (from qdg_q8_tile_mma) and MFMA-ordered activations xq, xl, xs (from
 * qdg_quantize_act_mma with the same B): the same terms in the same order (the
 * int8 MFMA's exact block dots, partial g mod 4, (P0 + P2) + (P1 + P3)), so out
 * is bit-identical to qdg_gemv_q8 over the plain weights and the plain
 * activations of the same x with the same B and splits, and every row to its
 * batch-1 result.  QDG_INT8ACT or QDG_TWOPASS (xl NULL for QDG_INT8ACT;
 * QDG_DEQUANT gives QDG_EMODE).  splits == 1: out is y [B][N]; splits > 1:
 * partials [splits][B][N] for qdg_sk_combine.  Shapes as qdg_q8_tile_mma (else
 * QDG_ESHAPE).  wt, xq, xl 16-byte aligned, xs and out 4-byte.  Needs no
 * workspace.
 */
int qdg_gemv_q8_mma_tiled(int mode, const uint8_t *wt, int64_t N, int64_t K, const int8_t *xq,
                          const int8_t *xl, const float *xs, int64_t B, int splits, float *out,
                          qdg_stream stream);

/*
 * The gate and up projections of 1 <= B <= QDG_MAX_B activation rows with the
 * gated product and the quantizer as the epilogue, in one launch (lane kernel
 * library page, GLU: lk_gemv_glu with a quantized output and its ACT; lk_act),
 * over MFMA-tiled gate and up weights wgt, wut (qdg_q8_tile_mma of Wg, Wu, each
 * [F][K]) and MFMA-ordered activations xq, xl, xs (qdg_quantize_act_mma with the
 * same B).  g = Wg x and u = Wu x as qdg_gemv_q8_mma_tiled computes them with
 * splits 1, h = act(g) * u as qdg_glu_quantize computes it, and h quantized in
 * the same mode and written in the MFMA order of qdg_quantize_act_mma for a
 * projection with K = F: hq (and hl under QDG_TWOPASS) 16*T*F bytes, hs
 * 16*T*F/32 floats, T as qdg_quantize_act_mma for B, rows B..16*T-1 those of a
 * zero row.  So (hq, hl, hs) are the bytes of qdg_gemv_q8_mma_tiled twice,
 * qdg_glu_quantize (h) and qdg_quantize_act_mma on h -- the down projection's
 * operands -- and h [B][F] (optional, NULL to skip) the producer's h, bit for
 * bit; g and u never reach memory.  act one of QDG_ACT_*, mode QDG_INT8ACT or
 * QDG_TWOPASS (xl, hl NULL under QDG_INT8ACT), else QDG_EINVAL.  K as
 * qdg_q8_tile_mma and F a positive multiple of 256 (the down projection's K),
 * else QDG_ESHAPE.  wgt, wut, xq, xl, h 16-byte aligned; xs, hq, hl, hs 4-byte.
 * No output may overlap an input (QDG_EINVAL).  Needs no workspace.
 */
int qdg_gemv_glu_mma_tiled(int act, int mode, const uint8_t *wgt, const uint8_t *wut, int64_t F,
                           int64_t K, const int8_t *xq, const int8_t *xl, const float *xs, int64_t B,
                           float *h, int8_t *hq, int8_t *hl, float *hs, qdg_stream stream);

/*
 * Tuning and test hooks.  Process-wide settings that choose among the library's
 * kernels, staging forms and launch shapes for the same call -- never the
 * arithmetic or its order, so every setting gives the same output bits -- for
 * tests that compare two kernels on one shape and for sweeps.  Every knob starts
 * at -1 (the library's own choice) and only these calls change it: the
 * environment is never read.  Not meant to be changed while another thread is
 * inside the library.
 */
enum {
  QDG_TUNE_SK_WSPLIT = 0,  /* 0: qdg_gemv_q8_sk always combines through the workspace      */
  QDG_TUNE_WS_DMA = 1,     /* 0: the in-workgroup split and the GLU kernel copy their staged */
                           /*    bytes through registers instead of LDS DMA                  */
  QDG_TUNE_WS_LOCAL = 2,   /* 1: per-wave staging, 0: workgroup-wide staging                 */
  QDG_TUNE_WS_ROWS = 3,    /* 1..4: row groups a workgroup of the in-workgroup split         */
  QDG_TUNE_DQ_SEG = 4,     /* 0: Dequant split-K takes the last-arriver kernel               */
  QDG_TUNE_DQ_ROWS = 5,    /* 1..4: row groups a workgroup of the Dequant chunk waves        */
  QDG_TUNE_DQ_X64 = 6,     /* 0: the unsplit Dequant kernel keeps its window in binary32     */
  QDG_TUNE_MFMA_GENERAL = 7, /* 1: the batched GEMV on its general (register) path           */
  QDG_TUNE_MFMA_SHAPE = 8, /* 100*waves + 10*tiles + ring of the batched fast path (B <= 16);
                              1000 + 10*tiles + ring: one wave per workgroup, own ring       */
  QDG_TUNE_MFMA_WIDE = 9,  /* the same for 16 < B <= 64                                      */
  QDG_TUNE_GEMV_ORDER = 10, /* 0: tile-major, 1: chunk-major workgroup order (split GEMV)    */
  QDG_TUNE_GEMV_RPW = 11,  /* 4 or 8 rows a wave (batch-1 GEMV)                              */
  QDG_TUNE_GEMV_UNROLL = 12, /* 2, 4 or 8 steps in flight with eight rows a wave             */
  QDG_TUNE_REJECT_LAUNCH = 13, /* 1: every launch asks for a 2048-thread workgroup, which the */
                           /*    HIP runtime refuses before anything is enqueued: the calls  */
                           /*    then return QDG_EHIP (the error path's test hook)           */
  QDG_TUNE_FMT_WAVES = 14, /* 1..16 chunk waves a row group of the block-format GEMV; each   */
                           /*    wave sums every W-th non-empty chunk in turn               */
  QDG_TUNE_DQ_WAVES = 15,  /* 1..16 chunk waves a row group of the Dequant chunk-wave kernel */
  QDG_TUNE_MT_GROUPS = 16, /* 1 or 2 64-row record groups a workgroup of qdg_gemv_q8_mma_tiled */
  QDG_TUNE_COUNT = 17
};

/* Sets knob to value (-1 restores the default).  QDG_EINVAL for an unknown knob. */
int qdg_set_tuning(int knob, int value);
/* The knob's current value (-1: default); QDG_EINVAL for an unknown knob. */
int qdg_get_tuning(int knob);

/*
 * Measurement hook: the next kernel that a call of this thread launches carries
 * the two events (hipEvent_t, created by the caller) on its own dispatch
 * (hipExtLaunchKernel): hipEventElapsedTime(start, stop) is then that kernel's
 * device duration, the time a kernel trace reports, without the stream work of
 * separately recorded events.  The binding covers one launch and is cleared by
 * it; for a call that launches more than one kernel, the first is timed.
 * Passing NULLs clears it.  Returns QDG_OK.
 */
int qdg_time_next_launch(void *start, void *stop);

/*
 * Host only: the split-K chunk boundaries in 32-value blocks (QWEN38 page,
 * gk_gemv_hl_sk): K runs in 512-value superblocks, per = ceil((K/512)/splits),
 * chunk s takes superblocks [s*per, min((s+1)*per, K/512)) and the last chunk
 * also takes the K mod 512 tail.  first_block (host, splits + 1 entries)
 * receives the boundaries: chunk s is blocks [first_block[s], first_block[s+1]).
 */
int qdg_split_bounds(int64_t K, int splits, int32_t *first_block);

#ifdef __cplusplus
}
#endif

#endif /* QDG_H */
