// qdg_producers.hip -- the kernels that produce the GEMV's activation words.
// They fuse the quantizer into the step before the projection, so the f32
// activation makes no round trip through HBM and needs no launch of its own.
//
//  * k_rmsnorm_quant: the residual add and RMSNorm (lane kernel library page,
//    RMSNORM: v = x + r, y = v / sqrt(mean(v^2) + eps) * w; QWEN38 page,
//    gk_add_rmsnorm_q8f: the add writes the residual stream back), then the
//    32-value block quantizer on y.
//  * k_glu_quant: h = act(g) * u -- silu (SwiGLU), sigmoid or the tanh-form
//    GELU (lane kernel library page, lk_act and GLU; QWEN38 page,
//    gk_silu_had_q8; the megakernel page's gelu-gated MLP) -- then the same
//    quantizer on h.
//
// Arithmetic: the residual sum is one binary32 addition.  The norm and act are
// evaluated in binary64 from binary32 operands and rounded once to binary32.
// The squares are exact in binary64, and the row's sum of squares runs in a
// fixed order: per thread, then a butterfly inside each wave, then the waves in
// ascending order.  So a row's result does not change from run to run.  Each
// binary32 result is within one unit in the last place of the exactly rounded
// value.  The quantizer then runs on those binary32 values, exactly as
// qdg_quantize_act would on them.
//
// Layout: a row's K values are K/4 float4 chunks.  Chunk c of a row belongs to
// thread c mod T (round c / T).  A 32-value block is 8 consecutive chunks, so
// its 8 chunks sit in 8 consecutive lanes of one wave, the layout quant_lane4
// expects.
#include "qdg_device.h"

namespace qdg {
namespace {

constexpr int NT = 1024;  // threads of a norm workgroup (one workgroup per row)

// x, s and y may be the same buffer: every chunk is read and written by one
// thread only, each read before that thread's write.  KEEP holds the row's
// values in registers between the two passes; without it (the largest K, where
// they would not fit) the second pass reads them again: from s when s is
// written (s may be x), else x + r once more.
template <int MODE, int PER, bool KEEP>
__global__ __launch_bounds__(NT) void k_rmsnorm_quant(const float* x, const float* __restrict__ r, float* s,
                                                      const float* __restrict__ w, float eps, int64_t K, float* y,
                                                      int8_t* __restrict__ xq, int8_t* __restrict__ xl,
                                                      float* __restrict__ xs) {
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x, nc = K / 4;
  auto sum_in = [&](int64_t c) {
    const float4 v = *(const float4*)(x + row * K + 4 * c);
    return r ? add4(v, *(const float4*)(r + row * K + 4 * c)) : v;
  };
  float4 v[KEEP ? PER : 1];
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int64_t c = tid + (int64_t)j * NT;
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < nc) {
      t = sum_in(c);
      if (s) *(float4*)(s + row * K + 4 * c) = t;
    }
    acc += sq4(t);
    if constexpr (KEEP) v[j] = t;
  }
  // wave butterfly, then the NT/64 wave sums in ascending order (every thread the same)
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  __shared__ double red[NT / 64];
  if ((tid & 63) == 0) red[tid >> 6] = acc;
  __syncthreads();
  double sum = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) sum += red[i];
  const double den = norm_den(sum, K, eps);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int64_t c = tid + (int64_t)j * NT;
    const bool on = c < nc;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (on) {
      float4 t;
      if constexpr (KEEP)
        t = v[j];
      else
        t = s ? *(const float4*)(s + row * K + 4 * c) : sum_in(c);
      o = norm4(t, den, w != nullptr, w ? *(const float4*)(w + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f));
      if (y) *(float4*)(y + row * K + 4 * c) = o;
    }
    if constexpr (MODE != 0) {
      // every lane of the wave takes part in the block maximum; a block is wholly in or out
      int h, l;
      const float sc = quant_lane4<MODE>(o, &h, &l);
      if (on) {
        const int64_t e = row * K + 4 * c;
        *(int*)(xq + e) = h;
        if constexpr (MODE == 2) *(int*)(xl + e) = l;
        if ((c & 7) == 0) xs[e / QK] = sc;
      }
    }
  }
}

// Eight lanes a 32-value block, four values a lane, as k_quantize.  h may be g or u.
template <int MODE, int ACT>
__global__ __launch_bounds__(256) void k_glu_quant(const float* g, const float* u, float* h,
                                                      int8_t* __restrict__ xq, int8_t* __restrict__ xl,
                                                      float* __restrict__ xs, int64_t nblocks) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = gid >> 3;
  const bool on = blk < nblocks;
  const int64_t e = blk * QK + (gid & 7) * 4;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (on) {
    const float4 a = *(const float4*)(g + e), b = *(const float4*)(u + e);
    o = make_float4(glu_mul<ACT>(a.x, b.x), glu_mul<ACT>(a.y, b.y), glu_mul<ACT>(a.z, b.z), glu_mul<ACT>(a.w, b.w));
    if (h) *(float4*)(h + e) = o;
  }
  if constexpr (MODE != 0) {
    int hw, lw;
    const float sc = quant_lane4<MODE>(o, &hw, &lw);
    if (!on) return;
    *(int*)(xq + e) = hw;
    if constexpr (MODE == 2) *(int*)(xl + e) = lw;
    if ((gid & 7) == 0) xs[blk] = sc;
  }
}

template <int MODE>
hipError_t launch_rms(const float* x, const float* r, float* s, const float* w, float eps, int64_t B, int64_t K,
                      float* y, int8_t* xq, int8_t* xl, float* xs, hipStream_t st) {
  const int64_t per = (K / 4 + NT - 1) / NT;
  const dim3 grid((unsigned)B), block(NT);
#define QDG_RMS(P, KEEP)                                                                                      \
  return launch((k_rmsnorm_quant<MODE, P, KEEP>), grid, block, 0, st, x, r, s, w, eps, K, y, xq, xl, xs);
  if (per <= 1) { QDG_RMS(1, true) }
  if (per <= 2) { QDG_RMS(2, true) }
  if (per <= 4) { QDG_RMS(4, true) }
  QDG_RMS(8, false)
#undef QDG_RMS
}

template <int MODE, int ACT>
hipError_t launch_glu_ma(const float* g, const float* u, int64_t nblocks, float* h, int8_t* xq, int8_t* xl,
                         float* xs, hipStream_t st) {
  const int64_t threads = nblocks * 8;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  return launch(k_glu_quant<MODE, ACT>, grid, block, 0, st, g, u, h, xq, xl, xs, nblocks);
}

template <int ACT>
hipError_t launch_glu_a(int mode, const float* g, const float* u, int64_t nblocks, float* h, int8_t* xq,
                        int8_t* xl, float* xs, hipStream_t st) {
  if (mode == 0) return launch_glu_ma<0, ACT>(g, u, nblocks, h, xq, xl, xs, st);
  if (mode == 1) return launch_glu_ma<1, ACT>(g, u, nblocks, h, xq, xl, xs, st);
  return launch_glu_ma<2, ACT>(g, u, nblocks, h, xq, xl, xs, st);
}

}  // namespace

int64_t rmsnorm_max_k() { return (int64_t)NT * 8 * 4; }

hipError_t launch_rmsnorm_quant(int mode, const float* x, const float* r, float* s, const float* w, float eps,
                                int64_t B, int64_t K, float* y, int8_t* xq, int8_t* xl, float* xs, hipStream_t st) {
  if (mode == 0) return launch_rms<0>(x, r, s, w, eps, B, K, y, xq, xl, xs, st);
  if (mode == 1) return launch_rms<1>(x, r, s, w, eps, B, K, y, xq, xl, xs, st);
  return launch_rms<2>(x, r, s, w, eps, B, K, y, xq, xl, xs, st);
}

hipError_t launch_glu_quant(int act, int mode, const float* g, const float* u, int64_t nblocks, float* h,
                            int8_t* xq, int8_t* xl, float* xs, hipStream_t st) {
  if (act == 0) return launch_glu_a<0>(mode, g, u, nblocks, h, xq, xl, xs, st);
  if (act == 1) return launch_glu_a<1>(mode, g, u, nblocks, h, xq, xl, xs, st);
  return launch_glu_a<2>(mode, g, u, nblocks, h, xq, xl, xs, st);
}

}  // namespace qdg
