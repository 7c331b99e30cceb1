// qdg_dequant.hip -- the batch-1 Q8_0 GEMV under the Dequant numerics: the f32
// activation meets the scaled int8 weight and every product and sum is binary64,
// rounded once to binary32 at the end (lane kernel library page: module doc on the
// Dequant mode, lk_acc<0>, the Q == 0 branch of lk_q8_rows_dot, accumulator()).
//
// Any fixed binary64 order computes the plain definition to within a few binary64
// roundings; this kernel's order is:
//  * a lane holds 16 consecutive values of a block (the lane pair (2j, 2j+1)
//    holds block j of its step) and forms sum_i w_i*x_i by binary64 fused
//    multiply-adds from +0 in ascending i (every product w_i*x_i is exact);
//  * the pair's two half-block sums are added (low half + high half), and the
//    block's term is sigma * that sum (one binary64 rounding);
//  * terms go into partial g mod 4 in ascending block order, and the row is
//    (P0 + P2) + (P1 + P3), then one rounding to binary32.
// The lane layout, the LDS staging of the window (the f32 activation and the
// rows' weight scales) and the load pipeline are those of the quantized kernel
// (qdg_gemv.hip).
#include "qdg_device.h"

namespace qdg {
namespace {

constexpr int WG = 256;
constexpr int LDS_BUDGET = 56 * 1024;

__device__ __forceinline__ double half_dot16(int4 w, const float* __restrict__ x) {
  const int ww[4] = {w.x, w.y, w.z, w.w};
  double acc = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 xv = *(const float4*)(x + 4 * q);
    const float xx[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int wi = (int)(signed char)((ww[q] >> (8 * i)) & 255);
      acc = __fma_rn((double)wi, (double)xx[i], acc);
    }
  }
  return acc;
}

template <int RPW, int U>
__global__ __launch_bounds__(WG) void k_gemv_dequant(const int8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
                                                    const float* __restrict__ x, int64_t N, int64_t K, int win,
                                                    float* __restrict__ out) {
  constexpr int LPR = 64 / RPW;
  constexpr int BPS = LPR / 2;
  constexpr int TPP = BPS / 4;
  constexpr int ROWS = (WG / 64) * RPW;
  static_assert(TPP == 1 || TPP == 2, "RPW must be 4 or 8");
  extern __shared__ __align__(16) unsigned char lds[];
  float* lx = (float*)lds;                            // [win][32]
  uint16_t* lsg = (uint16_t*)(lx + (int64_t)win * QK);  // [ROWS][win]

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane / LPR, li = lane % LPR, j = li >> 1, hf = li & 1;
  const int64_t nb = K / QK;
  const int64_t o_wg = (int64_t)blockIdx.x * ROWS;
  const int rr = wave * RPW + r;
  const int64_t o = o_wg + rr;
  const bool row_ok = o < N;
  const int8_t* wrow = wq + (row_ok ? o : N - 1) * K + hf * 16;
  const uint16_t* my_sg = lsg + rr * win;

  double p = 0.0;
  for (int64_t wb0 = 0; wb0 < nb; wb0 += win) {
    const int64_t wb1 = wb0 + win < nb ? wb0 + win : nb;
    const int nwb = (int)(wb1 - wb0);
    const int nsteps = (nwb + BPS - 1) / BPS;
    const int ngroups = (nsteps + U - 1) / U;
    int4 wcur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int bl = u * BPS + j;
      wcur[u] = bl < nwb ? ld16_stream(wrow + (wb0 + bl) * QK) : make_int4(0, 0, 0, 0);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nwb * 8; i += WG) ((float4*)lx)[i] = ((const float4*)(x + wb0 * QK))[i];
    stage_scales(lsg, win, ws, nb, N, o_wg, ROWS, wb0, nwb, threadIdx.x, WG);
    __syncthreads();

    for (int gi = 0; gi < ngroups; ++gi) {
      int4 wnxt[U];
      const bool more = gi + 1 < ngroups;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int bl = ((gi + 1) * U + u) * BPS + j;
        wnxt[u] = more && bl < nwb ? ld16_stream(wrow + (wb0 + bl) * QK) : make_int4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int bl = (gi * U + u) * BPS + j;
        const bool ok = bl < nwb;
        const int blc = ok ? bl : 0;
        const double hsum = half_dot16(wcur[u], lx + blc * QK + hf * 16);
        const double other = dpp_f64<DPP_QUAD_SWAP1>(hsum);
        const double blk = __dadd_rn(hsum, other);  // the same bits in both lanes of the pair
        const double term = __dmul_rn((double)half_bits_to_float(my_sg[blc]), blk);
        p = ok ? __dadd_rn(p, term) : p;
        if constexpr (TPP == 2) {
          const double term2 = dpp_f64<DPP_ROW_SHL8>(term);
          p = bl + 4 < nwb ? __dadd_rn(p, term2) : p;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) wcur[u] = wnxt[u];
    }
  }
  const double t = __dadd_rn(p, dpp_f64<DPP_ROW_SHL4>(p));
  const double y = __dadd_rn(t, dpp_f64<DPP_ROW_SHL2>(t));
  if (li == 0 && row_ok) out[o] = (float)y;
}

}  // namespace

hipError_t launch_gemv_dequant(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                               float* out, hipStream_t st) {
  constexpr int RPW = 4, U = 4;
  constexpr int rows_per_wg = (WG / 64) * RPW;
  const int64_t nb = K / QK;
  const int cap = (LDS_BUDGET / (QK * 4 + 2 * rows_per_wg)) / SUPER * SUPER;
  int win = (int)(((nb + SUPER - 1) / SUPER) * SUPER);
  if (win > cap) win = cap;
  const size_t lds = (size_t)win * (QK * 4 + 2 * rows_per_wg);
  const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg)), block(WG);
  hipLaunchKernelGGL((k_gemv_dequant<RPW, U>), grid, block, lds, st, wq, ws, x, N, K, win, out);
  return hipGetLastError();
}

}  // namespace qdg
