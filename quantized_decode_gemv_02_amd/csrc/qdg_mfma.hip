// qdg_mfma.hip -- the batched (2 <= B <= 16) Q8_0 GEMV on int8 MFMA, Int8Act and
// TwoPass (lane kernel library page: lk_gemv_mma and its sizing helpers; the
// megakernel page's batched decode, whose rows sum exactly as a single row does).
//
// Every (t, o) output is summed exactly as the batch-1 kernel sums it: block g's
// exact int32 dot D (and E), the step p <- fma(a, b, p) of lk_q8_term into
// partial g mod 4, ascending blocks, then (P0 + P2) + (P1 + P3).  Only where the
// block dots come from differs: here one v_mfma_i32_16x16x64_i8 gives the 16x16
// dots of 16 activation rows t by 16 weight rows o over one 64-byte span.
//
//  * A wave owns TILES tiles of 16 weight rows.  Lane (col = l%16, grp = l/16)
//    loads 16 bytes at offset 16*grp of a 64-byte span (two blocks) of weight
//    row o0+col (B operand) and of activation row t = col (A operand), so the
//    MFMA sums the products of matching bytes.  With the A operand of lane
//    groups 2-3 set to zero the sum is the first block's dot; with groups 0-1
//    zero, the second block's.  A "quad" of 4 blocks (128 bytes a row, blocks
//    g = 4m..4m+3) takes two spans and four MFMAs, block 4m+k landing in
//    partial k -- compile-time register indices.
//  * The MFMA result gives lane (col, grp) the dots of t = 4*grp + i (i < 4)
//    with o = o0 + col; that lane keeps the 4 partials of those 4 (t, o) pairs,
//    so every chain lives in one lane, in ascending block order.
//  * Activation scales of the chunk are staged in LDS transposed, [block][t],
//    so a lane reads the 4 scales it needs with one ds_read_b128.
//  * Weight rows past N read row N-1 and store nothing; activation rows t >= B
//    are zero and store nothing.
#include "qdg_device.h"

namespace qdg {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int WG = 256;
constexpr int LDS_BUDGET = 56 * 1024;

__device__ __forceinline__ v4i as_v4i(int4 v) {
  v4i r;
  r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
  return r;
}

__device__ __forceinline__ v4i mfma16x16x64(v4i a, v4i b) {
  const v4i z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, z, 0, 0, 0);
}

template <int MODE, int TILES, int QD>
__global__ __launch_bounds__(WG) void k_gemv_mfma(const int8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
                                                 const int8_t* __restrict__ xq, const int8_t* __restrict__ xl,
                                                 const float* __restrict__ xs, int64_t N, int64_t K, int B, int S,
                                                 int win, float* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char lds[];
  float* sT = (float*)lds;  // [win][16]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t nb = K / QK;
  const int s_idx = blockIdx.y;
  int32_t g0, g1;
  split_range(K, S, s_idx, g0, g1);

  const int64_t o0 = ((int64_t)blockIdx.x * (WG / 64) + wave) * TILES * 16;
  const int8_t* wrow[TILES];
  const uint16_t* srow[TILES];
#pragma unroll
  for (int tl = 0; tl < TILES; ++tl) {
    int64_t o = o0 + tl * 16 + col;
    if (o >= N) o = N - 1;
    wrow[tl] = wq + o * K + grp * 16;
    srow[tl] = ws + o * nb;
  }
  const bool t_ok = col < B;
  const int8_t* arow = xq + (int64_t)(t_ok ? col : 0) * K + grp * 16;
  const int8_t* lrow = MODE == 2 ? xl + (int64_t)(t_ok ? col : 0) * K + grp * 16 : nullptr;
  const bool lo_half = grp < 2;  // lane groups 0-1 carry the first block of a span

  float p[TILES][4][4];
#pragma unroll
  for (int tl = 0; tl < TILES; ++tl)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) p[tl][i][q] = 0.0f;

  const int4 z4 = make_int4(0, 0, 0, 0);
  for (int wb0 = g0; wb0 < g1; wb0 += win) {
    const int wb1 = min(wb0 + win, g1);
    const int nwb = wb1 - wb0;
    __syncthreads();
    for (int i = threadIdx.x; i < nwb * 16; i += WG) {
      const int bl = i >> 4, t = i & 15;
      sT[i] = t < B ? xs[(int64_t)t * nb + wb0 + bl] : 0.0f;
    }
    __syncthreads();

    // QD quads (4*QD blocks) per iteration: every load of the iteration is issued
    // before the first MFMA, so a wave keeps QD*TILES*2 KB of weights in flight.
    for (int bq = wb0; bq < wb1; bq += 4 * QD) {
      int4 wv[QD][TILES][2];
      unsigned short sgb[QD][TILES][4];
      int4 av[QD][2], lv[QD][2];
#pragma unroll
      for (int qd = 0; qd < QD; ++qd) {
        const int b = bq + 4 * qd;
        const bool v0 = b < wb1, v1 = b + 1 < wb1, v2 = b + 2 < wb1, v3 = b + 3 < wb1;
        const bool span0 = v0 && (lo_half || v1), span1 = v2 && (lo_half || v3);
        av[qd][0] = t_ok && span0 ? *(const int4*)(arow + (int64_t)b * QK) : z4;
        av[qd][1] = t_ok && span1 ? *(const int4*)(arow + (int64_t)b * QK + 64) : z4;
        if constexpr (MODE == 2) {
          lv[qd][0] = t_ok && span0 ? *(const int4*)(lrow + (int64_t)b * QK) : z4;
          lv[qd][1] = t_ok && span1 ? *(const int4*)(lrow + (int64_t)b * QK + 64) : z4;
        }
#pragma unroll
        for (int tl = 0; tl < TILES; ++tl) {
          wv[qd][tl][0] = span0 ? *(const int4*)(wrow[tl] + (int64_t)b * QK) : z4;
          wv[qd][tl][1] = span1 ? *(const int4*)(wrow[tl] + (int64_t)b * QK + 64) : z4;
          sgb[qd][tl][0] = v0 ? srow[tl][b] : (unsigned short)0;
          sgb[qd][tl][1] = v1 ? srow[tl][b + 1] : (unsigned short)0;
          sgb[qd][tl][2] = v2 ? srow[tl][b + 2] : (unsigned short)0;
          sgb[qd][tl][3] = v3 ? srow[tl][b + 3] : (unsigned short)0;
        }
      }
#pragma unroll
      for (int qd = 0; qd < QD; ++qd) {
        const int b = bq + 4 * qd;  // b - g0 is a multiple of 4: block b + k is partial k
        if (b >= wb1) break;        // uniform over the wave
        const bool vk[4] = {true, b + 1 < wb1, b + 2 < wb1, b + 3 < wb1};
        const v4i A[4] = {as_v4i(lo_half ? av[qd][0] : z4), as_v4i(lo_half ? z4 : av[qd][0]),
                          as_v4i(lo_half ? av[qd][1] : z4), as_v4i(lo_half ? z4 : av[qd][1])};
        v4i L[4];
        if constexpr (MODE == 2) {
          L[0] = as_v4i(lo_half ? lv[qd][0] : z4);
          L[1] = as_v4i(lo_half ? z4 : lv[qd][0]);
          L[2] = as_v4i(lo_half ? lv[qd][1] : z4);
          L[3] = as_v4i(lo_half ? z4 : lv[qd][1]);
        }
        float sv[4][4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 s4 = vk[k] ? *(const float4*)(sT + (b + k - wb0) * 16 + grp * 4) : make_float4(0, 0, 0, 0);
          sv[k][0] = s4.x; sv[k][1] = s4.y; sv[k][2] = s4.z; sv[k][3] = s4.w;
        }
#pragma unroll
        for (int tl = 0; tl < TILES; ++tl) {
          const v4i W0 = as_v4i(wv[qd][tl][0]), W1 = as_v4i(wv[qd][tl][1]);
          v4i D[4], E[4];
          D[0] = mfma16x16x64(A[0], W0);
          D[1] = mfma16x16x64(A[1], W0);
          D[2] = mfma16x16x64(A[2], W1);
          D[3] = mfma16x16x64(A[3], W1);
          if constexpr (MODE == 2) {
            E[0] = mfma16x16x64(L[0], W0);
            E[1] = mfma16x16x64(L[1], W0);
            E[2] = mfma16x16x64(L[2], W1);
            E[3] = mfma16x16x64(L[3], W1);
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (!vk[k]) continue;  // uniform over the wave
            const float sg = half_bits_to_float(sgb[qd][tl][k]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float ta, tb;
              q8_term<MODE>(sg, sv[k][i], D[k][i], MODE == 2 ? E[k][i] : 0, ta, tb);
              p[tl][i][k] = __fmaf_rn(ta, tb, p[tl][i][k]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int tl = 0; tl < TILES; ++tl) {
    const int64_t o = o0 + tl * 16 + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = grp * 4 + i;
      const float y = __fadd_rn(__fadd_rn(p[tl][i][0], p[tl][i][2]), __fadd_rn(p[tl][i][1], p[tl][i][3]));
      if (t < B && o < N) out[((int64_t)s_idx * B + t) * N + o] = y;
    }
  }
}

}  // namespace

hipError_t launch_gemv_mfma(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K,
                            const int8_t* xq, const int8_t* xl, const float* xs, int64_t B, int splits,
                            float* out, hipStream_t st) {
  constexpr int TILES = 1, QD = 4;
  int32_t mx = 0;
  for (int s = 0; s < splits; ++s) {
    int32_t g0, g1;
    split_range(K, splits, s, g0, g1);
    mx = g1 - g0 > mx ? g1 - g0 : mx;
  }
  const int cap = (LDS_BUDGET / 64) / SUPER * SUPER;
  int win = ((mx + SUPER - 1) / SUPER) * SUPER;
  if (win > cap) win = cap;
  if (win < SUPER) win = SUPER;
  const size_t lds = (size_t)win * 64;
  const int rows_per_wg = (WG / 64) * TILES * 16;
  const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg), (unsigned)splits), block(WG);
  if (mode == 1)
    hipLaunchKernelGGL((k_gemv_mfma<1, TILES, QD>), grid, block, lds, st, wq, ws, xq, xl, xs, N, K, (int)B, splits,
                       win, out);
  else
    hipLaunchKernelGGL((k_gemv_mfma<2, TILES, QD>), grid, block, lds, st, wq, ws, xq, xl, xs, N, K, (int)B, splits,
                       win, out);
  return hipGetLastError();
}

}  // namespace qdg
