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
//  * A wave owns one tile of 16 weight rows.  Lane (col = l%16, grp = l/16)
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
//  * The window's activation scales are staged in LDS as [t][block] and the
//    weight scales of the workgroup's rows as [row][block]; a lane reads its 4
//    activation rows' scales of a quad with four ds_read_b128 and its weight
//    row's 4 scales with one ds_read_b64.
//  * QD quads of loads are issued before the first MFMA of an iteration; the
//    weight stream uses the nontemporal hint.
//  * Weight rows past N read row N-1 and store nothing; activation rows t >= B
//    are zero and store nothing.
#include "qdg_device.h"

namespace qdg {
namespace {

typedef unsigned v2u __attribute__((ext_vector_type(2)));

constexpr int WAVES = 2;
constexpr int WG = 64 * WAVES;
constexpr int LDS_BUDGET = 48 * 1024;
constexpr int LDS_PER_BLOCK = 16 * 4 + WAVES * 16 * 2;  // activation scales + weight scales

__device__ __forceinline__ v4i mfma16x16x64(v4i a, v4i b) {
  const v4i z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, z, 0, 0, 0);
}

__device__ __forceinline__ v4i ld16v(const int8_t* p) { return *(const v4i*)p; }
__device__ __forceinline__ v4i ld16v_stream(const int8_t* p) { return __builtin_nontemporal_load((const v4i*)p); }

template <int MODE, int QD>
__global__ __launch_bounds__(WG) void k_gemv_mfma(const int8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
                                                 const int8_t* __restrict__ xq, const int8_t* __restrict__ xl,
                                                 const float* __restrict__ xs, int64_t N, int64_t K, int B, int S,
                                                 int win, float* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char lds[];
  float* sx = (float*)lds;                         // [16][win]: activation scales, t-major
  uint16_t* sgl = (uint16_t*)(sx + 16 * win);      // [WAVES*16][win]: weight scales of the rows
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t nb = K / QK;
  const int s_idx = blockIdx.y;
  int32_t g0, g1;
  split_range(K, S, s_idx, g0, g1);

  const int64_t o0 = ((int64_t)blockIdx.x * WAVES + wave) * 16;
  int64_t o = o0 + col;
  if (o >= N) o = N - 1;
  const int8_t* wrow = wq + o * K + grp * 16;
  const uint16_t* my_sg = sgl + (wave * 16 + col) * win;
  const bool t_ok = col < B;
  const int8_t* arow = xq + (int64_t)(t_ok ? col : 0) * K + grp * 16;
  const int8_t* lrow = MODE == 2 ? xl + (int64_t)(t_ok ? col : 0) * K + grp * 16 : nullptr;
  const bool lo_half = grp < 2;  // lane groups 0-1 carry the first block of a span
  const v4i z4 = {0, 0, 0, 0};

  float p[4][4];  // [i][partial]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) p[i][q] = 0.0f;

  for (int wb0 = g0; wb0 < g1; wb0 += win) {
    const int wb1 = min(wb0 + win, g1);
    const int nwb = wb1 - wb0;
    __syncthreads();
    for (int i = threadIdx.x; i < 16 * nwb; i += WG) {
      const int t = i / nwb, bl = i - t * nwb;
      sx[t * win + bl] = t < B ? xs[(int64_t)t * nb + wb0 + bl] : 0.0f;
    }
    stage_scales(sgl, win, ws, nb, N, (int64_t)blockIdx.x * WAVES * 16, WAVES * 16, wb0, nwb, threadIdx.x, WG);
    __syncthreads();

    for (int bq = wb0; bq < wb1; bq += 4 * QD) {
      v4i wv[QD][2], av[QD][2], lv[QD][2];
#pragma unroll
      for (int qd = 0; qd < QD; ++qd) {
        const int b = bq + 4 * qd;
        const bool v0 = b < wb1, v1 = b + 1 < wb1, v2 = b + 2 < wb1, v3 = b + 3 < wb1;
        const bool span0 = v0 && (lo_half || v1), span1 = v2 && (lo_half || v3);
        wv[qd][0] = span0 ? ld16v_stream(wrow + (int64_t)b * QK) : z4;
        wv[qd][1] = span1 ? ld16v_stream(wrow + (int64_t)b * QK + 64) : z4;
        av[qd][0] = t_ok && span0 ? ld16v(arow + (int64_t)b * QK) : z4;
        av[qd][1] = t_ok && span1 ? ld16v(arow + (int64_t)b * QK + 64) : z4;
        if constexpr (MODE == 2) {
          lv[qd][0] = t_ok && span0 ? ld16v(lrow + (int64_t)b * QK) : z4;
          lv[qd][1] = t_ok && span1 ? ld16v(lrow + (int64_t)b * QK + 64) : z4;
        }
      }
#pragma unroll
      for (int qd = 0; qd < QD; ++qd) {
        const int b = bq + 4 * qd;  // b - g0 is a multiple of 4: block b + k is partial k
        if (b >= wb1) break;        // uniform over the wave
        const bool vk[4] = {true, b + 1 < wb1, b + 2 < wb1, b + 3 < wb1};
        v4i D[4], E[4];
        D[0] = mfma16x16x64(lo_half ? av[qd][0] : z4, wv[qd][0]);
        D[1] = mfma16x16x64(lo_half ? z4 : av[qd][0], wv[qd][0]);
        D[2] = mfma16x16x64(lo_half ? av[qd][1] : z4, wv[qd][1]);
        D[3] = mfma16x16x64(lo_half ? z4 : av[qd][1], wv[qd][1]);
        if constexpr (MODE == 2) {
          E[0] = mfma16x16x64(lo_half ? lv[qd][0] : z4, wv[qd][0]);
          E[1] = mfma16x16x64(lo_half ? z4 : lv[qd][0], wv[qd][0]);
          E[2] = mfma16x16x64(lo_half ? lv[qd][1] : z4, wv[qd][1]);
          E[3] = mfma16x16x64(lo_half ? z4 : lv[qd][1], wv[qd][1]);
        }
        const v2u sg2 = *(const v2u*)(my_sg + (b - wb0));  // the row's 4 weight scales of the quad
        const unsigned short sg[4] = {(unsigned short)(sg2[0] & 0xffffu), (unsigned short)(sg2[0] >> 16),
                                      (unsigned short)(sg2[1] & 0xffffu), (unsigned short)(sg2[1] >> 16)};
        float sv[4][4];  // [i][k]: scale of activation row 4*grp + i at block b + k
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 s4 = *(const float4*)(sx + (grp * 4 + i) * win + (b - wb0));
          sv[i][0] = s4.x; sv[i][1] = s4.y; sv[i][2] = s4.z; sv[i][3] = s4.w;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (!vk[k]) continue;  // uniform over the wave
          const float sgm = half_bits_to_float(sg[k]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float ta, tb;
            q8_term<MODE>(sgm, sv[i][k], D[k][i], MODE == 2 ? E[k][i] : 0, ta, tb);
            p[i][k] = __fmaf_rn(ta, tb, p[i][k]);
          }
        }
      }
    }
  }
  const int64_t oo = o0 + col;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = grp * 4 + i;
    const float y = __fadd_rn(__fadd_rn(p[i][0], p[i][2]), __fadd_rn(p[i][1], p[i][3]));
    if (t < B && oo < N) out[((int64_t)s_idx * B + t) * N + oo] = y;
  }
}

}  // namespace

hipError_t launch_gemv_mfma(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K,
                            const int8_t* xq, const int8_t* xl, const float* xs, int64_t B, int splits,
                            float* out, hipStream_t st) {
  constexpr int QD = 4;
  int32_t mx = 0;
  for (int s = 0; s < splits; ++s) {
    int32_t g0, g1;
    split_range(K, splits, s, g0, g1);
    mx = g1 - g0 > mx ? g1 - g0 : mx;
  }
  // window: a multiple of 16 blocks (so a quad's four scales are 16-byte aligned in LDS)
  const int cap = (LDS_BUDGET / LDS_PER_BLOCK) / SUPER * SUPER;
  int win = ((mx + SUPER - 1) / SUPER) * SUPER;
  if (win > cap) win = cap;
  if (win < SUPER) win = SUPER;
  const size_t lds = (size_t)win * LDS_PER_BLOCK;
  const int rows_per_wg = WAVES * 16;
  const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg), (unsigned)splits), block(WG);
  if (mode == 1)
    hipLaunchKernelGGL((k_gemv_mfma<1, QD>), grid, block, lds, st, wq, ws, xq, xl, xs, N, K, (int)B, splits, win,
                       out);
  else
    hipLaunchKernelGGL((k_gemv_mfma<2, QD>), grid, block, lds, st, wq, ws, xq, xl, xs, N, K, (int)B, splits, win,
                       out);
  return hipGetLastError();
}

}  // namespace qdg
