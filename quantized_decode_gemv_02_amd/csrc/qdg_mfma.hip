// qdg_mfma.hip -- the batched (2 <= B <= 16) Q8_0 GEMV on int8 MFMA, Int8Act and
// TwoPass (lane kernel library page: lk_gemv_mma and its sizing helpers; the
// megakernel page's batched decode, whose rows sum exactly as a single row does).
//
// Every (t, o) output is summed exactly as the batch-1 kernel sums it: block g's
// exact int32 dot D (and E), the step p <- fma(a, b, p) of lk_q8_term into
// partial g mod 4, ascending blocks, then (P0 + P2) + (P1 + P3).  Only where the
// block dots come from differs: here one v_mfma_i32_16x16x32_i8 gives the 16x16
// dots of 16 activation rows t by 16 weight rows o over one 32-value block.
//
//  * A wave owns one tile of 16 weight rows.  Lane (col = l%16, grp = l/16)
//    loads 16 bytes at offset 16*grp of a 64-byte span (two blocks) of weight
//    row o0+col (B operand) and of activation row t = col (A operand); two
//    v_permlane32_swap per fragment regroup the bytes so that each block is one
//    16x16x32 MFMA (split_span).  A "quad" of 4 blocks (128 bytes a row, blocks
//    g = 4m..4m+3) takes two spans and four MFMAs, block 4m+k landing in
//    partial k -- compile-time register indices.
//  * The MFMA result gives lane (col, grp) the dots of t = 4*grp + i (i < 4)
//    with o = o0 + col; that lane keeps the 4 partials of those 4 (t, o) pairs,
//    so every chain lives in one lane, in ascending block order.
//  * The window of the chunk is staged in LDS once per workgroup of 4 waves (64
//    weight rows): the 16 activation rows' words (read as the MFMA A operand with
//    ds_read_b128; rows padded so the 16 rows fall on distinct banks), their
//    scales as [t][block] (four ds_read_b128 give a lane its 4 rows' scales of a
//    quad), and the weight scales of the 64 rows (one ds_read_b64 per quad).
//  * Weight loads run a group of QD quads ahead of the MFMAs (the next group is
//    requested before the current group is computed; the first group before the
//    window's barrier); the weight stream uses the nontemporal hint.
//  * Weight rows past N read row N-1 and store nothing; activation rows t >= B
//    are zero and store nothing.
#include "qdg_device.h"

namespace qdg {
namespace {

typedef unsigned v2u __attribute__((ext_vector_type(2)));

constexpr int WAVES = 4;
constexpr int WG = 64 * WAVES;
constexpr int LDS_BUDGET = 78 * 1024;  // two workgroups of 4 waves per CU

// LDS bytes per block of the window: the 16 activation rows' words (both words
// under TwoPass; rows padded by 16 bytes so that the 16 rows of a ds_read_b128
// fall on distinct banks), their scales, and the weight scales of the rows.
template <int MODE>
constexpr int lds_per_block() { return (MODE == 2 ? 2 : 1) * 16 * QK + 16 * 4 + WAVES * 16 * 2; }
constexpr int ROW_PAD = 16;

// One 32-value block's 16x16 dots: A and B hold 8 bytes a lane, k-group l/16.
__device__ __forceinline__ v4i mfma16x16x32(long a, long b) {
  const v4i z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, z, 0, 0, 0);
}

// A 16-byte fragment loaded at offset 16*g of a 64-byte span (two blocks) holds,
// in lane groups g = 0..3, bytes [0,16) and [16,32) of the first block and
// [0,16), [16,32) of the second.  Swapping registers 2-3 of the lower 32 lanes
// with registers 0-1 of the upper 32 lanes (v_permlane32_swap) leaves registers
// 0-1 of the four groups holding the first block's bytes [0,8), [16,24), [8,16),
// [24,32) and registers 2-3 the second block's in the same arrangement: one
// 16x16x32 MFMA per block, no masking.  Both operands take the same swap, so the
// bytes they multiply pairwise are the same k.
struct Halves {
  long first, second;
};
__device__ __forceinline__ Halves split_span(v4i v) {
  const auto p02 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  const auto p13 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  Halves h;
  h.first = (long)(((unsigned long)(unsigned)p13[0] << 32) | (unsigned)p02[0]);
  h.second = (long)(((unsigned long)(unsigned)p13[1] << 32) | (unsigned)p02[1]);
  return h;
}

__device__ __forceinline__ v4i ld16v_stream(const int8_t* p) { return __builtin_nontemporal_load((const v4i*)p); }

template <int MODE, int QD>
__global__ __launch_bounds__(WG) void k_gemv_mfma(const int8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
                                                 const int8_t* __restrict__ xq, const int8_t* __restrict__ xl,
                                                 const float* __restrict__ xs, int64_t N, int64_t K, int B, int S,
                                                 int win, float* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int apitch = win * QK + ROW_PAD;                       // bytes per activation row in LDS
  int8_t* la = (int8_t*)lds;                                   // [16][apitch] high words
  int8_t* ll = la + 16 * apitch;                               // [16][apitch] low words (TwoPass)
  float* sx = (float*)(lds + (MODE == 2 ? 2 : 1) * 16 * apitch);  // [16][win] activation scales
  uint16_t* sgl = (uint16_t*)(sx + 16 * win);                  // [WAVES*16][win] weight scales
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t nb = K / QK;
  const int s_idx = blockIdx.y;
  int32_t g0, g1;
  split_range(K, S, s_idx, g0, g1);

  const int64_t o_wg = (int64_t)blockIdx.x * WAVES * 16;
  const int64_t o0 = o_wg + wave * 16;
  int64_t o = o0 + col;
  if (o >= N) o = N - 1;
  const int8_t* wrow = wq + o * K + grp * 16;
  const uint16_t* my_sg = sgl + (wave * 16 + col) * win;
  const int8_t* my_a = la + col * apitch + grp * 16;  // A operand: activation row t = col
  const int8_t* my_l = ll + col * apitch + grp * 16;
  const bool lo_half = grp < 2;  // lane groups 0-1 load the first block of a span
  const v4i z4 = {0, 0, 0, 0};

  float p[4][4];  // [i][partial]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) p[i][q] = 0.0f;

  // Weight loads of QD quads (blocks bq .. bq + 4*QD - 1, none at or past `end`).
  auto issue = [&](int bq, int end, v4i (&w)[QD][2]) {
#pragma unroll
    for (int qd = 0; qd < QD; ++qd) {
      const int b = bq + 4 * qd;
      const bool v0 = b < end, v1 = b + 1 < end, v2 = b + 2 < end, v3 = b + 3 < end;
      w[qd][0] = v0 && (lo_half || v1) ? ld16v_stream(wrow + (int64_t)b * QK) : z4;
      w[qd][1] = v2 && (lo_half || v3) ? ld16v_stream(wrow + (int64_t)b * QK + 64) : z4;
    }
  };
  v4i wv[QD][2];
  issue(g0, min(g0 + win, g1), wv);  // the first group's weights fly across the first barrier
  for (int wb0 = g0; wb0 < g1; wb0 += win) {
    const int wb1 = min(wb0 + win, g1);
    const int nwb = wb1 - wb0;
    __syncthreads();
    // activation words of the window: 16 rows x nwb blocks, 16 bytes a thread-step (rows t >= B are zero)
    for (int i = threadIdx.x; i < 16 * nwb * 2; i += WG) {
      const int t = i / (nwb * 2), c = i - t * nwb * 2;
      int4 h = make_int4(0, 0, 0, 0), l = h;
      if (t < B) {
        h = *(const int4*)(xq + (int64_t)t * K + (int64_t)wb0 * QK + 16 * c);
        if constexpr (MODE == 2) l = *(const int4*)(xl + (int64_t)t * K + (int64_t)wb0 * QK + 16 * c);
      }
      *(int4*)(la + t * apitch + 16 * c) = h;
      if constexpr (MODE == 2) *(int4*)(ll + t * apitch + 16 * c) = l;
    }
    for (int i = threadIdx.x; i < 16 * nwb; i += WG) {
      const int t = i / nwb, bl = i - t * nwb;
      sx[t * win + bl] = t < B ? xs[(int64_t)t * nb + wb0 + bl] : 0.0f;
    }
    stage_scales(sgl, win, ws, nb, N, o_wg, WAVES * 16, wb0, nwb, threadIdx.x, WG);
    __syncthreads();

    // Groups of QD quads (win and the chunk start are multiples of 16 = 4*QD
    // blocks, so groups never straddle a window); the next group's weights --
    // across a window boundary too -- are requested before the current group's
    // MFMAs.  b - g0 is a multiple of 4, so block b + k is partial k.
    for (int bq = wb0; bq < wb1; bq += 4 * QD) {
      v4i wn[QD][2];
      if (bq + 4 * QD < wb1)
        issue(bq + 4 * QD, wb1, wn);
      else if (wb1 < g1)
        issue(wb1, min(wb1 + win, g1), wn);  // the next window's first group
#pragma unroll
      for (int qd = 0; qd < QD; ++qd) {
        const int b = bq + 4 * qd;
        if (b >= wb1) break;  // uniform over the wave
        const int bl = b - wb0;
        const bool vk[4] = {true, b + 1 < wb1, b + 2 < wb1, b + 3 < wb1};
        const Halves a0 = split_span(*(const v4i*)(my_a + bl * QK));
        const Halves a1 = split_span(*(const v4i*)(my_a + bl * QK + 64));
        const Halves w0 = split_span(wv[qd][0]), w1 = split_span(wv[qd][1]);
        v4i D[4], E[4];
        D[0] = mfma16x16x32(a0.first, w0.first);
        D[1] = mfma16x16x32(a0.second, w0.second);
        D[2] = mfma16x16x32(a1.first, w1.first);
        D[3] = mfma16x16x32(a1.second, w1.second);
        if constexpr (MODE == 2) {
          const Halves l0 = split_span(*(const v4i*)(my_l + bl * QK));
          const Halves l1 = split_span(*(const v4i*)(my_l + bl * QK + 64));
          E[0] = mfma16x16x32(l0.first, w0.first);
          E[1] = mfma16x16x32(l0.second, w0.second);
          E[2] = mfma16x16x32(l1.first, w1.first);
          E[3] = mfma16x16x32(l1.second, w1.second);
        }
        const v2u sg2 = *(const v2u*)(my_sg + bl);  // the row's 4 weight scales of the quad
        const unsigned short sg[4] = {(unsigned short)(sg2[0] & 0xffffu), (unsigned short)(sg2[0] >> 16),
                                      (unsigned short)(sg2[1] & 0xffffu), (unsigned short)(sg2[1] >> 16)};
        float sv[4][4];  // [i][k]: scale of activation row 4*grp + i at block b + k
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 s4 = *(const float4*)(sx + (grp * 4 + i) * win + bl);
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
#pragma unroll
      for (int qd = 0; qd < QD; ++qd) {
        wv[qd][0] = wn[qd][0];
        wv[qd][1] = wn[qd][1];
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

template <int MODE>
hipError_t launch_m(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq, const int8_t* xl,
                    const float* xs, int64_t B, int splits, float* out, hipStream_t st) {
  constexpr int QD = 4;
  int32_t mx = 0;
  for (int s = 0; s < splits; ++s) {
    int32_t g0, g1;
    split_range(K, splits, s, g0, g1);
    mx = g1 - g0 > mx ? g1 - g0 : mx;
  }
  // window: a multiple of 16 blocks (chunk starts are, so quads stay aligned to partials)
  const int cap = ((LDS_BUDGET - (MODE == 2 ? 2 : 1) * 16 * ROW_PAD) / lds_per_block<MODE>()) / SUPER * SUPER;
  int win = ((mx + SUPER - 1) / SUPER) * SUPER;
  if (win > cap) win = cap;
  if (win < SUPER) win = SUPER;
  const size_t lds = (size_t)win * lds_per_block<MODE>() + (MODE == 2 ? 2 : 1) * 16 * ROW_PAD;
  const int rows_per_wg = WAVES * 16;
  const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg), (unsigned)splits), block(WG);
  // windows above 64 KiB of LDS need the kernel's dynamic-LDS limit raised (once)
  static const hipError_t attr = hipFuncSetAttribute((const void*)&k_gemv_mfma<MODE, QD>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BUDGET + 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_gemv_mfma<MODE, QD>), grid, block, lds, st, wq, ws, xq, xl, xs, N, K, (int)B, splits, win,
                     out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_mfma(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K,
                            const int8_t* xq, const int8_t* xl, const float* xs, int64_t B, int splits,
                            float* out, hipStream_t st) {
  if (mode == 1) return launch_m<1>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
  return launch_m<2>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
}

}  // namespace qdg
