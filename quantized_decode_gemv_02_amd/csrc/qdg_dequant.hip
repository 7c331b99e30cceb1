// qdg_dequant.hip -- the batch-1 Q8_0 GEMV under the Dequant numerics: the f32
// activation meets the scaled int8 weight and every product and sum is binary64,
// rounded once to binary32 at the end (lane kernel library page: module doc on the
// Dequant mode, lk_acc<0>, the Q == 0 branch of lk_q8_rows_dot, accumulator()).
//
// Any fixed binary64 order computes the plain definition to within a few binary64
// roundings; this kernel's order is:
//  * a lane holds 16 consecutive values of a block (the lane pair (2j, 2j+1)
//    holds block j of its step) and forms sum_i w_i*x_i in four binary64 chains
//    by i mod 4, each by fused multiply-adds from +0 in ascending i (every
//    product w_i*x_i is exact), then (c0 + c1) + (c2 + c3) -- four independent
//    chains keep the FMA pipeline busy;
//  * the lane folds each half-block sum h into its accumulator as
//    acc <- fma(sigma, h, acc), in ascending block order from +0 (its blocks are
//    j, j + BPS, ... of the window, sigma the block's scale);
//  * the row's lanes meet by a butterfly over lane distances 1, 2, 4 (, 8), then
//    one rounding to binary32.
// One FMA a half block replaces the pair's addition, the multiplication by sigma
// and the DPP moves of a block-sum-first order: 11-12% faster on the 5120-row
// projections and the 151936-row LM head at S = 1.
// The lane layout, the LDS staging of the window (the f32 activation and the
// rows' weight scales) and the load pipeline are those of the quantized kernel
// (qdg_gemv.hip): four named one-step weight buffers at four rows a wave (dq_fold).
//
// Split-K (S > 1, the QWEN38 page's chunk rule, gk_gemv_hl_sk): chunk s of a row
// sums its blocks in the order above into a binary64 partial; the last workgroup
// of each row tile to finish (an atomic ticket per tile, the protocol of the
// quantized kernel's in-kernel combine) adds the tile's S partials from +0 in
// ascending chunk order in binary64 and rounds once to binary32.  Every sum is
// still binary64 and there is still one rounding to binary32, so the result
// stays within the Dequant tolerance of the plain definition.

#include "qdg_device.h"

namespace qdg {
namespace {

constexpr int WG = 256;
constexpr int LDS_BUDGET = 56 * 1024;

// sum_i w_i*x_i over one lane's 16 values: chains by i mod 4, then (c0+c1)+(c2+c3).
// XF64: the window holds the activation already in binary64.
template <bool XF64>
__device__ __forceinline__ double half_dot16(int4 w, const void* __restrict__ xv) {
  const int ww[4] = {w.x, w.y, w.z, w.w};
  double c[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    double xx[4];
    if constexpr (XF64) {
      const double2 a = ((const double2*)xv)[2 * q], b = ((const double2*)xv)[2 * q + 1];
      xx[0] = a.x; xx[1] = a.y; xx[2] = b.x; xx[3] = b.y;
    } else {
      const float4 f = ((const float4*)xv)[q];
      xx[0] = f.x; xx[1] = f.y; xx[2] = f.z; xx[3] = f.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int wi = (int)(signed char)((ww[q] >> (8 * i)) & 255);
      c[i] = __fma_rn((double)wi, xx[i], c[i]);
    }
  }
  return __dadd_rn(__dadd_rn(c[0], c[1]), __dadd_rn(c[2], c[3]));
}

// One step group's half blocks (four rows a wave: lane pair j takes block j of
// each 8-block step, lane hf its half): acc <- fma(sigma, half-block sum, acc) in
// ascending block order.  lx and my_sg are the window's (index = block - wb0).
template <bool XF64, int U, int SEG>
__device__ __forceinline__ void dq_terms(const int4 (&w)[U], const unsigned char* lx, const uint16_t* my_sg, int nwb,
                                         int j, int hf, int gi, double& p) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int bl = (gi * U + u) * 8 + j;
    const bool ok = bl < nwb;
    const int blc = ok ? bl : 0;
    const double hsum = half_dot16<XF64>(w[u], lx + (2 * blc + hf) * SEG);
    p = ok ? __fma_rn((double)half_bits_to_float(my_sg[blc]), hsum, p) : p;
  }
}

// The window [wb0, wb1) through NB named one-step buffers (w[k] holds step group k
// on entry), each refilled NB groups ahead: the quantized kernels' chunk_fold with
// the binary64 half-block terms.
template <bool XF64, int U, int NB, int SEG>
__device__ __forceinline__ void dq_fold(const int8_t* wrow, const unsigned char* lx, const uint16_t* my_sg, int wb0,
                                        int wb1, int j, int hf, int4 (&w)[NB][U], double& p) {
  const int nwb = wb1 - wb0;
  const int ngroups = ((nwb + 7) / 8 + U - 1) / U;
  int gi = 0;
  for (; gi + 2 * NB - 1 < ngroups; gi += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      dq_terms<XF64, U, SEG>(w[k], lx, my_sg, nwb, j, hf, gi + k, p);
      group_load<U>(w[k], wrow, wb0, wb1, gi + NB + k, j);
    }
  }
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    dq_terms<XF64, U, SEG>(w[k], lx, my_sg, nwb, j, hf, gi + k, p);
    if (gi + NB + k < ngroups) group_load<U>(w[k], wrow, wb0, wb1, gi + NB + k, j);
  }
#pragma unroll
  for (int k = 0; k + 1 < NB; ++k)
    if (gi + NB + k < ngroups) dq_terms<XF64, U, SEG>(w[k], lx, my_sg, nwb, j, hf, gi + NB + k, p);
}

constexpr int DQ_U = 1, DQ_NB = 4;  // four rows a wave: one-step weight groups, four in flight

// AMAX (S == 1): the workgroup also writes the arg-max key of its rows' largest
// output to keys[blockIdx.x] (as the quantized kernel's epilogue does).
template <int RPW, int U, bool XF64, bool AMAX = false>
__global__ __launch_bounds__(WG) void k_gemv_dequant(const int8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
                                                    const float* __restrict__ x, int64_t N, int64_t K, int S,
                                                    int win, float* __restrict__ out, double* __restrict__ part,
                                                    unsigned* __restrict__ tickets,
                                                    unsigned long long* __restrict__ keys = nullptr) {
  constexpr int LPR = 64 / RPW;
  constexpr int BPS = LPR / 2;
  constexpr int TPP = BPS / 4;
  constexpr int ROWS = (WG / 64) * RPW;
  static_assert(TPP == 1 || TPP == 2, "RPW must be 4 or 8");
  extern __shared__ __align__(16) unsigned char lds[];
  // The window's activation: each half block (16 values) is one segment, padded
  // by 16 bytes so that the 16 lanes of a row, which read 16 consecutive
  // segments in the same instruction, fall on 16 different groups of 4 banks.
  constexpr int XB = XF64 ? 8 : 4;  // bytes per staged activation value
  constexpr int SEG = 16 * XB + 16;  // bytes per padded half-block segment
  unsigned char* lx = lds;                                   // [win][2] segments
  uint16_t* lsg = (uint16_t*)(lds + (int64_t)win * 2 * SEG);  // [ROWS][win]

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPR, li = lane % LPR, j = li >> 1, hf = li & 1;
  const int64_t nb = K / QK;
  int32_t g0, g1;
  split_range(K, S, blockIdx.y, g0, g1);
  const int64_t o_wg = (int64_t)blockIdx.x * ROWS;
  const int rr = wave * RPW + r;
  const int64_t o = o_wg + rr;
  const bool row_ok = o < N;
  const int8_t* wrow = wq + (row_ok ? o : N - 1) * K + hf * 16;
  const uint16_t* my_sg = lsg + rr * win;

  double p = 0.0;
  for (int64_t wb0 = g0; wb0 < g1; wb0 += win) {
    const int64_t wb1 = wb0 + win < g1 ? wb0 + win : g1;
    const int nwb = (int)(wb1 - wb0);
    const int nsteps = (nwb + BPS - 1) / BPS;
    const int ngroups = (nsteps + U - 1) / U;
    // four rows a wave: the first DQ_NB one-step groups of the named-buffer
    // pipeline; eight rows a wave: the first U steps of a copy-based double buffer
    int4 w[DQ_NB][DQ_U];
    int4 wcur[U];
    if constexpr (RPW == 4) {
#pragma unroll
      for (int k = 0; k < DQ_NB; ++k) group_load<DQ_U>(w[k], wrow, (int)wb0, (int)wb1, k, j);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int bl = u * BPS + j;
        wcur[u] = bl < nwb ? ld16_stream(wrow + (wb0 + bl) * QK) : make_int4(0, 0, 0, 0);
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nwb * 8; i += WG) {  // i: 4 values, segment i/4, quarter i%4
      const float4 f = ((const float4*)(x + wb0 * QK))[i];
      unsigned char* d = lx + (i >> 2) * SEG + (i & 3) * 4 * XB;
      if constexpr (XF64) {
        ((double2*)d)[0] = make_double2((double)f.x, (double)f.y);
        ((double2*)d)[1] = make_double2((double)f.z, (double)f.w);
      } else {
        *(float4*)d = f;
      }
    }
    stage_scales(lsg, win, ws, nb, N, o_wg, ROWS, wb0, nwb, threadIdx.x, WG);
    __syncthreads();

    if constexpr (RPW == 4) {
      dq_fold<XF64, DQ_U, DQ_NB, SEG>(wrow, lx, my_sg, (int)wb0, (int)wb1, j, hf, w, p);
      continue;
    }
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
        const double hsum = half_dot16<XF64>(wcur[u], lx + (2 * blc + hf) * SEG);
        p = ok ? __fma_rn((double)half_bits_to_float(my_sg[blc]), hsum, p) : p;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) wcur[u] = wnxt[u];
    }
  }
  // the row's LPR lanes (a contiguous, aligned group of the wave) by a butterfly
  double y = p;
#pragma unroll
  for (int d = 1; d < LPR; d <<= 1) y = __dadd_rn(y, __shfl_xor(y, d, 64));
  if constexpr (AMAX) {
    __shared__ unsigned long long row_keys[ROWS];
    if (li == 0) {
      const float yf = (float)y;
      if (row_ok) out[o] = yf;
      row_keys[rr] = row_ok ? amax_key(yf, (unsigned)o) : 0ull;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long best = row_keys[0];
#pragma unroll
      for (int i = 1; i < ROWS; ++i) best = row_keys[i] > best ? row_keys[i] : best;
      keys[blockIdx.x] = best;
    }
    return;
  }
  if (S == 1) {
    if (li == 0 && row_ok) out[o] = (float)y;
    return;
  }
  // Hand the chunk's binary64 partial to the tile's last-arriving workgroup
  // (publish_partial / take_partial: marked slots, all accesses atomic).
  unsigned long long* slots = (unsigned long long*)part;
  if (li == 0 && row_ok) publish_partial(slots + (int64_t)blockIdx.y * N + o, y);
  __syncthreads();
  __shared__ int last_arrival;
  if (threadIdx.x == 0)
    last_arrival = __hip_atomic_fetch_add(&tickets[blockIdx.x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (unsigned)(S - 1);
  __syncthreads();
  if (!last_arrival) return;
  if (threadIdx.x < ROWS && o_wg + threadIdx.x < N) {
    const int64_t oo = o_wg + threadIdx.x;
    double a = 0.0;
    for (int s = 0; s < S; ++s) a = __dadd_rn(a, take_partial(slots + (int64_t)s * N + oo));
    out[oo] = (float)a;
  }
  if (threadIdx.x == 0) __hip_atomic_store(&tickets[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool XF64, bool AMAX = false>
hipError_t launch_dq(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x, int splits,
                     float* y, void* workspace, hipStream_t st, unsigned long long* keys = nullptr) {
  constexpr int RPW = 4, U = 4;
  constexpr int rows_per_wg = (WG / 64) * RPW;
  constexpr int bpb = 2 * (16 * (XF64 ? 8 : 4) + 16) + 2 * rows_per_wg;  // LDS bytes per block of the window
  int32_t mx = 0;
  for (int s = 0; s < splits; ++s) {
    int32_t g0, g1;
    split_range(K, splits, s, g0, g1);
    mx = g1 - g0 > mx ? g1 - g0 : mx;
  }
  const int cap = (LDS_BUDGET / bpb) / SUPER * SUPER;
  int win = ((mx + SUPER - 1) / SUPER) * SUPER;
  if (win > cap) win = cap;
  if (win < SUPER) win = SUPER;
  const size_t lds = (size_t)win * bpb;
  unsigned* tickets = (unsigned*)workspace;
  double* part = splits == 1 ? nullptr : (double*)((char*)workspace + sk_partials_offset(N));
  const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg), (unsigned)splits), block(WG);
  return launch((k_gemv_dequant<RPW, U, XF64, AMAX>), grid, block, lds, st, wq, ws, x, N, K, splits, win, y,
                     part, tickets, keys);
}

// Activation staged in binary32 (converted by every row's lanes) or binary64
// (converted once per workgroup, the default); QDG_TUNE_DQ_X64 = 0 picks binary32.
bool dq_x64() { return tune(QDG_TUNE_DQ_X64) != 0; }

}  // namespace

// The unsplit call (qdg_gemv_q8, and its arg-max form, which must give the same
// logits) runs the chunk-wave kernel with its own chunk count: two from 8192 rows
// up, four below.  Measured on the 151936x5120 LM head, two chunks take 153 us
// against 224-230 us at five; on the 5120-row projections four is the best of
// 2..8.  0 when that kernel does not serve the shape or QDG_TUNE_DQ_SEG = 0
// asks for this file's kernel.
int dq_unsplit_order(int64_t N) { return N >= 8192 ? 2 : 4; }

int dq_unsplit_chunks(int64_t N, int64_t K) {
  if (tune(QDG_TUNE_DQ_SEG) == 0) return 0;
  const int S = dq_unsplit_order(N);
  return dq_seg_chunks(K, S) > 0 ? S : 0;
}

hipError_t launch_gemv_dequant(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                               float* out, hipStream_t st) {
  const int S = dq_unsplit_chunks(N, K);
  if (S > 0) return launch_gemv_dq_seg(wq, ws, N, K, x, S, out, st);
  if (dq_x64()) return launch_dq<true>(wq, ws, N, K, x, 1, out, nullptr, st);
  return launch_dq<false>(wq, ws, N, K, x, 1, out, nullptr, st);
}

// The same kernel as launch_gemv_dequant, so the logits are its bits; the
// chunk-wave kernel has no arg-max epilogue, so a pass over y writes the tile keys.
hipError_t launch_gemv_dequant_argmax(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                                      float* y, unsigned long long* keys, hipStream_t st) {
  const int S = dq_unsplit_chunks(N, K);
  if (S > 0) {
    const hipError_t e = launch_gemv_dq_seg(wq, ws, N, K, x, S, y, st);
    if (e != hipSuccess) return e;
    return launch_tile_keys(y, N, keys, st);
  }
  if (dq_x64()) return launch_dq<true, true>(wq, ws, N, K, x, 1, y, nullptr, st, keys);
  return launch_dq<false, true>(wq, ws, N, K, x, 1, y, nullptr, st, keys);
}

hipError_t launch_gemv_dequant_sk(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                                  int splits, float* y, void* workspace, hipStream_t st) {
  // the chunks as waves of one workgroup (qdg_dequant_seg.hip) wherever that
  // kernel serves the shape; QDG_TUNE_DQ_SEG = 0 forces this file's kernel
  if (tune(QDG_TUNE_DQ_SEG) != 0 && dq_seg_chunks(K, splits) > 0) return launch_gemv_dq_seg(wq, ws, N, K, x, splits, y, st);
  if (dq_x64()) return launch_dq<true>(wq, ws, N, K, x, splits, y, workspace, st);
  return launch_dq<false>(wq, ws, N, K, x, splits, y, workspace, st);
}

}  // namespace qdg
