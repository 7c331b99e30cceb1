// qdg_dequant_seg.hip -- the batch-1 Q8_0 GEMV under the Dequant numerics with
// the chunks of a row tile as the waves of one workgroup (lane kernel library
// page: module doc on the Dequant mode, lk_acc<0>; QWEN38 page: the split-K
// chunk rule of gk_gemv_hl_sk, partials added in ascending chunk order as
// gk_sk_combine adds them).  Every product and sum is binary64 and the row is
// rounded once to binary32, as in k_gemv_dequant; only the fixed order and the
// mapping onto the GPU differ.
//
// Mapping: a wave takes four rows of one chunk.  Lane l takes the l-th 8-value
// piece of each 512-value step of the chunk (four lanes are a block) for all
// four rows, so the piece's activation -- read once from the L1/L2-resident f32
// vector and widened to binary64 in registers -- serves four rows, and each
// weight load instruction reads 512 contiguous bytes of one row.
//
// Order (fixed, so repeats are bit-identical; the Dequant contract is the
// binary64 sum within its tolerance, not one association):
//  * a lane's 8 products w_i*x_i (exact in binary64) are summed in two chains by
//    i mod 2 from +0 in ascending i, then c0 + c1: the piece sum v;
//  * the lane folds its pieces into the row's accumulator in ascending step
//    order from +0, acc <- fma(sigma, v, acc), with sigma its block's scale
//    (a quarter of a block per lane: the block's four pieces sit in four lanes);
//  * the chunk's partial is the sum of the 64 lanes' accumulators by a
//    butterfly over lane distances 1, 2, 4, 8, 16, 32;
//  * the row adds its chunks' partials in ascending chunk order from +0 (empty
//    chunks skipped: their partial is +0) and rounds once to binary32.
// Folding each piece straight into the accumulator takes one binary64 FMA a
// row and step, where summing the block's four pieces across its lanes first
// took two DPP moves, two additions and a multiplication: 8% faster on the
// 5120x25600 projection at S = 8 (35.7 -> 32.7 us).

#include <atomic>

#include "qdg_device.h"

namespace qdg {
namespace {

constexpr int DS_NT = 1024;

__device__ __forceinline__ double piece_dot8(int2 w, const double* xd) {
  const int ww[2] = {w.x, w.y};
  double c0 = 0.0, c1 = 0.0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      c0 = __fma_rn((double)(int)(signed char)((ww[q] >> (8 * i)) & 255), xd[4 * q + i], c0);
      c1 = __fma_rn((double)(int)(signed char)((ww[q] >> (8 * i + 8)) & 255), xd[4 * q + i + 1], c1);
    }
  }
  return __dadd_rn(c0, c1);
}

__device__ __forceinline__ int2 ld8_stream(const int8_t* p) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i t = __builtin_nontemporal_load((const v2i*)p);
  return make_int2(t[0], t[1]);
}

// One step's operands of a lane: the piece's weights in the wave's four rows,
// its eight activation values and the four rows' scales of its block.
struct DqStep {
  int2 w[4];
  float4 x0, x1;
  unsigned short sg[4];
};

// Requests piece p's operands (p already clamped into the chunk: a lane past the
// chunk's end re-reads its last piece, whose step dq_fold then drops, so every
// wave issues the same loads and the compiler's wait counts stay exact).
__device__ __forceinline__ void dq_load(DqStep& b, const int8_t* const (&wrow)[4], const uint16_t* const (&srow)[4],
                                        const float* __restrict__ x, int p) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 4; ++r) b.w[r] = ld8_stream(wrow[r] + (unsigned)(8 * p));
  b.x0 = *(const float4*)(x + (unsigned)(8 * p));
  b.x1 = *(const float4*)(x + (unsigned)(8 * p + 4));
#pragma unroll
  for (int r = 0; r < 4; ++r) b.sg[r] = srow[r][(unsigned)(p >> 2)];
  __builtin_amdgcn_sched_barrier(0);
}

// The step's terms: each row's piece sum v, folded as acc <- fma(sigma, v, acc)
// when the lane's piece lies in the chunk.
__device__ __forceinline__ void dq_fold(const DqStep& b, bool act, double (&acc)[4]) {
  const double xd[8] = {b.x0.x, b.x0.y, b.x0.z, b.x0.w, b.x1.x, b.x1.y, b.x1.z, b.x1.w};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const double v = piece_dot8(b.w[r], xd);
    const double f = __fma_rn((double)half_bits_to_float(b.sg[r]), v, acc[r]);
    acc[r] = act ? f : acc[r];
  }
}

// The partials of one row group's chunks: the wave takes chunks cw, cw + W, ...
// (chunks 0..m-1, then S-1) of the four rows at wrow/srow and leaves chunk c's
// four partials in lp[c].  The operands stream through NB named step buffers:
// buffer k's terms are taken, then it is refilled NB steps ahead, so NB - 1
// later steps stay in flight while a step is folded and no register copy waits
// for a load.  The earlier loop loaded a step and waited for all of it before
// its terms (one step in flight a wave), with a predicate that made every load
// and term a branch.
template <int NB>
__device__ __forceinline__ void dq_chunk_partials(const int8_t* const (&wrow)[4], const uint16_t* const (&srow)[4],
                                                  const float* __restrict__ x, int64_t K, int S, int m, int ceff,
                                                  int cw, int W, int lane, double (*lp)[4]) {
  const int nq = (int)(K >> 9), nbk = (int)(K / QK), per = (nq + S - 1) / S;  // K <= 2^31
  for (int c = cw; c < ceff; c += W) {
  int32_t g0, g1;
  split_range32(nq, nbk, per, S, c < m ? c : S - 1, g0, g1);
  // 8-value pieces of the row (32-bit offsets: K < 2^31)
  const int p0 = 4 * g0, p1 = 4 * g1;
  const int nsteps = (p1 - p0 + 63) / 64;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  if (nsteps > 0) {
    const int plast = p1 - 1;
    auto piece = [&](int st) { return p0 + 64 * st + lane; };
    auto clamp = [&](int p) { return p < plast ? p : plast; };
    DqStep b[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) dq_load(b[k], wrow, srow, x, clamp(piece(k)));
    int st = 0;
    // while every refill is due (only a chunk's last step can be partial -- a
    // chunk is whole 512-value superblocks, 64 pieces, but for the K mod 512
    // tail -- so every lane's piece here lies in the chunk)
    for (; st + 2 * NB - 1 < nsteps; st += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        dq_fold(b[k], true, acc);
        dq_load(b[k], wrow, srow, x, clamp(piece(st + k + NB)));
      }
    }
    // the last 1 .. 2*NB - 1 steps, in order
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (st + k < nsteps) dq_fold(b[k], piece(st + k) < p1, acc);
      if (st + k + NB < nsteps) dq_load(b[k], wrow, srow, x, clamp(piece(st + k + NB)));
    }
#pragma unroll
    for (int k = 0; k + 1 < NB; ++k)
      if (st + NB + k < nsteps) dq_fold(b[k], piece(st + NB + k) < p1, acc);
  }
  // the 64 lanes' accumulators by a fixed butterfly
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int d = 1; d <= 32; d <<= 1) acc[r] = __dadd_rn(acc[r], __shfl_xor(acc[r], d, 64));
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) lp[c][r] = acc[r];
  }
  }
}

// The four rows from o of one matrix, clamped into its N rows (a clamped row's
// partials are computed and never written).
__device__ __forceinline__ void dq_rows(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, int64_t o,
                                        const int8_t* (&wrow)[4], const uint16_t* (&srow)[4]) {
  const int64_t nb = K / QK;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t q = o + r < N ? o + r : N - 1;
    wrow[r] = wq + q * K;
    srow[r] = ws + q * nb;
  }
}

// The wave index is a scalar (readfirstlane), so the chunk bounds and the four
// rows' pointers sit in SGPRs.
template <int R, int NB>
__global__ __launch_bounds__(DS_NT) void k_gemv_dq_seg(const PartTable tab, const float* __restrict__ x, int64_t K,
                                                        int S, int m, int ceff) {
  constexpr int ROWS = 4 * R;
  __shared__ double lpart[DS_NT / 64][4];  // [row group * ceff + chunk][row]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = (int)(blockDim.x >> 6) / R;  // chunk waves a row group
  const int rg = wave / W, cw = wave % W;
  int64_t o_wg;
  const int part = find_part(tab, (int)blockIdx.x, ROWS, o_wg);
  float* __restrict__ y = tab.y[part];
  const int64_t N = tab.N[part];
  const int8_t* wrow[4];
  const uint16_t* srow[4];
  dq_rows(tab.wq[part], tab.ws[part], N, K, o_wg + rg * 4, wrow, srow);
  dq_chunk_partials<NB>(wrow, srow, x, K, S, m, ceff, cw, W, lane, lpart + rg * ceff);
  __syncthreads();
  if (tid < ROWS && o_wg + tid < N) {
    const int g = tid >> 2, q = tid & 3;
    double a = 0.0;
    for (int cc = 0; cc < ceff; ++cc) a = __dadd_rn(a, lpart[g * ceff + cc][q]);
    y[o_wg + tid] = (float)a;
  }
}

// The gate and up projections of four rows side by side (lane kernel library
// page, GLU / lk_gemv_glu under the Dequant accumulator with a binary32
// output): the first W waves take the gate's four rows, the next W the up's, each
// row group in the chunk order of k_gemv_dq_seg, so g and u are the bits that
// kernel writes at the same chunk count; four lanes then round both rows once
// and write h = act(g) * u with the producer's glu_mul.
template <int NB, int ACT>
__global__ __launch_bounds__(DS_NT) void k_gemv_dq_glu(const int8_t* __restrict__ wg, const uint16_t* __restrict__ sg,
                                                        const int8_t* __restrict__ wu, const uint16_t* __restrict__ su,
                                                        int64_t F, int64_t K, const float* __restrict__ x, int S,
                                                        int m, int ceff, float* __restrict__ h) {
  __shared__ double lpart[DS_NT / 64][4];  // [matrix * ceff + chunk][row]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = (int)(blockDim.x >> 6) / 2;
  const int rg = wave / W, cw = wave % W;
  const int64_t o = (int64_t)blockIdx.x * 4;
  const int8_t* wrow[4];
  const uint16_t* srow[4];
  dq_rows(rg ? wu : wg, rg ? su : sg, F, K, o, wrow, srow);
  dq_chunk_partials<NB>(wrow, srow, x, K, S, m, ceff, cw, W, lane, lpart + rg * ceff);
  __syncthreads();
  if (tid < 4 && o + tid < F) {
    double a = 0.0, b = 0.0;
    for (int cc = 0; cc < ceff; ++cc) {
      a = __dadd_rn(a, lpart[cc][tid]);
      b = __dadd_rn(b, lpart[ceff + cc][tid]);
    }
    h[o + tid] = glu_mul<ACT>((float)a, (float)b);
  }
}

void ds_chunks(int64_t K, int S, int& m, int& ceff) {
  const int64_t nq = K / 512, per = (nq + S - 1) / S;
  m = per > 0 ? (int)((nq + per - 1) / per) : 0;
  if (m > S) m = S;
  ceff = m;
  if (m < S && ((K % 512) != 0 || m == 0)) ceff = m + 1;
}

#ifndef QDG_DS_NB
#define QDG_DS_NB 2
#endif
constexpr int DS_NB = QDG_DS_NB;  // step buffers: DS_NB - 1 steps in flight beyond the one being folded

// Workgroups of R row groups of W chunk waves that a compute unit holds at once
// (the HIP occupancy calculator: the kernel keeps 75 VGPRs, six waves a SIMD),
// asked once a row-group count and W.
template <int R>
int ds_resident(int W) {
  static std::atomic<int> cache[17];
  int n = cache[W].load(std::memory_order_relaxed);
  if (n <= 0) {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, (const void*)k_gemv_dq_seg<R, DS_NB>, 64 * R * W, 0) !=
        hipSuccess) {
      (void)hipGetLastError();
      b = 1;
    }
    n = b > 0 ? b : 1;
    cache[W].store(n, std::memory_order_relaxed);
  }
  return n;
}

// W chunk waves a row group (pick_chunk_waves): at 5120 rows and S = 8 eight
// waves a workgroup would take 1.67 rounds of three workgroups a CU; four waves
// of two chunks fit one round.  QDG_TUNE_DQ_WAVES overrides.
template <int R>
int ds_waves(int64_t wgs, int64_t K, int S, int m, int ceff) {
  return pick_chunk_waves(wgs, 16 / R, K, S, m, ceff, tune(QDG_TUNE_DQ_WAVES), [](int w) { return ds_resident<R>(w); });
}

template <int R>
hipError_t launch_ds(const PartTable& tab, int64_t K, const float* x, int S, int m, int ceff, hipStream_t st) {
  const int64_t wgs = tab.tile_end[tab.n - 1];
  const int W = ds_waves<R>(wgs, K, S, m, ceff);
  const dim3 grid((unsigned)wgs), block((unsigned)(64 * R * W));
  return launch((k_gemv_dq_seg<R, DS_NB>), grid, block, 0, st, tab, x, K, S, m, ceff);
}

// The gate/up kernel's workgroups (two row groups of W chunk waves) a compute
// unit holds at once, asked once an activation and W.
template <int ACT>
int dg_resident(int W) {
  static std::atomic<int> cache[9];
  int n = cache[W].load(std::memory_order_relaxed);
  if (n <= 0) {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, (const void*)k_gemv_dq_glu<DS_NB, ACT>, 128 * W, 0) !=
        hipSuccess) {
      (void)hipGetLastError();
      b = 1;
    }
    n = b > 0 ? b : 1;
    cache[W].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int ACT>
hipError_t launch_dg(const int8_t* wg, const uint16_t* sg, const int8_t* wu, const uint16_t* su, int64_t F, int64_t K,
                     const float* x, int S, int m, int ceff, float* h, hipStream_t st) {
  const int64_t wgs = (F + 3) / 4;
  const int W = pick_chunk_waves(wgs, 8, K, S, m, ceff, tune(QDG_TUNE_DQ_WAVES),
                                 [](int w) { return dg_resident<ACT>(w); });
  const dim3 grid((unsigned)wgs), block((unsigned)(128 * W));
  return launch((k_gemv_dq_glu<DS_NB, ACT>), grid, block, 0, st, wg, sg, wu, su, F, K, x, S, m, ceff, h);
}

}  // namespace

// The chunk count the kernel uses: the caller's S, or 5 when it asks for none
// (the order is the kernel's own; five chunks of 5120 values make one round of
// workgroups on the 5120-row projections).  0 when the kernel does not serve the
// shape (more than 16 chunk waves).
int dq_seg_chunks(int64_t K, int splits) {
  const int S = splits == 1 ? 5 : splits;
  int m, ceff;
  ds_chunks(K, S, m, ceff);
  return ceff <= 16 ? S : 0;
}

// Row groups a workgroup: one (measured on the 5120-row projections: R = 1 is
// 10-25% faster than 2-4 at S = 4, 5 and 8); QDG_TUNE_DQ_ROWS overrides.
int ds_rows(int ceff) {
  int R = 1;
  if (tune(QDG_TUNE_DQ_ROWS) > 0) R = tune(QDG_TUNE_DQ_ROWS);
  if (R < 1) R = 1;
  if (R > 4) R = 4;
  while (R > 1 && R * ceff > 16) --R;
  return R;
}

int dq_chunk_waves(int64_t N, int64_t K, int splits) {
  const int S = dq_seg_chunks(K, splits);
  if (S == 0) return 0;
  int m, ceff;
  ds_chunks(K, S, m, ceff);
  const int R = ds_rows(ceff);
  const int64_t wgs = (N + 4 * R - 1) / (4 * R);
  switch (R) {
    case 1: return ds_waves<1>(wgs, K, S, m, ceff);
    case 2: return ds_waves<2>(wgs, K, S, m, ceff);
    case 3: return ds_waves<3>(wgs, K, S, m, ceff);
    default: return ds_waves<4>(wgs, K, S, m, ceff);
  }
}

hipError_t launch_gemv_dq_seg_parts(int nparts, const int8_t* const* wq, const uint16_t* const* ws, const int64_t* N,
                                    float* const* y, int64_t K, const float* x, int splits, hipStream_t st) {
  const int S = dq_seg_chunks(K, splits);
  int m, ceff;
  ds_chunks(K, S, m, ceff);
  const int R = ds_rows(ceff);
  PartTable tab;
  if (!make_parts(tab, nparts, wq, ws, y, N, 4 * R)) return hipErrorInvalidValue;
  switch (R) {
    case 1: return launch_ds<1>(tab, K, x, S, m, ceff, st);
    case 2: return launch_ds<2>(tab, K, x, S, m, ceff, st);
    case 3: return launch_ds<3>(tab, K, x, S, m, ceff, st);
    default: return launch_ds<4>(tab, K, x, S, m, ceff, st);
  }
}

hipError_t launch_gemv_dq_seg(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x, int splits,
                              float* y, hipStream_t st) {
  return launch_gemv_dq_seg_parts(1, &wq, &ws, &N, &y, K, x, splits, st);
}

// The gate and up projections of F rows with the gated product, S chunks a row
// (at most 8 chunk partials a matrix: both sit in the workgroup's 16 slots).
hipError_t launch_gemv_dq_glu(int act, const int8_t* wg, const uint16_t* sg, const int8_t* wu, const uint16_t* su,
                              int64_t F, int64_t K, const float* x, int S, float* h, hipStream_t st) {
  int m, ceff;
  ds_chunks(K, S, m, ceff);
  if (ceff < 1 || ceff > 8 || (F + 3) / 4 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (act == 0) return launch_dg<0>(wg, sg, wu, su, F, K, x, S, m, ceff, h, st);
  if (act == 1) return launch_dg<1>(wg, sg, wu, su, F, K, x, S, m, ceff, h, st);
  return launch_dg<2>(wg, sg, wu, su, F, K, x, S, m, ceff, h, st);
}

}  // namespace qdg
