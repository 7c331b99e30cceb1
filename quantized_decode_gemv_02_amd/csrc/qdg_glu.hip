// qdg_glu.hip -- the gate and up projections of one activation in one launch,
// with the gated product and the quantizer as the epilogue (lane kernel library
// page, GLU / lk_gemv_glu: a block of warps takes 32 outputs, gates them, and
// writes one quantized block of the next projection's activation; lk_act for
// the activation: silu, sigmoid or the tanh-form GELU).
//
// A workgroup of 16 waves owns outputs [32b, 32b + 32): waves 0-7 the 32 gate
// rows, waves 8-15 the 32 up rows, four rows a wave over all of K, each row
// summed exactly as the batch-1 GEMV sums it (chunk_dot4 over the whole row).
// The 64 results meet in LDS; then eight lanes form h = act(g) * u for the 32
// outputs (glu_mul, the producer's own arithmetic) and quantize them as one
// block (quant_lane4).  So g, u, h and the words are bit-identical to two
// qdg_gemv_q8 calls followed by qdg_glu_quantize, without the g/u round trip or
// the extra launch.
//
// Staging (DMA): as in the split-K GEMV, the activation and the 64 rows' weight
// scales go straight from global memory into LDS (global_load_lds_dwordx4)
// while each wave's first step groups of weights are in flight, when K is a
// multiple of 256 and every staged array is 16-byte aligned; otherwise they are
// copied through registers.

#include "qdg_device.h"

namespace qdg {
namespace {

constexpr int GL_NT = 1024;
constexpr int GL_ROWS = 64;                // 32 gate rows + 32 up rows
constexpr int GL_U = 1, GL_NB = 4;         // steps a group, groups in flight
constexpr int GL_LDS_MAX = 79 * 1024;      // two workgroups a CU

template <int MODE>
constexpr int gl_bytes_per_block() { return (MODE == 2 ? 2 : 1) * QK + 4 + 2 * GL_ROWS; }

template <int MODE, bool DMA, int ACT>
__global__ __launch_bounds__(GL_NT) __attribute__((amdgpu_waves_per_eu(8))) void k_gemv_glu(
    const int8_t* __restrict__ wg, const uint16_t* __restrict__ sg, const int8_t* __restrict__ wu,
    const uint16_t* __restrict__ su, int64_t K, const int8_t* __restrict__ xq, const int8_t* __restrict__ xl,
    const float* __restrict__ xs, float* __restrict__ h, int8_t* __restrict__ hq, int8_t* __restrict__ hl,
    float* __restrict__ hs) {
  constexpr int U = GL_U, NB = GL_NB, LPR = 16;
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ float lout[GL_ROWS];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane / LPR, li = lane % LPR, j = li >> 1, hf = li & 1;
  const int64_t nb = K / QK;
  const int64_t o0 = (int64_t)blockIdx.x * 32;
  const bool up = wave >= 8;
  const int rr = 4 * (wave & 7) + r;  // row within the gate (or up) tile
  const int8_t* wrow = (up ? wu : wg) + (o0 + rr) * K + hf * 16;

  int8_t* lq = (int8_t*)lds;                                   // [nb][32]
  int8_t* ll = lq + nb * QK;                                   // [nb][32] (TwoPass)
  float* lsx = (float*)(lds + nb * QK * (MODE == 2 ? 2 : 1));  // [nb]
  uint16_t* lsg = (uint16_t*)(lsx + nb);                       // [64][nb]: gate rows, then up rows

  // With LDS DMA the staged bytes are requested first and the first NB step
  // groups of weights after them, and the barrier waits for the staging only (the
  // weights stay in flight; loads complete in issue order).  With the register
  // copies the first group is requested ahead of the copies.
  int4 w[NB][U];
  if constexpr (!DMA) group_load<U>(w[0], wrow, 0, (int)nb, 0, j);
  if constexpr (DMA) {
    const int64_t nsx = nb * 4, nsg = 32 * nb * 2;  // multiples of 16 bytes (nb is a multiple of 8)
    for (int64_t base = (int64_t)wave * 1024; base < K; base += 16 * 1024) {
      if (base + lane * 16 < K) {
        lds_dma16(xq + base + lane * 16, lq + base);
        if constexpr (MODE == 2) lds_dma16(xl + base + lane * 16, ll + base);
      }
    }
    for (int64_t base = (int64_t)wave * 1024; base < nsx; base += 16 * 1024)
      if (base + lane * 16 < nsx) lds_dma16((const int8_t*)xs + base + lane * 16, (int8_t*)lsx + base);
    // the 32 gate rows, then the 32 up rows: each a consecutive run of scales
    for (int64_t base = (int64_t)wave * 1024; base < 2 * nsg; base += 16 * 1024) {
      const int64_t off = base + lane * 16;  // a wave's piece may straddle the two runs: each lane picks its own
      if (off < 2 * nsg) {
        const int8_t* src = off < nsg ? (const int8_t*)(sg + o0 * nb) + off : (const int8_t*)(su + o0 * nb) + (off - nsg);
        lds_dma16(src, (int8_t*)lsg + base);
      }
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) group_load<U>(w[k], wrow, 0, (int)nb, k, j);
    wait_barrier<NB * U>();
  } else {
    for (int64_t i = tid; i < nb * 2; i += GL_NT) {
      ((int4*)lq)[i] = ld16(xq + 16 * i);
      if constexpr (MODE == 2) ((int4*)ll)[i] = ld16(xl + 16 * i);
    }
    for (int64_t i = tid; i < nb; i += GL_NT) lsx[i] = xs[i];
    // rows past F do not occur: F is a multiple of 32
    stage_scales(lsg, (int)nb, sg, nb, o0 + 32, o0, 32, 0, (int)nb, tid, GL_NT);
    stage_scales(lsg + 32 * nb, (int)nb, su, nb, o0 + 32, o0, 32, 0, (int)nb, tid, GL_NT);
    __syncthreads();
#pragma unroll
    for (int k = 1; k < NB; ++k) group_load<U>(w[k], wrow, 0, (int)nb, k, j);
  }

  const float yv = chunk_dot4<MODE, U, NB>(wrow, lq, ll, lsx, lsg + (up ? 32 + rr : rr) * nb, 0, (int)nb, j, hf, w);
  if (li == 0) lout[(up ? 32 : 0) + rr] = yv;
  __syncthreads();
  if (wave == 0) {
    // lanes 0..7 take outputs 4*lane .. 4*lane + 3; every lane takes part in the block maximum
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane < 8) {
      const int i = 4 * lane;
      v = make_float4(glu_mul<ACT>(lout[i], lout[32 + i]), glu_mul<ACT>(lout[i + 1], lout[33 + i]),
                      glu_mul<ACT>(lout[i + 2], lout[34 + i]), glu_mul<ACT>(lout[i + 3], lout[35 + i]));
      if (h) *(float4*)(h + o0 + i) = v;
    }
    int hw, lw;
    const float sc = quant_lane4<MODE>(v, &hw, &lw);
    if (lane < 8) {
      *(int*)(hq + o0 + 4 * lane) = hw;
      if constexpr (MODE == 2) *(int*)(hl + o0 + 4 * lane) = lw;
      if (lane == 0) hs[o0 / QK] = sc;
    }
  }
}

template <int MODE, bool DMA, int ACT>
hipError_t launch_glu_s(const int8_t* wg, const uint16_t* sg, const int8_t* wu, const uint16_t* su, int64_t F,
                        int64_t K, const int8_t* xq, const int8_t* xl, const float* xs, float* h, int8_t* hq,
                        int8_t* hl, float* hs, hipStream_t st) {
  static const hipError_t attr = hipFuncSetAttribute((const void*)&k_gemv_glu<MODE, DMA, ACT>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, GL_LDS_MAX);
  if (attr != hipSuccess) return attr;
  const size_t lds = (size_t)(K / QK) * gl_bytes_per_block<MODE>();
  const dim3 grid((unsigned)(F / 32)), block(GL_NT);
  return launch((k_gemv_glu<MODE, DMA, ACT>), grid, block, lds, st, wg, sg, wu, su, K, xq, xl, xs, h, hq, hl, hs);
}

// LDS DMA staging when K is a multiple of 256 and every staged array starts
// 16-byte aligned; the knob QDG_TUNE_WS_DMA = 0 turns it off.
template <int MODE, int ACT>
hipError_t launch_glu_m(const int8_t* wg, const uint16_t* sg, const int8_t* wu, const uint16_t* su, int64_t F,
                        int64_t K, const int8_t* xq, const int8_t* xl, const float* xs, float* h, int8_t* hq,
                        int8_t* hl, float* hs, hipStream_t st) {
  bool dma = K % 256 == 0 && (((uintptr_t)xq | (uintptr_t)xs | (uintptr_t)sg | (uintptr_t)su) & 15) == 0 &&
             (MODE == 1 || ((uintptr_t)xl & 15) == 0);
  if (tune(QDG_TUNE_WS_DMA) == 0) dma = false;
  if (dma) return launch_glu_s<MODE, true, ACT>(wg, sg, wu, su, F, K, xq, xl, xs, h, hq, hl, hs, st);
  return launch_glu_s<MODE, false, ACT>(wg, sg, wu, su, F, K, xq, xl, xs, h, hq, hl, hs, st);
}

}  // namespace

bool glu_fits(int mode, int64_t K) {
  const int64_t bpb = (mode == 2 ? 2 : 1) * QK + 4 + 2 * GL_ROWS;
  return (K / QK) * bpb <= GL_LDS_MAX;
}

namespace {
template <int ACT>
hipError_t launch_gemv_glu_a(int mode, const int8_t* wg, const uint16_t* sg, const int8_t* wu, const uint16_t* su,
                        int64_t F, int64_t K, const int8_t* xq, const int8_t* xl, const float* xs, float* h,
                        int8_t* hq, int8_t* hl, float* hs, hipStream_t st) {
  if (mode == 1) return launch_glu_m<1, ACT>(wg, sg, wu, su, F, K, xq, xl, xs, h, hq, hl, hs, st);
  return launch_glu_m<2, ACT>(wg, sg, wu, su, F, K, xq, xl, xs, h, hq, hl, hs, st);
}
}  // namespace

hipError_t launch_gemv_glu(int act, int mode, const int8_t* wg, const uint16_t* sg, const int8_t* wu,
                           const uint16_t* su, int64_t F, int64_t K, const int8_t* xq, const int8_t* xl,
                           const float* xs, float* h, int8_t* hq, int8_t* hl, float* hs, hipStream_t st) {
  if (act == 0) return launch_gemv_glu_a<0>(mode, wg, sg, wu, su, F, K, xq, xl, xs, h, hq, hl, hs, st);
  if (act == 1) return launch_gemv_glu_a<1>(mode, wg, sg, wu, su, F, K, xq, xl, xs, h, hq, hl, hs, st);
  return launch_gemv_glu_a<2>(mode, wg, sg, wu, su, F, K, xq, xl, xs, h, hq, hl, hs, st);
}

}  // namespace qdg
