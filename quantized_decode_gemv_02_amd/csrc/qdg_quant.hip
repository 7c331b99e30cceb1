// qdg_quant.hip -- the activation quantizer (lane kernel library page: module doc on
// the activation quantizer, lk_quant_lane, lk_two_scale, lk_two_words, kernel
// lk_quant; QWEN38 page, two-pass int8 activations).
//
// Layout: B rows of K values are B*K/32 consecutive 32-value blocks.  Eight lanes
// take one block, four consecutive values each (one 16-byte load), so a wave64
// quantizes 8 blocks and every global access is a full, aligned word:
//   x   16 B per lane, xq/xl 4 B per lane (packed int8x4, first value lowest),
//   xs  written by the block's first lane.
// The block maximum is a max over the 8 lanes (a butterfly; max is exact and
// order-free, so its shape does not matter).  Every other step is the page's:
// IEEE division, round-to-nearest-even, one fused multiply-add for the residual.
#include "qdg_device.h"

namespace qdg {
namespace {

template <int MODE>
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ x, int8_t* __restrict__ xq,
                                                  int8_t* __restrict__ xl, float* __restrict__ xs,
                                                  int64_t nblocks) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = gid >> 3;
  const int sub = (int)(gid & 7);
  const bool on = blk < nblocks;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (on) v = *(const float4*)(x + blk * QK + sub * 4);
  int h, l;
  const float s = quant_lane4<MODE>(v, &h, &l);
  if (!on) return;
  *(int*)(xq + blk * QK + sub * 4) = h;
  if constexpr (MODE == 2) *(int*)(xl + blk * QK + sub * 4) = l;
  if (sub == 0) xs[blk] = s;
}

}  // namespace

hipError_t launch_quantize(int mode, const float* x, int64_t nblocks, int8_t* xq, int8_t* xl, float* xs,
                           hipStream_t st) {
  const int64_t threads = nblocks * 8;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (mode == 1)
    return launch(k_quantize<1>, grid, block, 0, st, x, xq, xl, xs, nblocks);
  else
    return launch(k_quantize<2>, grid, block, 0, st, x, xq, xl, xs, nblocks);
}

}  // namespace qdg
