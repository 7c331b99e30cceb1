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

__device__ __forceinline__ float lanes8_max(float a) {
  a = fmaxf(a, __shfl_xor(a, 1, 64));
  a = fmaxf(a, __shfl_xor(a, 2, 64));
  a = fmaxf(a, __shfl_xor(a, 4, 64));
  return a;
}

// rn() of the page with a saturating clamp to int8 (no-op inside the contract).
__device__ __forceinline__ int rn_clamp8(float v) {
  const float r = __builtin_rintf(v);
  return (int)__builtin_fminf(__builtin_fmaxf(r, -128.0f), 127.0f);
}

__device__ __forceinline__ int pack4(int a, int b, int c, int d) {
  return (int)((unsigned)(a & 255) | ((unsigned)(b & 255) << 8) | ((unsigned)(c & 255) << 16) |
               ((unsigned)(d & 255) << 24));
}

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
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = lanes8_max(a);
  if (!on) return;
  const float vv[4] = {v.x, v.y, v.z, v.w};
  int h[4], l[4];
  float s;
  if constexpr (MODE == 1) {
    s = a > 0.0f ? a / 127.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = rn_clamp8(vv[i] / s);
  } else {
    s = (a > 1e-30f ? a : 1e-30f) / 127.0f;
    const float lsc = __fmul_rn(s, 0.0078125f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = rn_clamp8(vv[i] / s);
      const float r = __fmaf_rn(-(float)h[i], s, vv[i]);
      l[i] = rn_clamp8(r / lsc);
    }
    *(int*)(xl + blk * QK + sub * 4) = pack4(l[0], l[1], l[2], l[3]);
  }
  *(int*)(xq + blk * QK + sub * 4) = pack4(h[0], h[1], h[2], h[3]);
  if (sub == 0) xs[blk] = s;
}

}  // namespace

hipError_t launch_quantize(int mode, const float* x, int64_t nblocks, int8_t* xq, int8_t* xl, float* xs,
                           hipStream_t st) {
  const int64_t threads = nblocks * 8;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (mode == 1)
    hipLaunchKernelGGL(k_quantize<1>, grid, block, 0, st, x, xq, xl, xs, nblocks);
  else
    hipLaunchKernelGGL(k_quantize<2>, grid, block, 0, st, x, xq, xl, xs, nblocks);
  return hipGetLastError();
}

}  // namespace qdg
