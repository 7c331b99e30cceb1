// qdg_device.h -- device helpers and launcher declarations shared by the gfx950
// kernels of libqdg.so (internal; the public interface is include/qdg.h).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>

#include "../../include/qdg.h"

namespace qdg {

// The process-wide tuning knobs (qdg_set_tuning; -1 = the library's choice) and
// the calling thread's measurement events for its next launch
// (qdg_time_next_launch), taken and cleared by that launch.  Both live in
// qdg_api.hip.
int tune(int knob);
struct LaunchTiming {
  hipEvent_t start, stop;
};
LaunchTiming take_launch_timing();

// Every kernel of the library is launched through here.  The dispatch carries
// the thread's measurement events when some are bound (hipExtLaunchKernel takes
// them on the kernel's own packet), and the error-path test hook
// (QDG_TUNE_REJECT_LAUNCH) asks for a workgroup of 2048 threads, which the
// runtime refuses before anything is enqueued.  A refused launch leaves no
// pending error behind for the caller's next HIP call.
template <typename... P, typename... A>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t st, A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<std::decay_t<P>...> vals{static_cast<std::decay_t<P>>(args)...};
  void* ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1];
  std::apply([&ptrs](auto&... v) {
    int i = 0;
    ((ptrs[i++] = (void*)&v), ...);
  }, vals);
  if (tune(QDG_TUNE_REJECT_LAUNCH) == 1) block = dim3(2048, 1, 1);
  const LaunchTiming t = take_launch_timing();
  const hipError_t e = hipExtLaunchKernel((const void*)kernel, grid, block, ptrs, lds, st, t.start, t.stop, 0);
  if (e != hipSuccess) (void)hipGetLastError();
  return e;
}

constexpr int QK = 32;          // values per Q8_0 block
constexpr int SUPER = 16;       // blocks per 512-value superblock of the split-K chunk rule

// The split-K chunk rule of the QWEN38 page (gk_gemv_hl_sk): 512-value
// superblocks, per = ceil(nq/S), chunk s = superblocks [s*per, min((s+1)*per, nq)),
// the K mod 512 tail in the last chunk.  Returned as 32-value block bounds.
// The same with K < 2^31 given as nq = K/512 superblocks, nb = K/32 blocks and
// per = ceil(nq/S), in 32-bit arithmetic (a kernel that walks several chunks
// forms these once).
__host__ __device__ inline void split_range32(int nq, int nb, int per, int S, int s, int32_t& g0, int32_t& g1) {
  const int q0 = s * per < nq ? s * per : nq, q1 = (s + 1) * per < nq ? (s + 1) * per : nq;
  g0 = q0 * SUPER;
  g1 = s == S - 1 ? nb : q1 * SUPER;
}
__host__ __device__ inline void split_range(int64_t K, int S, int s, int32_t& g0, int32_t& g1) {
  const int64_t nq = K / 512, nb = K / QK, per = (nq + S - 1) / S;
  int64_t q0 = (int64_t)s * per;
  if (q0 > nq) q0 = nq;
  int64_t q1 = (int64_t)(s + 1) * per;
  if (q1 > nq) q1 = nq;
  g0 = (int32_t)(q0 * SUPER);
  g1 = (s == S - 1) ? (int32_t)nb : (int32_t)(q1 * SUPER);
}

// Chunk waves a row group for the kernels whose workgroups hold the S chunks of
// their rows as waves, W of them each summing chunks w, w + W, ... in turn (so W
// changes no bit).  A compute unit holds a bounded number of a kernel's
// workgroups at once (resident(W), from the HIP occupancy calculator); with a
// wave a chunk the 5120-row projections at S = 8 ask for more than fit and run
// their last workgroups as a second, thinly occupied round.  The choice: the
// smallest W for which every workgroup (wgs of them) is resident at once and
// whose busiest wave holds the fewest blocks; where no W fits one round,
// min(ceff, cap).  `forced` (> 0) overrides.
int device_cus();
template <typename Resident>
int pick_chunk_waves(int64_t wgs, int cap, int64_t K, int S, int m, int ceff, int forced, Resident resident) {
  cap = ceff < cap ? ceff : cap;
  if (forced > 0) return forced < cap ? forced : cap;
  const int64_t cus = device_cus();
  int best = cap;
  int64_t best_load = INT64_MAX;
  for (int W = 1; W <= cap; ++W) {
    if ((int64_t)resident(W) * cus < wgs) break;
    int64_t load = 0;
    for (int w = 0; w < W; ++w) {
      int64_t l = 0;
      for (int c = w; c < ceff; c += W) {
        int32_t g0, g1;
        split_range(K, S, c < m ? c : S - 1, g0, g1);
        l += g1 - g0;
      }
      load = l > load ? l : load;
    }
    if (load < best_load) best_load = load, best = W;
  }
  return best;
}

// DPP lane moves (GFX9 encodings).  A lane whose source lies outside its
// 16-lane row reads 0; callers only consume lanes whose source is inside.
enum : int {
  DPP_QUAD_SWAP1 = 0xB1,  // quad_perm [1,0,3,2]: lane i <- lane i^1
  DPP_ROW_SHL2 = 0x102,   // lane i <- lane i+2 within the row
  DPP_ROW_SHL4 = 0x104,   // lane i <- lane i+4 within the row
  DPP_ROW_SHL8 = 0x108,   // lane i <- lane i+8 within the row
};

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  // bound_ctrl: a lane whose source is outside its row reads 0 (the same as an
  // old value of 0 with bound_ctrl off, without the move that sets it up)
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp_i32<CTRL>((int)(b & 0xffffffffll));
  const int hi = dpp_i32<CTRL>((int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

typedef int v4i __attribute__((ext_vector_type(4)));

// 16-byte loads.  The weight stream is read once per call, so it is loaded with
// the nontemporal hint (the cache lines are not kept for reuse); activations,
// which every workgroup re-reads, use ordinary loads.
__device__ __forceinline__ int4 to_int4(v4i t) { return make_int4(t[0], t[1], t[2], t[3]); }
__device__ __forceinline__ int4 ld16_stream(const int8_t* p) {
  return to_int4(__builtin_nontemporal_load((const v4i*)p));
}
__device__ __forceinline__ int4 ld16(const int8_t* p) { return to_int4(*(const v4i*)p); }
__device__ __forceinline__ unsigned short ld_u16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load((const unsigned short*)p);
}

// Copies the weight scales of `rows` consecutive rows (first row o0, rows at or
// past N read row N-1) over blocks [b0, b0 + n) into LDS as [row][n_pitch]
// (binary16 bits), with `nthreads` threads of index `tid`.  When a row's segment
// starts 16-byte aligned (ws 16-byte aligned, nb and b0 multiples of 8) the bulk
// moves in 16-byte words and only the last n mod 8 scales of a row move one by one.
__device__ __forceinline__ void stage_scales(uint16_t* __restrict__ dst, int pitch, const uint16_t* __restrict__ ws,
                                             int64_t nb, int64_t N, int64_t o0, int rows, int64_t b0, int n,
                                             int tid, int nthreads) {
  const bool wide = (nb % 8) == 0 && (b0 % 8) == 0 && (pitch % 8) == 0 && ((uintptr_t)ws & 15) == 0;
  const int nv = wide ? n / 8 : 0;  // 16-byte words per row
  for (int i = tid; i < rows * nv; i += nthreads) {
    const int r = i / nv, c = i - r * nv;
    int64_t o = o0 + r;
    if (o >= N) o = N - 1;
    *(int4*)(dst + r * pitch + 8 * c) = *(const int4*)(ws + o * nb + b0 + 8 * c);
  }
  const int rest = n - 8 * nv;
  for (int i = tid; i < rows * rest; i += nthreads) {
    const int r = i / rest, c = 8 * nv + (i - r * rest);
    int64_t o = o0 + r;
    if (o >= N) o = N - 1;
    dst[r * pitch + c] = ws[o * nb + b0 + c];
  }
}

// Exact int32 dot of 16 int8 pairs held in one lane (four v_dot4 steps).
__device__ __forceinline__ int dot16_i8(int4 w, int4 a) {
  int d = __builtin_amdgcn_sdot4(w.x, a.x, 0, false);
  d = __builtin_amdgcn_sdot4(w.y, a.y, d, false);
  d = __builtin_amdgcn_sdot4(w.z, a.z, d, false);
  d = __builtin_amdgcn_sdot4(w.w, a.w, d, false);
  return d;
}

// A 32-value block's exact int32 dot, the block split over the lane pair
// (2j, 2j+1) with 16 values each: both lanes return the block's dot.
__device__ __forceinline__ int block_dot_pair(int4 w, int4 a) {
  const int d = dot16_i8(w, a);
  return d + dpp_i32<DPP_QUAD_SWAP1>(d);
}

__device__ __forceinline__ float half_bits_to_float(unsigned short h) {
  return __half2float(__ushort_as_half(h));
}

// Arg-max keys (megakernel page, amax_key): the float's bits mapped to an
// unsigned integer that orders as the floats do, above the complement of the
// index, so the largest key is the largest value and, among equal values, the
// smallest index.  -0 is folded onto +0 first so that the two compare equal as
// IEEE floats do; the maximum of keys is order-free, which makes the result
// independent of how the values are split over lanes and workgroups.
__device__ __forceinline__ unsigned long long amax_key(float v, unsigned idx) {
  unsigned u = __float_as_uint(v);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(0xffffffffu - idx);
}

// Split-K partials handed to the last-arriving workgroup of a row tile.  A slot
// holds the partial's bits XOR a signalling-NaN pattern: no arithmetic result is
// a signalling NaN, so no published slot is zero, and a zero slot means "not yet
// published".  Every access to a slot (and to the tile's ticket) is an
// agent-scope atomic, so nothing races; the result does not rest on the order in
// which another workgroup's stores become visible: the last arriver waits,
// boundedly, until each slot it adds is nonzero, then clears it for the next
// call (the workspace is zero-filled before its first use).  Were the bound ever
// reached, the stale zero decodes to the pattern itself, a NaN in the output.
constexpr unsigned PART_MARK32 = 0x7f80deadu;                 // binary32 signalling NaN
constexpr unsigned long long PART_MARK64 = 0x7ff0deadbeef0001ull;  // binary64 signalling NaN
constexpr int PART_SPIN_LIMIT = 1 << 22;

__device__ __forceinline__ void publish_partial(unsigned* slot, float v) {
  __hip_atomic_store(slot, __float_as_uint(v) ^ PART_MARK32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_partial(unsigned long long* slot, double v) {
  __hip_atomic_store(slot, (unsigned long long)__double_as_longlong(v) ^ PART_MARK64, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T take_slot(T* slot) {
  T v = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int spin = 0; v == 0 && spin < PART_SPIN_LIMIT; ++spin) {
    __builtin_amdgcn_s_sleep(1);
    v = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __hip_atomic_store(slot, (T)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}
__device__ __forceinline__ float take_partial(unsigned* slot) { return __uint_as_float(take_slot(slot) ^ PART_MARK32); }
__device__ __forceinline__ double take_partial(unsigned long long* slot) {
  return __longlong_as_double((long long)(take_slot(slot) ^ PART_MARK64));
}

// One quantized step's factors (lane kernel library page, lk_q8_term):
// Int8Act a = fl(sigma*s), b = D; TwoPass a = sigma, b = fma(s, D, fl(fl(s/128)*E)).
template <int MODE>
__device__ __forceinline__ void q8_term(float sigma, float s, int d, int e, float& a, float& b) {
  if constexpr (MODE == 1) {
    a = __fmul_rn(sigma, s);
    b = (float)d;
  } else {
    const float lo = __fmul_rn(__fmul_rn(s, 0.0078125f), (float)e);
    a = sigma;
    b = __fmaf_rn(s, (float)d, lo);
  }
}

// The activation quantizer of one 32-value block, for the four values v of one
// lane of the block's 8-lane group (lane kernel library page: lk_quant_lane,
// lk_two_scale, lk_two_words).  All 64 lanes must call it (the block maximum is
// a butterfly over the 8 lanes; max is exact and order-free).  Returns the four
// words packed first-lowest in *h (and *l under TwoPass) and the block scale.
__device__ __forceinline__ int pack4_i8(int a, int b, int c, int d) {
  return (int)((unsigned)(a & 255) | ((unsigned)(b & 255) << 8) | ((unsigned)(c & 255) << 16) |
               ((unsigned)(d & 255) << 24));
}
// round to nearest, ties to even, then saturate to int8 (a no-op inside the contract)
__device__ __forceinline__ int rn_clamp8(float v) {
  const float r = __builtin_rintf(v);
  return (int)__builtin_fminf(__builtin_fmaxf(r, -128.0f), 127.0f);
}
template <int MODE>
__device__ __forceinline__ float quant_lane4(float4 v, int* h, int* l) {
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = fmaxf(a, __shfl_xor(a, 1, 64));
  a = fmaxf(a, __shfl_xor(a, 2, 64));
  a = fmaxf(a, __shfl_xor(a, 4, 64));
  const float vv[4] = {v.x, v.y, v.z, v.w};
  int hh[4], ll[4];
  float s;
  if constexpr (MODE == 1) {
    s = a > 0.0f ? a / 127.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) hh[i] = rn_clamp8(vv[i] / s);
    *l = 0;
  } else {
    s = (a > 1e-30f ? a : 1e-30f) / 127.0f;
    const float lsc = __fmul_rn(s, 0.0078125f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hh[i] = rn_clamp8(vv[i] / s);
      const float r = __fmaf_rn(-(float)hh[i], s, vv[i]);
      ll[i] = rn_clamp8(r / lsc);
    }
    *l = pack4_i8(ll[0], ll[1], ll[2], ll[3]);
  }
  *h = pack4_i8(hh[0], hh[1], hh[2], hh[3]);
  return s;
}

// The RMSNorm's arithmetic (lane kernel library page, RMSNORM: v = x + r,
// y = v / sqrt(mean(v^2) + eps) * w), shared by the norm producer and the norm
// epilogue of the split-K GEMV so that the two give the same bits: the residual
// add is one binary32 addition a value; the squares are exact in binary64 and
// summed there; the divisor is the correctly rounded binary64 square root; each
// value is divided and scaled in binary64 and rounded once to binary32.
__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(__fadd_rn(a.x, b.x), __fadd_rn(a.y, b.y), __fadd_rn(a.z, b.z), __fadd_rn(a.w, b.w));
}
__device__ __forceinline__ double sq4(float4 v) {
  double a = (double)v.x * (double)v.x;
  a += (double)v.y * (double)v.y;
  a += (double)v.z * (double)v.z;
  a += (double)v.w * (double)v.w;
  return a;
}
__device__ __forceinline__ double norm_den(double sumsq, int64_t n, float eps) {
  return __dsqrt_rn(sumsq / (double)n + (double)eps);
}
// four values of the row, normed; g holds their four weights when has_w
__device__ __forceinline__ float4 norm4(float4 t, double den, bool has_w, float4 g) {
  double ox = (double)t.x / den, oy = (double)t.y / den;
  double oz = (double)t.z / den, ow = (double)t.w / den;
  if (has_w) {
    ox *= (double)g.x;
    oy *= (double)g.y;
    oz *= (double)g.z;
    ow *= (double)g.w;
  }
  return make_float4((float)ox, (float)oy, (float)oz, (float)ow);
}

// The gated product of one value, act(g) * u (lane kernel library page, lk_act
// and GLU): act 0 silu g / (1 + e^-g), 1 sigmoid 1 / (1 + e^-g), 2 the GELU in its
// tanh form g / (1 + e^-2z) with z = sqrt(2/pi) * (g + 0.044715 g^3), g^3 as
// (g*g)*g; every step in binary64 from the binary32 operands, in the order
// written, and rounded once to binary32.  Shared by the producer and the gate/up
// GEMV epilogue, so the two give the same bits.
template <int ACT>
__device__ __forceinline__ float glu_mul(float g, float u) {
  const double gd = (double)g;
  double a;
  if constexpr (ACT == 0) {
    a = gd / (1.0 + exp(-gd));
  } else if constexpr (ACT == 1) {
    a = 1.0 / (1.0 + exp(-gd));
  } else {
    const double z = 0.79788456080286535588 * (gd + 0.044715 * ((gd * gd) * gd));
    a = gd / (1.0 + exp(-2.0 * z));
  }
  return (float)(a * (double)u);
}

// The s_waitcnt operand that waits until at most n vector-memory loads of the
// wave are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt at their no-wait maxima).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

// Waits until at most N of the wave's vector-memory loads are outstanding and
// its LDS accesses are done, then meets the workgroup.  Unlike __syncthreads(),
// whose workgroup fences wait for every outstanding global load (LDS DMA writes
// count as such), the wave's last N loads stay in flight across it; loads
// complete in issue order, so every earlier load -- LDS DMA included -- has
// landed.  The empty asm statements keep the compiler from moving memory
// accesses across.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);  // vmcnt(N) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A workgroup barrier for LDS only: the wave's global loads and stores stay in
// flight (a store need not be acknowledged before the wave goes on).
__device__ __forceinline__ void lds_barrier() { wait_barrier<63>(); }

// LDS DMA (gfx950 global_load_lds_dwordx4): each active lane's 16 bytes at g
// land at l + 16*lane, with l the same for the whole wave (it goes to M0).  The
// load counts in vmcnt like any other; it needs no VGPR for the data.
__device__ __forceinline__ void lds_dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}

// Requests step group gi's weights of the lane (U loads of 16 bytes, blocks
// g0 + (gi*U + u)*8 + j).  The loads are always issued, so every wave has the
// same number in flight and the compiler can count them: a lane whose block lies
// at or past g1 reads block g1 - 1 again, and chunk_dot4 never adds its term.
// The scheduling barriers keep the requests where they are written.
//
// TL selects the row-tiled weight layout (tiles of four rows by 256 values,
// tile after tile; the megakernel page's tiled-weights option with a tile that
// is one wave instruction's bytes): block b of a row then sits at
// (b/8)*1024 + (b%8)*32 from the row's first piece, wrow pointing at the row's
// tile plus 256 * (row mod 4) + 16*hf, so a wave's 64 lanes read one
// contiguous KiB.  The values and their order are those of the plain layout.
template <bool TL>
__device__ __forceinline__ int64_t block_offset(int b) {
  return TL ? ((int64_t)(b >> 3) << 10) + ((b & 7) << 5) : (int64_t)b * QK;
}

template <int U, bool TL = false>
__device__ __forceinline__ void group_load(int4 (&w)[U], const int8_t* wrow, int g0, int g1, int gi, int j) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int b = g0 + (gi * U + u) * 8 + j;
    w[u] = ld16_stream(wrow + block_offset<TL>(b < g1 ? b : g1 - 1));
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Step group gi's terms: U steps of 8 blocks; block bl of the chunk (lane pair
// j = bl mod 8) adds its step to partial bl mod 4 -- lanes j < 4 take blocks j
// and then j + 4 of each step, the latter moved over by DPP.  Blocks at or past
// nwb add nothing.  The LDS arrays hold block b at index b - lb.
template <int MODE, int U>
__device__ __forceinline__ void group_terms(const int4 (&w)[U], const int8_t* lq, const int8_t* ll, const float* lsx,
                                            const uint16_t* my_sg, int g0, int nwb, int j, int hf, int gi, float& p,
                                            int lb = 0) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int bl = (gi * U + u) * 8 + j;  // block within the chunk
    const bool ok = bl < nwb;
    const int blc = g0 - lb + (ok ? bl : 0);  // LDS index
    const int d = block_dot_pair(w[u], *(const int4*)(lq + blc * QK + hf * 16));
    int e = 0;
    if constexpr (MODE == 2) e = block_dot_pair(w[u], *(const int4*)(ll + blc * QK + hf * 16));
    float ta, tb;
    q8_term<MODE>(half_bits_to_float(my_sg[blc]), lsx[blc], d, e, ta, tb);
    p = ok ? __fmaf_rn(ta, tb, p) : p;
    const float ta2 = dpp_f32<DPP_ROW_SHL8>(ta), tb2 = dpp_f32<DPP_ROW_SHL8>(tb);
    p = bl + 4 < nwb ? __fmaf_rn(ta2, tb2, p) : p;
  }
}

// One wave's chunk partial of four rows (16 lanes a row, a lane pair a block),
// the lane kernel library page's row order restricted to blocks [g0, g1): block
// g's step p <- fma(a, b, p) goes into partial g mod 4 (lane pair g mod 4 of the
// row, blocks j and j+4 of each 8-block step), each partial ascending from +0,
// then (P0 + P2) + (P1 + P3), returned in lane 0 of the row (the other lanes
// hold partial sums).  wrow points at the lane's row plus 16*hf; lq, ll and lsx
// hold the activation words and scales by absolute block, my_sg the row's
// weight scales by absolute block.
//
// The weights stream through NB named buffers of U steps: w[k] holds step group
// k on entry (requested by the caller with group_load, so they can be in flight
// across its staging), and each buffer is refilled NB groups ahead right after
// its terms are taken.  Up to NB groups stay in flight, and no register copy has
// to wait for a load (a copy-based double buffer drains every load at each
// copy).  The wave-uniform bounds keep the loop scalar.
//
// chunk_fold adds blocks [g0, g1) into the lane's partial p (so a row split into
// LDS windows keeps one chain per partial across them; the window's arrays hold
// block b at index b - lb); chunk_dot4 starts from +0 and ends with the
// (P0 + P2) + (P1 + P3) reduction.
template <int MODE, int U, int NB, bool TL = false>
__device__ __forceinline__ void chunk_fold(const int8_t* wrow, const int8_t* lq, const int8_t* ll, const float* lsx,
                                           const uint16_t* my_sg, int g0, int g1, int j, int hf,
                                           int4 (&w)[NB][U], float& p, int lb = 0) {
  const int nwb = g1 - g0;
  const int ngroups = ((nwb + 7) / 8 + U - 1) / U;
  int gi = 0;
  // while every refill is due: no branch inside, so each group waits for its own loads only
  for (; gi + 2 * NB - 1 < ngroups; gi += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      group_terms<MODE, U>(w[k], lq, ll, lsx, my_sg, g0, nwb, j, hf, gi + k, p, lb);
      group_load<U, TL>(w[k], wrow, g0, g1, gi + NB + k, j);
    }
  }
  // the last 1 .. 2*NB - 1 groups, in order (a group past the chunk adds nothing)
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    group_terms<MODE, U>(w[k], lq, ll, lsx, my_sg, g0, nwb, j, hf, gi + k, p, lb);
    if (gi + NB + k < ngroups) group_load<U, TL>(w[k], wrow, g0, g1, gi + NB + k, j);
  }
#pragma unroll
  for (int k = 0; k + 1 < NB; ++k)
    if (gi + NB + k < ngroups) group_terms<MODE, U>(w[k], lq, ll, lsx, my_sg, g0, nwb, j, hf, gi + NB + k, p, lb);
}

// (P0 + P2) + (P1 + P3): partial q sits in lane pair q of the row's 16 lanes.
__device__ __forceinline__ float row_sum4(float p) {
  const float t = __fadd_rn(p, dpp_f32<DPP_ROW_SHL4>(p));
  return __fadd_rn(t, dpp_f32<DPP_ROW_SHL2>(t));
}

template <int MODE, int U, int NB, bool TL = false>
__device__ __forceinline__ float chunk_dot4(const int8_t* wrow, const int8_t* lq, const int8_t* ll, const float* lsx,
                                            const uint16_t* my_sg, int g0, int g1, int j, int hf,
                                            int4 (&w)[NB][U]) {
  float p = 0.0f;
  chunk_fold<MODE, U, NB, TL>(wrow, lq, ll, lsx, my_sg, g0, g1, j, hf, w, p);
  return row_sum4(p);
}

// Up to MAX_PARTS weight matrices over one activation in one launch (lane kernel
// library page, GEMV_PARTS and lk_part_y: q, k and v, or gate and up, side by
// side).  Workgroups [tile_end[p-1], tile_end[p]) take part p's row tiles; a
// single matrix is a table of one part.  Passed by value as a kernel argument.
constexpr int MAX_PARTS = 6;
struct PartTable {
  const int8_t* wq[MAX_PARTS];
  const uint16_t* ws[MAX_PARTS];
  float* y[MAX_PARTS];
  int64_t N[MAX_PARTS];
  int tile_end[MAX_PARTS];
  int n;
};

// The part of workgroup `tile` and its first row (a scan of at most six uniform values).
__device__ __forceinline__ int find_part(const PartTable& t, int tile, int rows, int64_t& o_wg) {
  int p = 0;
  while (p + 1 < t.n && tile >= t.tile_end[p]) ++p;
  o_wg = (int64_t)(tile - (p > 0 ? t.tile_end[p - 1] : 0)) * rows;
  return p;
}

// A table of `n` parts of `rows`-row workgroups; false if it overflows an int grid.
inline bool make_parts(PartTable& t, int n, const int8_t* const* wq, const uint16_t* const* ws, float* const* y,
                       const int64_t* N, int rows) {
  int64_t end = 0;
  t.n = n;
  for (int p = 0; p < MAX_PARTS; ++p) {
    t.wq[p] = p < n ? wq[p] : nullptr;
    t.ws[p] = p < n ? ws[p] : nullptr;
    t.y[p] = p < n ? y[p] : nullptr;
    t.N[p] = p < n ? N[p] : 0;
    if (p < n) end += (N[p] + rows - 1) / rows;
    if (end >= ((int64_t)1 << 31)) return false;
    t.tile_end[p] = (int)end;
  }
  return true;
}

// Launchers (one translation unit each); all return the launch's hipError_t.
hipError_t launch_quantize(int mode, const float* x, int64_t nblocks, int8_t* xq, int8_t* xl, float* xs,
                           hipStream_t st);
hipError_t launch_gemv_dot4(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K,
                            const int8_t* xq, const int8_t* xl, const float* xs, int splits, float* out,
                            hipStream_t st);
hipError_t launch_gemv_dequant(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                               float* out, hipStream_t st);
hipError_t launch_gemv_dequant_sk(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                                  int splits, float* y, void* workspace, hipStream_t st);
int64_t sk_partials_offset(int64_t N);
hipError_t launch_gemv_dequant_argmax(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                                      float* y, unsigned long long* keys, hipStream_t st);
hipError_t launch_gemv_mfma(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K,
                            const int8_t* xq, const int8_t* xl, const float* xs, int64_t B, int splits,
                            float* out, hipStream_t st);
hipError_t launch_block_dots(int mode, const int8_t* wq, int64_t N, int64_t K, const int8_t* xq,
                             const int8_t* xl, int64_t B, int32_t* dh, int32_t* dl, hipStream_t st);
hipError_t launch_combine(const float* part, int splits, int64_t count, float* y, hipStream_t st);
size_t sk_workspace_bytes(int64_t N, int splits);
hipError_t launch_gemv_sk(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq,
                          const int8_t* xl, const float* xs, int splits, float* y, void* workspace, hipStream_t st);
hipError_t launch_gemv_x(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                         int splits, float* y, void* workspace, hipStream_t st);
int argmax_groups(int64_t N);
hipError_t launch_stream_read(const void* buf, int64_t bytes, unsigned* sink, hipStream_t st);
bool wsplit_fits(int mode, int64_t K, int splits);
int dq_seg_chunks(int64_t K, int splits);
hipError_t launch_gemv_dq_seg(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x, int splits,
                              float* y, hipStream_t st);
hipError_t launch_gemv_dq_seg_parts(int nparts, const int8_t* const* wq, const uint16_t* const* ws, const int64_t* N,
                                    float* const* y, int64_t K, const float* x, int splits, hipStream_t st);
// the unsplit Dequant call's chunk count for N rows (qdg_dequant.hip), and the
// gate/up kernel with the gated product in that order (qdg_dequant_seg.hip)
int dq_unsplit_order(int64_t N);
hipError_t launch_gemv_dq_glu(int act, const int8_t* wg, const uint16_t* sg, const int8_t* wu, const uint16_t* su,
                              int64_t F, int64_t K, const float* x, int S, float* h, hipStream_t st);
void wsplit_shape(int64_t K, int splits, int& rows, int& waves);
// tiled: the weights in row tiles of four rows by 256 values (launch_tile_rows)
hipError_t launch_gemv_wsplit(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K,
                              const int8_t* xq, const int8_t* xl, const float* xs, int splits, float* y,
                              hipStream_t st, bool tiled = false);
hipError_t launch_gemv_wsplit_parts(int mode, int nparts, const int8_t* const* wq, const uint16_t* const* ws,
                                    const int64_t* N, float* const* y, int64_t K, const int8_t* xq,
                                    const int8_t* xl, const float* xs, int splits, hipStream_t st,
                                    bool tiled = false);
// the in-workgroup split with the residual add, RMSNorm and quantizer run by
// one more workgroup over the published rows (one activation row; workspace:
// one word a row)
size_t gemv_norm_workspace_bytes(int64_t N);
int64_t gemv_norm_max_n();
hipError_t launch_gemv_wsplit_norm(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K,
                                   const int8_t* xq, const int8_t* xl, const float* xs, int splits, float* y,
                                   const float* r, float* s, const float* w, float eps, int qmode, float* yn,
                                   int8_t* hq, int8_t* hl, float* hs, void* workspace, hipStream_t st);
hipError_t launch_tile_rows(const int8_t* wq, int64_t N, int64_t K, int8_t* wt, hipStream_t st);
int64_t tile_mma_bytes(int64_t N, int64_t K);
hipError_t launch_tile_mma(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, uint8_t* wt, hipStream_t st);
hipError_t launch_quantize_mma(int mode, const float* x, int64_t B, int64_t K, int8_t* xq, int8_t* xl, float* xs,
                               hipStream_t st);
hipError_t launch_gemv_mma_tiled(int mode, const uint8_t* wt, int64_t N, int64_t K, const int8_t* xq,
                                 const int8_t* xl, const float* xs, int64_t B, int splits, float* out,
                                 hipStream_t st);
int mma_act_tiles(int64_t B);
hipError_t launch_gemv_glu_mma(int act, int mode, const uint8_t* wgt, const uint8_t* wut, int64_t F, int64_t K,
                               const int8_t* xq, const int8_t* xl, const float* xs, int64_t B, float* h, int8_t* hq,
                               int8_t* hl, float* hs, hipStream_t st);
int64_t rmsnorm_max_k();
hipError_t launch_rmsnorm_quant(int mode, const float* x, const float* r, float* s, const float* w, float eps,
                                int64_t B, int64_t K, float* y, int8_t* xq, int8_t* xl, float* xs, hipStream_t st);
bool glu_fits(int mode, int64_t K);
void fmt_geometry(int fmt, int& values, int& bytes);
int fmt_chunk_waves(int fmt, int mode, int64_t N, int64_t K, int S);
int dq_chunk_waves(int64_t N, int64_t K, int splits);
hipError_t launch_gemv_fmt(int fmt, int mode, const uint8_t* w, int64_t N, int64_t K, const float* x,
                           const int8_t* xq, const int8_t* xl, const float* xs, int splits, float* y,
                           hipStream_t st);
hipError_t launch_gemv_glu(int act, int mode, const int8_t* wg, const uint16_t* sg, const int8_t* wu,
                           const uint16_t* su, int64_t F, int64_t K, const int8_t* xq, const int8_t* xl,
                           const float* xs, float* h, int8_t* hq, int8_t* hl, float* hs, hipStream_t st);
hipError_t launch_glu_quant(int act, int mode, const float* g, const float* u, int64_t nblocks, float* h,
                            int8_t* xq, int8_t* xl, float* xs, hipStream_t st);
hipError_t launch_argmax_final(const unsigned long long* keys, int64_t B, int G, int32_t* idx, hipStream_t st);
hipError_t launch_tile_keys(const float* y, int64_t N, unsigned long long* keys, hipStream_t st);
int64_t gemv_tiles(int64_t N);
hipError_t launch_gemv_argmax(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                              const int8_t* xq, const int8_t* xl, const float* xs, float* y, int32_t* idx,
                              unsigned long long* keys, hipStream_t st);
hipError_t launch_argmax(const float* y, int64_t B, int64_t N, int32_t* idx, unsigned long long* ws,
                         hipStream_t st);
}  // namespace qdg
