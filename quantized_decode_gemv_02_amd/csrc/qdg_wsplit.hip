// qdg_wsplit.hip -- the split-K GEMV with its combine inside one workgroup: the
// S chunks of a row tile are S waves of the same workgroup, and their partials
// meet in LDS.  It computes exactly what the QWEN38 page's split-K GEMV
// (gk_gemv_hl_sk) followed by its ascending combine (gk_sk_combine) computes:
// wave c forms chunk c's partial of its four rows in the lane kernel library
// page's row order (lk_q8_rows_dot restricted to the chunk, as k_gemv_dot4
// does), and one thread per row then adds the S partials in ascending chunk
// order from +0.  No partial leaves the workgroup, so there is no workspace, no
// ticket and no second launch.
//
// Layout: a workgroup has R row groups of four rows times one wave per
// non-empty chunk (at most 16 waves).  The workgroup stages the whole activation
// row (words, scales) and its rows' weight scales in LDS, since its waves
// between them cover all of K.  A wave's lanes work as in k_gemv_dot4 with four
// rows a wave: 16 lanes a row, a lane pair a block, partial q of the row in lane
// pair q.
//
// Staging (STAGE): WS_DMA moves the staged bytes straight from global memory
// into LDS (global_load_lds_dwordx4) after each wave has requested its first NB
// step groups of weights, so the weights, the activation and the scales are all
// in flight together and one wait covers them; it needs 16-byte aligned inputs
// and K a multiple of 256.  WS_BARRIER (the others) copies through registers
// with the whole workgroup; WS_LOCAL has each wave copy only its own chunk and
// start without a workgroup barrier (waves of different row groups that share a
// chunk write the same bytes).
//
// TL: the weight values in row tiles of four rows by 256 values (tile_rows
// below).  A row group's four rows are one tile row, so each weight request of
// a wave reads one contiguous KiB and a chunk wave streams one contiguous range;
// the terms, their order and the result are those of the plain layout.
//
// NORM (lane kernel library page, GEMV_Q8_NORM, lk_gemv_q8_norm: a projection
// with the residual add and the next norm in its epilogue): each workgroup
// writes its rows and publishes them to marked slots; one more workgroup, the
// grid's last, gathers the whole row from the slots as they fill (it starts with
// the others, so the gather overlaps the projection) and runs the residual add,
// the RMSNorm and the block quantizer over it exactly as k_rmsnorm_quant's
// 1024-thread workgroup does, its waves playing that workgroup's sixteen waves in
// turn (norm_tail).  So its outputs are the bits of qdg_gemv_q8_sk followed by
// qdg_rmsnorm_quantize, in one launch.  The page's kernel elects the norm's block
// by an arrival count instead; with one count for the whole grid, its hundreds
// of atomics on one word cost more (2.6 us on 5120x8192) than the norm workgroup
// waiting on the slots.

#include "qdg_device.h"

namespace qdg {
namespace {

constexpr int WS_NT = 1024;               // sixteen waves
enum { WS_BARRIER = 0, WS_LOCAL = 1, WS_DMA = 2 };
constexpr int WS_U = 1, WS_NB = 4;  // steps a group, groups in flight
constexpr int WS_LDS_MAX = 79 * 1024;     // two workgroups a CU (160 KiB) with the static part

// The norm epilogue's operands.  slots: one marked word a row (zero between
// launches).
struct NormArgs {
  const float* r;   // residual operand, or null
  float* s;         // y + r written back, or null
  const float* w;   // norm weight, or null
  float* yn;        // the normed row (binary32), or null
  int8_t* hq;       // the normed row's words (qmode 1, 2), or null (qmode 0)
  int8_t* hl;
  float* hs;
  float eps;
  int qmode;
  unsigned* slots;
};

// The norm workgroup's work over the n-value row in the slots, in three steps.
//  1. Gather: the workgroup's threads take the row's values in turn (value i to
//     thread i mod blockDim, coalesced), NT_BATCH a thread at a time: its slot,
//     r and w are all requested before the first is used, and the slots still
//     unwritten are requested again, together, until all are in (at most
//     PART_SPIN_LIMIT rounds a thread); each slot is cleared once read.  The sum
//     t = y + r goes to s and to vbuf, w to wbuf (both LDS).
//  2. k_rmsnorm_quant's sum of squares with its 1024 threads played by this
//     workgroup's nw waves, real wave w taking the norm's waves w, w + nw, ... in
//     turn: a norm thread's chunks are c = t, t + 1024, ...; its sum runs over
//     them in that order, then the butterfly inside its wave, then the sixteen
//     wave sums in ascending order.
//  3. The same waves norm and quantize their chunks from vbuf and wbuf.
// wbuf is used when both rows fit the LDS (w_lds); otherwise step 3 reads w
// from global memory.  The barriers wait for LDS only: no store of the tail
// waits to be acknowledged before the next step.
constexpr int NT_BATCH = 8;
__device__ __forceinline__ void norm_tail(const NormArgs& nm, int64_t n, float* vbuf, float* wbuf, bool w_lds,
                                          int tid, int nt, int wave, int nw, int lane) {
  constexpr int NW = 16;
  __shared__ double red[NW];
  int spins = 0;
  for (int64_t i0 = tid; i0 < n; i0 += (int64_t)nt * NT_BATCH) {
    unsigned u[NT_BATCH];
    float rv[NT_BATCH], wv[NT_BATCH];
#pragma unroll
    for (int b = 0; b < NT_BATCH; ++b) {
      const int64_t i = i0 + (int64_t)b * nt;
      const bool on = i < n;
      u[b] = on ? __hip_atomic_load(nm.slots + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1u;
      rv[b] = on && nm.r ? nm.r[i] : 0.0f;
      wv[b] = on && w_lds ? nm.w[i] : 0.0f;
    }
    for (;;) {
      bool waiting = false;
#pragma unroll
      for (int b = 0; b < NT_BATCH; ++b) waiting |= u[b] == 0;
      if (!waiting || spins >= PART_SPIN_LIMIT) break;
      ++spins;
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int b = 0; b < NT_BATCH; ++b)
        if (u[b] == 0) u[b] = __hip_atomic_load(nm.slots + i0 + (int64_t)b * nt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int b = 0; b < NT_BATCH; ++b) {
      const int64_t i = i0 + (int64_t)b * nt;
      if (i >= n) break;
      __hip_atomic_store(nm.slots + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      float t = __uint_as_float(u[b] ^ PART_MARK32);
      if (nm.r) t = __fadd_rn(t, rv[b]);
      if (nm.s) nm.s[i] = t;
      vbuf[i] = t;
      if (w_lds) wbuf[i] = wv[b];
    }
  }
  lds_barrier();
  const int64_t nc = n / 4;
  const int per = (int)((nc + NW * 64 - 1) / (NW * 64));
  for (int vw = wave; vw < NW; vw += nw) {
    double acc = 0.0;
    for (int j = 0; j < per; ++j) {
      const int64_t c = vw * 64 + lane + (int64_t)j * NW * 64;
      if (c < nc) acc += sq4(*(const float4*)(vbuf + 4 * c));  // past the row: +0 to a sum that is +0 or more
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (lane == 0) red[vw] = acc;
  }
  lds_barrier();
  double sum = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) sum += red[i];
  const double den = norm_den(sum, n, nm.eps);
  for (int vw = wave; vw < NW; vw += nw) {
    for (int j = 0; j < per; ++j) {
      const int64_t c = vw * 64 + lane + (int64_t)j * NW * 64;
      const bool on = c < nc;
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      if (on) {
        float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
        if (nm.w) g = *(const float4*)((w_lds ? wbuf : nm.w) + 4 * c);
        o = norm4(*(const float4*)(vbuf + 4 * c), den, nm.w != nullptr, g);
        if (nm.yn) *(float4*)(nm.yn + 4 * c) = o;
      }
      // every lane of the wave takes part in the block maximum; a block is wholly in or out
      if (nm.qmode != 0) {
        int h, l;
        const float sc = nm.qmode == 1 ? quant_lane4<1>(o, &h, &l) : quant_lane4<2>(o, &h, &l);
        if (on) {
          *(int*)(nm.hq + 4 * c) = h;
          if (nm.qmode == 2) *(int*)(nm.hl + 4 * c) = l;
          if ((c & 7) == 0) nm.hs[c / 8] = sc;
        }
      }
    }
  }
}

template <int MODE, int ROWS>
constexpr int ws_bytes_per_block() { return (MODE == 2 ? 2 : 1) * QK + 4 + 2 * ROWS; }

#ifdef QDG_PHASE_STAMPS
// Phase-stamp build only (never in the release library): each wave's lane 0
// records the 100 MHz constant clock at five points of its life -- 0 entry, 1
// all first loads issued, 2 staged bytes landed (after the barrier), 3 chunk
// terms done, 4 exit -- and, in word 5, the XCC and hardware id it ran on.  The
// stamps go to LDS (so they never wait on, or count in, the wave's outstanding
// global loads) and are written to stamp_buf[(workgroup * 16 + wave) * 8 + k] at
// exit.
__device__ unsigned long long* stamp_buf;
#define QDG_STAMP(w, k) \
  do {                                                                            \
    if ((threadIdx.x & 63) == 0) st_lds[w][k] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define QDG_STAMP(w, k) ((void)0)
#endif

template <int MODE, int R, int U, int NB, int STAGE, bool TL, bool NORM>
// eight waves a SIMD (64 VGPRs): two sixteen-wave workgroups a CU
__global__ __launch_bounds__(WS_NT) __attribute__((amdgpu_waves_per_eu(8))) void k_gemv_wsplit(
    const PartTable tab, const int8_t* __restrict__ xq, const int8_t* __restrict__ xl, const float* __restrict__ xs,
    int64_t K, int S, int m, int ceff, const NormArgs nm) {
  constexpr int ROWS = 4 * R;   // rows of the workgroup
  constexpr int LPR = 16;  // lanes a row (a lane pair a block, eight blocks a step)
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ float lpart[WS_NT / 64][4];

  // the wave index as a scalar: every per-chunk bound below is then wave-uniform
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if constexpr (NORM) {
    if (blockIdx.x == gridDim.x - 1) {  // the norm workgroup
      const int64_t n = tab.N[0];
      const bool w_lds = nm.w != nullptr && 8 * n <= WS_LDS_MAX;
      norm_tail(nm, n, (float*)lds, (float*)lds + n, w_lds, tid, (int)blockDim.x, wave, (int)(blockDim.x >> 6), lane);
      return;
    }
  }
#ifdef QDG_PHASE_STAMPS
  __shared__ unsigned long long st_lds[16][8];
  QDG_STAMP(wave, 0);
  if (lane == 0)  // XCC id (HW_REG_XCC_ID) and hardware id (HW_REG_HW_ID: CU, SE)
    st_lds[wave][5] = ((unsigned long long)__builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (15 << 11)) << 32) |
                      (unsigned)__builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11));
#endif
  // wave c of a row group takes the c-th non-empty chunk: chunks 0..m-1, then
  // chunk S-1 when it holds the K mod 512 tail; the empty chunks' partials are
  // +0 and adding +0 changes no partial sum (none is -0), so they are skipped
  const int rg = wave / ceff, c = wave % ceff;
  const int chunk = c < m ? c : S - 1;
  const int r = lane / LPR, li = lane % LPR, j = li >> 1, hf = li & 1;
  const int64_t nb = K / QK;
  int64_t o_wg;
  const int part = find_part(tab, (int)blockIdx.x, ROWS, o_wg);
  const int8_t* __restrict__ wq = tab.wq[part];
  const uint16_t* __restrict__ ws = tab.ws[part];
  float* __restrict__ y = tab.y[part];
  const int64_t N = tab.N[part];
  const int rr = rg * 4 + r;
  const int64_t o = o_wg + rr;
  const bool row_ok = o < N;
  const int64_t ro = row_ok ? o : N - 1;  // with tiled weights N is a multiple of 4: ro's tile is whole
  const int8_t* wrow = TL ? wq + (ro >> 2) * 4 * K + (ro & 3) * 256 + hf * 16 : wq + ro * K + hf * 16;
  int32_t g0, g1;
  split_range(K, S, chunk, g0, g1);
  const int nwb = g1 - g0;

  int8_t* lq = (int8_t*)lds;                                               // [nb][32]
  int8_t* ll = lq + nb * QK;                                               // [nb][32] (TwoPass)
  float* lsx = (float*)(lds + nb * QK * (MODE == 2 ? 2 : 1));              // [nb]
  uint16_t* lsg = (uint16_t*)(lsx + nb);                                   // [ROWS][nb]
  const uint16_t* my_sg = lsg + rr * nb;

  int4 w[NB][U];
  if constexpr (STAGE != WS_DMA) group_load<U, TL>(w[0], wrow, g0, g1, 0, j);  // ahead of the register copies
  if constexpr (STAGE == WS_DMA) {
    // The staged bytes are requested first and the wave's first NB step groups of
    // weights after them.  Loads complete in issue order, so the wait below for
    // all but the last NB*U loads covers exactly the staging, and the barrier
    // (wait_barrier: no workgroup fence, which would wait for every load) lets
    // the weights stay in flight.  Requesting the weights first made every wave
    // wait for them at the barrier: 0.2 us (5120x25600) and 0.3 us (5120x8192) a
    // launch.
    // Whole 1 KiB pieces a wave instruction; the byte counts are multiples of 16
    // (K and nb are multiples of 256 and 8), so a lane's 16 bytes are all in range
    const int nwv = (int)(blockDim.x >> 6);
    const int64_t rows_ok = N - o_wg < ROWS ? N - o_wg : ROWS;  // rows past N stay unstaged; their results are dropped
    const int64_t nsx = nb * 4, nsg = rows_ok * nb * 2;
    const int8_t* sgsrc = (const int8_t*)(ws + o_wg * nb);      // the workgroup's rows are consecutive
    for (int64_t base = (int64_t)wave * 1024; base < K; base += (int64_t)nwv * 1024) {
      if (base + lane * 16 < K) {
        lds_dma16(xq + base + lane * 16, lq + base);
        if constexpr (MODE == 2) lds_dma16(xl + base + lane * 16, ll + base);
      }
    }
    for (int64_t base = (int64_t)wave * 1024; base < nsx; base += (int64_t)nwv * 1024)
      if (base + lane * 16 < nsx) lds_dma16((const int8_t*)xs + base + lane * 16, (int8_t*)lsx + base);
    for (int64_t base = (int64_t)wave * 1024; base < nsg; base += (int64_t)nwv * 1024)
      if (base + lane * 16 < nsg) lds_dma16(sgsrc + base + lane * 16, (int8_t*)lsg + base);
#pragma unroll
    for (int k = 0; k < NB; ++k) group_load<U, TL>(w[k], wrow, g0, g1, k, j);
    QDG_STAMP(wave, 1);
    // the wave's staged bytes have landed (the NB*U weight loads may not have)
    wait_barrier<NB * U>();
  } else if constexpr (STAGE == WS_LOCAL) {
    for (int i = lane; i < nwb * 2; i += 64) {
      const int64_t k = (int64_t)g0 * 2 + i;
      ((int4*)lq)[k] = ld16(xq + 16 * k);
      if constexpr (MODE == 2) ((int4*)ll)[k] = ld16(xl + 16 * k);
    }
    for (int i = lane; i < nwb; i += 64) lsx[g0 + i] = xs[g0 + i];
    // stage_scales writes columns [0, n) of dst: point dst at column g0 of the row group's rows
    stage_scales(lsg + rg * 4 * nb + g0, (int)nb, ws, nb, N, o_wg + rg * 4, 4, g0, nwb, lane, 64);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    const int nt = (int)blockDim.x;
    for (int64_t i = tid; i < nb * 2; i += nt) {
      ((int4*)lq)[i] = ld16(xq + 16 * i);
      if constexpr (MODE == 2) ((int4*)ll)[i] = ld16(xl + 16 * i);
    }
    for (int64_t i = tid; i < nb; i += nt) lsx[i] = xs[i];
    stage_scales(lsg, (int)nb, ws, nb, N, o_wg, ROWS, 0, (int)nb, tid, nt);
    __syncthreads();
  }
  if constexpr (STAGE != WS_DMA) {
#pragma unroll
    for (int k = 1; k < NB; ++k) group_load<U, TL>(w[k], wrow, g0, g1, k, j);
  }

  // the chunk's partial of the row, in lane 0 of the row
  QDG_STAMP(wave, 2);
  const float yv = chunk_dot4<MODE, U, NB, TL>(wrow, lq, ll, lsx, my_sg, g0, g1, j, hf, w);
  QDG_STAMP(wave, 3);
  if (li == 0) lpart[wave][r] = yv;
  __syncthreads();
  if (tid < ROWS && o_wg + tid < N) {
    // row tid of the workgroup: row group tid/4, row tid%4; its partials are the
    // row group's waves in ascending chunk order
    const int g = tid >> 2, q = tid & 3;
    float a = 0.0f;
    for (int cc = 0; cc < ceff; ++cc) a = __fadd_rn(a, lpart[g * ceff + cc][q]);
    if (!NORM || y) y[o_wg + tid] = a;
    if constexpr (NORM) publish_partial(nm.slots + o_wg + tid, a);
  }
  QDG_STAMP(wave, 4);
#ifdef QDG_PHASE_STAMPS
  if (lane < 6 && stamp_buf) stamp_buf[((int64_t)blockIdx.x * 16 + wave) * 8 + lane] = st_lds[wave][lane];
#endif
}

// The chunk waves of one row group: the non-empty chunks of the S-chunk rule.
void ws_chunks(int64_t K, int S, int& m, int& ceff) {
  const int64_t nq = K / 512, per = (nq + S - 1) / S;
  m = per > 0 ? (int)((nq + per - 1) / per) : 0;  // chunks with superblocks (head)
  if (m > S) m = S;
  const bool tail = (K % 512) != 0;
  ceff = m;
  if (m < S && (tail || m == 0)) ceff = m + 1;      // chunk S-1: the tail (or all of K when nq = 0)
  if (m == S) ceff = S;
}

template <int MODE, int R>
size_t ws_lds_bytes(int64_t K) { return (size_t)(K / QK) * ws_bytes_per_block<MODE, 4 * R>(); }

template <int MODE, int R, int STAGE, bool TL, bool NORM>
hipError_t launch_ws(const PartTable& tab, int64_t K, const int8_t* xq, const int8_t* xl, const float* xs, int S,
                     const NormArgs& nm, hipStream_t st) {
  int m, ceff;
  ws_chunks(K, S, m, ceff);
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)&k_gemv_wsplit<MODE, R, WS_U, WS_NB, STAGE, TL, NORM>, hipFuncAttributeMaxDynamicSharedMemorySize,
      WS_LDS_MAX);
  if (attr != hipSuccess) return attr;
  // NORM: one more workgroup, the norm's
  const dim3 grid((unsigned)tab.tile_end[tab.n - 1] + (NORM ? 1 : 0)), block((unsigned)(64 * R * ceff));
  size_t lds = ws_lds_bytes<MODE, R>(K);
  if (NORM) {  // the norm's row, and its weights where both fit
    const size_t row = (size_t)tab.N[0] * 4, both = 2 * row;
    const size_t need = nm.w != nullptr && both <= (size_t)WS_LDS_MAX ? both : row;
    if (lds < need) lds = need;
  }
  return launch((k_gemv_wsplit<MODE, R, WS_U, WS_NB, STAGE, TL, NORM>), grid, block, lds, st, tab, xq, xl, xs, K, S,
                m, ceff, nm);
}

// The staging: per-wave copies when a row group is the whole workgroup (each
// wave's chunk is its own); otherwise LDS DMA when every staged array starts
// 16-byte aligned and K is a multiple of 256 (whole 16-byte pieces of every
// array), else the workgroup copy.  Measured on 5120x25600 / 5120x8192:
//   - three row groups (S = 5): the DMA staging is 4-10% faster than the copy;
//   - one row group (S = 16): per-wave copies beat the DMA on the 25600-value
//     rows by 2-8% and lose on the 8192-value rows by 4-8%;
//   - with the copy, per-wave staging was 4% faster with one row group and 1-6%
//     slower with two or four.
// QDG_TUNE_WS_LOCAL = 1 forces the per-wave copies, 0 the workgroup-wide
// staging; QDG_TUNE_WS_DMA = 0 turns the DMA off.
int ws_stage(int R, const PartTable& tab, int64_t K, int mode, const int8_t* xq, const int8_t* xl, const float* xs) {
  bool dma = K % 256 == 0 && ((uintptr_t)xq & 15) == 0 && ((uintptr_t)xs & 15) == 0 &&
             (mode == 1 || ((uintptr_t)xl & 15) == 0);
  for (int p = 0; p < tab.n; ++p) dma = dma && ((uintptr_t)tab.ws[p] & 15) == 0;
  if (tune(QDG_TUNE_WS_DMA) == 0) dma = false;
  const int loc = tune(QDG_TUNE_WS_LOCAL);
  if (loc >= 0 ? loc == 1 : R == 1) return WS_LOCAL;
  return dma ? WS_DMA : WS_BARRIER;
}

// Row groups a workgroup: three where they fit in 16 waves, else as many as fit.
// Measured on the 5120-row projections over R = 1..4 and S = 2, 4, 5, 8: three
// groups (427 workgroups, one round at two workgroups a CU) is the fastest or
// within 1% of it in every case, and four is 7-20% slower than three.
// QDG_TUNE_WS_ROWS (1..4) overrides.
int ws_groups(int ceff) {
  int R = 3 * ceff <= 16 ? 3 : 16 / ceff;
  if (tune(QDG_TUNE_WS_ROWS) > 0) R = tune(QDG_TUNE_WS_ROWS);
  if (R > 4) R = 4;
  if (R < 1) R = 1;
  while (R > 1 && R * ceff > 16) --R;
  return R;
}

template <int MODE, int R, bool TL, bool NORM>
hipError_t launch_ws_staged(const PartTable& tab, int64_t K, const int8_t* xq, const int8_t* xl, const float* xs,
                            int S, const NormArgs& nm, hipStream_t st) {
  switch (ws_stage(R, tab, K, MODE, xq, xl, xs)) {
    case WS_DMA: return launch_ws<MODE, R, WS_DMA, TL, NORM>(tab, K, xq, xl, xs, S, nm, st);
    case WS_LOCAL: return launch_ws<MODE, R, WS_LOCAL, TL, NORM>(tab, K, xq, xl, xs, S, nm, st);
    default: return launch_ws<MODE, R, WS_BARRIER, TL, NORM>(tab, K, xq, xl, xs, S, nm, st);
  }
}

template <int MODE, bool TL, bool NORM = false>
hipError_t launch_ws_mode(const PartTable& tab, int64_t K, const int8_t* xq, const int8_t* xl, const float* xs, int S,
                          int R, hipStream_t st, const NormArgs& nm = NormArgs{}) {
  switch (R) {
    case 1: return launch_ws_staged<MODE, 1, TL, NORM>(tab, K, xq, xl, xs, S, nm, st);
    case 2: return launch_ws_staged<MODE, 2, TL, NORM>(tab, K, xq, xl, xs, S, nm, st);
    case 3: return launch_ws_staged<MODE, 3, TL, NORM>(tab, K, xq, xl, xs, S, nm, st);
    default: return launch_ws_staged<MODE, 4, TL, NORM>(tab, K, xq, xl, xs, S, nm, st);
  }
}

// Row tiles: thread i moves the i-th 16 bytes of the tiled array, byte
// ((t*(K/256) + s)*4 + r)*256 + c <- row 4t + r, column 256s + c (c a multiple
// of 16).  Both sides are read and written in 256-byte runs.
__global__ __launch_bounds__(256) void k_tile_rows(const int8_t* __restrict__ wq, int64_t K, int64_t n16,
                                                   int8_t* __restrict__ wt) {
  const int64_t steps = K >> 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = (i & 15) << 4, q = i >> 4;
    const int64_t r = q & 3, q2 = q >> 2;
    const int64_t sidx = q2 % steps, t = q2 / steps;
    *(v4i*)(wt + (i << 4)) = *(const v4i*)(wq + (4 * t + r) * K + (sidx << 8) + c);
  }
}

}  // namespace

// Whether the in-workgroup split serves (mode, K, splits) for one activation row:
// the non-empty chunks fit in 16 waves and the staged row in the LDS budget.
bool wsplit_fits(int mode, int64_t K, int splits) {
  if (splits < 2 || splits > 16) return false;
  int m, ceff;
  ws_chunks(K, splits, m, ceff);
  if (ceff < 2) return false;
  const int R = ws_groups(ceff);
  const int64_t bpb = (mode == 2 ? 2 : 1) * QK + 4 + 2 * 4 * R;
  return (K / QK) * bpb <= WS_LDS_MAX;
}

void wsplit_shape(int64_t K, int splits, int& rows, int& waves) {
  int m, ceff;
  ws_chunks(K, splits, m, ceff);
  const int R = ws_groups(ceff);
  rows = 4 * R;
  waves = R * ceff;
}

hipError_t launch_gemv_wsplit_parts(int mode, int nparts, const int8_t* const* wq, const uint16_t* const* ws,
                                    const int64_t* N, float* const* y, int64_t K, const int8_t* xq,
                                    const int8_t* xl, const float* xs, int splits, hipStream_t st, bool tiled) {
  int m, ceff;
  ws_chunks(K, splits, m, ceff);
  const int R = ws_groups(ceff);
  PartTable tab;
  if (!make_parts(tab, nparts, wq, ws, y, N, 4 * R)) return hipErrorInvalidValue;
  if (tiled) {
    if (mode == 1) return launch_ws_mode<1, true>(tab, K, xq, xl, xs, splits, R, st);
    return launch_ws_mode<2, true>(tab, K, xq, xl, xs, splits, R, st);
  }
  if (mode == 1) return launch_ws_mode<1, false>(tab, K, xq, xl, xs, splits, R, st);
  return launch_ws_mode<2, false>(tab, K, xq, xl, xs, splits, R, st);
}

hipError_t launch_gemv_wsplit(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K,
                              const int8_t* xq, const int8_t* xl, const float* xs, int splits, float* y,
                              hipStream_t st, bool tiled) {
  return launch_gemv_wsplit_parts(mode, 1, &wq, &ws, &N, &y, K, xq, xl, xs, splits, st, tiled);
}

size_t gemv_norm_workspace_bytes(int64_t N) { return (size_t)((N * 4 + 255) / 256) * 256; }
int64_t gemv_norm_max_n() { return WS_LDS_MAX / 4; }

hipError_t launch_gemv_wsplit_norm(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K,
                                   const int8_t* xq, const int8_t* xl, const float* xs, int splits, float* y,
                                   const float* r, float* s, const float* w, float eps, int qmode, float* yn,
                                   int8_t* hq, int8_t* hl, float* hs, void* workspace, hipStream_t st) {
  int m, ceff;
  ws_chunks(K, splits, m, ceff);
  const int R = ws_groups(ceff);
  PartTable tab;
  if (!make_parts(tab, 1, &wq, &ws, &y, &N, 4 * R)) return hipErrorInvalidValue;
  NormArgs nm;
  nm.r = r;
  nm.s = s;
  nm.w = w;
  nm.yn = yn;
  nm.hq = hq;
  nm.hl = hl;
  nm.hs = hs;
  nm.eps = eps;
  nm.qmode = qmode;
  nm.slots = (unsigned*)workspace;
  if (mode == 1) return launch_ws_mode<1, false, true>(tab, K, xq, xl, xs, splits, R, st, nm);
  return launch_ws_mode<2, false, true>(tab, K, xq, xl, xs, splits, R, st, nm);
}

#ifdef QDG_PHASE_STAMPS
// Phase-stamp build only: points the in-workgroup split kernel's stamps at buf
// (device, 8 words a wave of 16 a workgroup; NULL stops stamping).
extern "C" int qdg_debug_phase_stamps(void* buf) {
  unsigned long long* p = (unsigned long long*)buf;
  return hipMemcpyToSymbol(HIP_SYMBOL(stamp_buf), &p, sizeof(p)) == hipSuccess ? 0 : -6;
}
#endif

hipError_t launch_tile_rows(const int8_t* wq, int64_t N, int64_t K, int8_t* wt, hipStream_t st) {
  const int64_t n16 = N * K / 16;
  const int64_t blocks = (n16 + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
  return launch(k_tile_rows, dim3(grid), dim3(256), 0, st, wq, K, n16, wt);
}

}  // namespace qdg
