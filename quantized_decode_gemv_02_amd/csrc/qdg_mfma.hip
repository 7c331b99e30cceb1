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
//  * A workgroup of 8 waves owns 32 weight rows (two tiles of 16) and walks its
//    chunk of K in steps of 8 blocks (256 bytes a row).  Wave v = 4*tau + r works
//    on tile tau and owns partial r: blocks r and r + 4 of every step (steps start
//    at multiples of 8 blocks from the chunk start, itself a multiple of 16, so
//    block k of a step is partial k mod 4).  Each of its chains runs in one lane,
//    in ascending block order, and the four partials meet once, at the end, in
//    the fixed order (P0 + P2) + (P1 + P3).
//  * Loads: wave v reads rows 4*v .. 4*v + 3 of the step, 256 contiguous bytes a
//    row (lane (r = l/16, c = l%16) takes 16 bytes at 16*c of row 4*v + r): whole
//    128-byte lines, the layout that streams HBM best.  The words go to a shared
//    LDS tile of 32 rows x 256 bytes, where the MFMA reads them transposed (lane
//    col = l%16 is a weight row, l/16 picks 8 of the block's 32 bytes).  The
//    16-byte chunks of row r sit at chunk index c ^ (r mod 16), so the writes
//    and the reads spread over all banks.
//  * The A operand is activation row t = col, the same 8 bytes of the block; the
//    MFMA result gives lane (col, grp = l/16) the dots of t = 4*grp + i (i < 4)
//    with weight row col of its tile.
//  * Shared step data -- the 32 rows' weight words, the 16 activation rows' words,
//    their scales and the 32 rows' weight scales -- lives in LDS in two slots:
//    step s's data is loaded into registers ahead of step s (weights P - 1 steps
//    ahead in a ring, the rest 2 steps ahead), written to slot s mod 2 at the
//    start of step s, and one workgroup barrier a step makes it visible.
//  * The loop is a uniform software pipeline: every step issues the same loads,
//    all unconditional (addresses past the chunk are clamped to its last block,
//    whose extra data is never summed), and the loop starts at the virtual step
//    -P, so the compiler's wait counts keep the look-ahead in flight.
//  * Weight rows past N read row N-1 and store nothing; activation rows t >= B
//    read row B-1 and store nothing (an MFMA row never mixes into another).

#include "qdg_device.h"

namespace qdg {
namespace {

constexpr int WAVES = 8;                  // 2 row tiles x 4 partials
constexpr int WG = 64 * WAVES;
constexpr int ROWS = 32;                  // weight rows a workgroup
constexpr int STEP = 8;                   // blocks per step: 256 bytes of a weight row
constexpr int WTILE = ROWS * STEP * QK;   // one slot of the shared weight tile
constexpr int APITCH = STEP * QK + 16;    // bytes per staged activation row (padded: rows on distinct banks)

// One LDS slot of staged step data besides the weights: activation words (both
// under TwoPass), activation scales [16][8], weight scales [32][8].
template <int MODE>
struct Slot {
  static constexpr int A = 0;
  static constexpr int L = A + 16 * APITCH;
  static constexpr int SX = L + (MODE == 2 ? 16 * APITCH : 0);
  static constexpr int SG = SX + 16 * STEP * 4;
  static constexpr int BYTES = SG + ROWS * STEP * 2;
};
template <int MODE>
constexpr int lds_bytes() { return 2 * WTILE + 2 * Slot<MODE>::BYTES; }
static_assert(2 * WTILE >= WAVES * 64 * 4 * 4, "the final reduction reuses the weight tile");

// One 32-value block's 16x16 dots: A and B hold 8 bytes a lane, k-group l/16.
__device__ __forceinline__ v4i mfma16x16x32(long a, long b) {
  const v4i z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, z, 0, 0, 0);
}

// Byte offset of 16-byte chunk c of row r in a weight tile slot.
__device__ __forceinline__ int tile_off(int r, int c) { return r * (STEP * QK) + (((c ^ r) & 15) << 4); }

// The shared data of one step besides the weights, in registers between its
// loads and its LDS store.  Thread tid (of 512) moves: activation word c = tid%16
// of row t = (tid%256)/16 -- high words for tid < 256, low words (TwoPass) for the
// rest; activation scale k = tid%8 of row (tid%128)/8; weight scales of row
// tid%32 -- all 8 in one 16-byte word when WIDE, else scale (tid%256)/32 of it.
// Threads whose share repeats another's load it too and store nothing, so every
// thread issues the same loads.
template <int MODE, bool WIDE>
struct StepStage {
  v4i h;
  float sx;
  v4i sw;            // WIDE
  unsigned short sh;  // not WIDE

  __device__ __forceinline__ void load(const int8_t* __restrict__ xq, const int8_t* __restrict__ xl,
                                       const float* __restrict__ xs, const uint16_t* __restrict__ ws,
                                       int64_t N, int64_t K, int B, int64_t o_wg, int blk0, int g1) {
    const int tid = threadIdx.x;
    const int64_t nb = K / QK;
    const int t = min((tid & 255) >> 4, B - 1), c = tid & 15;
    const int ba = min(blk0 + (c >> 1), g1 - 1);  // block of activation word c
    const int8_t* src = (MODE == 2 && tid >= 256) ? xl : xq;
    h = *(const v4i*)(src + (int64_t)t * K + (int64_t)ba * QK + 16 * (c & 1));
    const int ts = min((tid & 127) >> 3, B - 1), ks = tid & 7;
    sx = xs[(int64_t)ts * nb + min(blk0 + ks, g1 - 1)];
    int64_t o = o_wg + (tid & 31);
    if (o >= N) o = N - 1;
    if constexpr (WIDE) {
      // steps are whole when WIDE (K/32 and chunk ends are multiples of 8); the
      // clamp only keeps the look-ahead past the chunk in bounds
      sw = *(const v4i*)(ws + o * nb + min(blk0, g1 - STEP));
    } else {
      sh = ws[o * nb + min(blk0 + ((tid & 255) >> 5), g1 - 1)];
    }
  }

  __device__ __forceinline__ void store(unsigned char* slot) const {
    const int tid = threadIdx.x;
    const int t = (tid & 255) >> 4, c = tid & 15;
    if (tid < 256) *(v4i*)(slot + Slot<MODE>::A + t * APITCH + 16 * c) = h;
    if (MODE == 2 && tid >= 256) *(v4i*)(slot + Slot<MODE>::L + t * APITCH + 16 * c) = h;
    if (tid < 128) ((float*)(slot + Slot<MODE>::SX))[tid] = sx;  // [t][k] = tid
    uint16_t* sg = (uint16_t*)(slot + Slot<MODE>::SG);             // [row][8]
    if constexpr (WIDE) {
      if (tid < 32) *(v4i*)(sg + tid * STEP) = sw;
    } else {
      if (tid < 256) sg[(tid & 31) * STEP + (tid >> 5)] = sh;
    }
  }
};

template <int MODE, int P, bool WIDE>
__global__ __launch_bounds__(WG) void k_gemv_mfma(const int8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
                                                 const int8_t* __restrict__ xq, const int8_t* __restrict__ xl,
                                                 const float* __restrict__ xs, int64_t N, int64_t K, int B, int S,
                                                 float* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tau = wave >> 2, res = wave & 3;  // row tile, owned partial
  unsigned char* wtile = lds;                 // [2 slots][32 rows][256 bytes]
  unsigned char* slots = lds + 2 * WTILE;     // [2 slots] of Slot<MODE>
  const int col = lane & 15, grp = lane >> 4;
  const int s_idx = blockIdx.y;
  int32_t g0, g1;
  split_range(K, S, s_idx, g0, g1);
  const int nsteps = (g1 - g0 + STEP - 1) / STEP;

  const int64_t o_wg = (int64_t)blockIdx.x * ROWS;
  // load side: lane (r = grp, c = col) reads row 4*wave + r, 16-byte chunk c of
  // the step (half (c & 1) of block c >> 1)
  const int lrow = 4 * wave + grp;
  int64_t lo = o_wg + lrow;
  if (lo >= N) lo = N - 1;
  const int8_t* wrow = wq + lo * K + 16 * (col & 1);
  const int cblk = col >> 1;
  const int w_st = tile_off(lrow, col);  // where this lane's word goes in a tile slot
  // read side: rows 16*tau + col of the tile, blocks res and res + 4
  int w_rd[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) w_rd[h] = tile_off(16 * tau + col, 2 * (res + 4 * h) + (grp >> 1)) + 8 * (grp & 1);
  const int a_off = Slot<MODE>::A + col * APITCH + 8 * grp;  // A operand: activation row t = col
  const int l_off = Slot<MODE>::L + col * APITCH + 8 * grp;
  const int sx_off = Slot<MODE>::SX + grp * 4 * STEP * 4;    // rows 4*grp .. 4*grp + 3
  const int sg_off = Slot<MODE>::SG + (16 * tau + col) * STEP * 2;

  float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // partial `res` of (t = 4*grp + i, o = o_wg + 16*tau + col)

  StepStage<MODE, WIDE> st[2];
  v4i wr[P];
  // The loop starts at the virtual step -P: steps below 0 only issue loads (of
  // step 0 where they would look before it), so every iteration -- the first
  // ones included -- issues the same loads in the same order.  The start value
  // passes through an empty asm statement so that the compiler cannot peel the
  // first iterations into a prologue with a different load order.
  int first = -P;
  asm volatile("" : "+s"(first));
  // an empty chunk (K < 512 with several chunks) loads nothing: its partials stay +0
  if (g1 <= g0) first = nsteps;
  for (int s0 = first; s0 < nsteps; s0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int s = s0 + u;
      // uniform over the workgroup; leaves both loops, so no path runs from a
      // partial group back to the loop head (the wait counts stay exact)
      if (s >= nsteps) goto done;
      unsigned char* slot = slots + (u & 1) * Slot<MODE>::BYTES;  // P is even: slot s mod 2
      unsigned char* tile = wtile + (u & 1) * WTILE;
      if (s >= 0) {  // step s's data: weights loaded during step s - P + 1, the rest during s - 2
        st[u & 1].store(slot);
        *(v4i*)(tile + w_st) = wr[u];
      }
      st[u & 1].load(xq, xl, xs, ws, N, K, B, o_wg, g0 + max(s + 2, 0) * STEP, g1);
      {
        const int blk = min(g0 + max(s + P - 1, 0) * STEP + cblk, g1 - 1);
        wr[(u + P - 1) % P] = __builtin_nontemporal_load((const v4i*)(wrow + (int64_t)blk * QK));
      }
      __syncthreads();
      if (s >= 0) {  // uniform; steps below 0 only load
        const int b = g0 + s * STEP;
        const v4i sg8 = *(const v4i*)(slot + sg_off);  // the row's 8 weight scales of the step
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = res + 4 * h;
          if (b + k >= g1) break;  // uniform over the wave
          const long wk = *(const long*)(tile + w_rd[h]);
          const v4i D = mfma16x16x32(*(const long*)(slot + a_off + k * QK), wk);
          v4i E = {0, 0, 0, 0};
          if constexpr (MODE == 2) E = mfma16x16x32(*(const long*)(slot + l_off + k * QK), wk);
          const unsigned sgw = (unsigned)sg8[k >> 1];
          const float sgm = half_bits_to_float((unsigned short)((k & 1) ? (sgw >> 16) : (sgw & 0xffffu)));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sig = *(const float*)(slot + sx_off + (i * STEP + k) * 4);
            float ta, tb;
            q8_term<MODE>(sgm, sig, D[i], E[i], ta, tb);
            p[i] = __fmaf_rn(ta, tb, p[i]);
          }
        }
      }
    }
  }
done:
  // the four partials of each output meet in a fixed order: (P0 + P2) + (P1 + P3)
  __syncthreads();  // every wave is done with the tile, which now holds the partials
  float* red = (float*)lds;  // [wave][i][lane]
#pragma unroll
  for (int i = 0; i < 4; ++i) red[(wave * 4 + i) * 64 + lane] = p[i];
  __syncthreads();
  if (res == 0) {
    const int64_t oo = o_wg + 16 * tau + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = grp * 4 + i;
      const float q0 = red[((4 * tau + 0) * 4 + i) * 64 + lane], q1 = red[((4 * tau + 1) * 4 + i) * 64 + lane];
      const float q2 = red[((4 * tau + 2) * 4 + i) * 64 + lane], q3 = red[((4 * tau + 3) * 4 + i) * 64 + lane];
      const float y = __fadd_rn(__fadd_rn(q0, q2), __fadd_rn(q1, q3));
      if (t < B && oo < N) out[((int64_t)s_idx * B + t) * N + oo] = y;
    }
  }
}

template <int MODE, int P, bool WIDE>
hipError_t launch_mg(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq, const int8_t* xl,
                     const float* xs, int64_t B, int splits, float* out, hipStream_t st) {
  const dim3 grid((unsigned)((N + ROWS - 1) / ROWS), (unsigned)splits), block(WG);
  return launch((k_gemv_mfma<MODE, P, WIDE>), grid, block, lds_bytes<MODE>(), st, wq, ws, xq, xl, xs, N, K,
                     (int)B, splits, out);
}

template <int MODE, int P>
hipError_t launch_mp(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq, const int8_t* xl,
                     const float* xs, int64_t B, int splits, float* out, hipStream_t st) {
  // 16-byte weight-scale words need ws 16-byte aligned and K/32 a multiple of 8
  if ((K / QK) % 8 == 0 && ((uintptr_t)ws & 15) == 0)
    return launch_mg<MODE, P, true>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
  return launch_mg<MODE, P, false>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
}

// ---------------------------------------------------------------------------
// The fast path for K a multiple of 256 and ws 16-byte aligned.  Same sums and
// operand layouts as k_gemv_mfma, but a workgroup of WV waves (4 or 8) owns
// 16*(WV/4)*TPW weight rows: wave v = 4*g + r works on tiles g, g + WV/4, ...
// (TPW of them, one A operand read serving all) for partial r.  Every byte of a
// step -- weights, activation words, scales -- moves from global memory straight
// into LDS (global_load_lds), into a ring of P slots, P - 1 steps ahead.  More
// rows a workgroup means fewer re-reads of the activations, which every
// workgroup needs in full.  No data passes through registers, so nothing the
// compiler schedules can make a wave wait on loads that are still ahead of it;
// instead every wave issues exactly DMA_LOADS loads a step and waits, before
// each step's barrier, until only the later steps' loads are outstanding
// (s_waitcnt vmcnt).  The barrier then makes the whole workgroup's copies of the
// step visible, and the slot it refills for step s + P - 1 was last read in step
// s - 1, which every wave has finished.
//
// The shared loads of a step besides the weights are a list of jobs -- the
// activation words (4 loads of 4 rows, and 4 more for the TwoPass low words),
// the activation scales (2 dword loads) and the weight scales (one 16-byte load
// per 64 rows) -- dealt round-robin to the waves; a wave with no job left that
// step issues a one-dword placeholder load, so every wave issues the same count.
//
// Slot layout: W [rows][256] and A (L) [16 rows][256] with the 16-byte chunk c
// of row r at chunk index c ^ (r mod 16) -- a wave's load writes 1 KiB in lane
// order, so lane (r4 = l/16, j = l%16) fetches global chunk j ^ row to land it
// in place; SX [16][8] activation scales; SG [rows][8] weight scales; JUNK for
// the placeholders.
template <int MODE, int WV, int TPW, int AT = 1>
struct DSlot {
  static constexpr int TG = WV / 4;  // tile groups
  static constexpr int DROWS = 16 * TG * TPW;
  static constexpr int W = 0;
  static constexpr int A = W + DROWS * 256;                 // AT activation tiles of 16 rows
  static constexpr int L = A + AT * 16 * 256;
  static constexpr int SX = L + (MODE == 2 ? AT * 16 * 256 : 0);
  static constexpr int SG = SX + AT * 16 * STEP * 4;
  static constexpr int NG = (DROWS * 16 + 1023) / 1024;  // weight-scale loads (1 KiB each)
  static constexpr int JUNK = SG + NG * 1024;
  static constexpr int BYTES = JUNK + 64 * 4;
  static constexpr int JOBS = AT * ((MODE == 2 ? 8 : 4) + 2) + NG;
  static constexpr int AUX = (JOBS + WV - 1) / WV;  // aux loads a wave a step
  static constexpr int WLOADS = DROWS / (4 * WV);   // weight loads a wave a step
  static constexpr int DMA_LOADS = WLOADS + AUX;
  static_assert(DROWS % (4 * WV) == 0, "whole weight loads per wave");
};
template <int MODE, int WV, int TPW, int P, int AT = 1>
constexpr int dma_lds_bytes() { return P * DSlot<MODE, WV, TPW, AT>::BYTES; }

typedef __attribute__((address_space(3))) void* lds_ptr;

// global_load_lds of 16 or 4 bytes a lane; AUX 2 sets the nontemporal hint
template <int BYTES_, int AUXF>
__device__ __forceinline__ void dma(const void* g, unsigned char* l) {
  static_assert((BYTES_ == 16 || BYTES_ == 4) && (AUXF == 0 || AUXF == 2), "supported forms");
  if constexpr (BYTES_ == 16 && AUXF == 2)
    __builtin_amdgcn_global_load_lds(g, (lds_ptr)l, 16, 0, 2);
  else if constexpr (BYTES_ == 16)
    __builtin_amdgcn_global_load_lds(g, (lds_ptr)l, 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds(g, (lds_ptr)l, 4, 0, 0);
}

// Waits until at most N of this wave's vector-memory loads are outstanding (and
// its LDS accesses are done), then meets the workgroup; the empty asm
// statements keep the compiler from moving LDS accesses across.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);  // vmcnt(N) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// AT activation tiles of 16 rows (B up to 16*AT): every weight step is
// multiplied against all of them, so the weights are read once for the batch.
template <int MODE, int WV, int TPW, int P, int AT = 1>
__global__ __launch_bounds__(64 * WV) void k_gemv_mfma_dma(const int8_t* __restrict__ wq,
                                                          const uint16_t* __restrict__ ws,
                                                          const int8_t* __restrict__ xq,
                                                          const int8_t* __restrict__ xl,
                                                          const float* __restrict__ xs, int64_t N, int64_t K, int B,
                                                          int S, float* __restrict__ out) {
  using SL = DSlot<MODE, WV, TPW, AT>;
  constexpr int DROWS = SL::DROWS, TG = SL::TG;
  static_assert(P * SL::BYTES >= WV * TPW * AT * 4 * 64 * 4, "the final reduction reuses the slots");
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tg = wave >> 2, res = wave & 3;  // tile group (tiles tg, tg + TG, ...), owned partial
  const int col = lane & 15, grp = lane >> 4;
  const int s_idx = blockIdx.y;
  int32_t g0, g1;
  split_range(K, S, s_idx, g0, g1);
  const int nsteps = (g1 - g0) / STEP;  // whole steps: K/32 and chunk ends are multiples of 8 here
  const int64_t nb = K / QK;
  const int64_t o_wg = (int64_t)blockIdx.x * DROWS;

  // ---- load side (per lane, fixed over the steps)
  const int r4 = lane >> 4, j = lane & 15;
  const int8_t* wsrc[SL::WLOADS];  // load m of this wave: rows 4*(WV*m + wave) + r4
  int wcb[SL::WLOADS];
#pragma unroll
  for (int m = 0; m < SL::WLOADS; ++m) {
    const int row = 4 * (WV * m + wave) + r4;
    const int c = (j ^ row) & 15;  // fetched so that it lands at chunk j
    int64_t o = o_wg + row;
    if (o >= N) o = N - 1;
    wsrc[m] = wq + o * K + 16 * (c & 1);
    wcb[m] = c >> 1;
  }

  // one aux job (uniform over the wave): 4*AT high-word loads (tile at = job/4,
  // rows 4*(job%4)..), 4*AT low-word loads (TwoPass), then 2 activation-scale
  // loads a tile, then NG weight-scale loads
  constexpr int NW_JOBS = AT * (MODE == 2 ? 8 : 4);
  auto issue_job = [&](int job, int blk0, unsigned char* slot) {
    if (job < NW_JOBS) {
      const bool low = MODE == 2 && job >= 4 * AT;
      const int jj = low ? job - 4 * AT : job;
      const int at = jj >> 2, q = jj & 3;
      const int arow = 4 * q + r4;  // row within the tile
      const int ac = (j ^ arow) & 15;
      const int8_t* src = low ? xl : xq;
      const int blk = min(blk0 + (ac >> 1), g1 - 1);
      dma<16, 0>(src + (int64_t)min(16 * at + arow, B - 1) * K + (int64_t)blk * QK + 16 * (ac & 1),
                 slot + (low ? SL::L : SL::A) + at * 4096 + q * 1024);
    } else if (job < NW_JOBS + 2 * AT) {
      const int sq = job - NW_JOBS;
      const int at = sq >> 1, sh = sq & 1;
      const int sidx = 64 * sh + lane;  // [t][k] = sidx within the tile
      dma<4, 0>(xs + (int64_t)min(16 * at + (sidx >> 3), B - 1) * nb + min(blk0 + (sidx & 7), g1 - 1),
                slot + SL::SX + at * 512 + sh * 256);
    } else if (job < SL::JOBS) {
      const int gq = job - NW_JOBS - 2 * AT;
      int64_t o = o_wg + ((64 * gq + lane) % DROWS);
      if (o >= N) o = N - 1;
      // steps are whole when this path runs; the clamp keeps the look-ahead in bounds
      dma<16, 0>(ws + o * nb + min(blk0, g1 - STEP), slot + SL::SG + gq * 1024);
    } else {
      dma<4, 0>(xs, slot + SL::JUNK);
    }
  };
  auto issue = [&](int s) {  // every load of step s, into slot s mod P
    unsigned char* slot = lds + (s % P) * SL::BYTES;
    const int blk0 = g0 + min(s, nsteps - 1) * STEP;  // steps past the chunk repeat its last one
#pragma unroll
    for (int m = 0; m < SL::WLOADS; ++m)  // nontemporal: the weights are streamed once
      dma<16, 2>(wsrc[m] + (int64_t)(blk0 + wcb[m]) * QK, slot + SL::W + (WV * m + wave) * 1024);
#pragma unroll
    for (int a = 0; a < SL::AUX; ++a) issue_job(wave + WV * a, blk0, slot);
  };

  // ---- read side
  int w_rd[TPW][2], a_rd[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = 2 * (res + 4 * h) + (grp >> 1);
    a_rd[h] = SL::A + col * 256 + (((c ^ col) & 15) << 4) + 8 * (grp & 1);
#pragma unroll
    for (int m = 0; m < TPW; ++m)
      w_rd[m][h] = SL::W + (16 * (tg + TG * m) + col) * 256 + (((c ^ col) & 15) << 4) + 8 * (grp & 1);
  }
  const int sx_rd = SL::SX + grp * 4 * STEP * 4;  // rows 4*grp .. 4*grp + 3
  int sg_rd[TPW];
#pragma unroll
  for (int m = 0; m < TPW; ++m) sg_rd[m] = SL::SG + (16 * (tg + TG * m) + col) * 16;

  // partial `res` of (t = 16*at + 4*grp + i, o = o_wg + 16*(tg + TG*m) + col)
  float p[TPW][AT][4];
#pragma unroll
  for (int m = 0; m < TPW; ++m)
#pragma unroll
    for (int at = 0; at < AT; ++at)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[m][at][i] = 0.0f;
  // an empty chunk (K < 512 with several chunks) loads nothing: its partials stay +0
  if (nsteps > 0) {
#pragma unroll
    for (int q = 0; q < P - 1; ++q) issue(q);
  }
  for (int s = 0; s < nsteps; ++s) {
    wait_and_barrier<(P - 2) * SL::DMA_LOADS>();  // step s is in LDS, slot (s-1) mod P is free
    issue(s + P - 1);
    const unsigned char* slot = lds + (s % P) * SL::BYTES;
    // One activation tile: all operands first, then the products.  Several tiles
    // (prefill): one tile at a time, so its operands and products are dead before
    // the next tile's; each partial still takes one step per h, in order.
    // Measured: the first is 3% faster at B = 16 (TwoPass), the second 5% faster
    // at B = 64 (Int8Act), with 121 VGPRs instead of 171 (TwoPass, four tiles).
    if constexpr (AT == 1) {
  #pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = res + 4 * h;
        long ak[AT], lk[AT];
        float sig[AT][4];
  #pragma unroll
        for (int at = 0; at < AT; ++at) {
          ak[at] = *(const long*)(slot + a_rd[h] + at * 4096);
          lk[at] = 0;
          if constexpr (MODE == 2) lk[at] = *(const long*)(slot + a_rd[h] + at * 4096 + (SL::L - SL::A));
  #pragma unroll
          for (int i = 0; i < 4; ++i) sig[at][i] = *(const float*)(slot + sx_rd + at * 512 + (i * STEP + k) * 4);
        }
  #pragma unroll
        for (int m = 0; m < TPW; ++m) {
          const long wk = *(const long*)(slot + w_rd[m][h]);
          const float sgm = half_bits_to_float(*(const unsigned short*)(slot + sg_rd[m] + 2 * k));
  #pragma unroll
          for (int at = 0; at < AT; ++at) {
            const v4i D = mfma16x16x32(ak[at], wk);
            v4i E = {0, 0, 0, 0};
            if constexpr (MODE == 2) E = mfma16x16x32(lk[at], wk);
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              float ta, tb;
              q8_term<MODE>(sgm, sig[at][i], D[i], E[i], ta, tb);
              p[m][at][i] = __fmaf_rn(ta, tb, p[m][at][i]);
            }
          }
        }
      }
    } else {
  #pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = res + 4 * h;
        long wk[TPW];
        float sgm[TPW];
  #pragma unroll
        for (int m = 0; m < TPW; ++m) {
          wk[m] = *(const long*)(slot + w_rd[m][h]);
          sgm[m] = half_bits_to_float(*(const unsigned short*)(slot + sg_rd[m] + 2 * k));
        }
  #pragma unroll
        for (int at = 0; at < AT; ++at) {
          const long ak = *(const long*)(slot + a_rd[h] + at * 4096);
          long lk = 0;
          if constexpr (MODE == 2) lk = *(const long*)(slot + a_rd[h] + at * 4096 + (SL::L - SL::A));
          float sig[4];
  #pragma unroll
          for (int i = 0; i < 4; ++i) sig[i] = *(const float*)(slot + sx_rd + at * 512 + (i * STEP + k) * 4);
  #pragma unroll
          for (int m = 0; m < TPW; ++m) {
            const v4i D = mfma16x16x32(ak, wk[m]);
            v4i E = {0, 0, 0, 0};
            if constexpr (MODE == 2) E = mfma16x16x32(lk, wk[m]);
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              float ta, tb;
              q8_term<MODE>(sgm[m], sig[i], D[i], E[i], ta, tb);
              p[m][at][i] = __fmaf_rn(ta, tb, p[m][at][i]);
            }
          }
        }
      }
    }
  }
  // the four partials of each output meet in a fixed order: (P0 + P2) + (P1 + P3)
  wait_and_barrier<0>();  // every load has landed and every wave is done with the slots
  float* red = (float*)lds;  // [wave][m][at][i][lane]
#pragma unroll
  for (int m = 0; m < TPW; ++m)
#pragma unroll
    for (int at = 0; at < AT; ++at)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(((wave * TPW + m) * AT + at) * 4 + i) * 64 + lane] = p[m][at][i];
  wait_and_barrier<0>();
  if (res == 0) {
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int64_t oo = o_wg + 16 * (tg + TG * m) + col;
#pragma unroll
      for (int at = 0; at < AT; ++at) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * at + grp * 4 + i;
          float q[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) q[r] = red[((((4 * tg + r) * TPW + m) * AT + at) * 4 + i) * 64 + lane];
          const float y = __fadd_rn(__fadd_rn(q[0], q[2]), __fadd_rn(q[1], q[3]));
          if (t < B && oo < N) out[((int64_t)s_idx * B + t) * N + oo] = y;
        }
      }
    }
  }
}

template <int MODE, int WV, int TPW, int P, int AT = 1>
hipError_t launch_dma(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq,
                      const int8_t* xl, const float* xs, int64_t B, int splits, float* out, hipStream_t st) {
  constexpr int rows = DSlot<MODE, WV, TPW, AT>::DROWS;
  const dim3 grid((unsigned)((N + rows - 1) / rows), (unsigned)splits), block(64 * WV);
  constexpr int lds = dma_lds_bytes<MODE, WV, TPW, P, AT>();
  static_assert(lds <= 160 * 1024, "LDS of one workgroup");
  // above 64 KiB of LDS the kernel's dynamic-LDS limit is raised (once)
  static const hipError_t attr = hipFuncSetAttribute((const void*)&k_gemv_mfma_dma<MODE, WV, TPW, P, AT>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  return launch((k_gemv_mfma_dma<MODE, WV, TPW, P, AT>), grid, block, lds, st, wq, ws, xq, xl, xs, N, K,
                     (int)B, splits, out);
}

// ---------------------------------------------------------------------------
// The batched fast path for up to 16 activation rows: one wave a workgroup, with
// a ring of its own in LDS, so no wave ever waits for another.  Wave = TPW row
// tiles of 16 weight rows over the whole chunk; every step of 8 blocks moves the
// tiles' weights (4 rows x 256 bytes a DMA instruction, whole lines), the 16
// activation rows' words of the step (both words under TwoPass), their scales
// and the tiles' weight scales from global memory straight into the wave's slot
// (global_load_lds), P - 1 steps ahead.  The wave waits only for its own loads
// (s_waitcnt vmcnt: loads complete in issue order) -- no barrier -- and takes
// all 8 blocks of the step itself: block k's v_mfma_i32_16x16x32_i8 gives the
// dots of activation rows 4*grp + i against weight row col of a tile, and each
// output's step goes into partial k mod 4 in the lane that holds the output, so
// the four partial chains of an output (blocks r, r + 4, ... in ascending
// order) and their (P0 + P2) + (P1 + P3) stay in one lane: the batch-1 sums,
// bit for bit.  (The workgroup-shared ring above waits at a barrier every step,
// so a workgroup keeps one step in flight; a copy of it with the barrier taken
// out streamed the same loads a third faster.)
//
// Slot: W [16*TPW rows][256] and A (L) [16 rows][256] with 16-byte chunk c of
// row r at c ^ (r mod 16) -- lane (r4 = l/16, j = l%16) of a DMA instruction
// fetches global chunk j ^ row so that its lane-ordered write lands in place --;
// SX [16][8] activation scales; SG [16*TPW rows][8] weight scales.
// s_waitcnt vmcnt(min(after, A) * L), `after` wave-uniform, the count an immediate
template <int L, int A>
__device__ __forceinline__ void wait_steps(int after) {
  if constexpr (A == 0) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  } else {
    if (after >= A) __builtin_amdgcn_s_waitcnt(vmcnt_imm(A * L));
    else wait_steps<L, A - 1>(after);
  }
}

template <int MODE, int TPW>
struct RSlot {
  static constexpr int W = 0;
  static constexpr int A = W + 16 * TPW * 256;
  static constexpr int L = A + 16 * 256;
  static constexpr int SX = L + (MODE == 2 ? 16 * 256 : 0);
  static constexpr int SG = SX + 16 * STEP * 4;
  static constexpr int BYTES = SG + 16 * TPW * STEP * 2;
  static constexpr int LOADS = 4 * TPW + (MODE == 2 ? 8 : 4) + 2 + 1;  // DMA instructions a step
};

template <int MODE, int TPW, int P>
__global__ __launch_bounds__(64) void k_gemv_mfma_ring(const int8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
                                                       const int8_t* __restrict__ xq, const int8_t* __restrict__ xl,
                                                       const float* __restrict__ xs, int64_t N, int64_t K, int B,
                                                       int S, float* __restrict__ out) {
  using SL = RSlot<MODE, TPW>;
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int s_idx = blockIdx.y;
  int32_t g0, g1;
  split_range(K, S, s_idx, g0, g1);
  const int nsteps = (g1 - g0) / STEP;  // whole steps: K/32 and chunk ends are multiples of 8 here
  const int64_t nb = K / QK;
  const int64_t o_wg = (int64_t)blockIdx.x * 16 * TPW;

  // ---- load side: instruction m of the weights reads rows 4m .. 4m+3 of the wave
  const int r4 = lane >> 4, j = lane & 15;
  const int8_t* wsrc[4 * TPW];
#pragma unroll
  for (int m = 0; m < 4 * TPW; ++m) {
    const int row = 4 * m + r4;
    int64_t o = o_wg + row;
    if (o >= N) o = N - 1;
    wsrc[m] = wq + o * K + 16 * ((j ^ row) & 15);  // global chunk j ^ row of the row's step
  }
  int64_t aoff[4];  // activation rows 4q + r4, chunk j ^ row
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = 4 * q + r4;
    aoff[q] = (int64_t)min(t, B - 1) * K + 16 * ((j ^ t) & 15);
  }
  const float* xsrc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int sidx = 64 * h + lane;  // [t][k] within the step
    xsrc[h] = xs + (int64_t)min(sidx >> 3, B - 1) * nb + (sidx & 7);
  }
  int64_t so = o_wg + (lane < 16 * TPW ? lane : 0);
  if (so >= N) so = N - 1;
  const uint16_t* ssrc = ws + so * nb;

  // every load of step s, into slot s mod P: the same count (SL::LOADS) each step
  auto issue = [&](int s) {
    unsigned char* slot = lds + (s % P) * SL::BYTES;
    const int64_t b0 = g0 + (int64_t)s * STEP;
#pragma unroll
    for (int m = 0; m < 4 * TPW; ++m)  // nontemporal: the weights are streamed once
      dma<16, 2>(wsrc[m] + b0 * QK, slot + SL::W + m * 1024);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma<16, 0>(xq + aoff[q] + b0 * QK, slot + SL::A + q * 1024);
    if constexpr (MODE == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) dma<16, 0>(xl + aoff[q] + b0 * QK, slot + SL::L + q * 1024);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) dma<4, 0>(xsrc[h] + b0, slot + SL::SX + h * 256);
    // lane i < 16*TPW moves row i's 8 scales (16 bytes); the other lanes are masked off
    if (lane < 16 * TPW) dma<16, 0>(ssrc + b0, slot + SL::SG);
  };
  // waits until step s has landed: after it, `after` later steps' loads may be outstanding
  auto wait_step = [&](int after) {
    asm volatile("" ::: "memory");
    wait_steps<SL::LOADS, P - 1>(after);
    asm volatile("" ::: "memory");
  };
  static_assert(P >= 2 && (P - 1) * SL::LOADS < 64, "ring depth and wait counts");

  // ---- read side (lane col, grp): block k's 8 bytes of row col of a tile
  float p[TPW][4][4];  // [tile][partial][i]: output (t = 4*grp + i, o = o_wg + 16*tile + col)
#pragma unroll
  for (int m = 0; m < TPW; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[m][r][i] = 0.0f;

  // Only the chunk's own steps are loaded (an empty chunk, K < 512 with several
  // chunks, loads nothing: its partials stay +0); near the end fewer steps are in
  // flight, and the waits count them.
#pragma unroll
  for (int q = 0; q < P - 1; ++q)
    if (q < nsteps) issue(q);
  for (int s = 0; s < nsteps; ++s) {
    asm volatile("" ::: "memory");
    if (s + P - 1 < nsteps) issue(s + P - 1);  // into slot (s - 1) mod P, whose reads (step s - 1) are done
    wait_step(min(P - 1, nsteps - 1 - s));
    const unsigned char* slot = lds + (s % P) * SL::BYTES;
#pragma unroll
    for (int k = 0; k < STEP; ++k) {
      const int off = ((((2 * k + (grp >> 1)) ^ col) & 15) << 4) + 8 * (grp & 1);
      const long ak = *(const long*)(slot + SL::A + col * 256 + off);
      long lk = 0;
      if constexpr (MODE == 2) lk = *(const long*)(slot + SL::L + col * 256 + off);
      float sig[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sig[i] = *(const float*)(slot + SL::SX + ((4 * grp + i) * STEP + k) * 4);
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        const long wk = *(const long*)(slot + SL::W + (16 * m + col) * 256 + off);
        const float sgm =
            half_bits_to_float(*(const unsigned short*)(slot + SL::SG + ((16 * m + col) * STEP + k) * 2));
        const v4i D = mfma16x16x32(ak, wk);
        v4i E = {0, 0, 0, 0};
        if constexpr (MODE == 2) E = mfma16x16x32(lk, wk);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float ta, tb;
          q8_term<MODE>(sgm, sig[i], D[i], E[i], ta, tb);
          p[m][k & 3][i] = __fmaf_rn(ta, tb, p[m][k & 3][i]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int64_t oo = o_wg + 16 * m + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * grp + i;
      const float y = __fadd_rn(__fadd_rn(p[m][0][i], p[m][2][i]), __fadd_rn(p[m][1][i], p[m][3][i]));
      if (t < B && oo < N) out[((int64_t)s_idx * B + t) * N + oo] = y;
    }
  }
}

template <int MODE, int TPW, int P>
hipError_t launch_ring(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq,
                       const int8_t* xl, const float* xs, int64_t B, int splits, float* out, hipStream_t st) {
  constexpr int lds = P * RSlot<MODE, TPW>::BYTES;
  static_assert(lds <= 160 * 1024, "LDS of one workgroup");
  static const hipError_t attr = hipFuncSetAttribute((const void*)&k_gemv_mfma_ring<MODE, TPW, P>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const dim3 grid((unsigned)((N + 16 * TPW - 1) / (16 * TPW)), (unsigned)splits), block(64);
  return launch((k_gemv_mfma_ring<MODE, TPW, P>), grid, block, lds, st, wq, ws, xq, xl, xs, N, K, (int)B, splits,
                out);
}

// Fast-path shape: QDG_TUNE_MFMA_SHAPE = 100*WV + 10*TPW + P among the compiled
// ones -- 4,4,2 (the default), 4,4,3, 4,2,2, 8,2,3.  On 25600x5120, B = 16:
// 4,4,2 streams 4.30 / 3.96 TB/s (Int8Act / TwoPass), 8,2,3 4.27 / 3.73,
// 4,4,3 4.06 / 3.80, 4,2,3 3.73 / 3.24.
struct DmaShape {
  int wv, tpw, ring;
};
DmaShape shape_knob(int knob, DmaShape def) {
  const int v = tune(knob);
  if (v < 0) return def;
  return DmaShape{v / 100, (v / 10) % 10, v % 10};
}
DmaShape dma_shape() { return shape_knob(QDG_TUNE_MFMA_SHAPE, DmaShape{4, 4, 2}); }

template <int MODE>
hipError_t launch_m(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq, const int8_t* xl,
                    const float* xs, int64_t B, int splits, float* out, hipStream_t st) {
  // more than 16 activation rows: 2 or 4 activation tiles against each weight
  // step (the fast path's layout; the caller has checked its conditions)
  if (B > 16) {
    // QDG_TUNE_MFMA_WIDE = 100*WV + 10*TPW + P among the compiled shapes (for sweeps)
    const DmaShape wide = shape_knob(QDG_TUNE_MFMA_WIDE, DmaShape{8, 2, 2});
    const int wv = wide.wv, tpw = wide.tpw, ring = wide.ring;
#define QDG_WIDE(WV_, TPW_, P_)                                                                   \
  if (wv == WV_ && tpw == TPW_ && ring == P_) {                                                    \
    if (B <= 32) return launch_dma<MODE, WV_, TPW_, P_, 2>(wq, ws, N, K, xq, xl, xs, B, splits, out, st); \
    return launch_dma<MODE, WV_, TPW_, P_, 4>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);            \
  }
    QDG_WIDE(8, 1, 3)
    QDG_WIDE(4, 2, 3)
    QDG_WIDE(8, 2, 3)
    QDG_WIDE(4, 1, 3)
#undef QDG_WIDE
    if (B <= 32) return launch_dma<MODE, 8, 2, 2, 2>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
    return launch_dma<MODE, 8, 2, 2, 4>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
  }
  // the fast path needs whole steps (K/32 a multiple of 8) and 16-byte weight-scale words
  if ((K / QK) % 8 == 0 && ((uintptr_t)ws & 15) == 0 && tune(QDG_TUNE_MFMA_GENERAL) != 1) {
    // the workgroup-shared ring (default; QDG_TUNE_MFMA_SHAPE = 100*WV + 10*TPW + P),
    // or the per-wave ring (1000 + 10*TPW + P), which measured slower: each wave
    // fetches the activation tile itself and its own steps serialise behind its loads
    const int knob = tune(QDG_TUNE_MFMA_SHAPE);
    if (knob >= 1000) {
      const int rt = (knob / 10) % 10, rp = knob % 10;
#define QDG_RING(T_, P_) \
  if (rt == T_ && rp == P_) return launch_ring<MODE, T_, P_>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
      QDG_RING(1, 3) QDG_RING(2, 2)
#undef QDG_RING
      return launch_ring<MODE, 2, 3>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
    }
    const DmaShape d = dma_shape();
#define QDG_DMA(WV_, TPW_, P_)                   \
  if (d.wv == WV_ && d.tpw == TPW_ && d.ring == P_) \
    return launch_dma<MODE, WV_, TPW_, P_>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
    QDG_DMA(4, 4, 3);
    QDG_DMA(4, 4, 4);
    QDG_DMA(4, 2, 2);
    QDG_DMA(4, 2, 3);
    QDG_DMA(4, 2, 4);
    QDG_DMA(8, 2, 3);
    QDG_DMA(8, 1, 3);
    QDG_DMA(8, 1, 4);
#undef QDG_DMA
    return launch_dma<MODE, 4, 4, 2>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
  }
  return launch_mp<MODE, 2>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
}

}  // namespace

hipError_t launch_gemv_mfma(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K,
                            const int8_t* xq, const int8_t* xl, const float* xs, int64_t B, int splits,
                            float* out, hipStream_t st) {
  if (mode == 1) return launch_m<1>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
  return launch_m<2>(wq, ws, N, K, xq, xl, xs, B, splits, out, st);
}

}  // namespace qdg
