// qdg_mma_tiled.hip -- the batched (B <= 64) Q8_0 GEMV on int8 MFMA over weights
// and activations stored in the MFMA's own operand order (megakernel page: the
// GEMV's tiled-weights option, where only the addresses of the weights change;
// lane kernel library page: lk_gemv_mma, whose rows sum exactly as a single row).
//
// The sums are k_gemv_mfma_dma's, term for term: block g's exact int32 dots D
// (and E) from v_mfma_i32_16x16x32_i8, the step p <- fma(a, b, p) of
// lk_q8_term into partial g mod 4 in ascending block order, then
// (P0 + P2) + (P1 + P3).  So every row equals qdg_gemv_q8's, bit for bit, for the
// same splits, whatever the batch.
//
// Layout.  A record holds what one wave consumes in one step: for a group of 64
// weight rows q (four 16-row tiles m), an 8-block step s and a residue r (the
// blocks 8s + r and 8s + r + 4, which feed partial r), 4096 weight bytes and 256
// scale bytes:
//  * weight byte 1024*m + 16*l + 8*h + j (lane l, column c = l % 16, group
//    u = l / 16) is byte 8*u + j of block 8s + r + 4h of row 64q + 16m + c -- so
//    a lane's 16 bytes are exactly its B operands of the step's two MFMAs;
//  * scale halfword 4096/2 + 8*c + 2*m + h is the binary16 scale of that row and
//    block.
// Records run (q, s, r) in row-major order; rows past N are zero.  A wave's
// weight load is one contiguous KiB, its scale load 256 bytes.
//
// The activations come in the same order (qdg_quantize_act_mma), in AT tiles of
// 16 rows (1, 2 or 4 of them, one after the other): for step s and residue r,
// lane l's 16 bytes of a tile are the A operands of the two blocks (tile row
// t = l % 16, 8 bytes from 8 * (l / 16) of blocks 8s + r and 8s + r + 4), and 32
// scales follow the same (s, r) order, [h][t].  The quantizer writes the rows
// past the batch as the words of a zero row.
//
// Kernel.  A workgroup of 4 * (4 * GW / TPW) waves owns GW 64-row groups and one
// chunk of K; wave (g, r) takes TPW tiles for residue r and walks the chunk's
// steps reading records (q, s, r) and the activation records (s, r) of every
// activation tile straight into registers -- no LDS tile, no workgroup barrier
// until the end -- with P - 1 steps in flight (named step buffers; every step
// issues the same loads, so the compiler's wait counts stay exact).  Each load
// is a contiguous run: 1 KiB a weight tile, 1 KiB of activation words and 128
// bytes of activation scales an activation tile.  A lane loads one activation
// scale a tile and the scales of its four batch rows reach it by ds_bpermute.
// The partial waves meet in LDS at the end, one activation tile at a time.

#include "qdg_device.h"

namespace qdg {
namespace {

constexpr int MT_ROWS = 64;               // weight rows of a record group
constexpr int MT_WBYTES = 4096;           // weight bytes of a record
constexpr int MT_REC = MT_WBYTES + 256;   // record bytes (weights, then scales)
constexpr int MT_STEP = 8;                // blocks a step

// One workgroup a (row group, step): its four records, one residue after the
// other, so the step's 256-byte row segments are fetched once and re-read from
// the cache for the later residues.
__global__ __launch_bounds__(256) void k_tile_mma(const int8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
                                                  int64_t N, int64_t K, uint8_t* __restrict__ wt) {
  const int64_t qs = blockIdx.x, nst = K / 256, nb = K / QK;  // qs = q * nst + s
  const int64_t s = qs % nst, q = qs / nst;
  const int tid = threadIdx.x, m = tid >> 6, l = tid & 63, c = l & 15, u = l >> 4;
  const int64_t row = q * MT_ROWS + 16 * m + c;
  for (int r = 0; r < 4; ++r) {
    const int64_t b0 = s * MT_STEP + r;
    int2 lo = make_int2(0, 0), hi = make_int2(0, 0);
    if (row < N) {
      lo = *(const int2*)(wq + row * K + b0 * QK + 8 * u);
      hi = *(const int2*)(wq + row * K + (b0 + 4) * QK + 8 * u);
    }
    uint8_t* dst = wt + (qs * 4 + r) * MT_REC;
    *(int4*)(dst + 16 * tid) = make_int4(lo.x, lo.y, hi.x, hi.y);
    if (tid < 16) {
      unsigned w[4];
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const int64_t rw = q * MT_ROWS + 16 * mm + tid;
        const unsigned a = rw < N ? ws[rw * nb + b0] : 0u, b = rw < N ? ws[rw * nb + b0 + 4] : 0u;
        w[mm] = a | (b << 16);
      }
      *(int4*)(dst + MT_WBYTES + 16 * tid) = make_int4((int)w[0], (int)w[1], (int)w[2], (int)w[3]);
    }
  }
}

// The activation quantizer of qdg_quantize_act (quant_lane4: eight lanes a
// 32-value block, four values a lane), writing the words and scales in the
// MFMA order above, AT tiles of 16 rows one after the other.  Rows B..16*AT-1
// quantize a zero row.
template <int MODE>
__global__ __launch_bounds__(256) void k_quantize_mma(const float* __restrict__ x, int B, int64_t K, int AT,
                                                      int8_t* __restrict__ xq, int8_t* __restrict__ xl,
                                                      float* __restrict__ xs) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nb = K / QK, blk = gid >> 3;  // blk over [16*AT][nb]
  const int sub = (int)(gid & 7);
  const bool on = blk < 16 * AT * nb;
  const int t = (int)(blk / nb);
  const int64_t b = blk - (int64_t)t * nb;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (on && t < B) v = *(const float4*)(x + (int64_t)t * K + b * QK + 4 * sub);
  int h, l;
  const float sc = quant_lane4<MODE>(v, &h, &l);
  if (!on) return;
  const int at = t >> 4, tt = t & 15;
  const int64_t rs = (b >> 3) * 4 + (b & 3);  // record (s, r)
  const int hh = (int)((b >> 2) & 1);
  const int64_t off = at * 16 * K + (rs * 64 + 16 * (sub >> 1) + tt) * 16 + 8 * hh + 4 * (sub & 1);
  *(int*)(xq + off) = h;
  if constexpr (MODE == 2) *(int*)(xl + off) = l;
  if (sub == 0) xs[at * (K / 2) + rs * 32 + 16 * hh + tt] = sc;
}

__device__ __forceinline__ v4i mma16x16x32(long a, long b) {
  const v4i z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, z, 0, 0, 0);
}

// One step's operands of a lane.
template <int MODE, int TPW, int AT>
struct MtStep {
  v4i w[TPW];   // the B operands of blocks 8s + r (.x, .y) and 8s + r + 4 (.z, .w), a tile each
  v4i sc;       // the scales of column c's four rows: word m = block 8s + r (low), 8s + r + 4 (high)
  v4i a[AT];    // A operands (activation row t = c of each activation tile) of the two blocks
  v4i al[AT];   // TwoPass low words
  float sx[AT]; // the scale of activation row t = l % 16, block 8s + r + 4 * ((l / 16) & 1)
};

__device__ __forceinline__ long lo64(v4i v) { return (long)(((unsigned long)(unsigned)v[1] << 32) | (unsigned)v[0]); }
__device__ __forceinline__ long hi64(v4i v) { return (long)(((unsigned long)(unsigned)v[3] << 32) | (unsigned)v[2]); }

// xa, xla, xsa point at this step's record of activation tile 0; tile `at`
// lies at + at * 16K bytes (words) and + at * K/2 scales.
template <int MODE, int TPW, int AT>
__device__ __forceinline__ void mt_load(MtStep<MODE, TPW, AT>& b, const uint8_t* rec, int m0, const int8_t* xa,
                                        const int8_t* xla, const float* xsa, int64_t K) {
  __builtin_amdgcn_sched_barrier(0);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 0; m < TPW; ++m)
    b.w[m] = __builtin_nontemporal_load((const v4i*)(rec + 1024 * (m0 + m) + 16 * lane));
  b.sc = *(const v4i*)(rec + MT_WBYTES + 16 * (lane & 15));
#pragma unroll
  for (int at = 0; at < AT; ++at) {
    b.a[at] = *(const v4i*)(xa + at * 16 * K + 16 * lane);
    if constexpr (MODE == 2) b.al[at] = *(const v4i*)(xla + at * 16 * K + 16 * lane);
    b.sx[at] = xsa[at * (K / 2) + (lane & 31)];
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int MODE, int TPW, int AT>
__device__ __forceinline__ void mt_terms(const MtStep<MODE, TPW, AT>& b, int m0, float (&p)[TPW][AT][4]) {
  const int lane = threadIdx.x & 63, u = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float sig[AT][4];
    long ak[AT], lk[AT];
#pragma unroll
    for (int at = 0; at < AT; ++at) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sig[at][i] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (16 * h + 4 * u + i), __float_as_int(b.sx[at])));
      ak[at] = h == 0 ? lo64(b.a[at]) : hi64(b.a[at]);
      lk[at] = 0;
      if constexpr (MODE == 2) lk[at] = h == 0 ? lo64(b.al[at]) : hi64(b.al[at]);
    }
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const long wk = h == 0 ? lo64(b.w[m]) : hi64(b.w[m]);
      const unsigned sw = (unsigned)b.sc[m0 + m];
      const float sgm = half_bits_to_float((unsigned short)(h == 0 ? (sw & 0xffffu) : (sw >> 16)));
#pragma unroll
      for (int at = 0; at < AT; ++at) {
        const v4i D = mma16x16x32(ak[at], wk);
        v4i E = {0, 0, 0, 0};
        if constexpr (MODE == 2) E = mma16x16x32(lk[at], wk);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float ta, tb;
          q8_term<MODE>(sgm, sig[at][i], D[i], E[i], ta, tb);
          p[m][at][i] = __fmaf_rn(ta, tb, p[m][at][i]);
        }
      }
    }
  }
}

// A wave's partials over its chunk: nsteps steps from record rec0 and
// activation records xa0 / xla0 / xsa0, tiles m0.. of the record group, P - 1
// steps in flight (named step buffers; past the chunk a load repeats its last
// step, so every step issues the same loads and the wait counts stay exact).
template <int MODE, int TPW, int P, int AT>
__device__ __forceinline__ void mt_partials(const uint8_t* rec0, const int8_t* xa0, const int8_t* xla0,
                                            const float* xsa0, int nsteps, int m0, int64_t K,
                                            float (&p)[TPW][AT][4]) {
#pragma unroll
  for (int m = 0; m < TPW; ++m)
#pragma unroll
    for (int at = 0; at < AT; ++at)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[m][at][i] = 0.0f;

  if (nsteps > 0) {
    auto load = [&](MtStep<MODE, TPW, AT>& b, int st) {
      const int64_t k = st < nsteps ? st : nsteps - 1;  // past the chunk: its last step again
      mt_load<MODE, TPW, AT>(b, rec0 + k * 4 * MT_REC, m0, xa0 + k * 4096, MODE == 2 ? xla0 + k * 4096 : nullptr,
                             xsa0 + k * 128, K);
    };
    MtStep<MODE, TPW, AT> b[P];
#pragma unroll
    for (int k = 0; k < P; ++k) load(b[k], k);
    int st = 0;
    // while every refill is due
    for (; st + 2 * P - 1 < nsteps; st += P) {
#pragma unroll
      for (int k = 0; k < P; ++k) {
        mt_terms<MODE, TPW, AT>(b[k], m0, p);
        load(b[k], st + k + P);
      }
    }
    // the last 1 .. 2P - 1 steps, in order
#pragma unroll
    for (int k = 0; k < P; ++k) {
      if (st + k < nsteps) mt_terms<MODE, TPW, AT>(b[k], m0, p);
      if (st + k + P < nsteps) load(b[k], st + k + P);
    }
#pragma unroll
    for (int k = 0; k + 1 < P; ++k)
      if (st + P + k < nsteps) mt_terms<MODE, TPW, AT>(b[k], m0, p);
  }
}

// Grid (workgroup row blocks of 64*GW rows, splits), 4 * (4*GW / TPW) waves a
// workgroup, AT activation tiles of 16 rows (B <= 16 * AT).  out [splits][B][N].
template <int MODE, int TPW, int P, int GW, int AT>
__global__ __launch_bounds__(256 * (4 * GW / TPW)) void k_gemv_mma_tiled(const uint8_t* __restrict__ wt,
                                                                    const int8_t* __restrict__ xq,
                                                                    const int8_t* __restrict__ xl,
                                                                    const float* __restrict__ xs, int64_t N, int64_t K,
                                                                    int B, int S, float* __restrict__ out) {
  constexpr int G = 4 * GW / TPW;      // tile groups a workgroup
  __shared__ float red[4 * G][TPW][4][64];  // [wave][tile][i][lane], one activation tile at a time
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = wave & 3, g = wave >> 2, m0 = (TPW * g) & 3;  // tile m0.. of record group q
  const int c = lane & 15, u = lane >> 4;
  const int s_idx = blockIdx.y;
  int32_t g0, g1;
  split_range(K, S, s_idx, g0, g1);
  const int64_t nst = K / 256;
  const int64_t q = (int64_t)blockIdx.x * GW + (TPW * g) / 4;  // this wave's record group
  // K is a multiple of 256: chunks are whole steps; a record group past the
  // matrix (the last workgroup's, when GW > 1) loads nothing
  const int nsteps = q < (N + MT_ROWS - 1) / MT_ROWS ? (g1 - g0) / MT_STEP : 0;
  const int gs0 = g0 / MT_STEP;
  // record (q, gs0 + st, r) and activation record (gs0 + st, r)
  const uint8_t* rec0 = wt + ((q * nst + gs0) * 4 + r) * (int64_t)MT_REC;
  const int8_t* xa0 = xq + ((int64_t)gs0 * 4 + r) * 1024;
  const int8_t* xla0 = MODE == 2 ? xl + ((int64_t)gs0 * 4 + r) * 1024 : nullptr;
  const float* xsa0 = xs + ((int64_t)gs0 * 4 + r) * 32;

  float p[TPW][AT][4];
#pragma unroll
  for (int m = 0; m < TPW; ++m)
#pragma unroll
    for (int at = 0; at < AT; ++at)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[m][at][i] = 0.0f;

  if (nsteps > 0) {
    auto load = [&](MtStep<MODE, TPW, AT>& b, int st) {
      const int64_t k = st < nsteps ? st : nsteps - 1;  // past the chunk: its last step again
      mt_load<MODE, TPW, AT>(b, rec0 + k * 4 * MT_REC, m0, xa0 + k * 4096, MODE == 2 ? xla0 + k * 4096 : nullptr,
                             xsa0 + k * 128, K);
    };
    MtStep<MODE, TPW, AT> b[P];
#pragma unroll
    for (int k = 0; k < P; ++k) load(b[k], k);
    int st = 0;
    // while every refill is due
    for (; st + 2 * P - 1 < nsteps; st += P) {
#pragma unroll
      for (int k = 0; k < P; ++k) {
        mt_terms<MODE, TPW, AT>(b[k], m0, p);
        load(b[k], st + k + P);
      }
    }
    // the last 1 .. 2P - 1 steps, in order
#pragma unroll
    for (int k = 0; k < P; ++k) {
      if (st + k < nsteps) mt_terms<MODE, TPW, AT>(b[k], m0, p);
      if (st + k + P < nsteps) load(b[k], st + k + P);
    }
#pragma unroll
    for (int k = 0; k + 1 < P; ++k)
      if (st + P + k < nsteps) mt_terms<MODE, TPW, AT>(b[k], m0, p);
  }

  // one activation tile at a time through LDS: wave (g, 0) writes its tiles,
  // lane (c, u) holding row 64q + 16(m0 + m) + c and batch rows 16 at + 4u + i
#pragma unroll
  for (int at = 0; at < AT; ++at) {
    if (at > 0) __syncthreads();  // the previous tile's reads are done
#pragma unroll
    for (int m = 0; m < TPW; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][m][i][lane] = p[m][at][i];
    __syncthreads();
    if (r == 0) {
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        const int64_t o = q * MT_ROWS + 16 * (m0 + m) + c;  // rows past the last record group: o >= N
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * at + 4 * u + i;
          const float y = __fadd_rn(__fadd_rn(red[4 * g][m][i][lane], red[4 * g + 2][m][i][lane]),
                                    __fadd_rn(red[4 * g + 1][m][i][lane], red[4 * g + 3][m][i][lane]));
          if (t < B && o < N) out[((int64_t)s_idx * B + t) * N + o] = y;
        }
      }
    }
  }
}

// The gate and up projections of a batch with the gated product and the
// quantizer as the epilogue (lane kernel library page, GLU / lk_gemv_glu with a
// quantized output, here for up to 64 activation rows): workgroup q's first
// four waves sum record group q of the gate records, the next four the same
// group of the up records, exactly as k_gemv_mma_tiled sums them unsplit.  Per
// activation tile the eight waves' partials meet in LDS; four waves then form,
// for each of the tile's 16 rows and the group's two 32-row blocks of outputs,
// g and u in that kernel's order, h = act(g) * u with the producer's glu_mul
// (+0 for a row past the batch), and quantize each 32-value block with eight
// lanes as the quantizer does -- writing the words in the activation record
// order of qdg_quantize_act_mma for a projection with K = F.  h [B][F] is
// written too when asked for.  Grid F / 64, 512 threads.
template <int MODE, int P, int AT, int ACT>
__global__ __launch_bounds__(512) void k_gemv_mma_glu(const uint8_t* __restrict__ wgt, const uint8_t* __restrict__ wut,
                                                      const int8_t* __restrict__ xq, const int8_t* __restrict__ xl,
                                                      const float* __restrict__ xs, int64_t F, int64_t K, int B,
                                                      float* __restrict__ h, int8_t* __restrict__ hq,
                                                      int8_t* __restrict__ hl, float* __restrict__ hs) {
  __shared__ float red[8][4][4][64];  // [wave][tile][i][lane], one activation tile at a time
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = wave & 3, g = wave >> 2;  // g = 0 gate, 1 up
  const int64_t nst = K / 256, q = blockIdx.x;
  const uint8_t* rec0 = (g ? wut : wgt) + (q * nst * 4 + r) * (int64_t)MT_REC;
  const int8_t* xa0 = xq + (int64_t)r * 1024;
  const int8_t* xla0 = MODE == 2 ? xl + (int64_t)r * 1024 : nullptr;
  const float* xsa0 = xs + (int64_t)r * 32;
  float p[4][AT][4];
  mt_partials<MODE, 4, P, AT>(rec0, xa0, xla0, xsa0, (int)nst, 0, K, p);

  // block bk of the group's 32 (16 tile rows x 2 output blocks), lane sub of its eight
  const int bk = 8 * (wave & 3) + (lane >> 3), tt = bk >> 1, half = bk & 1, sub = lane & 7;
  const int64_t b = 2 * q + half;                // output block along F
  const int64_t rs = (b >> 3) * 4 + (b & 3);     // its activation record (s, r) for K = F
  const int hh = (int)((b >> 2) & 1);
#pragma unroll
  for (int at = 0; at < AT; ++at) {
    if (at > 0) __syncthreads();  // the previous tile's reads are done
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][m][i][lane] = p[m][at][i];
    __syncthreads();
    if (wave < 4) {
      const int t = 16 * at + tt;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int o = 32 * half + 4 * sub + j;  // row of the group
        const int m = o >> 4, i = tt & 3, ln = (o & 15) + 16 * (tt >> 2);
        const float gv = __fadd_rn(__fadd_rn(red[0][m][i][ln], red[2][m][i][ln]),
                                   __fadd_rn(red[1][m][i][ln], red[3][m][i][ln]));
        const float uv = __fadd_rn(__fadd_rn(red[4][m][i][ln], red[6][m][i][ln]),
                                   __fadd_rn(red[5][m][i][ln], red[7][m][i][ln]));
        v[j] = t < B ? glu_mul<ACT>(gv, uv) : 0.0f;
      }
      const float4 v4 = make_float4(v[0], v[1], v[2], v[3]);
      if (h && t < B) *(float4*)(h + (int64_t)t * F + 64 * q + 32 * half + 4 * sub) = v4;
      int wh, wl;
      const float sc = quant_lane4<MODE>(v4, &wh, &wl);
      const int64_t off = at * 16 * F + (rs * 64 + 16 * (sub >> 1) + tt) * 16 + 8 * hh + 4 * (sub & 1);
      *(int*)(hq + off) = wh;
      if constexpr (MODE == 2) *(int*)(hl + off) = wl;
      if (sub == 0) hs[at * (F / 2) + rs * 32 + 16 * hh + tt] = sc;
    }
  }
}

// Steps in flight: P - 1 ahead of the one being summed (P = 4 measured best
// against 3 and 5 on 25600x5120, B = 16).
constexpr int MT_P = 4;

// Record groups a workgroup.  Two (eight waves, 128 rows) when the launch still
// spreads over most of the machine: the two waves of a residue read the same
// activation record, which the second finds in L1, so a compute unit moves half
// the activation bytes per weight byte -- 23.0 against 25.2 us (Int8Act) and
// 26.7 against 28.4 us (TwoPass) on 25600x5120, B = 16, though 56 compute units
// then stay idle.  QDG_TUNE_MT_GROUPS overrides.
int mt_groups(int64_t N, int splits) {
  const int f = tune(QDG_TUNE_MT_GROUPS);
  if (f == 1 || f == 2) return f;
  return (N + 127) / 128 * splits >= 192 ? 2 : 1;
}

// Activation tiles of 16 rows for B rows: 1, 2 or 4.
int mt_tiles(int64_t B) { return B <= 16 ? 1 : B <= 32 ? 2 : 4; }

// Steps in flight fall with the activation tiles a step holds in registers.
template <int MODE, int GW, int AT>
hipError_t launch_mta(const uint8_t* wt, int64_t N, int64_t K, const int8_t* xq, const int8_t* xl, const float* xs,
                      int64_t B, int splits, float* out, hipStream_t st) {
  constexpr int P = AT == 1 ? MT_P : AT == 2 ? 3 : 2;
  const dim3 grid((unsigned)((N + GW * MT_ROWS - 1) / (GW * MT_ROWS)), (unsigned)splits), block(256 * GW);
  return launch((k_gemv_mma_tiled<MODE, 4, P, GW, AT>), grid, block, 0, st, wt, xq, xl, xs, N, K, (int)B, splits,
                out);
}

template <int MODE, int GW>
hipError_t launch_mt(const uint8_t* wt, int64_t N, int64_t K, const int8_t* xq, const int8_t* xl, const float* xs,
                     int64_t B, int splits, float* out, hipStream_t st) {
  switch (mt_tiles(B)) {
    case 1: return launch_mta<MODE, GW, 1>(wt, N, K, xq, xl, xs, B, splits, out, st);
    case 2: return launch_mta<MODE, GW, 2>(wt, N, K, xq, xl, xs, B, splits, out, st);
    default: return launch_mta<MODE, GW, 4>(wt, N, K, xq, xl, xs, B, splits, out, st);
  }
}

template <int MODE, int AT, int ACT>
hipError_t launch_mga(const uint8_t* wgt, const uint8_t* wut, int64_t F, int64_t K, const int8_t* xq,
                      const int8_t* xl, const float* xs, int64_t B, float* h, int8_t* hq, int8_t* hl, float* hs,
                      hipStream_t st) {
  constexpr int P = AT == 1 ? MT_P : AT == 2 ? 3 : 2;
  return launch((k_gemv_mma_glu<MODE, P, AT, ACT>), dim3((unsigned)(F / MT_ROWS)), dim3(512), 0, st, wgt, wut, xq,
                xl, xs, F, K, (int)B, h, hq, hl, hs);
}

template <int MODE, int ACT>
hipError_t launch_mg(const uint8_t* wgt, const uint8_t* wut, int64_t F, int64_t K, const int8_t* xq, const int8_t* xl,
                     const float* xs, int64_t B, float* h, int8_t* hq, int8_t* hl, float* hs, hipStream_t st) {
  switch (mt_tiles(B)) {
    case 1: return launch_mga<MODE, 1, ACT>(wgt, wut, F, K, xq, xl, xs, B, h, hq, hl, hs, st);
    case 2: return launch_mga<MODE, 2, ACT>(wgt, wut, F, K, xq, xl, xs, B, h, hq, hl, hs, st);
    default: return launch_mga<MODE, 4, ACT>(wgt, wut, F, K, xq, xl, xs, B, h, hq, hl, hs, st);
  }
}

template <int ACT>
hipError_t launch_mg_a(int mode, const uint8_t* wgt, const uint8_t* wut, int64_t F, int64_t K, const int8_t* xq,
                       const int8_t* xl, const float* xs, int64_t B, float* h, int8_t* hq, int8_t* hl, float* hs,
                       hipStream_t st) {
  if (mode == 1) return launch_mg<1, ACT>(wgt, wut, F, K, xq, xl, xs, B, h, hq, hl, hs, st);
  return launch_mg<2, ACT>(wgt, wut, F, K, xq, xl, xs, B, h, hq, hl, hs, st);
}

template <int MODE>
hipError_t launch_qm(const float* x, int64_t B, int64_t K, int8_t* xq, int8_t* xl, float* xs, hipStream_t st) {
  const int AT = mt_tiles(B);
  const int64_t threads = 16 * AT * (K / QK) * 8;
  return launch(k_quantize_mma<MODE>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, x, (int)B, K, AT, xq,
                xl, xs);
}

}  // namespace

int64_t tile_mma_bytes(int64_t N, int64_t K) {
  return (N + MT_ROWS - 1) / MT_ROWS * (K / 256) * 4 * (int64_t)MT_REC;
}

hipError_t launch_tile_mma(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, uint8_t* wt, hipStream_t st) {
  const int64_t steps = (N + MT_ROWS - 1) / MT_ROWS * (K / 256);  // a workgroup a (row group, step)
  return launch(k_tile_mma, dim3((unsigned)steps), dim3(256), 0, st, wq, ws, N, K, wt);
}

hipError_t launch_quantize_mma(int mode, const float* x, int64_t B, int64_t K, int8_t* xq, int8_t* xl, float* xs,
                               hipStream_t st) {
  if (mode == 1) return launch_qm<1>(x, B, K, xq, xl, xs, st);
  return launch_qm<2>(x, B, K, xq, xl, xs, st);
}

hipError_t launch_gemv_mma_tiled(int mode, const uint8_t* wt, int64_t N, int64_t K, const int8_t* xq,
                                 const int8_t* xl, const float* xs, int64_t B, int splits, float* out,
                                 hipStream_t st) {
  const int gw = mt_groups(N, splits);
  if (mode == 1)
    return gw == 2 ? launch_mt<1, 2>(wt, N, K, xq, xl, xs, B, splits, out, st)
                   : launch_mt<1, 1>(wt, N, K, xq, xl, xs, B, splits, out, st);
  return gw == 2 ? launch_mt<2, 2>(wt, N, K, xq, xl, xs, B, splits, out, st)
                 : launch_mt<2, 1>(wt, N, K, xq, xl, xs, B, splits, out, st);
}

int mma_act_tiles(int64_t B) { return mt_tiles(B); }

hipError_t launch_gemv_glu_mma(int act, int mode, const uint8_t* wgt, const uint8_t* wut, int64_t F, int64_t K,
                               const int8_t* xq, const int8_t* xl, const float* xs, int64_t B, float* h, int8_t* hq,
                               int8_t* hl, float* hs, hipStream_t st) {
  if (act == 0) return launch_mg_a<0>(mode, wgt, wut, F, K, xq, xl, xs, B, h, hq, hl, hs, st);
  if (act == 1) return launch_mg_a<1>(mode, wgt, wut, F, K, xq, xl, xs, B, h, hq, hl, hs, st);
  return launch_mg_a<2>(mode, wgt, wut, F, K, xq, xl, xs, B, h, hq, hl, hs, st);
}

}  // namespace qdg
