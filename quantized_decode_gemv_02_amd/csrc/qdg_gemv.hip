// qdg_gemv.hip -- the batch-1 Q8_0 GEMV under the quantized numerics (Int8Act,
// TwoPass), with split-K partials; the lane kernel library page's lk_gemv_q8 /
// lk_q8_rows_dot / lk_q8_term / lk_q8_sum4, and the QWEN38 page's gk_gemv_hl_sk.
//
// What is summed, and in which order, is the page's: block g's step
// p <- fma(a, b, p) goes into partial g mod 4, each partial takes its blocks in
// ascending order starting from +0, and the row is (P0 + P2) + (P1 + P3).  How
// the work maps onto gfx950 is this file's own:
//
//  * A wave64 takes RPW rows at once; each row gets LPR = 64/RPW lanes, a lane
//    pair per 32-value block, so one step of a wave reads LPR*16 contiguous bytes
//    of each of its rows (whole 128-byte lines) with one 16-byte load per lane.
//  * A step covers BPS = LPR/2 consecutive blocks of a row.  Blocks are read in
//    groups of 4 that start at a multiple of 4, so block j of a step belongs to
//    partial j mod 4.  Lanes (2q, 2q+1) of a row own partial q for the whole
//    row: they fold their own block (j = q) and, when BPS = 8, the block j = q+4
//    that the lanes 8 to the right hold (one DPP row shift), in that order.  The
//    chain of every partial therefore stays in one lane pair, in ascending block
//    order, with no reduction tree at all; the pair's lanes hold equal values.
//  * The window of the workgroup's K-chunk -- activation words (TwoPass low
//    words too) and scales, and the weight scales of the workgroup's rows -- is
//    staged in LDS with 16-byte loads; a lane reads its block's activation with
//    one ds_read_b128 and its scales with two small LDS reads.
//  * With four rows a wave (the default) the weights stream through four named
//    one-step buffers (chunk_fold), each refilled four steps ahead, so four
//    steps (4 KiB a wave) stay in flight and the compiler's waits count exactly;
//    the four are requested before the window's barrier.  With eight rows a
//    wave, U steps are issued ahead of the steps being computed through a
//    copy-based double buffer.  Weights are read with the nontemporal hint
//    (streamed once, never re-read).
//  * one workgroup per (row tile, split): the split s of a row covers the QWEN38 chunk
//    [g0, g1) and writes partial[s][o]; an empty chunk writes +0.
//  * QX = true (one launch for a whole projection): the workgroup quantizes its
//    own window of the f32 activation into LDS -- the activation quantizer's
//    routine, eight lanes a block -- instead of copying words quantized by an
//    earlier launch; every workgroup of a chunk quantizes the same blocks, so
//    they all hold the words the quantizer kernel would write, bit for bit.

#include "qdg_device.h"

namespace qdg {
namespace {

constexpr int WG = 256;                // four waves
constexpr int DOT_U = 1, DOT_NB = 4;   // four rows a wave: one-step weight groups, four in flight
constexpr int LDS_BUDGET = 56 * 1024;  // window bytes per workgroup

// LDS bytes per block of the window: activation words (two under TwoPass), the
// activation scale, and the binary16 weight scales of the workgroup's rows.
template <int MODE, int RPW>
constexpr int window_bytes_per_block() { return (MODE == 2 ? 2 : 1) * QK + 4 + 2 * (WG / 64) * RPW; }

// FUSED = false: out receives y (S == 1) or the partials [S][N].
// FUSED = true: with S > 1 the workgroup writes its partials to out, and the
//   last workgroup of a row tile to finish (an atomic ticket per tile) sums the
//   tile's S partials in ascending order into y and resets the ticket -- which
//   chunk finishes last changes nothing in the result.
// AMAX (S == 1 only): the workgroup also writes the arg-max key (amax_key) of
// its rows' largest output to keys[tile]; a final pass over the tiles' keys gives
// the first index of the row's maximum (the megakernel page's per-block arg-max
// partials, in the GEMV's epilogue instead of a pass over the logits).
template <int MODE, int RPW, int U, bool FUSED, bool QX, bool AMAX = false>
__global__ __launch_bounds__(WG) void k_gemv_dot4(const int8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
                                                 const int8_t* __restrict__ xq, const int8_t* __restrict__ xl,
                                                 const float* __restrict__ xs, const float* __restrict__ x,
                                                 int64_t N, int64_t K, int S, int win, int ntiles, int chunk_major,
                                                 float* __restrict__ out, unsigned* __restrict__ tickets,
                                                 float* __restrict__ y, unsigned long long* __restrict__ keys = nullptr) {
  constexpr int LPR = 64 / RPW;  // lanes per row
  constexpr int BPS = LPR / 2;   // blocks per step of a row
  constexpr int TPP = BPS / 4;   // steps of one partial per step (1 or 2)
  constexpr int ROWS = (WG / 64) * RPW;
  static_assert(TPP == 1 || TPP == 2, "RPW must be 4 or 8");
  extern __shared__ __align__(16) unsigned char lds[];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPR, li = lane % LPR, j = li >> 1, hf = li & 1;
  const int64_t nb = K / QK;
  // one workgroup per (row tile, chunk) on a 1-D grid: chunk-major order walks
  // the S chunks of a tile consecutively (neighbouring workgroups read adjacent
  // parts of the same rows, and each XCD sees only a few activation chunks)
  const int tile = chunk_major ? (int)(blockIdx.x / S) : (int)(blockIdx.x % ntiles);
  const int s_idx = chunk_major ? (int)(blockIdx.x % S) : (int)(blockIdx.x / ntiles);
  int32_t g0, g1;
  split_range(K, S, s_idx, g0, g1);

  const int64_t o_wg = (int64_t)tile * ROWS;
  const int rr = wave * RPW + r;  // row within the workgroup
  const int64_t o = o_wg + rr;
  const bool row_ok = o < N;
  const int8_t* wrow = wq + (row_ok ? o : N - 1) * K + hf * 16;

  int8_t* lq = (int8_t*)lds;                                              // [win][32]
  int8_t* ll = lq + (int64_t)win * QK;                                    // [win][32] (TwoPass)
  float* lsx = (float*)(lds + (int64_t)win * (MODE == 2 ? 2 : 1) * QK);  // [win]
  uint16_t* lsg = (uint16_t*)(lsx + win);                                 // [ROWS][win]
  const uint16_t* my_sg = lsg + rr * win;

  float p = 0.0f;  // this lane pair's partial (j < 4)
  for (int wb0 = g0; wb0 < g1; wb0 += win) {
    const int wb1 = min(wb0 + win, g1);
    const int nwb = wb1 - wb0;
    const int nsteps = (nwb + BPS - 1) / BPS;
    const int ngroups = (nsteps + U - 1) / U;
    // the first weights are requested before the window is staged, so the weight
    // stream is already in flight across the barrier: with four rows a wave, the
    // first DOT_NB one-step groups of the named-buffer pipeline (chunk_fold);
    // with eight, the first U steps of the copy-based double buffer
    int4 w[DOT_NB][DOT_U];
    int4 wcur[U];
    if constexpr (RPW == 4) {
#pragma unroll
      for (int k = 0; k < DOT_NB; ++k) group_load<DOT_U>(w[k], wrow, wb0, wb1, k, j);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int b = wb0 + u * BPS + j;
        wcur[u] = b < wb1 ? ld16_stream(wrow + (int64_t)b * QK) : make_int4(0, 0, 0, 0);
      }
    }
    __syncthreads();
    if constexpr (QX) {
      // quantize the window: 8 lanes a block, 4 values a lane; two rounds of
      // loads are in flight before the first is quantized.  The trip count is
      // uniform, so all lanes of every 8-lane group take part in its maximum.
      for (int base = 0; base < nwb * 8; base += 2 * WG) {
        float4 v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = base + h * WG + threadIdx.x;
          v[h] = i < nwb * 8 ? *(const float4*)(x + (int64_t)(wb0 + (i >> 3)) * QK + (i & 7) * 4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = base + h * WG + threadIdx.x;
          int hw, lw;
          const float s = quant_lane4<MODE>(v[h], &hw, &lw);
          if (i < nwb * 8) {
            const int blk = i >> 3, sub = i & 7;
            *(int*)(lq + blk * QK + sub * 4) = hw;
            if constexpr (MODE == 2) *(int*)(ll + blk * QK + sub * 4) = lw;
            if (sub == 0) lsx[blk] = s;
          }
        }
      }
    } else {
      for (int i = threadIdx.x; i < nwb * 2; i += WG) {
        ((int4*)lq)[i] = ld16(xq + (int64_t)wb0 * QK + 16 * i);
        if constexpr (MODE == 2) ((int4*)ll)[i] = ld16(xl + (int64_t)wb0 * QK + 16 * i);
      }
      for (int i = threadIdx.x; i < nwb; i += WG) lsx[i] = xs[wb0 + i];
    }
    stage_scales(lsg, win, ws, nb, N, o_wg, ROWS, wb0, nwb, threadIdx.x, WG);
    __syncthreads();

    if constexpr (RPW == 4) {
      chunk_fold<MODE, DOT_U, DOT_NB>(wrow, lq, ll, lsx, my_sg, (int)wb0, (int)wb1, j, hf, w, p, (int)wb0);
      continue;
    }
    for (int gi = 0; gi < ngroups; ++gi) {
      int4 wnxt[U];
      const bool more = gi + 1 < ngroups;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int b = wb0 + ((gi + 1) * U + u) * BPS + j;
        wnxt[u] = more && b < wb1 ? ld16_stream(wrow + (int64_t)b * QK) : make_int4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int bl = (gi * U + u) * BPS + j;  // block within the window
        const bool ok = bl < nwb;
        const int blc = ok ? bl : 0;
        const int4 a = *(const int4*)(lq + blc * QK + hf * 16);
        const int d = block_dot_pair(wcur[u], a);
        int e = 0;
        if constexpr (MODE == 2) e = block_dot_pair(wcur[u], *(const int4*)(ll + blc * QK + hf * 16));
        float ta, tb;
        q8_term<MODE>(half_bits_to_float(my_sg[blc]), lsx[blc], d, e, ta, tb);
        p = ok ? __fmaf_rn(ta, tb, p) : p;
        if constexpr (TPP == 2) {
          const float ta2 = dpp_f32<DPP_ROW_SHL8>(ta), tb2 = dpp_f32<DPP_ROW_SHL8>(tb);
          p = bl + 4 < nwb ? __fmaf_rn(ta2, tb2, p) : p;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) wcur[u] = wnxt[u];
    }
  }
  // (P0 + P2) + (P1 + P3): partial q sits in lane 2q of the row.
  const float t = __fadd_rn(p, dpp_f32<DPP_ROW_SHL4>(p));
  const float yv = __fadd_rn(t, dpp_f32<DPP_ROW_SHL2>(t));
  if constexpr (AMAX) {
    // one key a row (0, below every real key, for rows past N), the workgroup's maximum to keys[tile]
    __shared__ unsigned long long row_keys[ROWS];
    if (li == 0) {
      if (row_ok) out[o] = yv;
      row_keys[rr] = row_ok ? amax_key(yv, (unsigned)o) : 0ull;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long best = row_keys[0];
#pragma unroll
      for (int i = 1; i < ROWS; ++i) best = row_keys[i] > best ? row_keys[i] : best;
      keys[tile] = best;
    }
    return;
  }
  if constexpr (!FUSED) {
    if (li == 0 && row_ok) out[(int64_t)s_idx * N + o] = yv;
  } else {
    if (S == 1) {
      if (li == 0 && row_ok) y[o] = yv;
      return;
    }
    // Hand the partials to the tile's last-arriving workgroup (publish_partial /
    // take_partial: marked slots, all accesses atomic, no ordering assumed).  The
    // barrier only makes the ticket come after the workgroup's own stores are
    // issued; which chunk arrives last changes nothing in the sum.
    unsigned* slots = (unsigned*)out;
    if (li == 0 && row_ok) publish_partial(slots + (int64_t)s_idx * N + o, yv);
    __syncthreads();
    __shared__ int last_arrival;
    if (threadIdx.x == 0)
      last_arrival = __hip_atomic_fetch_add(&tickets[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (unsigned)(S - 1);
    __syncthreads();
    if (!last_arrival) return;
    if (threadIdx.x < ROWS && o_wg + threadIdx.x < N) {
      const int64_t oo = o_wg + threadIdx.x;
      float a = 0.0f;
      for (int s = 0; s < S; ++s) a = __fadd_rn(a, take_partial(slots + (int64_t)s * N + oo));
      y[oo] = a;
    }
    if (threadIdx.x == 0) __hip_atomic_store(&tickets[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

struct Tuning {
  int rpw = 4;
  int unroll = 4;
  int order = -1;  // -1: by S (chunk-major for S <= 4), 0: tile-major, 1: chunk-major
};

// Tuning knobs for sweeps (QDG_TUNE_GEMV_RPW in {4, 8}, QDG_TUNE_GEMV_UNROLL in
// {2, 4, 8} -- the load depth of the eight-rows-a-wave layout only --,
// QDG_TUNE_GEMV_ORDER 0 tile-major / 1 chunk-major); they change the lane
// layout, load depth and workgroup order only, never the arithmetic or its order.
Tuning tuning() {
  Tuning v;
  const int order = tune(QDG_TUNE_GEMV_ORDER), rpw = tune(QDG_TUNE_GEMV_RPW), u = tune(QDG_TUNE_GEMV_UNROLL);
  if (order >= 0) v.order = order ? 1 : 0;
  if (rpw >= 0) v.rpw = rpw == 8 ? 8 : 4;
  if (u >= 0) v.unroll = (u == 2 || u == 8) ? u : 4;
  return v;
}

// Workgroup order.  Measured on the narrow projections: walking a tile's chunks
// consecutively is 3-6% faster at S = 4 (5120x8192), tiles first 20% faster at
// S = 16 (5120x25600).
int chunk_major(int splits) {
  const int o = tuning().order;
  return o >= 0 ? o : (splits <= 4 ? 1 : 0);
}

int window_blocks(int64_t K, int splits, int bytes_per_block) {
  int32_t mx = 0;
  for (int s = 0; s < splits; ++s) {
    int32_t g0, g1;
    split_range(K, splits, s, g0, g1);
    mx = g1 - g0 > mx ? g1 - g0 : mx;
  }
  const int cap = (LDS_BUDGET / bytes_per_block) / SUPER * SUPER;
  int win = ((mx + SUPER - 1) / SUPER) * SUPER;
  if (win > cap) win = cap;
  if (win < SUPER) win = SUPER;
  return win;
}

template <int MODE, int RPW, int U, bool FUSED, bool QX>
hipError_t launch_t(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq, const int8_t* xl,
                    const float* xs, const float* x, int splits, float* out, unsigned* tickets, float* y,
                    hipStream_t st) {
  constexpr int bpb = window_bytes_per_block<MODE, RPW>();
  const int win = window_blocks(K, splits, bpb);
  const int rows_per_wg = (WG / 64) * RPW;
  const int ntiles = (int)((N + rows_per_wg - 1) / rows_per_wg);
  const dim3 grid((unsigned)((int64_t)ntiles * splits)), block(WG);
  return launch((k_gemv_dot4<MODE, RPW, U, FUSED, QX>), grid, block, (size_t)win * bpb, st, wq, ws, xq, xl, xs,
                     x, N, K, splits, win, ntiles, chunk_major(splits), out, tickets, y, nullptr);
}

template <int MODE, bool FUSED, bool QX>
hipError_t launch_mode(const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq,
                       const int8_t* xl, const float* xs, const float* x, int splits, float* out, unsigned* tickets,
                       float* y, hipStream_t st) {
  const Tuning t = tuning();
#define QDG_LAUNCH(R_, U_) \
  return launch_t<MODE, R_, U_, FUSED, QX>(wq, ws, N, K, xq, xl, xs, x, splits, out, tickets, y, st)
  if (t.rpw == 8) {
    if (t.unroll == 2) QDG_LAUNCH(8, 2);
    if (t.unroll == 8) QDG_LAUNCH(8, 8);
    QDG_LAUNCH(8, 4);
  }
  if (t.unroll == 2) QDG_LAUNCH(4, 2);
  if (t.unroll == 8) QDG_LAUNCH(4, 8);
  QDG_LAUNCH(4, 4);
#undef QDG_LAUNCH
}

}  // namespace

hipError_t launch_gemv_dot4(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K,
                            const int8_t* xq, const int8_t* xl, const float* xs, int splits, float* out,
                            hipStream_t st) {
  if (mode == 1)
    return launch_mode<1, false, false>(wq, ws, N, K, xq, xl, xs, nullptr, splits, out, nullptr, nullptr, st);
  return launch_mode<2, false, false>(wq, ws, N, K, xq, xl, xs, nullptr, splits, out, nullptr, nullptr, st);
}

// Workspace of the in-kernel combine, each part 256-byte aligned: one ticket per
// row tile (room for 16-row tiles), then the split partials [S][N] -- binary32
// for the quantized modes, binary64 for Dequant (sized for the latter).
constexpr int64_t TILE_ROWS = 16;
int64_t pad256(int64_t b) { return (b + 255) / 256 * 256; }
int64_t sk_partials_offset(int64_t N) { return pad256(((N + TILE_ROWS - 1) / TILE_ROWS) * 4); }

size_t sk_workspace_bytes(int64_t N, int splits) {
  return (size_t)(sk_partials_offset(N) + pad256((int64_t)splits * N * 8));
}

hipError_t launch_gemv_sk(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const int8_t* xq,
                          const int8_t* xl, const float* xs, int splits, float* y, void* workspace, hipStream_t st) {
  if (splits == 1) return launch_gemv_dot4(mode, wq, ws, N, K, xq, xl, xs, 1, y, st);
  // the chunks as waves of one workgroup, combined in LDS, where the activation
  // fits (QDG_TUNE_SK_WSPLIT = 0 forces the workspace path)
  if (tune(QDG_TUNE_SK_WSPLIT) != 0 && wsplit_fits(mode, K, splits))
    return launch_gemv_wsplit(mode, wq, ws, N, K, xq, xl, xs, splits, y, st);
  unsigned* tickets = (unsigned*)workspace;
  float* part = (float*)((char*)workspace + sk_partials_offset(N));
  if (mode == 1) return launch_mode<1, true, false>(wq, ws, N, K, xq, xl, xs, nullptr, splits, part, tickets, y, st);
  return launch_mode<2, true, false>(wq, ws, N, K, xq, xl, xs, nullptr, splits, part, tickets, y, st);
}

int64_t gemv_tiles(int64_t N) { return (N + 15) / 16; }

hipError_t launch_gemv_argmax(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                              const int8_t* xq, const int8_t* xl, const float* xs, float* y, int32_t* idx,
                              unsigned long long* keys, hipStream_t st) {
  hipError_t e;
  if (mode == 0) {
    e = launch_gemv_dequant_argmax(wq, ws, N, K, x, y, keys, st);
  } else {
    // the default lane layout (RPW 4, U 4): 16-row tiles, one key each
    constexpr int bpb1 = window_bytes_per_block<1, 4>(), bpb2 = window_bytes_per_block<2, 4>();
    const int win = window_blocks(K, 1, mode == 1 ? bpb1 : bpb2);
    const int ntiles = (int)gemv_tiles(N);
    const dim3 grid((unsigned)ntiles), block(WG);
    const float* nox = nullptr;
    unsigned* not_ = nullptr;
    float* noy = nullptr;
    if (mode == 1)
      e = launch(k_gemv_dot4<1, 4, 4, false, false, true>, grid, block, (size_t)win * bpb1, st, wq, ws, xq, xl, xs,
                 nox, N, K, 1, win, ntiles, 0, y, not_, noy, keys);
    else
      e = launch(k_gemv_dot4<2, 4, 4, false, false, true>, grid, block, (size_t)win * bpb2, st, wq, ws, xq, xl, xs,
                 nox, N, K, 1, win, ntiles, 0, y, not_, noy, keys);
  }
  if (e != hipSuccess) return e;
  return launch_argmax_final(keys, 1, (int)gemv_tiles(N), idx, st);
}

hipError_t launch_gemv_x(int mode, const int8_t* wq, const uint16_t* ws, int64_t N, int64_t K, const float* x,
                         int splits, float* y, void* workspace, hipStream_t st) {
  unsigned* tickets = (unsigned*)workspace;
  float* part = splits == 1 ? y : (float*)((char*)workspace + sk_partials_offset(N));
  if (mode == 1)
    return launch_mode<1, true, true>(wq, ws, N, K, nullptr, nullptr, nullptr, x, splits, part, tickets, y, st);
  return launch_mode<2, true, true>(wq, ws, N, K, nullptr, nullptr, nullptr, x, splits, part, tickets, y, st);
}

}  // namespace qdg
