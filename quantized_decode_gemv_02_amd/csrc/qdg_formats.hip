// qdg_formats.hip -- the batch-1 GEMV of a matrix in another GGUF block format
// (lane kernel library page: module doc on the other formats; BLOCKS, lk_sub
// and its helpers for the layouts; lk_row_dot and lk_sub_dot for the sums).
//
// A 32-weight sub-block decodes to int8 levels with a scale d and an offset c
// per half of 16: weight = d*level + c.
//  * Int8Act / TwoPass: per sub-block, the exact int32 dots of each half with
//    the activation words, dh = sum level*h and sh = sum h (the latter a v_dot4
//    against ones; dl, sl with the low words); part = ((d0*dh0 + c0*sh0) +
//    d1*dh1) + c1*sh1, one rounding per operation; TwoPass adds fl(2^-7 * the
//    same with dl, sl).  The row is the Q8_0 row: p <- fma(s_g, part, p) into
//    partial g mod 4, ascending, then (P0 + P2) + (P1 + P3).
//  * Dequant: each weight fl(fl(d*level) + c), its products with x and their
//    sums in binary64 (a sub-block's half in four chains; where c = 0 the
//    half's scale applied once to its level-times-x sum, d*level being exact;
//    then the row's partials as above), one rounding to binary32.
// A format whose levels carry a constant offset (Q4_0: nibble - 8, Q5_0: - 16,
// Q3_K: - 4, Q6_K: - 32) is dotted on its raw unsigned levels and corrected by
// the offset times the activation sum, which is the same integer.
//
// Mapping: a wave takes 4 rows, 16 lanes a row, one sub-block a lane, so a
// step covers 16 consecutive sub-blocks of a row (two super-blocks of the
// K-quants).  Lane j < 4 of a row owns partial j: it folds its own sub-block,
// then those of lanes j + 4, j + 8 and j + 12 (DPP row shifts).  Each step's
// bytes are staged in the wave's LDS slot by aligned 16-byte loads, a step
// ahead.  Split-K (the QWEN38 page's chunk rule, gk_gemv_hl_sk /
// gk_sk_combine): the chunks are summed by the waves of one workgroup, each
// wave taking one or more in turn, and their partials are added in ascending
// order in LDS.

#include <atomic>

#include "qdg_device.h"

namespace qdg {
namespace {

enum : int {
  F_Q4_0 = 2, F_Q4_1 = 3, F_Q5_0 = 6, F_Q5_1 = 7, F_Q2_K = 10, F_Q3_K = 11, F_Q4_K = 12,
  F_Q5_K = 13, F_Q6_K = 14, F_IQ4_NL = 20, F_IQ4_XS = 23, F_MXFP4 = 39
};
constexpr int DPP_ROW_SHL1 = 0x101;

// GGUF geometry: values per block and bytes per block.
template <int F>
struct Geo;
template <> struct Geo<F_Q4_0> { static constexpr int V = 32, B = 18; };
template <> struct Geo<F_Q4_1> { static constexpr int V = 32, B = 20; };
template <> struct Geo<F_Q5_0> { static constexpr int V = 32, B = 22; };
template <> struct Geo<F_Q5_1> { static constexpr int V = 32, B = 24; };
template <> struct Geo<F_IQ4_NL> { static constexpr int V = 32, B = 18; };
template <> struct Geo<F_MXFP4> { static constexpr int V = 32, B = 17; };
template <> struct Geo<F_Q2_K> { static constexpr int V = 256, B = 84; };
template <> struct Geo<F_Q3_K> { static constexpr int V = 256, B = 110; };
template <> struct Geo<F_Q4_K> { static constexpr int V = 256, B = 144; };
template <> struct Geo<F_Q5_K> { static constexpr int V = 256, B = 176; };
template <> struct Geo<F_Q6_K> { static constexpr int V = 256, B = 210; };
template <> struct Geo<F_IQ4_XS> { static constexpr int V = 256, B = 136; };

__device__ __forceinline__ unsigned ld_u8(const uint8_t* p) { return *p; }
__device__ __forceinline__ unsigned ld_u16(const uint8_t* p) { return *(const unsigned short*)p; }
__device__ __forceinline__ unsigned ld_u32(const uint8_t* p) { return *(const unsigned*)p; }
__device__ __forceinline__ float h16(unsigned bits) { return half_bits_to_float((unsigned short)(bits & 0xffff)); }

// n dwords from p (in the wave's LDS slot) at any alignment.  REALIGN: the
// n + 1 aligned dwords that hold them, realigned by byte shifts (v_alignbyte);
// the extra dword is read only when p is misaligned, and then holds the last
// bytes wanted, so no read leaves the block.  Otherwise one byte copy, which
// the compiler turns into multi-dword reads at p's alignment.  The hardware
// splits a misaligned multi-dword LDS read into many accesses: the super-blocks
// of Q3_K (110 bytes) and Q6_K (210) decoded at the speed of those splits, and
// the realigned reads cut their GEMV from 40 to 27 and from 39 to 29 us on
// 5120x25600; on the 32-value blocks (17-22 bytes, fewer words a lane) the
// byte copy is 3-6% faster.
template <int NW, bool REALIGN = false>
__device__ __forceinline__ void ld_words(const uint8_t* p, unsigned* w) {
  if constexpr (REALIGN) {
    const unsigned mis = (unsigned)(uintptr_t)p & 3u;
    const unsigned* a = (const unsigned*)(p - mis);  // pointer arithmetic keeps the LDS address space
    unsigned d[NW + 1];
#pragma unroll
    for (int i = 0; i < NW; ++i) d[i] = a[i];
    d[NW] = a[mis ? NW : NW - 1];
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = __builtin_amdgcn_alignbyte(d[i + 1], d[i], mis);
  } else {
    __builtin_memcpy(w, p, 4 * NW);
  }
}

// A funnel window on the n dwords at p (in the wave's LDS slot): n + 1 aligned
// dwords d and a shift sh such that alignbit(d[i+1], d[i], sh) is dword i at p
// shifted right by `off` bits (-8 < off < 8: a field's place within each byte,
// negative to move it up) -- the realignment and the field's shift in one
// v_alignbit.  The total shift 8*mis + off is negative only for an aligned p and
// off < 0; then the window starts one dword early (p - 4: the slots sit 16
// bytes above the start of LDS, so that dword is always in the allocation) and
// shifts by 32 + off.  The last dword is read only when it holds wanted bytes.
template <int NW>
__device__ __forceinline__ unsigned ld_funnel(const uint8_t* p, int off, unsigned (&d)[NW + 1]) {
  const unsigned mis = (unsigned)(uintptr_t)p & 3u;
  const int s = 8 * (int)mis + off;
  const unsigned* a = (const unsigned*)(p - mis - (s < 0 ? 4 : 0));  // pointer arithmetic keeps the LDS address space
#pragma unroll
  for (int i = 0; i < NW; ++i) d[i] = a[i];
  d[NW] = a[(mis != 0 || s < 0) ? NW : NW - 1];
  return (unsigned)s & 31u;
}

// The low nibbles of a word's four bytes and the high ones, as bytes.
__device__ __forceinline__ unsigned lo_nib(unsigned q) { return q & 0x0f0f0f0fu; }
__device__ __forceinline__ unsigned hi_nib(unsigned q) { return (q >> 4) & 0x0f0f0f0fu; }

// Four nibbles (one a byte) mapped through a 16-entry int8 table held four
// entries a word (t[0] entries 0-3 ... t[3] 12-15), by byte permutes: the low
// three bits select within entries 0-7 and within 8-15, the fourth bit between.
__device__ __forceinline__ unsigned table16(unsigned nib, const unsigned (&t)[4]) {
  // v_perm_b32(a, b, sel): selector byte k < 4 picks byte k of b, 4..7 byte k-4 of a
  const unsigned sel = nib & 0x07070707u;
  const unsigned lo = __builtin_amdgcn_perm(t[1], t[0], sel);
  const unsigned hi = __builtin_amdgcn_perm(t[3], t[2], sel);
  const unsigned m = ((nib >> 3) & 0x01010101u) * 0xffu;  // 0xff in the bytes whose nibble is >= 8
  return (lo & ~m) | (hi & m);
}

// IQ4's sixteen levels and MXFP4's doubled E2M1 values, four to a word (little-endian).
__device__ __forceinline__ void iq4_table(unsigned (&t)[4]) {
  t[0] = 0xBFAD9881u; t[1] = 0xF6EADDCFu; t[2] = 0x26190D01u; t[3] = 0x71594535u;
}
__device__ __forceinline__ void e2m1_table(unsigned (&t)[4]) {
  t[0] = 0x03020100u; t[1] = 0x0C080604u; t[2] = 0xFDFEFF00u; t[3] = 0xF4F8FAFCu;
}

// The five-bit levels' fifth bits: bit i (i < 4) of x to bit 4 of byte i.
__device__ __forceinline__ unsigned spread4(unsigned x) {
  return ((x & 1u) | ((x & 2u) << 7) | ((x & 4u) << 14) | ((x & 8u) << 21)) << 4;
}

// One decoded sub-block: raw int8 levels, four a word, level = raw - off; the
// scale d and offset c of each half.
struct Sub {
  unsigned w[8];
  int off;
  float d[2], c[2];
};

// One sub-block (lane kernel library page, lk_sub: the same layouts): b is its
// 32-value block, or for the K-quants and IQ4_XS its 256-value super-block with
// the sub-block at position j (0-7).
template <int F>
__device__ __forceinline__ void decode(const uint8_t* __restrict__ b, int j, Sub& s) {
  s.off = 0;
  s.c[0] = s.c[1] = 0.0f;
  if constexpr (F == F_Q4_0 || F == F_IQ4_NL || F == F_Q4_1) {
    unsigned q[4];
    if constexpr (F == F_Q4_1) {
      const unsigned hd = ld_u32(b);
      s.d[0] = s.d[1] = h16(hd);
      s.c[0] = s.c[1] = h16(hd >> 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = ld_u32(b + 4 + 4 * i);
    } else {
      s.d[0] = s.d[1] = h16(ld_u16(b));
      ld_words<4>(b + 2, q);
    }
    if constexpr (F == F_IQ4_NL) {
      unsigned t[4];
      iq4_table(t);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s.w[i] = table16(lo_nib(q[i]), t);
        s.w[4 + i] = table16(hi_nib(q[i]), t);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s.w[i] = lo_nib(q[i]);
        s.w[4 + i] = hi_nib(q[i]);
      }
      if constexpr (F == F_Q4_0) s.off = 8;
    }
  } else if constexpr (F == F_Q5_0 || F == F_Q5_1) {
    unsigned qh, q[4];
    if constexpr (F == F_Q5_1) {
      const unsigned hd = ld_u32(b);
      s.d[0] = s.d[1] = h16(hd);
      s.c[0] = s.c[1] = h16(hd >> 16);
      qh = ld_u32(b + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = ld_u32(b + 8 + 4 * i);
    } else {
      s.d[0] = s.d[1] = h16(ld_u16(b));
      ld_words<1>(b + 2, &qh);
      ld_words<4>(b + 6, q);
      s.off = 16;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s.w[i] = lo_nib(q[i]) | spread4((qh >> (4 * i)) & 15u);
      s.w[4 + i] = hi_nib(q[i]) | spread4((qh >> (16 + 4 * i)) & 15u);
    }
  } else if constexpr (F == F_MXFP4) {
    const unsigned e = ld_u8(b);
    const unsigned bits = e < 2 ? (0x00200000u << e) : ((e - 1) << 23);  // 2^(e - 128)
    s.d[0] = s.d[1] = __uint_as_float(bits);
    unsigned t[4];
    e2m1_table(t);
    unsigned q[4];
    ld_words<4>(b + 1, q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s.w[i] = table16(lo_nib(q[i]), t);
      s.w[4 + i] = table16(hi_nib(q[i]), t);
    }
  } else if constexpr (F == F_Q4_K || F == F_Q5_K) {
    const int pair = j >> 1, upper = j & 1;
    const int4 hd = *(const int4*)b;  // d, dmin, 12 scale bytes
    const unsigned sw[3] = {(unsigned)hd.y, (unsigned)hd.z, (unsigned)hd.w};
    auto sbyte = [&](int i) { return (sw[i >> 2] >> (8 * (i & 3))) & 255u; };
    int sc, mn;
    if (j < 4) {
      sc = (int)(sbyte(j) & 63);
      mn = (int)(sbyte(j + 4) & 63);
    } else {
      sc = (int)((sbyte(j + 4) & 15) | ((sbyte(j - 4) >> 6) << 4));
      mn = (int)((sbyte(j + 4) >> 4) | ((sbyte(j) >> 6) << 4));
    }
    s.d[0] = s.d[1] = __fmul_rn(h16((unsigned)hd.x), (float)sc);
    s.c[0] = s.c[1] = -__fmul_rn(h16((unsigned)hd.x >> 16), (float)mn);
    const uint8_t* ql = b + (F == F_Q4_K ? 16 : 48) + 32 * pair;
    const int4 a0 = *(const int4*)ql, a1 = *(const int4*)(ql + 16);
    const unsigned q[8] = {(unsigned)a0.x, (unsigned)a0.y, (unsigned)a0.z, (unsigned)a0.w,
                           (unsigned)a1.x, (unsigned)a1.y, (unsigned)a1.z, (unsigned)a1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) s.w[i] = upper ? hi_nib(q[i]) : lo_nib(q[i]);
    if constexpr (F == F_Q5_K) {
      const int4 h0 = *(const int4*)(b + 16), h1 = *(const int4*)(b + 32);
      const unsigned qh[8] = {(unsigned)h0.x, (unsigned)h0.y, (unsigned)h0.z, (unsigned)h0.w,
                              (unsigned)h1.x, (unsigned)h1.y, (unsigned)h1.z, (unsigned)h1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) s.w[i] |= ((qh[i] >> j) & 0x01010101u) << 4;
    }
  } else if constexpr (F == F_Q6_K) {
    const int half = j >> 2, k = j & 3;
    unsigned qd[9], hd[9];
    // the nibble (low for k < 2, high otherwise) of each level byte to bits 0-3,
    // and bits 2k, 2k+1 of each high byte to bits 4, 5
    const unsigned nsh = ld_funnel<8>(b + 64 * half + 32 * (k & 1), 4 * (k >> 1), qd);
    const unsigned hsh = ld_funnel<8>(b + 128 + 32 * half, 2 * k - 4, hd);
    const unsigned scw = ld_u16(b + 192 + 8 * half + 2 * k);
    const float dd = h16(ld_u16(b + 208));
    s.d[0] = __fmul_rn(dd, (float)(int)(signed char)(scw & 255));
    s.d[1] = __fmul_rn(dd, (float)(int)(signed char)(scw >> 8));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      s.w[i] = (__builtin_amdgcn_alignbit(qd[i + 1], qd[i], nsh) & 0x0f0f0f0fu) |
               (__builtin_amdgcn_alignbit(hd[i + 1], hd[i], hsh) & 0x30303030u);
    s.off = 32;
  } else if constexpr (F == F_Q2_K) {
    const int half = j >> 2, k = j & 3;  // b 4-byte aligned: 84 is a multiple of 4
    unsigned q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = ld_u32(b + 16 + 32 * half + 4 * i);
    const unsigned scw = ld_u16(b + 8 * half + 2 * k);
    const unsigned dw = ld_u32(b + 80);
    const float dd = h16(dw), dm = h16(dw >> 16);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const unsigned sc = (scw >> (8 * h)) & 255u;
      s.d[h] = __fmul_rn(dd, (float)(sc & 15u));
      s.c[h] = -__fmul_rn(dm, (float)(sc >> 4));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) s.w[i] = (q[i] >> (2 * k)) & 0x03030303u;
  } else if constexpr (F == F_Q3_K) {
    const int half = j >> 2, k = j & 3;
    unsigned hd[9], qd[9];
    // bit 4*half + k (the sub-block's) of each high-mask byte to bit 2, and bits
    // 2k, 2k+1 of each level byte to bits 0, 1
    const unsigned hsh = ld_funnel<8>(b, 4 * half + k - 2, hd);
    const unsigned qsh = ld_funnel<8>(b + 32 + 32 * half, 2 * k, qd);
    // the 16 six-bit scales: scale i = low nibble of byte i & 7 (shifted by
    // 4*(i >> 3)) | bits 2*(i >> 2) of byte 8 + (i & 3) as its top two bits;
    // the lane's two, i = 8*half + 2*k + h, sit in the byte pairs 2k, 2k+1 and
    // 8 + 2(k & 1), +1 (the fields are 2-byte aligned)
    const unsigned lo16 = ld_u16(b + 96 + 2 * k), hi16 = ld_u16(b + 104 + 2 * (k & 1));
    const float dd = h16(ld_u16(b + 108));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const unsigned lo4 = (lo16 >> (8 * h + 4 * half)) & 15u;
      const unsigned hi2 = (hi16 >> (8 * h + 2 * (2 * half + (k >> 1)))) & 3u;
      s.d[h] = __fmul_rn(dd, (float)((int)(lo4 | (hi2 << 4)) - 32));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      s.w[i] = (__builtin_amdgcn_alignbit(qd[i + 1], qd[i], qsh) & 0x03030303u) |
               (__builtin_amdgcn_alignbit(hd[i + 1], hd[i], hsh) & 0x04040404u);
    s.off = 4;  // level = low2 - 4 + 4*high bit
  } else if constexpr (F == F_IQ4_XS) {
    const int ib = j;  // b 8-byte aligned
    const unsigned h0 = ld_u32(b), h1 = ld_u32(b + 4);
    const unsigned sh = h0 >> 16, sl = (h1 >> (8 * (ib >> 1))) & 255u;
    const int ls = (int)((sl >> (4 * (ib & 1))) & 15u) | (int)(((sh >> (2 * ib)) & 3u) << 4);
    s.d[0] = s.d[1] = __fmul_rn(h16(h0), (float)(ls - 32));
    unsigned t[4];
    iq4_table(t);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned q = ld_u32(b + 8 + 16 * ib + 4 * i);
      s.w[i] = table16(lo_nib(q), t);
      s.w[4 + i] = table16(hi_nib(q), t);
    }
  }
}

// Formats whose halves carry an offset c.
template <int F>
constexpr bool has_offsets() {
  return F == F_Q4_1 || F == F_Q5_1 || F == F_Q2_K || F == F_Q4_K || F == F_Q5_K;
}
// Formats that need the activation sums sh: an offset c, or levels dotted raw
// and corrected by a constant.
template <int F>
constexpr bool needs_sums() {
  return has_offsets<F>() || F == F_Q4_0 || F == F_Q5_0 || F == F_Q3_K || F == F_Q6_K;
}

// The activation sums of a sub-block's two halves (sh0, sh1): each half's
// four words dotted with ones.  Each lane forms them for its own sub-block (a
// wave's four rows repeat them): forming them once per wave into LDS measured
// 5-15% slower, its registers and LDS reads costing more than the dots.
__device__ __forceinline__ int2 act_sums(const int (&a)[8]) {
  int s0 = 0, s1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s0 = __builtin_amdgcn_sdot4(0x01010101, a[i], s0, false);
    s1 = __builtin_amdgcn_sdot4(0x01010101, a[4 + i], s1, false);
  }
  return make_int2(s0, s1);
}

// part = ((d0*dh0 + c0*sh0) + d1*dh1) + c1*sh1 with the activation words a[8]
// and their half sums sh (for the formats that need them).
// Where c = 0 and the levels are signed (IQ4_NL, IQ4_XS, MXFP4) the c terms are
// left out: each is a zero, which can change only the sign of a zero part, and
// fma(s, +-0, p) is p for every p the row can hold (it starts at +0 and a sum
// of nonzero terms that cancels rounds to +0), so the row's bits are the same.
template <int F>
__device__ __forceinline__ float sub_part(const Sub& s, const int (&a)[8], int2 sh) {
  int dh0 = 0, dh1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dh0 = __builtin_amdgcn_sdot4((int)s.w[i], a[i], dh0, false);
    dh1 = __builtin_amdgcn_sdot4((int)s.w[4 + i], a[4 + i], dh1, false);
  }
  if constexpr (!needs_sums<F>()) return __fadd_rn(__fmul_rn(s.d[0], (float)dh0), __fmul_rn(s.d[1], (float)dh1));
  const int sh0 = sh.x, sh1 = sh.y;
  dh0 -= s.off * sh0;
  dh1 -= s.off * sh1;
  float part = __fmul_rn(s.d[0], (float)dh0);
  part = __fadd_rn(part, __fmul_rn(s.c[0], (float)sh0));
  part = __fadd_rn(part, __fmul_rn(s.d[1], (float)dh1));
  return __fadd_rn(part, __fmul_rn(s.c[1], (float)sh1));
}

// The activation of one 32-value block in registers: Dequant's 32 binary32
// values, or the quantized modes' words (h, and l under TwoPass) and scale.
template <int MODE>
struct Act {
  int a[8], l[8];
  float s;
  int2 sh, sl;  // half sums of a and of l (formats that need them)
};
template <>
struct Act<0> {
  float4 x[8];
};

template <int MODE>
__device__ __forceinline__ void load_act(int gc, const float* __restrict__ x, const int8_t* __restrict__ xq,
                                         const int8_t* __restrict__ xl, const float* __restrict__ xs, Act<MODE>& A) {
  // 32-bit offsets (K < 2^31): a scalar base plus a lane offset, no 64-bit address arithmetic
  const unsigned e = (unsigned)gc * QK;
  if constexpr (MODE == 0) {
    const float4* xv = (const float4*)(x + e);
#pragma unroll
    for (int q4 = 0; q4 < 8; ++q4) A.x[q4] = xv[q4];
  } else {
    const int4 a0 = *(const int4*)(xq + e), a1 = *(const int4*)(xq + e + 16u);
    A.a[0] = a0.x; A.a[1] = a0.y; A.a[2] = a0.z; A.a[3] = a0.w; A.a[4] = a1.x; A.a[5] = a1.y; A.a[6] = a1.z; A.a[7] = a1.w;
    if constexpr (MODE == 2) {
      const int4 b0 = *(const int4*)(xl + e), b1 = *(const int4*)(xl + e + 16u);
      A.l[0] = b0.x; A.l[1] = b0.y; A.l[2] = b0.z; A.l[3] = b0.w; A.l[4] = b1.x; A.l[5] = b1.y; A.l[6] = b1.z; A.l[7] = b1.w;
    }
    A.s = xs[(unsigned)gc];
  }
}

// A sub-block (decoded from b, j) against its activation: Dequant's binary64
// sum of its 32 products (ta), or the quantized modes' scale (ta) and part (tb).
template <int F, int MODE, typename Acc>
__device__ __forceinline__ void sub_term(const uint8_t* __restrict__ b, int j, const Act<MODE>& A, Acc& ta, Acc& tb) {
  Sub s;
  decode<F>(b, j, s);
  if constexpr (MODE == 0) {
    // four binary64 chains (products i mod 4, ascending), then (c0 + c2) + (c1 + c3)
    // per half; any fixed binary64 order meets the Dequant tolerance
    double h[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      double c4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 xv = A.x[4 * half + q4];
        const float xe[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * half + 4 * q4 + e;
          const int lvl = (int)(signed char)((s.w[i >> 2] >> (8 * (i & 3))) & 255u) - s.off;
          if constexpr (has_offsets<F>()) {
            const float wt = __fadd_rn(__fmul_rn(s.d[half], (float)lvl), s.c[half]);
            c4[e] = __fma_rn((double)wt, (double)xe[e], c4[e]);
          } else {
            c4[e] = __fma_rn((double)lvl, (double)xe[e], c4[e]);  // the scale is applied per half below
          }
        }
      }
      h[half] = __dadd_rn(__dadd_rn(c4[0], c4[2]), __dadd_rn(c4[1], c4[3]));
    }
    if constexpr (has_offsets<F>()) {
      ta = __dadd_rn(h[0], h[1]);
    } else {
      // c = 0: every weight fl(d*level) is d*level exactly (at most 23 significant
      // bits in every such format), so d factors out of the half's products
      ta = __fma_rn((double)s.d[0], h[0], __dmul_rn((double)s.d[1], h[1]));
    }
    tb = 0.0;
  } else {
    float part = sub_part<F>(s, A.a, A.sh);
    if constexpr (MODE == 2) part = __fadd_rn(part, __fmul_rn(0.0078125f, sub_part<F>(s, A.l, A.sl)));
    ta = A.s;
    tb = part;
  }
}

// A wave's geometry: ROWS rows of LPR = 64/ROWS lanes, one sub-block a lane,
// so a step covers LPR consecutive sub-blocks of each row (LPR/8 super-blocks
// of the K-quants); the row's step bytes and the 16-byte pieces that cover
// them at any offset.
template <int F, int ROWS>
struct Seg {
  static constexpr bool SUP = Geo<F>::V == 256;
  static constexpr int LPR = 64 / ROWS;
  static constexpr int L = SUP ? LPR / 8 * Geo<F>::B : LPR * Geo<F>::B;
  static constexpr int CPR = (L + 30) / 16;
  static constexpr int NCH = ROWS * CPR;  // weight pieces a wave stages a step
};

// The wave slots start 16 bytes into the workgroup's LDS, so that a funnel
// window that starts a dword before a field (ld_funnel) stays in the allocation.
constexpr int SLOT_BASE = 16;

// A wave's LDS slot for one step: the rows' weight pieces, then under Dequant
// the step's activation (LPR sub-blocks of 32 binary32 values, 8 pieces each).
// The quantized modes read their activation words and scales from global
// memory instead (L1/L2-resident): measured on the 5120-row projections,
// staging them too left Int8Act unchanged and made TwoPass 5-15% slower (a
// third load a lane a step), while Dequant, whose activation is four times
// larger, gains 25-30%.
template <int F, int MODE, int ROWS>
struct Stage {
  using G = Seg<F, ROWS>;
  static constexpr bool ACT = MODE == 0;            // activation staged with the weights
  static constexpr int NA = ACT ? 8 * G::LPR : 0;
  static constexpr int NT = G::NCH + NA;           // pieces a step
  static constexpr int NPL = (NT + 63) / 64;       // loads a lane a step
  static constexpr int SLOT = NT * 16;
  // 16 chunk waves' slots and the partials of QDG_MAX_SPLITS chunks stay within
  // the 64 KiB a launch gets without raising the kernel's LDS limit
  static_assert(SLOT_BASE + 16 * SLOT + QDG_MAX_SPLITS * ROWS * 8 <= 65536, "LDS of a 16-wave workgroup");
};

// The 16 bytes at w + a with those at or past `total` read as 0 (a < total),
// in two halves so that every piece is one 16-byte load: piece_addr gives the
// load's offset -- a, or for the last piece of a matrix whose size is not a
// multiple of 16 the 16 bytes that end at `total` (every matrix holds at least
// 17) -- and the count of bytes to drop from its bottom; piece_fix drops them.
__device__ __forceinline__ int64_t piece_addr(int64_t a, int64_t total, int& sh) {
  const bool tail = a + 16 > total;
  sh = tail ? (int)(16 - (total - a)) : 0;
  return tail ? total - 16 : a;
}
__device__ __forceinline__ uint4 piece_fix(uint4 t, int sh) {
  if (sh == 0) return t;
  uint64_t lo = (uint64_t)t.x | ((uint64_t)t.y << 32), hi = (uint64_t)t.z | ((uint64_t)t.w << 32);
  if (sh >= 8) {
    lo = sh == 8 ? hi : hi >> (8 * (sh - 8));
    hi = 0;
  } else {
    lo = (lo >> (8 * sh)) | (hi << (64 - 8 * sh));
    hi >>= 8 * sh;
  }
  return make_uint4((unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi, (unsigned)(hi >> 32));
}

constexpr int DPP_ROW_SHL12 = 0x10C;

// A workgroup: R row groups of ROWS rows times W chunk waves a group.  The
// non-empty chunks of the S-chunk split rule (S = 1: the whole row), ceff of
// them, go to the group's waves in turn: wave w sums chunks w, w + W, ... one
// after another, each from +0 into its own partial (W = ceff: a wave a chunk).
// The chunk partials meet in LDS and a thread per row adds them in ascending
// chunk order from 0 (empty chunks, whose partial is +0, skipped).
// Each step the wave copies its rows' bytes for the step into its own LDS slot
// with aligned 16-byte loads (issued one step ahead), and the lanes decode their
// sub-blocks from there; the LDS copy keeps every byte's address mod 16, so the
// decoders' alignment holds.  The quantized modes read the activation straight
// from global memory (L1/L2-resident; the rows of a wave share each
// sub-block's); Dequant's travels with the weight pieces into the slot.
// Lane j < 4 of a row owns partial j (blocks g = j mod 4): it folds its own
// sub-block, then those of lanes j + 4, j + 8, j + 12 (DPP row shifts), so each
// partial takes its blocks in ascending order.
template <int F, int MODE, int ROWS, int R>
__global__ __launch_bounds__(1024) void k_gemv_fmt(const uint8_t* __restrict__ w, int64_t rb, int64_t N, int64_t total,
                                                   const float* __restrict__ x, const int8_t* __restrict__ xq,
                                                   const int8_t* __restrict__ xl, const float* __restrict__ xs,
                                                   int64_t K, int S, int m, int ceff, float* __restrict__ y) {
  using Acc = typename std::conditional<MODE == 0, double, float>::type;
  using G = Seg<F, ROWS>;
  using T = Stage<F, MODE, ROWS>;
  constexpr bool SUP = G::SUP;
  constexpr int B = Geo<F>::B, LPR = G::LPR, CPR = G::CPR, NCH = G::NCH, NT = T::NT, NPL = T::NPL;
  extern __shared__ uint4 lds_dyn[];  // [waves] slots, then the chunk partials [R][ceff][ROWS]
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nwaves = blockDim.x >> 6;
  uint8_t* slot = (uint8_t*)lds_dyn + SLOT_BASE + wave * T::SLOT;
  uint4* lw = (uint4*)slot;
  Acc* lpart = (Acc*)((uint8_t*)lds_dyn + SLOT_BASE + nwaves * T::SLOT);
  const int W = nwaves / R;  // chunk waves a row group
  const int rg = wave / W, cw = wave % W;
  const int r = lane / LPR, j = lane % LPR;
  const int64_t o_wg = (int64_t)blockIdx.x * (ROWS * R);
  const int64_t o = o_wg + ROWS * rg + r;
  const int64_t myrow = (o < N ? o : N - 1) * rb;
  // chunk c of the wave's list: chunks 0..m-1, then S-1 (the tail chunk); every
  // one of them holds at least one sub-block
  const int nq = (int)(K >> 9), nb = (int)(K / QK), per = (nq + S - 1) / S;  // K < 2^31
  auto range = [&](int c, int32_t& a, int32_t& b) { split_range32(nq, nb, per, S, c < m ? c : S - 1, a, b); };
  int c = cw;
  int32_t g0, g1;
  range(c, g0, g1);

  auto seg_off = [&](int st) -> int64_t { return SUP ? (int64_t)(st >> 3) * B : (int64_t)st * B; };
  auto seg_len = [&](int st, int32_t ge) -> int {
    const int n = ge - st < LPR ? ge - st : LPR;  // sub-blocks of the step (whole super-blocks for SUP)
    return SUP ? (n >> 3) * B : n * B;
  };
  // A fetch: piece t = lane + 64k is weight piece t % CPR of row t / CPR
  // (t < NCH), or under Dequant activation piece t - NCH (t < NT).  The next
  // step's fetch (the first of the wave's next chunk after a chunk's last step)
  // is issued before this step is summed.  Every fetch issues the
  // same loads whatever the step, so no load sits behind a branch.  A piece's
  // row base is fixed for the launch; away from the matrix end (a scalar test
  // on the wave's last row) every piece is simply the 16 bytes at the row's
  // step offset plus 16*pc -- bytes past the step's are loaded and never
  // decoded -- and only a step that reaches the matrix end takes the clamped
  // form (pieces past the chunk's sub-blocks reread a valid piece; the last
  // piece of a matrix whose size is not a multiple of 16 is shifted into place).
  // pbase[k]: w + the piece's row start + 16*pc, so that a plain step's piece
  // is the 16 bytes at (pbase[k] + step offset) rounded down to 16 (w is
  // 16-byte aligned).
  uintptr_t pbase[NPL];
  int pcs[NPL];
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int t = lane + 64 * k;
    const int tw = t < NCH ? t : 0;
    const int64_t po = o_wg + ROWS * rg + tw / CPR;
    pcs[k] = tw % CPR;
    pbase[k] = (uintptr_t)w + (uintptr_t)((po < N ? po : N - 1) * rb) + 16u * (unsigned)pcs[k];
  }
  // Steps st <= st_plain are plain: the wave's highest row (its pieces reach
  // furthest) keeps all CPR pieces inside the matrix, i.e. its step offset
  // rounded down to 16 plus 16*CPR is at most total.
  const int64_t last_row = o_wg + ROWS * rg + ROWS - 1 < N ? o_wg + ROWS * rg + ROWS - 1 : N - 1;
  int32_t st_plain;
  {
    const int64_t room = total - 16 * CPR + 16 - last_row * rb;  // plain iff seg_off(st) < room
    const int64_t units = room <= 0 ? 0 : (room + B - 1) / B;   // segments (blocks or super-blocks) below room
    st_plain = (int32_t)((SUP ? 8 * units : units) - 1 < INT32_MAX ? (SUP ? 8 * units : units) - 1 : INT32_MAX);
  }
  uint4 v[NPL];
  int vsh[NPL];
  bool fixed = false;  // whether the fetch in v took the clamped form (wave-uniform)
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) const v4u gv4u;
  auto fetch = [&](int st, int32_t ge) {  // ge: the end of st's chunk
    const bool plain = st <= st_plain;
    fixed = !plain;
    const uintptr_t soff = (uintptr_t)seg_off(st);
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int t = lane + 64 * k;
      const bool wpiece = t < NCH || t >= NT;
      int sh = 0;
      const gv4u* src;
      if (plain) {
        src = (const gv4u*)((pbase[k] + soff) & ~(uintptr_t)15);
      } else {
        const int pc = pcs[k];
        const int64_t so = (int64_t)(pbase[k] - (uintptr_t)w) - 16 * pc + (int64_t)soff;  // row start + step offset
        const bool need = t < NCH && 16 * pc < (int)(so & 15) + seg_len(st, ge);
        src = (const gv4u*)(w + piece_addr((so & ~(int64_t)15) + (need ? 16 * pc : 0), total, sh));
      }
      if (!wpiece) {
        const int i = t - NCH;
        const int sb = st + (i >> 3);
        src = (const gv4u*)((const uint8_t*)(x + (int64_t)(sb < ge ? sb : st) * QK) + 16 * (i & 7));
        sh = 0;
      }
      vsh[k] = sh;
      v4u tt;
      if (64 * k + 63 < NCH) {  // a constant once the loop is unrolled
        tt = __builtin_nontemporal_load(src);  // weights only: streamed once
      } else {
        tt = *src;
      }
      v[k] = make_uint4(tt[0], tt[1], tt[2], tt[3]);
    }
  };
  fetch(g0, g1);

  // One step's terms.  FULL: the step's LPR sub-blocks all lie in the chunk, so
  // every lane's own term and the three it folds from lanes j + 4, j + 8, j + 12
  // are taken without a test (lanes j >= 4 fold values that are never used);
  // the chunk's last step, when partial, tests each one.
  Acc p = 0;
  auto terms = [&](int st, auto full) {
    constexpr bool FULL = decltype(full)::value;
    const int g = st + j;  // this lane's sub-block
    const bool ok = FULL || g < g1;
    const int jj = ok ? j : 0;
    Act<MODE> A;
    if constexpr (T::ACT) {
      const float4* xa = (const float4*)(slot + 16 * NCH + 128 * jj);
#pragma unroll
      for (int q4 = 0; q4 < 8; ++q4) A.x[q4] = xa[q4];
    } else {
      load_act<MODE>(ok ? g : st, x, xq, xl, xs, A);
      if constexpr (needs_sums<F>()) {
        A.sh = act_sums(A.a);
        if constexpr (MODE == 2) A.sl = act_sums(A.l);
      }
    }
    const uint8_t* seg = slot + 16 * r * CPR + (int)((myrow + seg_off(st)) & 15);
    Acc ta, tb;
    sub_term<F, MODE>(SUP ? seg + (jj >> 3) * B : seg + jj * B, jj & 7, A, ta, tb);
    if constexpr (MODE == 0) {
      p = ok ? __dadd_rn(p, ta) : p;
      const double t4 = dpp_f64<DPP_ROW_SHL4>(ta);
      p = FULL || g + 4 < g1 ? __dadd_rn(p, t4) : p;
      if constexpr (LPR == 16) {
        const double t8 = dpp_f64<DPP_ROW_SHL8>(ta), t12 = dpp_f64<DPP_ROW_SHL12>(ta);
        p = FULL || g + 8 < g1 ? __dadd_rn(p, t8) : p;
        p = FULL || g + 12 < g1 ? __dadd_rn(p, t12) : p;
      }
    } else {
      p = ok ? __fmaf_rn(ta, tb, p) : p;
      const float a4 = dpp_f32<DPP_ROW_SHL4>(ta), b4 = dpp_f32<DPP_ROW_SHL4>(tb);
      p = FULL || g + 4 < g1 ? __fmaf_rn(a4, b4, p) : p;
      if constexpr (LPR == 16) {
        const float a8 = dpp_f32<DPP_ROW_SHL8>(ta), b8 = dpp_f32<DPP_ROW_SHL8>(tb);
        const float a12 = dpp_f32<DPP_ROW_SHL12>(ta), b12 = dpp_f32<DPP_ROW_SHL12>(tb);
        p = FULL || g + 8 < g1 ? __fmaf_rn(a8, b8, p) : p;
        p = FULL || g + 12 < g1 ? __fmaf_rn(a12, b12, p) : p;
      }
    }
  };
  for (int st = g0;;) {
    if (fixed) {
#pragma unroll
      for (int k = 0; k < NPL; ++k) v[k] = piece_fix(v[k], vsh[k]);
    }
#pragma unroll
    for (int k = 0; k < NPL; ++k)
      if (lane + 64 * k < NT) lw[lane + 64 * k] = v[k];
    // the next step's bytes (the first of the wave's next chunk after a chunk's
    // last step; past the wave's last step this one's again, so that every step
    // issues the same loads), in flight while this one is summed
    int32_t ns = st + LPR, ne = g1;
    bool more = true;
    if (ns >= g1) {
      more = c + W < ceff;
      if (more)
        range(c + W, ns, ne);
      else
        ns = st;
    }
    fetch(ns, ne);
    if (st + LPR <= g1)
      terms(st, std::integral_constant<bool, true>());
    else
      terms(st, std::integral_constant<bool, false>());
    st += LPR;
    if (st < g1) continue;
    // the chunk's partial: (P0 + P2) + (P1 + P3), partial q in lane q of the row's lanes
    Acc pr;
    if constexpr (MODE == 0) {
      const double t = __dadd_rn(p, dpp_f64<DPP_ROW_SHL2>(p));
      pr = __dadd_rn(t, dpp_f64<DPP_ROW_SHL1>(t));
    } else {
      const float t = __fadd_rn(p, dpp_f32<DPP_ROW_SHL2>(p));
      pr = __fadd_rn(t, dpp_f32<DPP_ROW_SHL1>(t));
    }
    if (j == 0) lpart[(rg * ceff + c) * ROWS + r] = pr;
    if (!more) break;
    c += W;
    st = ns;
    g1 = ne;
    p = 0;
  }
  __syncthreads();
  if ((int)threadIdx.x < ROWS * R) {
    const int gq = threadIdx.x / ROWS, rq = threadIdx.x % ROWS;
    const int64_t oo = o_wg + threadIdx.x;
    if (oo < N) {
      if (ceff == 1) {
        y[oo] = (float)lpart[gq * ROWS + rq];
      } else {
        Acc acc = 0;
        for (int cc = 0; cc < ceff; ++cc) acc = acc + lpart[(gq * ceff + cc) * ROWS + rq];
        y[oo] = (float)acc;
      }
    }
  }
}

// The non-empty chunks of the S-chunk rule: chunks 0..m-1, then chunk S-1 when
// it holds the K mod 512 tail (or all of K when K < 512).
void f_chunks(int64_t K, int S, int& m, int& ceff) {
  const int64_t nq = K / 512, per = (nq + S - 1) / S;
  m = per > 0 ? (int)((nq + per - 1) / per) : 0;
  if (m > S) m = S;
  ceff = m;
  if (m < S && ((K % 512) != 0 || m == 0)) ceff = m + 1;
}

template <int F, int MODE, int ROWS, int R>
size_t fr_lds(int W, int ceff) {
  using Acc = typename std::conditional<MODE == 0, double, float>::type;
  return SLOT_BASE + (size_t)R * W * Stage<F, MODE, ROWS>::SLOT + (size_t)R * ceff * ROWS * sizeof(Acc);
}

template <int F, int MODE, int ROWS, int R>
hipError_t launch_fr(const uint8_t* w, int64_t N, int64_t K, const float* x, const int8_t* xq, const int8_t* xl,
                     const float* xs, int S, int m, int ceff, int W, float* y, hipStream_t st) {
  const int64_t rb = K / Geo<F>::V * Geo<F>::B;
  const dim3 grid((unsigned)((N + ROWS * R - 1) / (ROWS * R))), block((unsigned)(64 * R * W));
  return launch((k_gemv_fmt<F, MODE, ROWS, R>), grid, block, fr_lds<F, MODE, ROWS, R>(W, ceff), st, w, rb, N,
                N * rb, x, xq, xl, xs, K, S, m, ceff, y);
}

// Workgroups of W chunk waves that a compute unit holds at once: the HIP
// occupancy calculator over the kernel's VGPRs, LDS and wave slots (8 waves a
// SIMD at most 64 VGPRs, 7 at 72, 6 at 80, 5 at 96), asked once a kernel and W
// with the partials of QDG_MAX_SPLITS chunks.
template <int F, int MODE, int ROWS, int R>
int fr_resident(int W) {
  static std::atomic<int> cache[17];
  int n = cache[W].load(std::memory_order_relaxed);
  if (n <= 0) {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, (const void*)k_gemv_fmt<F, MODE, ROWS, R>, 64 * R * W,
                                                     fr_lds<F, MODE, ROWS, R>(W, QDG_MAX_SPLITS)) != hipSuccess) {
      (void)hipGetLastError();
      b = 1;
    }
    n = b > 0 ? b : 1;
    cache[W].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Four rows a wave (16 lanes a row) and one row group a workgroup.  Measured on
// the 5120 x 25600 projection: 8 rows a wave was slower in 70 of 72 format,
// mode and S (4, 5, 8) cases, by up to 43%; two row groups a workgroup and
// fetching two or three steps ahead were slower too.
template <int F, int MODE>
int f_waves(int64_t N, int64_t K, int S, int& m, int& ceff) {
  f_chunks(K, S, m, ceff);
  if (S == 1) m = 1, ceff = 1;
  // at 5120 rows and S = 8: four waves of two chunks; at S = 16, five or six
  return pick_chunk_waves((N + 3) / 4, 16, K, S, m, ceff, tune(QDG_TUNE_FMT_WAVES),
                          [](int w) { return fr_resident<F, MODE, 4, 1>(w); });
}

template <int F, int MODE>
hipError_t launch_f(const uint8_t* w, int64_t N, int64_t K, const float* x, const int8_t* xq, const int8_t* xl,
                    const float* xs, int S, float* y, hipStream_t st) {
  int m, ceff;
  const int W = f_waves<F, MODE>(N, K, S, m, ceff);
  return launch_fr<F, MODE, 4, 1>(w, N, K, x, xq, xl, xs, S, m, ceff, W, y, st);
}

template <int F>
int fm_waves(int mode, int64_t N, int64_t K, int S) {
  int m, ceff;
  if (mode == 0) return f_waves<F, 0>(N, K, S, m, ceff);
  if (mode == 1) return f_waves<F, 1>(N, K, S, m, ceff);
  return f_waves<F, 2>(N, K, S, m, ceff);
}

template <int F>
hipError_t launch_fm(int mode, const uint8_t* w, int64_t N, int64_t K, const float* x, const int8_t* xq,
                     const int8_t* xl, const float* xs, int S, float* y, hipStream_t st) {
  if (mode == 0) return launch_f<F, 0>(w, N, K, x, xq, xl, xs, S, y, st);
  if (mode == 1) return launch_f<F, 1>(w, N, K, x, xq, xl, xs, S, y, st);
  return launch_f<F, 2>(w, N, K, x, xq, xl, xs, S, y, st);
}

}  // namespace

// Compute units of the current device (256 on the MI355X), asked once a device.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Values per block and bytes per block of a format (0, 0 if unknown).
void fmt_geometry(int fmt, int& values, int& bytes) {
  values = 32;
  switch (fmt) {
    case F_Q4_0: bytes = 18; break;
    case F_Q4_1: bytes = 20; break;
    case F_Q5_0: bytes = 22; break;
    case F_Q5_1: bytes = 24; break;
    case F_IQ4_NL: bytes = 18; break;
    case F_MXFP4: bytes = 17; break;
    case F_Q2_K: values = 256; bytes = 84; break;
    case F_Q3_K: values = 256; bytes = 110; break;
    case F_Q4_K: values = 256; bytes = 144; break;
    case F_Q5_K: values = 256; bytes = 176; break;
    case F_Q6_K: values = 256; bytes = 210; break;
    case F_IQ4_XS: values = 256; bytes = 136; break;
    default: values = 0; bytes = 0;
  }
}

int fmt_chunk_waves(int fmt, int mode, int64_t N, int64_t K, int S) {
  switch (fmt) {
    case F_Q4_0: return fm_waves<F_Q4_0>(mode, N, K, S);
    case F_Q4_1: return fm_waves<F_Q4_1>(mode, N, K, S);
    case F_Q5_0: return fm_waves<F_Q5_0>(mode, N, K, S);
    case F_Q5_1: return fm_waves<F_Q5_1>(mode, N, K, S);
    case F_IQ4_NL: return fm_waves<F_IQ4_NL>(mode, N, K, S);
    case F_MXFP4: return fm_waves<F_MXFP4>(mode, N, K, S);
    case F_Q2_K: return fm_waves<F_Q2_K>(mode, N, K, S);
    case F_Q3_K: return fm_waves<F_Q3_K>(mode, N, K, S);
    case F_Q4_K: return fm_waves<F_Q4_K>(mode, N, K, S);
    case F_Q5_K: return fm_waves<F_Q5_K>(mode, N, K, S);
    case F_Q6_K: return fm_waves<F_Q6_K>(mode, N, K, S);
    default: return fm_waves<F_IQ4_XS>(mode, N, K, S);
  }
}

hipError_t launch_gemv_fmt(int fmt, int mode, const uint8_t* w, int64_t N, int64_t K, const float* x,
                           const int8_t* xq, const int8_t* xl, const float* xs, int S, float* y, hipStream_t st) {
  switch (fmt) {
    case F_Q4_0: return launch_fm<F_Q4_0>(mode, w, N, K, x, xq, xl, xs, S, y, st);
    case F_Q4_1: return launch_fm<F_Q4_1>(mode, w, N, K, x, xq, xl, xs, S, y, st);
    case F_Q5_0: return launch_fm<F_Q5_0>(mode, w, N, K, x, xq, xl, xs, S, y, st);
    case F_Q5_1: return launch_fm<F_Q5_1>(mode, w, N, K, x, xq, xl, xs, S, y, st);
    case F_IQ4_NL: return launch_fm<F_IQ4_NL>(mode, w, N, K, x, xq, xl, xs, S, y, st);
    case F_MXFP4: return launch_fm<F_MXFP4>(mode, w, N, K, x, xq, xl, xs, S, y, st);
    case F_Q2_K: return launch_fm<F_Q2_K>(mode, w, N, K, x, xq, xl, xs, S, y, st);
    case F_Q3_K: return launch_fm<F_Q3_K>(mode, w, N, K, x, xq, xl, xs, S, y, st);
    case F_Q4_K: return launch_fm<F_Q4_K>(mode, w, N, K, x, xq, xl, xs, S, y, st);
    case F_Q5_K: return launch_fm<F_Q5_K>(mode, w, N, K, x, xq, xl, xs, S, y, st);
    case F_Q6_K: return launch_fm<F_Q6_K>(mode, w, N, K, x, xq, xl, xs, S, y, st);
    default: return launch_fm<F_IQ4_XS>(mode, w, N, K, x, xq, xl, xs, S, y, st);
  }
}

}  // namespace qdg
