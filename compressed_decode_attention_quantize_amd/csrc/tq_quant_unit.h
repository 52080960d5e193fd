// tq_quant_unit.h -- the per-group quantiser of the append path, shared by
// the append kernel and the fused append + decode kernel.  See tq_quant.hip
// for the method and the lane layout.
//
// Everything here must round exactly as the format defines: no floating-point
// contraction (the residual's single rounding is an explicit fmaf).  The
// pragma below holds for the rest of the including file; a file that wants
// contraction back re-enables it after the include.
#pragma once

#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"

#pragma clang fp contract(off)

namespace tq {
namespace qunit {

constexpr int kWavesPerWg = 8;
// padded LDS row of the sketch halves (fp16 high and low parts of S): 16-byte
// reads of 16 rows fall on distinct banks
constexpr int kSRowH = kD + 8;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t norm_to_f16(float n) {
  return __half_as_ushort(__float2half_rn(fminf(n, 65504.0f)));
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return __half2float(__ushort_as_half(h)); }
// floor(log2 x) of a positive finite x (subnormals give -127)
__device__ __forceinline__ int exponent_of_f(float x) { return static_cast<int>((__float_as_uint(x) >> 23) & 0xffu) - 127; }

// ---------------------------------------------------------------- exchanges
// xswap<LB>(a, b): afterwards, in every lane, a holds the value whose lane
// bit LB is 0 and b the value whose lane bit LB is 1, both of register a in
// lanes with bit LB clear and of register b in the others.  The lane bit
// then indexes the former register pair and the register slot the former
// lane bit.
template <int LB>
__device__ __forceinline__ void xswap_u(uint32_t& a, uint32_t& b) {
  if constexpr (LB == 5) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
  }
}
template <int LB>
__device__ __forceinline__ void xswap(float& a, float& b) {
  uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  xswap_u<LB>(ua, ub);
  a = __uint_as_float(ua);
  b = __uint_as_float(ub);
}
template <int LB>
__device__ __forceinline__ void xswap(double& a, double& b) {
  const uint64_t ua = static_cast<uint64_t>(__double_as_longlong(a));
  const uint64_t ub = static_cast<uint64_t>(__double_as_longlong(b));
  uint32_t alo = static_cast<uint32_t>(ua), ahi = static_cast<uint32_t>(ua >> 32);
  uint32_t blo = static_cast<uint32_t>(ub), bhi = static_cast<uint32_t>(ub >> 32);
  xswap_u<LB>(alo, blo);
  xswap_u<LB>(ahi, bhi);
  a = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(ahi) << 32) | alo));
  b = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(bhi) << 32) | blo));
}
// v + (v of lane ^ (1 << LB)), identical in both lanes.
template <int LB>
__device__ __forceinline__ double pair_sum(double v) {
  double a = v, b = v;
  xswap<LB>(a, b);
  return a + b;
}
template <int LB>
__device__ __forceinline__ uint32_t partner(uint32_t v) {
  uint32_t a = v, b = v;
  xswap_u<LB>(a, b);
  return ((threadIdx.x >> LB) & 1) ? a : b;
}

// 2 w + (bit of this lane in mask m): shifts one code bit into a packed word.
__device__ __forceinline__ uint32_t shift_in(uint32_t w, uint64_t m) {
  uint32_t r;
  uint64_t carry_out;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(w), "s"(m));
  return r;
}

// One step of a 16 x 16 bit transpose inside each 16-lane row: lane p holds
// row p of two matrices (bits 0..15 and 16..31); the off-diagonal K x K
// blocks of every 2K x 2K block trade places with lane p ^ K.
template <int K>
__device__ __forceinline__ uint32_t transpose_step(uint32_t w, int p) {
  constexpr uint32_t M = K == 8 ? 0xFF00FF00u : K == 4 ? 0xF0F0F0F0u : K == 2 ? 0xCCCCCCCCu : 0xAAAAAAAAu;
  const uint32_t o = static_cast<uint32_t>(lane_xor_i<K>(static_cast<int>(w)));
  return (p & K) ? ((w & M) | ((o >> K) & ~M)) : ((w & ~M) | ((o << K) & M));
}
// Afterwards lane p holds, at bit c (+ 16), bit p (+ 16) of lane c's word.
__device__ __forceinline__ uint32_t transpose16(uint32_t w, int p) {
  w = transpose_step<8>(w, p);
  w = transpose_step<4>(w, p);
  w = transpose_step<2>(w, p);
  return transpose_step<1>(w, p);
}

// ------------------------------------------------------------- norm tree
// fp64 pairwise tree of squares over the 128 coordinates of each position,
// level 64 (pairs c, c + 64) first, then 32, ..., 1.  v holds coordinate bit
// 6 on register bit 4 and bits 0..3 on register bits 0..3; lane bit C5 holds
// coordinate bit 5 and the other of lane bits 4/5 coordinate bit 4.  Every
// lane of the position returns the sum.
template <int C5>
__device__ __forceinline__ double tree_sumsq(const float (&v)[32]) {
  constexpr int C4 = 9 - C5;
  double t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {   // level 64: a^2 and b^2 are exact, one rounding
    const double a = static_cast<double>(v[i]), b = static_cast<double>(v[i + 16]);
    t[i] = fma(a, a, b * b);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {    // level 32 (coordinate bit 5 on lane bit C5)
    xswap<C5>(t[i], t[i + 8]);
    t[i] = t[i] + t[i + 8];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {    // level 16 (bit 4 on lane bit C4)
    xswap<C4>(t[i], t[i + 4]);
    t[i] = t[i] + t[i + 4];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {    // level 8 (bit 3, moved to lane bit C5)
    xswap<C5>(t[i], t[i + 2]);
    t[i] = t[i] + t[i + 2];
  }
  xswap<C4>(t[0], t[1]);           // level 4 (bit 2, moved to lane bit C4)
  t[0] = t[0] + t[1];
  t[0] = pair_sum<C5>(t[0]);       // level 2 (bit 1 on lane bit C5)
  return pair_sum<C4>(t[0]);       // level 1 (bit 0 on lane bit C4)
}

// ------------------------------------------------------------------ FWHT
__device__ __forceinline__ void bfly(float& a, float& b) {
  const float x = a, y = b;
  a = x + y;
  b = x - y;
}
// Raw Sylvester FWHT, stages h = 1, 2, ..., 64 in that order.  On entry v
// holds coordinate bits 0..3 on register bits 0..3, bit 6 on register bit 4,
// bit 5 on lane bit 4 and bit 4 on lane bit 5.  On exit bits 0..3 and 6 are
// where they were, bit 4 is on lane bit 4 and bit 5 on lane bit 5.
__device__ __forceinline__ void fwht_tile(float (&v)[32]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if ((i & h) == 0) bfly(v[i], v[i + h]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {   // h = 16: bit 4 to register bit 4, bit 6 to lane bit 5
    xswap<5>(v[i], v[i + 16]);
    bfly(v[i], v[i + 16]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {   // h = 32: bit 5 to register bit 4, bit 4 to lane bit 4
    xswap<4>(v[i], v[i + 16]);
    bfly(v[i], v[i + 16]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {   // h = 64: bit 6 to register bit 4, bit 5 to lane bit 5
    xswap<5>(v[i], v[i + 16]);
    bfly(v[i], v[i + 16]);
  }
}

// -------------------------------------------------------------- codebook
// Bits of the code of y: the number of thresholds below y (thresholds sorted
// ascending), found by a binary search; bit[k] is bit k of the code.
template <int B>
__device__ __forceinline__ void code_bits(float y, const float (&thr)[15], bool (&bit)[4]) {
#pragma unroll
  for (int k = B - 1; k >= 0; --k) {
    constexpr int kMax = 1 << (B - 1);
    float cand[kMax];
    const int n = 1 << (B - 1 - k);
#pragma unroll
    for (int m = 0; m < kMax; ++m)
      if (m < n) cand[m] = thr[m * (2 << k) + (1 << k) - 1];
#pragma unroll
    for (int j = k + 1; j < B; ++j) {   // select by the known bits, lowest first
      const int half = 1 << (B - 1 - j);
#pragma unroll
      for (int m = 0; m < kMax / 2; ++m)
        if (m < half) cand[m] = bit[j] ? cand[2 * m + 1] : cand[2 * m];
    }
    bit[k] = y > cand[0];
  }
}
// The centroid of a code.  The codebook is antisymmetric (centroid
// 2^B - 1 - c is minus centroid c, exactly: the host mirrors the positive
// half), so the top bit is the sign and the other bits, complemented for a
// negative code, pick the magnitude among the positive half: B - 1 levels of
// selects over 2^(B-1) values instead of B levels over 2^B.
template <int B>
__device__ __forceinline__ float centroid(const float (&cv)[16], const bool (&bit)[4]) {
  constexpr int H = 1 << (B - 1);
  const bool pos = bit[B - 1];
  float cand[H];
#pragma unroll
  for (int m = 0; m < H; ++m) cand[m] = cv[H + m];
#pragma unroll
  for (int j = 0; j < B - 1; ++j) {
    const bool up = bit[j] == pos;   // bit j of the code's mirror image in the positive half
    const int half = 1 << (B - 2 - j);
#pragma unroll
    for (int m = 0; m < H / 2; ++m)
      if (m < half) cand[m] = up ? cand[2 * m + 1] : cand[2 * m];
  }
  return pos ? cand[0] : -cand[0];
}

// ----------------------------------------------------------------- loads
// The 32 input values at element offset idx (coordinates 32 g .. 32 g + 31).
__device__ __forceinline__ void load_row(const void* p, int64_t idx, int dtype, float (&v)[32]) {
  if (dtype == IN_F32) {
    const float4* s = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + idx);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = s[i];
      v[4 * i] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
  } else {
    const uint4* s = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + idx);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = s[i];
      w[4 * i] = u.x;
      w[4 * i + 1] = u.y;
      w[4 * i + 2] = u.z;
      w[4 * i + 3] = u.w;
    }
    if (dtype == IN_BF16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        v[2 * i] = f16_to_f32(static_cast<uint16_t>(w[i]));
        v[2 * i + 1] = f16_to_f32(static_cast<uint16_t>(w[i] >> 16));
      }
    }
  }
}

// D x for the 32 coordinates 32 g + i of this lane (D = +/-1, exact).
__device__ __forceinline__ void apply_signs(float (&v)[32], const float* D, int g) {
  const float4* d4 = reinterpret_cast<const float4*>(D + 32 * g);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 d = d4[i];
    v[4 * i] *= d.x;
    v[4 * i + 1] *= d.y;
    v[4 * i + 2] *= d.z;
    v[4 * i + 3] *= d.w;
  }
}

// Rotation and radius of a tile: v (loaded, natural layout) becomes y = H D x
// in the FWHT's exit layout; returns the fp32 radius (rounded once from the
// fp64 tree) of this lane's position.
__device__ __forceinline__ float rotate(float (&v)[32], const float* D, int g) {
  apply_signs(v, D, g);
#pragma unroll
  for (int i = 0; i < 16; ++i) xswap<5>(v[i], v[i + 16]);   // bit 6 to register bit 4, bit 4 to lane bit 5
  const double ss = tree_sumsq<4>(v);
  fwht_tile(v);
  return static_cast<float>(sqrt(ss));
}

struct Unit {
  int b, h, t0, t1, grp;
  uint8_t* kblk;
  uint8_t* vblk;
};

// --------------------------------------------------------------- kernel
// The sketch S in shared memory as two fp16 tables, S = hi + lo (hi = S
// rounded to fp16, lo = the remainder rounded to fp16), rows kSRowH halves
// apart in natural coordinate order.
struct SHalves {
  const _Float16* hi;
  const _Float16* lo;
};

template <int KB, int VB, bool QJL>
__device__ void quant_unit(const QuantArgs& a, const Unit& u, const SHalves& sh, int lane) {
  constexpr bool kPolar = KB > 0;
  const int p = lane & 15;
  const int g = lane >> 4;
  const int k_codec = a.k_codec;
  const int plane_words = (kD / 32) * kBlock;
  float kthr_b[15], vthr_b[15], kc[16];
#pragma unroll
  for (int j = 0; j < 15; ++j) {
    kthr_b[j] = (kPolar && j < (1 << KB) - 1) ? a.tb.kb[j] : 0.0f;
    vthr_b[j] = (VB > 0 && j < (1 << VB) - 1) ? a.tb.vb[j] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) kc[j] = (kPolar && j < (1 << KB)) ? a.tb.ck[j] : 0.0f;

  // value bit-plane words owned by this lane: coordinates p + 16 g and p + 16 g + 64
  uint32_t vw_lo[4] = {}, vw_hi[4] = {};   // per plane: tile 0 / tile 1 transposed words
  const int base = u.grp * 32;

#pragma unroll 1
  for (int tile = 0; tile < 2; ++tile) {
    const int tb = base + 16 * tile;
    if (tb + 16 <= u.t0 || tb >= u.t1) continue;   // uniform
    const int pos = tb + p;
    const bool valid = pos >= u.t0 && pos < u.t1;
    const int pos_c = min(max(pos, u.t0), u.t1 - 1);
    const int t = pos_c % kBlock;
    const int start = a.seq_lens[u.b];
    const int64_t in_idx = ((static_cast<int64_t>(u.b) * a.n_new + (pos_c - start)) * a.n_kv + u.h) * kD + 32 * g;

    // ---------------------------------------------------------- keys
    float v[32];
    load_row(a.k_new, in_idx, a.in_dtype, v);
    if (!kPolar && k_codec == RAW_F32) {
      if (valid) {
        float4* row = reinterpret_cast<float4*>(reinterpret_cast<float*>(u.kblk) + t * kD + 32 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) row[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
      }
    } else if (!kPolar && k_codec == Q8_BLOCK32) {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
      const uint16_t s16 = norm_to_f16(m / 127.0f);
      const float sf = f16_to_f32(s16);
      // k = rint(x / sf) with the quotient rounded once (fp32 division): from
      // x times the block's reciprocal, kept when the exact remainder
      // x - k sf (one fma) puts x / sf more than 2^-12 inside the interval
      // (k - 1/2, k + 1/2), where every rounding of the quotient gives k;
      // otherwise (about 1 in 2000 values) from the division itself
      const float rs = (sf > 0.0f) ? 1.0f / sf : 0.0f;
      const float lim = (0.5f - 0x1p-12f) * sf;
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int k = 0;
          if (sf > 0.0f) {
            const float x = v[4 * i + e];
            float kq = rintf(x * rs);
            if (!(fabsf(fmaf(-kq, sf, x)) < lim)) kq = rintf(x / sf);
            k = static_cast<int>(fminf(fmaxf(kq, -127.0f), 127.0f));
          }
          word |= (static_cast<uint32_t>(k) & 0xFFu) << (8 * e);
        }
        w[i] = word;
      }
      if (valid) {
        uint4* row = reinterpret_cast<uint4*>(u.kblk + t * kD + 32 * g);
        row[0] = make_uint4(w[0], w[1], w[2], w[3]);
        row[1] = make_uint4(w[4], w[5], w[6], w[7]);
        reinterpret_cast<uint16_t*>(u.kblk + kBlock * kD)[t * (kD / 32) + g] = s16;
      }
    } else if constexpr (kPolar) {
      const float n = rotate(v, a.tb.dk, g);
      const uint16_t n16 = norm_to_f16(n);
      const float nf = f16_to_f32(n16);
      float thr[15];
#pragma unroll
      for (int j = 0; j < 15; ++j) thr[j] = kthr_b[j] * n;
      uint32_t hw[4] = {0, 0, 0, 0};
#pragma unroll
      for (int s = 31; s >= 0; --s) {
        bool bit[4] = {false, false, false, false};
        code_bits<KB>(v[s], thr, bit);
#pragma unroll
        for (int q = 0; q < KB; ++q) hw[q] = shift_in(hw[q], __ballot(bit[q]));
        if constexpr (QJL) {
          v[s] = fmaf(-nf, centroid<KB>(kc, bit), v[s]);   // residual
          asm volatile("" : "+v"(v[s]));   // here, while the code masks are live
        }
      }
      // plane words: the lane's bits s < 16 are bits 16 (g & 1) + s of word
      // g >> 1, bits s >= 16 those of word (g >> 1) + 2; the lane of the other
      // g & 1 holds the other halves
      const bool odd = g & 1;
      const int word = (g >> 1) + (odd ? 2 : 0);
      const int slot = slot_of(t);
      uint32_t* planes = reinterpret_cast<uint32_t*>(u.kblk);
#pragma unroll
      for (int q = 0; q < KB; ++q) {
        const uint32_t o = partner<4>(hw[q]);
        const uint32_t wv = odd ? ((o >> 16) | (hw[q] & 0xFFFF0000u)) : ((hw[q] & 0xFFFFu) | (o << 16));
        if (valid) planes[q * plane_words + word * kBlock + slot] = wv;
      }
      uint8_t* after = u.kblk + 4 * KB * plane_words;
      if constexpr (QJL) {
        const double sr = tree_sumsq<5>(v);
        const float rho = static_cast<float>(sqrt(sr / static_cast<double>(kD)));
        // sketch Z = S R: rows = sketch rows, columns = the tile's positions,
        // on the fp16 matrix instruction with both factors split into fp16
        // high and low parts (hi hi + lo hi + hi lo: products exact in fp32,
        // the dropped lo lo and the splits' remainders below 2^-21 of each
        // term), the residual first scaled by a power of two to |r| < 1 (the
        // signs do not change).  Instruction b of a row tile takes, from lane
        // group g, the 8 coordinates this lane holds in registers 8 b .. 8 b
        // + 7: coordinates 16 g + 8 (b & 1) + 64 (b >> 1) + i, in natural
        // order in the tables.  neg[w] collects, in this lane, the signs of
        // its position's rows 32 w + 16 (mt & 1) + 4 g + i at bit
        // 16 (mt & 1) + i.
        const float rn = static_cast<float>(sqrt(sr));
        const int re = (rn > 0.0f) ? exponent_of_f(rn) + 1 : 0;
        v8h rh[4], rl[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float x = __builtin_amdgcn_ldexpf(v[8 * b + i], -re);
            const _Float16 hx = static_cast<_Float16>(x);
            rh[b][i] = hx;
            rl[b][i] = static_cast<_Float16>(x - static_cast<float>(hx));
          }
        uint32_t neg[4] = {0, 0, 0, 0};
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          const _Float16* shi = sh.hi + (16 * mt + p) * kSRowH + 16 * g;
          const _Float16* slo = sh.lo + (16 * mt + p) * kSRowH + 16 * g;
          v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int c0 = 8 * (b & 1) + 64 * (b >> 1);
            const v8h ah = *reinterpret_cast<const v8h*>(shi + c0);
            const v8h al = *reinterpret_cast<const v8h*>(slo + c0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, rh[b], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, rh[b], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, rl[b], acc, 0, 0, 0);
          }
          // acc[i]: sketch row 16 mt + 4 g + i of position p; a zero sum is +0
#pragma unroll
          for (int i = 0; i < 4; ++i)
            neg[mt >> 1] |= (__float_as_uint(acc[i]) >> 31) << (16 * (mt & 1) + i);
        }
        // sign bit [z >= 0] at 16 (mt & 1) + 4 g + i; then OR over the four
        // lanes of the position, leaving word g in lane g
        uint32_t sw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) sw[w] = (~neg[w] & 0x000F000Fu) << (4 * g);
        xswap_u<4>(sw[0], sw[1]);
        xswap_u<4>(sw[2], sw[3]);
        uint32_t sa = sw[0] | sw[1], sb = sw[2] | sw[3];   // words g & 1 and (g & 1) + 2
        xswap_u<5>(sa, sb);
        if (valid) {
          uint32_t* sgn = reinterpret_cast<uint32_t*>(after);
          sgn[g * kBlock + slot] = sa | sb;
        }
        after += 4 * (kM / 32) * kBlock;
        if (valid && g == 0) reinterpret_cast<uint16_t*>(after + 2 * kBlock)[slot] = norm_to_f16(rho);
      }
      if (valid && g == 0) reinterpret_cast<uint16_t*>(after)[slot] = n16;
    }

    // -------------------------------------------------------- values
    load_row(a.v_new, in_idx, a.in_dtype, v);
    if constexpr (VB == 0) {
      if (valid && a.v_codec == RAW_F32) {   // recursive polar values have their own kernel
        float4* row = reinterpret_cast<float4*>(reinterpret_cast<float*>(u.vblk) + t * kD + 32 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) row[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
      }
    } else {
      const float n = rotate(v, a.tb.dv, g);
      const uint16_t n16 = norm_to_f16(n);
      float thr[15];
#pragma unroll
      for (int j = 0; j < 15; ++j) thr[j] = vthr_b[j] * n;
      // bit s of wv[q]: plane q of coordinate (s & 15) + 16 g + 64 (s >> 4)
      uint32_t wv[4] = {0, 0, 0, 0};
#pragma unroll
      for (int s = 31; s >= 0; --s) {
        bool bit[4] = {false, false, false, false};
        code_bits<VB>(v[s], thr, bit);
#pragma unroll
        for (int q = 0; q < VB; ++q) wv[q] = shift_in(wv[q], __ballot(bit[q]));
      }
      // transposed: bit p (+ 16) = position p of coordinate p' + 16 g (+ 64), p' = this lane's p
#pragma unroll
      for (int q = 0; q < VB; ++q) {
        const uint32_t tw = transpose16(wv[q], p);
        if (tile == 0) {
          vw_lo[q] = tw;
        } else {
          vw_hi[q] = tw;
        }
      }
      if (valid && g == 0) reinterpret_cast<uint16_t*>(u.vblk + 4 * VB * 4 * kD)[slot_of(t)] = n16;
    }
  }

  if constexpr (VB > 0) {
    // coordinate-major words of this 32-position group; bits of positions
    // outside [t0, t1) keep what the cache holds
    const int lo = u.t0 - base, hi = u.t1 - base;   // 0 <= lo < hi <= 32
    const uint32_t keep = ~(((hi == 32) ? 0xFFFFFFFFu : ((1u << hi) - 1u)) & ~((1u << lo) - 1u));
    uint32_t* planes = reinterpret_cast<uint32_t*>(u.vblk);
    const int j = (base % kBlock) / 32;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int coord = p + 16 * g + 64 * half;
#pragma unroll
      for (int q = 0; q < VB; ++q) {
        uint32_t* w = planes + q * 4 * kD + j * kD + coord;
        const uint32_t nw = half ? ((vw_lo[q] >> 16) | (vw_hi[q] & 0xFFFF0000u))
                                 : ((vw_lo[q] & 0xFFFFu) | (vw_hi[q] << 16));
        *w = keep ? ((*w & keep) | (nw & ~keep)) : nw;
      }
    }
  }
}

// ------------------------------------------------------------ one position
// A single new position of one (sequence, KV head) per wavefront (the
// serving step's append): lane l holds coordinates l and l + 64.  Codes,
// radii and residual norms are those of quant_unit bit for bit (the same
// FWHT stage order, fp64 norm tree, thresholds, binary search and residual);
// the QJL sketch is a per-lane fp32 dot product over the coordinates in
// order, so a sign can differ from quant_unit's only where the sketch value
// is within rounding of zero (a sign bit set, -0 included, counts as
// negative in both).

__device__ __forceinline__ float token_in(const void* p, int64_t idx, int dtype) {
  if (dtype == IN_F32) return static_cast<const float*>(p)[idx];
  const uint16_t h = static_cast<const uint16_t*>(p)[idx];
  if (dtype == IN_BF16) return __uint_as_float(static_cast<uint32_t>(h) << 16);
  return f16_to_f32(h);
}

// the format's fp64 tree of squares over (lo = coordinate l, hi = l + 64):
// level 64 in the lane, then levels 32 .. 1 across lanes; every lane gets it
__device__ __forceinline__ double token_sumsq(float lo, float hi) {
  double s = static_cast<double>(lo) * static_cast<double>(lo) + static_cast<double>(hi) * static_cast<double>(hi);
  s += lane_xor<32>(s);
  s += lane_xor<16>(s);
  s += lane_xor<8>(s);
  s += lane_xor<4>(s);
  s += lane_xor<2>(s);
  s += lane_xor<1>(s);
  return __shfl(s, 0, 64);
}

// Keys of one position: POLAR (KB bits, QJL sketch if QJL), q8 or RAW.
// in_idx: element offset of the vector in k_new; t: position in its block.
// S: sketch row j at S + j * SROW.  r_lds: 128 floats of shared memory owned
// by this wavefront (QJL only).
template <int KB, bool QJL, int SROW>
__device__ void token_keys(const QuantArgs& a, int64_t in_idx, uint8_t* kblk, int t, const float* S, float* r_lds,
                           int lane) {
  const float x0 = token_in(a.k_new, in_idx + lane, a.in_dtype);
  const float x1 = token_in(a.k_new, in_idx + lane + 64, a.in_dtype);
  const int slot = slot_of(t);
  if constexpr (KB == 0) {
    if (a.k_codec == RAW_F32) {
      float* row = reinterpret_cast<float*>(kblk) + t * kD;
      row[lane] = x0;
      row[lane + 64] = x1;
    } else if (a.k_codec == Q8_BLOCK32) {
      // per 32-coordinate block: lanes 0..31 / 32..63 hold blocks 0 / 1 (lo) and 2 / 3 (hi)
      float m0 = fabsf(x0), m1 = fabsf(x1);
      m0 = fmaxf(m0, lane_xor<1>(m0));
      m1 = fmaxf(m1, lane_xor<1>(m1));
      m0 = fmaxf(m0, lane_xor<2>(m0));
      m1 = fmaxf(m1, lane_xor<2>(m1));
      m0 = fmaxf(m0, lane_xor<4>(m0));
      m1 = fmaxf(m1, lane_xor<4>(m1));
      m0 = fmaxf(m0, lane_xor<8>(m0));
      m1 = fmaxf(m1, lane_xor<8>(m1));
      m0 = fmaxf(m0, lane_xor<16>(m0));
      m1 = fmaxf(m1, lane_xor<16>(m1));
      const uint16_t s0 = norm_to_f16(m0 / 127.0f), s1 = norm_to_f16(m1 / 127.0f);
      const float f0 = f16_to_f32(s0), f1 = f16_to_f32(s1);
      const int k0 = (f0 > 0.0f) ? static_cast<int>(fminf(fmaxf(rintf(x0 / f0), -127.0f), 127.0f)) : 0;
      const int k1 = (f1 > 0.0f) ? static_cast<int>(fminf(fmaxf(rintf(x1 / f1), -127.0f), 127.0f)) : 0;
      int8_t* row = reinterpret_cast<int8_t*>(kblk) + t * kD;
      row[lane] = static_cast<int8_t>(k0);
      row[lane + 64] = static_cast<int8_t>(k1);
      uint16_t* sc = reinterpret_cast<uint16_t*>(kblk + kBlock * kD) + t * (kD / 32);
      if ((lane & 31) == 0) {
        sc[lane >> 5] = s0;
        sc[2 + (lane >> 5)] = s1;
      }
    }
  } else {
    float kthr[15], kc[16];
#pragma unroll
    for (int j = 0; j < 15; ++j) kthr[j] = (j < (1 << KB) - 1) ? a.tb.kb[j] : 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) kc[j] = (j < (1 << KB)) ? a.tb.ck[j] : 0.0f;
    const float n = static_cast<float>(sqrt(token_sumsq(x0, x1)));
    const uint16_t n16 = norm_to_f16(n);
    const float nf = f16_to_f32(n16);
    float lo = a.tb.dk[lane] * x0, hi = a.tb.dk[lane + 64] * x1;
    wave_fwht128(lo, hi, lane);
    float thr[15];
#pragma unroll
    for (int j = 0; j < 15; ++j) thr[j] = kthr[j] * n;
    bool blo[4] = {false, false, false, false}, bhi[4] = {false, false, false, false};
    code_bits<KB>(lo, thr, blo);
    code_bits<KB>(hi, thr, bhi);
    // token-major plane words: word j holds coordinates 32 j .. 32 j + 31
    uint32_t* planes = reinterpret_cast<uint32_t*>(kblk);
    const int plane_words = (kD / 32) * kBlock;
#pragma unroll
    for (int q = 0; q < KB; ++q) {
      const uint64_t ml = __ballot(blo[q]), mh = __ballot(bhi[q]);
      const uint32_t wsel = (lane & 2) ? static_cast<uint32_t>(((lane & 1) ? mh : ml) >> 32)
                                       : static_cast<uint32_t>((lane & 1) ? mh : ml);
      // lane 0: word 0, lane 1: word 2, lane 2: word 1, lane 3: word 3
      if (lane < 4) planes[q * plane_words + ((lane & 1) * 2 + (lane >> 1)) * kBlock + slot] = wsel;
    }
    uint8_t* after = kblk + 4 * KB * plane_words;
    if constexpr (QJL) {
      const float rlo = fmaf(-nf, centroid<KB>(kc, blo), lo);
      const float rhi = fmaf(-nf, centroid<KB>(kc, bhi), hi);
      const float rho = static_cast<float>(sqrt(token_sumsq(rlo, rhi) / static_cast<double>(kD)));
      r_lds[lane] = rlo;
      r_lds[lane + 64] = rhi;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // sketch rows lane and lane + 64
      const float* s0 = S + lane * SROW;
      const float* s1 = S + (lane + 64) * SROW;
      float z0 = 0.0f, z1 = 0.0f;
#pragma unroll 4
      for (int i = 0; i < kD; i += 4) {
        const float4 r4 = *reinterpret_cast<const float4*>(r_lds + i);
        const float4 a4 = *reinterpret_cast<const float4*>(s0 + i);
        const float4 b4 = *reinterpret_cast<const float4*>(s1 + i);
        z0 = fmaf(a4.x, r4.x, z0);
        z0 = fmaf(a4.y, r4.y, z0);
        z0 = fmaf(a4.z, r4.z, z0);
        z0 = fmaf(a4.w, r4.w, z0);
        z1 = fmaf(b4.x, r4.x, z1);
        z1 = fmaf(b4.y, r4.y, z1);
        z1 = fmaf(b4.z, r4.z, z1);
        z1 = fmaf(b4.w, r4.w, z1);
      }
      const uint64_t p0 = __ballot((__float_as_uint(z0) >> 31) == 0u);
      const uint64_t p1 = __ballot((__float_as_uint(z1) >> 31) == 0u);
      uint32_t* sgn = reinterpret_cast<uint32_t*>(after);
      const uint32_t wsel = (lane & 2) ? static_cast<uint32_t>(((lane & 1) ? p1 : p0) >> 32)
                                       : static_cast<uint32_t>((lane & 1) ? p1 : p0);
      if (lane < 4) sgn[((lane & 1) * 2 + (lane >> 1)) * kBlock + slot] = wsel;
      after += 4 * (kM / 32) * kBlock;
      if (lane == 0) reinterpret_cast<uint16_t*>(after + 2 * kBlock)[slot] = norm_to_f16(rho);
    }
    if (lane == 0) reinterpret_cast<uint16_t*>(after)[slot] = n16;
  }
}

// Values of one position: POLAR (VB bits) or RAW.  Coordinate-major words:
// each lane rewrites the bit of this position in its two coordinates' words.
template <int VB>
__device__ void token_values(const QuantArgs& a, int64_t in_idx, uint8_t* vblk, int t, int lane) {
  const float x0 = token_in(a.v_new, in_idx + lane, a.in_dtype);
  const float x1 = token_in(a.v_new, in_idx + lane + 64, a.in_dtype);
  if constexpr (VB == 0) {
    if (a.v_codec == RAW_F32) {
      float* row = reinterpret_cast<float*>(vblk) + t * kD;
      row[lane] = x0;
      row[lane + 64] = x1;
    }
  } else {
    float vthr[15];
#pragma unroll
    for (int j = 0; j < 15; ++j) vthr[j] = (j < (1 << VB) - 1) ? a.tb.vb[j] : 0.0f;
    const float n = static_cast<float>(sqrt(token_sumsq(x0, x1)));
    float lo = a.tb.dv[lane] * x0, hi = a.tb.dv[lane + 64] * x1;
    wave_fwht128(lo, hi, lane);
    float thr[15];
#pragma unroll
    for (int j = 0; j < 15; ++j) thr[j] = vthr[j] * n;
    bool blo[4] = {false, false, false, false}, bhi[4] = {false, false, false, false};
    code_bits<VB>(lo, thr, blo);
    code_bits<VB>(hi, thr, bhi);
    uint32_t* planes = reinterpret_cast<uint32_t*>(vblk);
    const int j = t >> 5, e = t & 31;
    const uint32_t bitm = 1u << e;
#pragma unroll
    for (int q = 0; q < VB; ++q) {
      uint32_t* w0 = planes + q * 4 * kD + j * kD + lane;
      uint32_t* w1 = w0 + 64;
      *w0 = (*w0 & ~bitm) | (blo[q] ? bitm : 0u);
      *w1 = (*w1 & ~bitm) | (bhi[q] ? bitm : 0u);
    }
    if (lane == 0) reinterpret_cast<uint16_t*>(vblk + 4 * VB * 4 * kD)[slot_of(t)] = norm_to_f16(n);
  }
}

}  // namespace qunit
}  // namespace tq
