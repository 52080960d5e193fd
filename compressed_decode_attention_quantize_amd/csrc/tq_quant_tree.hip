// tq_quant_tree.hip -- quantize-on-append for the recursive polar codec.
//
// What is computed (wis-web.com reader, TurboQuant article: the PolarQuant
// paragraph's Walsh-Hadamard rotation and its Cartesian-to-polar step, one
// radius plus angles whose law is known in advance, taken literally as a
// pairwise tree): y = H (D . x) with the raw FWHT in the same stage order as
// the per-coordinate codec; the radius n = |x| (fp64 pairwise tree of x^2,
// one rounding to fp32, then fp16); then 127 angles.  Level 1 pairs
// (y_2i, y_2i+1) and codes its angle on the circle with b + 1 bits (uniform
// cells); level l >= 2 pairs the radii of two sibling nodes and codes
// atan2(r_right, r_left) in [0, pi/2] with b - 1 bits (Lloyd-Max for the law
// sin(2t)^(2^(l-1) - 1)).  A code counts the boundaries below its angle, so
// ties go to the lower cell.  No angle is formed: the quadrant comes from
// signs, and "angle above boundary B" is r_right^2 cos^2 B > r_left^2 sin^2 B
// with squared radii and both products in fp64.
//
// Angles sit in heap slots: slot 64 + i is level-1 pair i, slot
// 2^(7 - l) + k is node k of level l, slot 1 the root, slot 0 unused.
//
// Mapping: one workgroup per (32-position group, KV head, sequence).  Its
// four wavefronts encode one vector at a time (lane l holds coordinates l and
// l + 64; level-l nodes end up in the lanes that are multiples of 2^l; every
// lane evaluates each level's comparisons, with the code bits a template
// parameter so they unroll over boundaries read through the scalar cache)
// and leave the codes in LDS; then the workgroup writes the packed words,
// each from 32 consecutive code bytes: keys token-major (one position's 32
// slots per word), values slot-major (32 positions per word, bits of
// positions outside this append kept).

#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint16_t norm_to_f16(float n) {
  return __half_as_ushort(__float2half_rn(fminf(n, 65504.0f)));
}

__device__ __forceinline__ float load_in(const void* base, int64_t idx, int dtype) {
  if (dtype == IN_F32) return static_cast<const float*>(base)[idx];
  const uint16_t h = static_cast<const uint16_t*>(base)[idx];
  if (dtype == IN_BF16) return __uint_as_float(static_cast<uint32_t>(h) << 16);
  return __half2float(__ushort_as_half(h));
}

// The tables are read at wave-uniform addresses: through the scalar cache.
typedef __attribute__((address_space(4))) const double cdouble;

// number of boundaries j < N with r_right^2 cos^2 B_j > r_left^2 sin^2 B_j
template <int N>
__device__ __forceinline__ int count_above(double sl, double sr, const double* c2, const double* s2) {
  int c = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const double cj = ((cdouble*)c2)[j], sj = ((cdouble*)s2)[j];
    c += (__dmul_rn(sr, cj) > __dmul_rn(sl, sj)) ? 1 : 0;
  }
  return c;
}

// level-1 code of the pair (a, b) = (y_2i, y_2i+1): quadrant of the circle
// (cells close on their upper end, so (0, +) is the top of quadrant 0), then
// the cell inside it from the local coordinates rotated into quadrant 0
template <int PER_Q>
__device__ __forceinline__ int level1_code(float a, float b, const TreeTab& T) {
  int q;
  float u, v;
  if (a >= 0.0f && b >= 0.0f) {
    q = 0; u = a; v = b;
  } else if (a < 0.0f && b >= 0.0f) {
    q = 1; u = b; v = -a;
  } else if (a <= 0.0f && b < 0.0f) {
    q = 2; u = -a; v = -b;
  } else {
    q = 3; u = -b; v = a;
  }
  const double uu = static_cast<double>(u) * static_cast<double>(u);
  const double vv = static_cast<double>(v) * static_cast<double>(v);
  return q * PER_Q + count_above<PER_Q - 1>(uu, vv, T.c2_1, T.s2_1);
}

// Encode one vector held as (x0 = x_lane, x1 = x_lane+64); the code of heap
// slot s goes to row[s * stride] (LDS), the fp16 radius is returned in every
// lane.
template <int BITS>
__device__ __forceinline__ uint16_t encode_tree(float x0, float x1, const float* D, const TreeTab* Tp, int lane,
                                                uint8_t* row, int stride) {
  const TreeTab& T = *Tp;
  double s = static_cast<double>(x0) * static_cast<double>(x0) + static_cast<double>(x1) * static_cast<double>(x1);
  s += lane_xor<32>(s);
  s += lane_xor<16>(s);
  s += lane_xor<8>(s);
  s += lane_xor<4>(s);
  s += lane_xor<2>(s);
  s += lane_xor<1>(s);
  s = __shfl(s, 0, 64);
  const uint16_t n16 = norm_to_f16(static_cast<float>(sqrt(s)));

  float lo = D[lane] * x0, hi = D[lane + 64] * x1;
  wave_fwht128(lo, hi, lane);

  // level 1: even lanes hold pairs lane / 2 (lo half) and 32 + lane / 2 (hi half)
  constexpr int kPerQ = 1 << (BITS - 1);
  constexpr int kNb = kPerQ - 1;   // boundaries of the b - 1 bit codebooks
  const float plo = lane_xor<1>(lo), phi = lane_xor<1>(hi);
  double slo = static_cast<double>(lo) * static_cast<double>(lo) + static_cast<double>(plo) * static_cast<double>(plo);
  double shi = static_cast<double>(hi) * static_cast<double>(hi) + static_cast<double>(phi) * static_cast<double>(phi);
  if ((lane & 1) == 0) {
    row[(64 + (lane >> 1)) * stride] = static_cast<uint8_t>(level1_code<kPerQ>(lo, plo, T));
    row[(96 + (lane >> 1)) * stride] = static_cast<uint8_t>(level1_code<kPerQ>(hi, phi, T));
  }
  // levels 2..6: the node of lane L (L a multiple of 2^l) pairs lanes L and L + 2^(l-1)
#define TQ_TREE_LEVEL(l)                                                                           \
  {                                                                                                \
    const double rlo = lane_xor<(1 << ((l) - 1))>(slo);                                            \
    const double rhi = lane_xor<(1 << ((l) - 1))>(shi);                                            \
    const int clo = count_above<kNb>(slo, rlo, T.c2[l], T.s2[l]);                                  \
    const int chi = count_above<kNb>(shi, rhi, T.c2[l], T.s2[l]);                                  \
    if ((lane & ((1 << (l)) - 1)) == 0) {                                                          \
      const int first = 1 << (7 - (l));                                                            \
      row[(first + (lane >> (l))) * stride] = static_cast<uint8_t>(clo);                           \
      row[(first + (64 >> (l)) + (lane >> (l))) * stride] = static_cast<uint8_t>(chi);             \
    }                                                                                              \
    slo += rlo;                                                                                    \
    shi += rhi;                                                                                    \
  }
  TQ_TREE_LEVEL(2)
  TQ_TREE_LEVEL(3)
  TQ_TREE_LEVEL(4)
  TQ_TREE_LEVEL(5)
  TQ_TREE_LEVEL(6)
#undef TQ_TREE_LEVEL
  const int root = count_above<kNb>(slo, shi, T.c2[7], T.s2[7]);   // lo half vs hi half
  if (lane == 0) {
    row[1 * stride] = static_cast<uint8_t>(root);
    row[0] = 0;
  }
  return n16;
}

// Bit p of each of the four code bytes of d, as four contiguous bits.
__device__ __forceinline__ uint32_t gather_bits(uint32_t d, int p) {
  return (((d >> p) & 0x01010101u) * 0x01020408u) >> 24 & 0xFu;
}
// Bit p of 32 consecutive code bytes (16-byte aligned in LDS) as one word.
__device__ __forceinline__ uint32_t plane_word(const uint8_t* bytes, int p) {
  const uint4 a = *reinterpret_cast<const uint4*>(bytes);
  const uint4 b = *reinterpret_cast<const uint4*>(bytes + 16);
  return gather_bits(a.x, p) | gather_bits(a.y, p) << 4 | gather_bits(a.z, p) << 8 | gather_bits(a.w, p) << 12 |
         gather_bits(b.x, p) << 16 | gather_bits(b.y, p) << 20 | gather_bits(b.z, p) << 24 | gather_bits(b.w, p) << 28;
}

// KT, VT: code bits of recursive polar keys / values, 0 where that side uses
// another codec (its own kernel stores it).
template <int KT, int VT>
__global__ __launch_bounds__(kThreads) void quant_tree_kernel(QuantArgs a) {
  // key codes position-major (one position's 128 slots contiguous), value
  // codes slot-major (one slot's 32 positions contiguous): each packed word
  // reads 32 consecutive bytes
  __shared__ __attribute__((aligned(16))) uint8_t kcodes[KT ? 32 : 1][kD];
  __shared__ __attribute__((aligned(16))) uint8_t vcodes[VT ? kD : 1][32];
  __shared__ uint16_t radius[2][32];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int start = a.seq_lens[b];
  const int grp = start / 32 + static_cast<int>(blockIdx.x);
  const int base = grp * 32;
  const int t0 = max(start, base);
  const int t1 = min(min(start + a.n_new, base + 32), a.max_ctx);
  if (t0 >= t1) return;   // the whole workgroup
  const int64_t cslot = (static_cast<int64_t>(b) * a.n_kv + h) * a.n_blocks + base / kBlock;

  for (int item = wave; item < 64; item += kThreads / 64) {
    const int tt = item >> 5;
    const int e = item & 31;
    const int pos = base + e;
    if ((tt ? VT : KT) == 0 || pos < t0 || pos >= t1) continue;   // uniform in the wavefront
    const void* src = tt ? a.v_new : a.k_new;
    const int64_t in_idx = ((static_cast<int64_t>(b) * a.n_new + (pos - start)) * a.n_kv + h) * kD;
    const float x0 = load_in(src, in_idx + lane, a.in_dtype);
    const float x1 = load_in(src, in_idx + lane + 64, a.in_dtype);
    uint16_t n16 = 0;
    if constexpr (VT > 0) {
      if (tt) n16 = encode_tree<VT>(x0, x1, a.tb.dv, a.tb.tv, lane, &vcodes[0][e], 32);
    }
    if constexpr (KT > 0) {
      if (!tt) n16 = encode_tree<KT>(x0, x1, a.tb.dk, a.tb.tk, lane, &kcodes[e][0], 1);
    }
    if (lane == 0) radius[tt][e] = n16;
  }
  __syncthreads();

  const int lo = t0 - base, hi = t1 - base;   // 0 <= lo < hi <= 32
  const int jg = (base % kBlock) / 32;        // this group inside its block
  if constexpr (KT > 0) {
    // keys: per position, (b - 1) planes x 4 words over all slots, then the two
    // extra level-1 planes x 2 words over slots 64..127
    constexpr int nb = KT;
    constexpr int per_pos = 4 * nb;
    uint32_t* words = reinterpret_cast<uint32_t*>(a.kc + cslot * a.k_block_bytes);
    uint32_t* l1 = words + (nb - 1) * 4 * kBlock;
    for (int idx = threadIdx.x; idx < 32 * per_pos; idx += kThreads) {
      const int e = idx / per_pos, w = idx % per_pos;
      if (e < lo || e >= hi) continue;
      const int sl = slot_of((base + e) % kBlock);
      const uint8_t* row = &kcodes[e][0];
      if (w < 4 * (nb - 1)) {
        const int p = w >> 2, j = w & 3;
        words[p * 4 * kBlock + j * kBlock + sl] = plane_word(row + 32 * j, p);
      } else {
        const int x = (w - 4 * (nb - 1)) >> 1, j = (w - 4 * (nb - 1)) & 1;
        l1[x * 2 * kBlock + j * kBlock + sl] = plane_word(row + 64 + 32 * j, nb - 1 + x);
      }
    }
    if (threadIdx.x < 32 && threadIdx.x >= lo && threadIdx.x < hi) {
      uint16_t* n16 = reinterpret_cast<uint16_t*>(l1 + 4 * kBlock);
      n16[slot_of((base + threadIdx.x) % kBlock)] = radius[0][threadIdx.x];
    }
  }
  if constexpr (VT > 0) {
    // values: per slot, 32 positions per word; bits of positions outside [lo, hi) kept
    constexpr int nb = VT;
    const uint32_t mine = ((hi == 32) ? 0xFFFFFFFFu : ((1u << hi) - 1u)) & ~((1u << lo) - 1u);
    uint32_t* words = reinterpret_cast<uint32_t*>(a.vc + cslot * a.v_block_bytes);
    uint32_t* l1 = words + (nb - 1) * 4 * kD;
    constexpr int n_words = kD * (nb - 1) + kD;
    for (int idx = threadIdx.x; idx < n_words; idx += kThreads) {
      uint32_t word;
      uint32_t* dst;
      if (idx < kD * (nb - 1)) {
        const int p = idx / kD, sl = idx % kD;
        word = plane_word(&vcodes[sl][0], p);
        dst = words + p * 4 * kD + jg * kD + sl;
      } else {
        const int r = idx - kD * (nb - 1);
        const int x = r / (kD / 2), sl = kD / 2 + r % (kD / 2);
        word = plane_word(&vcodes[sl][0], nb - 1 + x);
        dst = l1 + x * 4 * (kD / 2) + jg * (kD / 2) + (sl - kD / 2);
      }
      word &= mine;   // bytes of positions outside [lo, hi) are stale
      *dst = (mine == 0xFFFFFFFFu) ? word : ((*dst & ~mine) | word);
    }
    if (threadIdx.x >= 32 && threadIdx.x < 64) {
      const int e = threadIdx.x - 32;
      if (e >= lo && e < hi) {
        uint16_t* n16 = reinterpret_cast<uint16_t*>(l1 + 2 * 4 * (kD / 2));
        n16[slot_of((base + e) % kBlock)] = radius[1][e];
      }
    }
  }
}

template <int KT>
hipError_t launch_vt(const QuantArgs& a, int vt, hipStream_t stream) {
  const dim3 grid(a.groups_per_seq, a.n_kv, a.batch);
  switch (vt) {
    case 0:
      if constexpr (KT == 0) return hipErrorInvalidValue;
      else hipLaunchKernelGGL((quant_tree_kernel<KT, 0>), grid, dim3(kThreads), 0, stream, a);
      break;
    case 2: hipLaunchKernelGGL((quant_tree_kernel<KT, 2>), grid, dim3(kThreads), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((quant_tree_kernel<KT, 3>), grid, dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((quant_tree_kernel<KT, 4>), grid, dim3(kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_tree(const QuantArgs& a, hipStream_t stream) {
  if (a.n_new <= 0 || a.batch <= 0) return hipSuccess;
  const int kt = a.k_codec == POLAR_TREE ? a.k_bits : 0;
  const int vt = a.v_codec == POLAR_TREE ? a.v_bits : 0;
  switch (kt) {
    case 0: return launch_vt<0>(a, vt, stream);
    case 2: return launch_vt<2>(a, vt, stream);
    case 3: return launch_vt<3>(a, vt, stream);
    case 4: return launch_vt<4>(a, vt, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
