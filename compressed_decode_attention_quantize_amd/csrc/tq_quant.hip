// tq_quant.hip -- quantize-on-append for gfx950 (wave64).
//
// Method (wis-web.com reader, article on TurboQuant in a llama.cpp fork,
// PolarQuant and QJL paragraphs): rotate each vector with a seeded,
// randomised Walsh-Hadamard transform so its coordinates follow a known law,
// keep the radius (fp16) and code the direction per coordinate with a fixed
// codebook for that law; for keys, add the signs of a Gaussian sketch of the
// residual and the residual's norm (the 1-bit QJL corrector).
//
// Mapping: one wavefront owns one (sequence, KV head, 32-position group) of
// the append and walks its positions in order.  Lane l holds coordinates l
// and l + 64 of the current vector:
//   * FWHT stages h = 1..32 pair lane l with lane l ^ h (cross-lane
//     butterflies through DPP / swizzle / permute); stage h = 64 pairs the
//     two registers of a lane.  The
//     stage order and the pairing are those of the format, and add/sub are
//     exact IEEE operations, so the rotated values are bit-identical to any
//     other engine that follows the format.
//   * sums of squares are fp64 pairwise trees (register pair, then xor
//     butterflies 32..1), the tree the format fixes.
//   * the b code bit-planes and the sign plane are wave ballots; key planes
//     are token-major words (at the position's slot inside its block), value
//     planes accumulate one bit per position in
//     coordinate-major words that the wavefront owns for the whole group
//     (read-modify-write keeps bits of positions it does not write).
//   * the sketch S r (m = 128 rows) reads S^T from LDS, one row pair per lane,
//     broadcasting r_i with readlane.
// This file is compiled with -ffp-contract=off: the residual uses an explicit
// fmaf and nothing else may be fused.

#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWavesPerWg = 16;   // one copy of S^T in LDS serves 16 wavefronts

__device__ __forceinline__ float load_in(const void* p, int64_t idx, int dtype) {
  if (dtype == IN_F32) return reinterpret_cast<const float*>(p)[idx];
  const uint16_t h = reinterpret_cast<const uint16_t*>(p)[idx];
  if (dtype == IN_BF16) return __uint_as_float(static_cast<uint32_t>(h) << 16);
  return __half2float(__ushort_as_half(h));
}

__device__ __forceinline__ uint16_t norm_to_f16(float n) {
  return __half_as_ushort(__float2half_rn(fminf(n, 65504.0f)));
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// fp64 pairwise tree of squares: level 64 in-lane, then xor butterflies.
__device__ __forceinline__ double wave_tree_sumsq(float lo, float hi) {
  const double a = static_cast<double>(lo) * static_cast<double>(lo);
  const double b = static_cast<double>(hi) * static_cast<double>(hi);
  double s = a + b;
  s = s + lane_xor<32>(s);
  s = s + lane_xor<16>(s);
  s = s + lane_xor<8>(s);
  s = s + lane_xor<4>(s);
  s = s + lane_xor<2>(s);
  s = s + lane_xor<1>(s);
  return s;
}

__device__ __forceinline__ uint32_t pick_word(uint64_t mlo, uint64_t mhi, int j) {
  const uint64_t m = (j < 2) ? mlo : mhi;
  return (j & 1) ? static_cast<uint32_t>(m >> 32) : static_cast<uint32_t>(m);
}

struct PolarOut {
  int c_lo, c_hi;
  float y_lo, y_hi;
  uint16_t n16;
};

// Rotation, radius and angle codes of one vector; also writes its code planes
// (token-major) when `kplanes` is non-null.
__device__ __forceinline__ PolarOut polar_codes(float x_lo, float x_hi, const float* D,
                                                const float* bounds, int bits, int lane) {
  PolarOut o;
  float y_lo = D[lane] * x_lo;
  float y_hi = D[lane + 64] * x_hi;
  wave_fwht128(y_lo, y_hi, lane);
  const double ss = wave_tree_sumsq(x_lo, x_hi);
  const float n = static_cast<float>(sqrt(ss));
  o.n16 = norm_to_f16(n);
  int c_lo = 0, c_hi = 0;
  const int levels = 1 << bits;
  for (int j = 0; j + 1 < levels; ++j) {
    const float thr = bounds[j] * n;
    c_lo += (y_lo > thr) ? 1 : 0;
    c_hi += (y_hi > thr) ? 1 : 0;
  }
  o.c_lo = c_lo;
  o.c_hi = c_hi;
  o.y_lo = y_lo;
  o.y_hi = y_hi;
  return o;
}

__global__ __launch_bounds__(64 * kWavesPerWg) void quant_kernel(QuantArgs a) {
  extern __shared__ float st_lds[];   // [128][128] S^T when the key codec has QJL
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  if (a.k_codec == POLAR_QJL) {
    const float4* src = reinterpret_cast<const float4*>(a.tb.st);
    float4* dst = reinterpret_cast<float4*>(st_lds);
    for (int i = threadIdx.x; i < kD * kM / 4; i += blockDim.x) dst[i] = src[i];
    __syncthreads();
  }

  const int item = blockIdx.x * kWavesPerWg + wave;
  const int total = a.batch * a.n_kv * a.groups_per_seq;
  if (item >= total) return;
  const int g = item % a.groups_per_seq;
  const int rest = item / a.groups_per_seq;
  const int h = rest % a.n_kv;
  const int b = rest / a.n_kv;
  const int start = a.seq_lens[b];
  const int end = start + a.n_new;
  const int grp = start / 32 + g;
  int t0 = max(start, grp * 32);
  int t1 = min(end, grp * 32 + 32);
  t1 = min(t1, a.max_ctx);
  if (t0 >= t1) return;
  const int blk = t0 / kBlock;
  const int64_t slot = (static_cast<int64_t>(b) * a.n_kv + h) * a.n_blocks + blk;
  uint8_t* kblk = a.kc + slot * a.k_block_bytes;
  uint8_t* vblk = a.vc + slot * a.v_block_bytes;

  // value bit words for this group: plane p, coordinates lane and lane+64
  uint32_t vw_lo[4] = {0, 0, 0, 0};
  uint32_t vw_hi[4] = {0, 0, 0, 0};
  uint32_t vmask = 0;

  for (int pos = t0; pos < t1; ++pos) {
    const int t = pos % kBlock;
    const int64_t in_idx = ((static_cast<int64_t>(b) * a.n_new + (pos - start)) * a.n_kv + h) * kD;

    // ------------------------------------------------------------ keys
    const float xk_lo = load_in(a.k_new, in_idx + lane, a.in_dtype);
    const float xk_hi = load_in(a.k_new, in_idx + lane + 64, a.in_dtype);
    if (a.k_codec == RAW_F32) {
      float* row = reinterpret_cast<float*>(kblk) + t * kD;
      row[lane] = xk_lo;
      row[lane + 64] = xk_hi;
    } else if (a.k_codec == Q8_BLOCK32) {
      float m_lo = fabsf(xk_lo), m_hi = fabsf(xk_hi);
      // max inside each 32-lane block
      m_lo = fmaxf(m_lo, lane_xor<16>(m_lo));
      m_hi = fmaxf(m_hi, lane_xor<16>(m_hi));
      m_lo = row_max16(m_lo);
      m_hi = row_max16(m_hi);
      const uint16_t s_lo = norm_to_f16(m_lo / 127.0f);
      const uint16_t s_hi = norm_to_f16(m_hi / 127.0f);
      const float sf_lo = f16_to_f32(s_lo), sf_hi = f16_to_f32(s_hi);
      int k_lo = 0, k_hi = 0;
      if (sf_lo > 0.0f) k_lo = static_cast<int>(fminf(fmaxf(rintf(xk_lo / sf_lo), -127.0f), 127.0f));
      if (sf_hi > 0.0f) k_hi = static_cast<int>(fminf(fmaxf(rintf(xk_hi / sf_hi), -127.0f), 127.0f));
      int8_t* row = reinterpret_cast<int8_t*>(kblk) + t * kD;
      row[lane] = static_cast<int8_t>(k_lo);
      row[lane + 64] = static_cast<int8_t>(k_hi);
      uint16_t* sc = reinterpret_cast<uint16_t*>(kblk + kBlock * kD) + t * (kD / 32);
      if ((lane & 31) == 0) {
        sc[lane >> 5] = s_lo;          // blocks 0, 1
        sc[2 + (lane >> 5)] = s_hi;    // blocks 2, 3
      }
    } else {
      const PolarOut o = polar_codes(xk_lo, xk_hi, a.tb.dk, a.tb.kb, a.k_bits, lane);
      uint32_t* planes = reinterpret_cast<uint32_t*>(kblk);
      const int plane_words = (kD / 32) * kBlock;
      for (int p = 0; p < a.k_bits; ++p) {
        const uint64_t mlo = __ballot((o.c_lo >> p) & 1);
        const uint64_t mhi = __ballot((o.c_hi >> p) & 1);
        if (lane < 4) planes[p * plane_words + lane * kBlock + slot_of(t)] = pick_word(mlo, mhi, lane);
      }
      uint8_t* after = kblk + 4 * a.k_bits * plane_words;
      if (a.k_codec == POLAR_QJL) {
        const float nf = f16_to_f32(o.n16);
        const float r_lo = fmaf(-nf, a.tb.ck[o.c_lo], o.y_lo);
        const float r_hi = fmaf(-nf, a.tb.ck[o.c_hi], o.y_hi);
        const double sr = wave_tree_sumsq(r_lo, r_hi);
        const float rho = static_cast<float>(sqrt(sr / static_cast<double>(kD)));
        float z_lo = 0.0f, z_hi = 0.0f;
        for (int i = 0; i < 64; ++i) {
          const float rl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r_lo), i));
          const float rh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r_hi), i));
          z_lo = fmaf(st_lds[i * kM + lane], rl, z_lo);
          z_lo = fmaf(st_lds[(i + 64) * kM + lane], rh, z_lo);
          z_hi = fmaf(st_lds[i * kM + lane + 64], rl, z_hi);
          z_hi = fmaf(st_lds[(i + 64) * kM + lane + 64], rh, z_hi);
        }
        const uint64_t slo = __ballot(z_lo >= 0.0f);
        const uint64_t shi = __ballot(z_hi >= 0.0f);
        uint32_t* sgn = reinterpret_cast<uint32_t*>(after);
        if (lane < 4) sgn[lane * kBlock + slot_of(t)] = pick_word(slo, shi, lane);
        after += 4 * (kM / 32) * kBlock;
        if (lane == 0) reinterpret_cast<uint16_t*>(after + 2 * kBlock)[slot_of(t)] = norm_to_f16(rho);
      }
      if (lane == 0) reinterpret_cast<uint16_t*>(after)[slot_of(t)] = o.n16;
    }

    // ---------------------------------------------------------- values
    const float xv_lo = load_in(a.v_new, in_idx + lane, a.in_dtype);
    const float xv_hi = load_in(a.v_new, in_idx + lane + 64, a.in_dtype);
    if (a.v_codec == RAW_F32) {
      float* row = reinterpret_cast<float*>(vblk) + t * kD;
      row[lane] = xv_lo;
      row[lane + 64] = xv_hi;
    } else {
      const PolarOut o = polar_codes(xv_lo, xv_hi, a.tb.dv, a.tb.vb, a.v_bits, lane);
      const uint32_t bit = 1u << (t & 31);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if (p < a.v_bits) {
          if ((o.c_lo >> p) & 1) vw_lo[p] |= bit;
          if ((o.c_hi >> p) & 1) vw_hi[p] |= bit;
        }
      }
      vmask |= bit;
      if (lane == 0) reinterpret_cast<uint16_t*>(vblk + 4 * a.v_bits * 4 * kD)[slot_of(t)] = o.n16;
    }
  }

  if (a.v_codec == POLAR) {
    uint32_t* planes = reinterpret_cast<uint32_t*>(vblk);
    const int j = (t0 % kBlock) / 32;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p < a.v_bits) {
        uint32_t* w = planes + p * 4 * kD + j * kD;
        w[lane] = (w[lane] & ~vmask) | vw_lo[p];
        w[lane + 64] = (w[lane + 64] & ~vmask) | vw_hi[p];
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
  const int total = a.batch * a.n_kv * a.groups_per_seq;
  if (total <= 0 || a.n_new <= 0) return hipSuccess;
  const int grid = (total + kWavesPerWg - 1) / kWavesPerWg;
  const size_t lds = (a.k_codec == POLAR_QJL) ? sizeof(float) * kD * kM : 0;
  hipLaunchKernelGGL(quant_kernel, dim3(grid), dim3(64 * kWavesPerWg), lds, stream, a);
  return hipGetLastError();
}

}  // namespace tq
