// tq_dequant.hip -- packed records back to fp32 vectors.
//
// x_hat = D H (n16 C[code]) / d inverts the rotation of the PolarQuant step
// (wis-web.com reader, TurboQuant article, PolarQuant paragraph: H H = d I,
// so H / d undoes the raw transform).  With TQ_DEQ_QJL keys also get the
// QJL correction rho sqrt(pi/2)/m R^T S^T sign (R = H D / sqrt d), whose
// inner product with a query is the estimator's correction term (the
// article's QJL paragraph).  q8 keys are s16 * k8; RAW is a copy.
// Recursive polar records (the radius + angle step read as a pairwise tree)
// give y_hat = sqrt(d) n16 u, coordinate i of u being the product over the 7
// levels of the cos or sin of its ancestors' centroid angles (sin when i lies
// in the right half of the ancestor), then the same inverse rotation.
//
// Mapping: one wavefront per (position, KV head); lane l produces
// coordinates l and l + 64; the transform is the same cross-lane FWHT as on
// the append side.

#include <hip/hip_fp16.h>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWavesPerWg = 4;

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return __half2float(__ushort_as_half(h)); }

__device__ __forceinline__ void wave_fwht128(float& lo, float& hi, int lane) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const float plo = __shfl_xor(lo, h, 64);
    const float phi = __shfl_xor(hi, h, 64);
    if (lane & h) {
      lo = plo - lo;
      hi = phi - hi;
    } else {
      lo = lo + plo;
      hi = hi + phi;
    }
  }
  const float a = lo, b = hi;
  lo = a + b;
  hi = a - b;
}

// u_i from the codes of its ancestors: code(s) returns the code of angle slot s
template <typename CodeOf>
__device__ __forceinline__ float tree_coord(int i, const TreeTab* T, CodeOf code) {
  const float2 c1 = T->cs1[code(64 + (i >> 1))];
  float u = (i & 1) ? c1.y : c1.x;
#pragma unroll
  for (int l = 2; l <= 7; ++l) {
    const float2 cs = T->cs[l][code((1 << (7 - l)) + (i >> l))];
    u *= ((i >> (l - 1)) & 1) ? cs.y : cs.x;
  }
  return u;
}

__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * kWavesPerWg + (threadIdx.x >> 6);
  if (item >= a.count * a.n_kv) return;
  const int h = item % a.n_kv;
  const int k = item / a.n_kv;
  const int pos = a.start + k;
  const int t = pos % kBlock;
  const int sl = slot_of(t);
  const int64_t slot = (static_cast<int64_t>(a.b) * a.n_kv + h) * a.n_blocks + pos / kBlock;
  const int64_t out_idx = (static_cast<int64_t>(k) * a.n_kv + h) * kD;
  const float inv_d = 1.0f / static_cast<float>(kD);

  if (a.k_out != nullptr) {
    const uint8_t* kb = a.kc + slot * a.k_block_bytes;
    float lo, hi;
    if (a.k_codec == RAW_F32) {
      const float* row = reinterpret_cast<const float*>(kb) + t * kD;
      lo = row[lane];
      hi = row[lane + 64];
    } else if (a.k_codec == Q8_BLOCK32) {
      const int8_t* row = reinterpret_cast<const int8_t*>(kb) + t * kD;
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(kb + kBlock * kD) + t * (kD / 32);
      lo = f16_to_f32(sc[lane >> 5]) * static_cast<float>(row[lane]);
      hi = f16_to_f32(sc[2 + (lane >> 5)]) * static_cast<float>(row[lane + 64]);
    } else if (a.k_codec == POLAR_TREE) {
      const uint32_t* planes = reinterpret_cast<const uint32_t*>(kb);
      const int nb1 = a.k_bits - 1;
      const uint32_t* l1 = planes + nb1 * 4 * kBlock;
      auto code = [&](int s) {
        int c = 0;
        for (int p = 0; p < nb1; ++p) c |= ((planes[(p * 4 + (s >> 5)) * kBlock + sl] >> (s & 31)) & 1u) << p;
        if (s >= 64)
          for (int x = 0; x < 2; ++x) c |= ((l1[(x * 2 + (s >> 5) - 2) * kBlock + sl] >> (s & 31)) & 1u) << (nb1 + x);
        return c;
      };
      const float r = 11.313708498984761f * f16_to_f32(reinterpret_cast<const uint16_t*>(l1 + 4 * kBlock)[sl]);
      lo = r * tree_coord(lane, a.tb.tk, code);
      hi = r * tree_coord(lane + 64, a.tb.tk, code);
      wave_fwht128(lo, hi, lane);
      lo = a.tb.dk[lane] * lo * inv_d;
      hi = a.tb.dk[lane + 64] * hi * inv_d;
    } else {
      const uint32_t* planes = reinterpret_cast<const uint32_t*>(kb);
      const int plane_words = (kD / 32) * kBlock;
      int c_lo = 0, c_hi = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if (p < a.k_bits) {
          c_lo |= ((planes[p * plane_words + (lane >> 5) * kBlock + sl] >> (lane & 31)) & 1u) << p;
          c_hi |= ((planes[p * plane_words + (2 + (lane >> 5)) * kBlock + sl] >> (lane & 31)) & 1u) << p;
        }
      }
      const uint8_t* after = kb + 4 * a.k_bits * plane_words;
      const uint8_t* norms = after + ((a.k_codec == POLAR_QJL) ? 4 * (kM / 32) * kBlock : 0);
      const float n16 = f16_to_f32(reinterpret_cast<const uint16_t*>(norms)[sl]);
      lo = n16 * a.tb.ck[c_lo];
      hi = n16 * a.tb.ck[c_hi];
      wave_fwht128(lo, hi, lane);
      lo = a.tb.dk[lane] * lo * inv_d;
      hi = a.tb.dk[lane + 64] * hi * inv_d;
      if (a.k_codec == POLAR_QJL && a.qjl) {
        const uint32_t* sg = reinterpret_cast<const uint32_t*>(after);
        float u_lo = 0.0f, u_hi = 0.0f;
        for (int j = 0; j < kM; ++j) {
          const bool pos_sign = (sg[(j >> 5) * kBlock + sl] >> (j & 31)) & 1u;
          const float s_lo = a.tb.s[j * kD + lane];
          const float s_hi = a.tb.s[j * kD + lane + 64];
          u_lo += pos_sign ? s_lo : -s_lo;
          u_hi += pos_sign ? s_hi : -s_hi;
        }
        wave_fwht128(u_lo, u_hi, lane);
        const float rho = f16_to_f32(reinterpret_cast<const uint16_t*>(norms + 2 * kBlock)[sl]);
        const float kq = rho * 1.2533141373155003f / static_cast<float>(kM) * 0.08838834764831845f;
        lo += kq * a.tb.dk[lane] * u_lo;
        hi += kq * a.tb.dk[lane + 64] * u_hi;
      }
    }
    a.k_out[out_idx + lane] = lo;
    a.k_out[out_idx + lane + 64] = hi;
  }

  if (a.v_out != nullptr) {
    const uint8_t* vb = a.vc + slot * a.v_block_bytes;
    float lo, hi;
    if (a.v_codec == RAW_F32) {
      const float* row = reinterpret_cast<const float*>(vb) + t * kD;
      lo = row[lane];
      hi = row[lane + 64];
    } else if (a.v_codec == POLAR_TREE) {
      const uint32_t* planes = reinterpret_cast<const uint32_t*>(vb);
      const int nb1 = a.v_bits - 1;
      const uint32_t* l1 = planes + nb1 * 4 * kD;
      const int j = t >> 5, e = t & 31;
      auto code = [&](int s) {
        int c = 0;
        for (int p = 0; p < nb1; ++p) c |= ((planes[(p * 4 + j) * kD + s] >> e) & 1u) << p;
        if (s >= 64)
          for (int x = 0; x < 2; ++x) c |= ((l1[(x * 4 + j) * (kD / 2) + s - 64] >> e) & 1u) << (nb1 + x);
        return c;
      };
      const float r = 11.313708498984761f * f16_to_f32(reinterpret_cast<const uint16_t*>(l1 + 2 * 4 * (kD / 2))[sl]);
      lo = r * tree_coord(lane, a.tb.tv, code);
      hi = r * tree_coord(lane + 64, a.tb.tv, code);
      wave_fwht128(lo, hi, lane);
      lo = a.tb.dv[lane] * lo * inv_d;
      hi = a.tb.dv[lane + 64] * hi * inv_d;
    } else {
      const uint32_t* planes = reinterpret_cast<const uint32_t*>(vb);
      int c_lo = 0, c_hi = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if (p < a.v_bits) {
          c_lo |= ((planes[p * 4 * kD + (t >> 5) * kD + lane] >> (t & 31)) & 1u) << p;
          c_hi |= ((planes[p * 4 * kD + (t >> 5) * kD + lane + 64] >> (t & 31)) & 1u) << p;
        }
      }
      const float n16 = f16_to_f32(reinterpret_cast<const uint16_t*>(vb + 4 * a.v_bits * 4 * kD)[sl]);
      lo = n16 * a.tb.cv[c_lo];
      hi = n16 * a.tb.cv[c_hi];
      wave_fwht128(lo, hi, lane);
      lo = a.tb.dv[lane] * lo * inv_d;
      hi = a.tb.dv[lane + 64] * hi * inv_d;
    }
    a.v_out[out_idx + lane] = lo;
    a.v_out[out_idx + lane + 64] = hi;
  }
}

}  // namespace

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t stream) {
  const int total = a.count * a.n_kv;
  if (total <= 0) return hipSuccess;
  const int grid = (total + kWavesPerWg - 1) / kWavesPerWg;
  hipLaunchKernelGGL(dequant_kernel, dim3(grid), dim3(64 * kWavesPerWg), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
