// tq_quant.hip -- quantize-on-append for gfx950 (wave64).
//
// Method (wis-web.com reader, article on TurboQuant in a llama.cpp fork,
// PolarQuant and QJL paragraphs): rotate each vector with a seeded,
// randomised Walsh-Hadamard transform so its coordinates follow a known law,
// keep the radius (fp16) and code the direction per coordinate with a fixed
// codebook for that law; for keys, add the signs of a Gaussian sketch of the
// residual and the residual's norm (the 1-bit QJL corrector).
//
// Mapping: a wavefront owns one (sequence, KV head, 32-position group) of the
// append and takes it as two tiles of 16 positions.  Inside a tile, lane l
// serves position l & 15 with 32 of its 128 coordinates in registers; the
// four lanes l & 15 + 16 g (g = 0..3) of a position hold the rest.  Which
// coordinate bit sits on a register-index bit and which on lane bit 4 or 5
// changes as the work proceeds: a permlane swap of a register pair across
// lane bit 4 or 5 exchanges the roles of that lane bit and that register bit.
// With it,
//   * every FWHT stage and every level of the fp64 pairwise norm tree is an
//     in-lane add/sub: stages and levels keep the format's order (stages
//     h = 1..64, tree levels 64..1) and pairing, so the rotated values and
//     the norms are bit-identical to any engine that follows the format;
//   * the residual of a tile, r[16 positions][128], is already the B operand
//     of the fp16 matrix instruction (8 of a lane's coordinates per
//     instruction), so the sketch S r of 16 positions is 96 MFMA 16x16x32:
//     S staged once per workgroup in LDS as fp16 high and low parts, the
//     residual split the same way, hi hi + lo hi + hi lo (products exact in
//     fp32, far inside the sign band the format allows);
//   * code bits come from a binary search over the sorted boundaries and
//     are shifted into in-lane words (an add with the compare mask as carry);
//     key bit-planes (token-major words) take them as they are, value
//     bit-planes (coordinate-major words, one bit per position) after a
//     16 x 16 bit transpose across the 16 lanes of a row.
// This file is compiled with -ffp-contract=off: the residual uses an explicit
// fmaf and nothing else may be fused.

#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_quant_unit.h"

namespace tq {
namespace {

using namespace qunit;

template <int KB, int VB, bool QJL>
__global__ __launch_bounds__(64 * kWavesPerWg) __attribute__((amdgpu_waves_per_eu(4))) void quant_kernel(QuantArgs a) {
  // S as fp16 high and low parts, row j = sketch row, padded rows
  __shared__ __attribute__((aligned(16))) _Float16 s_hi[QJL ? kM * kSRowH : 8];
  __shared__ __attribute__((aligned(16))) _Float16 s_lo[QJL ? kM * kSRowH : 8];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  if constexpr (QJL) {
    const float4* src = reinterpret_cast<const float4*>(a.tb.s);
    for (int i = threadIdx.x; i < kM * kD / 4; i += blockDim.x) {
      const int row = i / (kD / 4), c4 = i % (kD / 4);
      const float4 f = src[i];
      const float x[4] = {f.x, f.y, f.z, f.w};
      _Float16 h[4], l[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[k] = static_cast<_Float16>(x[k]);
        l[k] = static_cast<_Float16>(x[k] - static_cast<float>(h[k]));
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        s_hi[row * kSRowH + 4 * c4 + k] = h[k];
        s_lo[row * kSRowH + 4 * c4 + k] = l[k];
      }
    }
    __syncthreads();
  }

  const int item = blockIdx.x * kWavesPerWg + wave;
  const int total = a.batch * a.n_kv * a.groups_per_seq;
  if (item >= total) return;
  Unit u;
  const int gi = item % a.groups_per_seq;
  const int rest = item / a.groups_per_seq;
  u.h = rest % a.n_kv;
  u.b = rest / a.n_kv;
  const int start = a.seq_lens[u.b];
  const int end = start + a.n_new;
  u.grp = start / 32 + gi;
  u.t0 = max(start, u.grp * 32);
  u.t1 = min(min(end, u.grp * 32 + 32), a.max_ctx);
  if (u.t0 >= u.t1) return;
  const int blk = u.t0 / kBlock;
  const int64_t slot = (static_cast<int64_t>(u.b) * a.n_kv + u.h) * a.n_blocks + blk;
  u.kblk = a.kc + slot * a.k_block_bytes;
  u.vblk = a.vc + slot * a.v_block_bytes;
  quant_unit<KB, VB, QJL>(a, u, SHalves{s_hi, s_lo}, lane);
}

// One new position per sequence (serving appends): two wavefronts per
// (sequence, KV head), the even one for its key, the odd one for its value.
template <int KB, int VB, bool QJL>
__global__ __launch_bounds__(256) void token_kernel(QuantArgs a) {
  __shared__ __attribute__((aligned(16))) float r_lds[2][kD];   // residuals of the two key wavefronts
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int unit = blockIdx.x * 2 + (wave >> 1);
  if (unit >= a.batch * a.n_kv) return;
  const int h = unit % a.n_kv;
  const int b = unit / a.n_kv;
  const int pos = a.seq_lens[b];
  if (pos >= a.max_ctx) return;
  const int64_t cslot = (static_cast<int64_t>(b) * a.n_kv + h) * a.n_blocks + pos / kBlock;
  const int64_t in_idx = (static_cast<int64_t>(b) * a.n_kv + h) * kD;
  if ((wave & 1) == 0) {
    token_keys<KB, QJL, kD>(a, in_idx, a.kc + cslot * a.k_block_bytes, pos % kBlock, a.tb.s, r_lds[wave >> 1], lane);
  } else {
    token_values<VB>(a, in_idx, a.vc + cslot * a.v_block_bytes, pos % kBlock, lane);
  }
}

template <int KB, bool QJL>
hipError_t launch_token(const QuantArgs& a, hipStream_t stream) {
  const dim3 grid((a.batch * a.n_kv + 1) / 2), blk(256);
  switch (a.v_codec == POLAR ? a.v_bits : 0) {
    case 0: hipLaunchKernelGGL((token_kernel<KB, 0, QJL>), grid, blk, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((token_kernel<KB, 2, QJL>), grid, blk, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((token_kernel<KB, 3, QJL>), grid, blk, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((token_kernel<KB, 4, QJL>), grid, blk, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KB, bool QJL>
hipError_t launch_k(const QuantArgs& a, int grid, hipStream_t stream) {
  if (a.n_new == 1) return launch_token<KB, QJL>(a, stream);
  const dim3 blk(64 * kWavesPerWg);
  switch (a.v_codec == POLAR ? a.v_bits : 0) {
    case 0: hipLaunchKernelGGL((quant_kernel<KB, 0, QJL>), dim3(grid), blk, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((quant_kernel<KB, 2, QJL>), dim3(grid), blk, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((quant_kernel<KB, 3, QJL>), dim3(grid), blk, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((quant_kernel<KB, 4, QJL>), dim3(grid), blk, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
  const int total = a.batch * a.n_kv * a.groups_per_seq;
  if (total <= 0 || a.n_new <= 0) return hipSuccess;
  const int grid = (total + kWavesPerWg - 1) / kWavesPerWg;
  // recursive polar tensors have their own kernel: with K stored that way the
  // K part below matches no branch and writes nothing
  if (a.k_codec == POLAR_TREE && a.v_codec == POLAR_TREE) return hipSuccess;
  if (a.k_codec == POLAR_QJL) {
    switch (a.k_bits) {
      case 2: return launch_k<2, true>(a, grid, stream);
      case 3: return launch_k<3, true>(a, grid, stream);
      case 4: return launch_k<4, true>(a, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (a.k_codec == POLAR) {
    switch (a.k_bits) {
      case 2: return launch_k<2, false>(a, grid, stream);
      case 3: return launch_k<3, false>(a, grid, stream);
      case 4: return launch_k<4, false>(a, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  return launch_k<0, false>(a, grid, stream);
}

}  // namespace tq
