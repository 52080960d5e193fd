// tq_device.h -- small device helpers shared by the decode kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace tq {

// In-place raw FWHT over buf[rows][128] in shared memory; every thread of the
// block participates (contains barriers).
__device__ inline void block_fwht128(float* buf, int rows, int nthreads) {
  for (int h = 1; h < kD; h <<= 1) {
    __syncthreads();
    for (int k = threadIdx.x; k < rows * (kD / 2); k += nthreads) {
      const int g = k / (kD / 2);
      const int r = k % (kD / 2);
      const int lo = (r / h) * 2 * h + (r % h);
      float* v = buf + g * kD;
      const float x = v[lo], y = v[lo + h];
      v[lo] = x + y;
      v[lo + h] = x - y;
    }
  }
  __syncthreads();
}

// Block range of a split: splits [0, n_long) take long_blocks blocks each,
// the later ones chunk_blocks.
__device__ __forceinline__ int split_first_block(const DecodeArgs& a, int split) {
  return (split < a.n_long) ? split * a.long_blocks
                            : a.n_long * a.long_blocks + (split - a.n_long) * a.chunk_blocks;
}
__device__ __forceinline__ int split_block_count(const DecodeArgs& a, int split) {
  return (split < a.n_long) ? a.long_blocks : a.chunk_blocks;
}
// The split whose range holds block blk.
__device__ __forceinline__ int split_of_block(const DecodeArgs& a, int blk) {
  const int lb = a.n_long * a.long_blocks;
  return (blk < lb) ? blk / a.long_blocks : a.n_long + (blk - lb) / a.chunk_blocks;
}

// Max / sum over the 16 lanes of a row (DPP: xor 1, xor 2, half-row mirror,
// row mirror); every lane of the row ends with the result.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

// Value of lane (l ^ H) for lane l, by the cheapest cross-lane route: DPP
// within 16-lane rows (xor 1, 2 as quad permutations; xor 4 = xor 3 then
// xor 7; xor 8 = xor 7 then xor 15 via the half-row and row mirrors), the
// 32-lane swizzle for xor 16, a 32-lane swap for xor 32.
template <int H>
__device__ __forceinline__ int lane_xor_i(int v) {
  if constexpr (H == 1) return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  if constexpr (H == 2) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  if constexpr (H == 4) {
    const int u = __builtin_amdgcn_update_dpp(0, v, 0x1B, 0xF, 0xF, false);
    return __builtin_amdgcn_update_dpp(0, u, 0x141, 0xF, 0xF, false);
  }
  if constexpr (H == 8) {
    const int u = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
    return __builtin_amdgcn_update_dpp(0, u, 0x140, 0xF, 0xF, false);
  }
  if constexpr (H == 16) return __builtin_amdgcn_ds_swizzle(v, 0x401F);
  if constexpr (H == 32) {   // one swap of the register with itself, then each half takes the other's copy
    const auto r = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(v), static_cast<unsigned>(v), false, false);
    return static_cast<int>((__lane_id() & 32) ? r[0] : r[1]);
  }
  return v;
}
template <int H>
__device__ __forceinline__ float lane_xor(float x) {
  return __int_as_float(lane_xor_i<H>(__float_as_int(x)));
}
template <int H>
__device__ __forceinline__ double lane_xor(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t lo = static_cast<uint32_t>(lane_xor_i<H>(static_cast<int>(u)));
  const uint32_t hi = static_cast<uint32_t>(lane_xor_i<H>(static_cast<int>(u >> 32)));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

template <int H>
__device__ __forceinline__ void butterfly(float& lo, float& hi, int lane) {
  const float plo = lane_xor<H>(lo), phi = lane_xor<H>(hi);
  const bool up = (lane & H) != 0;
  lo = up ? plo - lo : lo + plo;
  hi = up ? phi - hi : hi + phi;
}

// Raw Sylvester FWHT of 128 values held as (lo = coord lane, hi = coord lane+64).
__device__ __forceinline__ void wave_fwht128(float& lo, float& hi, int lane) {
  butterfly<1>(lo, hi, lane);
  butterfly<2>(lo, hi, lane);
  butterfly<4>(lo, hi, lane);
  butterfly<8>(lo, hi, lane);
  butterfly<16>(lo, hi, lane);
  butterfly<32>(lo, hi, lane);
  const float x = lo, y = hi;
  lo = x + y;
  hi = x - y;
}

__device__ __forceinline__ float wave_max64(float x) {
  x = row_max16(x);
  x = fmaxf(x, lane_xor<16>(x));
  return fmaxf(x, lane_xor<32>(x));
}
__device__ __forceinline__ float wave_sum64(float x) {
  x = row_sum16(x);
  x += lane_xor<16>(x);
  return x + lane_xor<32>(x);
}

// Partials travel between workgroups on different XCDs (each with its own L2)
// as agent-scope atomic stores, which write through to the device-coherent
// level, so the writers need no device-wide cache write-back (a
// __threadfence).  A workgroup publishes its partials, waits for its stores
// to complete, then bumps the (sequence, KV head) counter; the workgroup that
// takes the counter to n_splits acquires (drops its own L2's stale lines) and
// merges with ordinary vector loads.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns true in every thread of the workgroup that arrives last.
__device__ inline bool arrive_last(uint32_t* counter, int n_splits, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (prev == static_cast<uint32_t>(n_splits - 1)) ? 1 : 0;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Split-K merge done by the last workgroup of a (sequence, KV head): partials
// hold, per query head and split, acc[128] (rotated frame for POLAR and
// recursive polar values), the running max m (natural-log units) and the
// softmax denominator l.  Writes out = D_V H (sum_s acc_s e^{m_s - M}) /
// (d sum_s l_s e^{m_s - M}) for rotated values, the same without the inverse
// rotation for RAW values.  obuf is a
// shared buffer of G*128 floats.  One wavefront per query head; splits are
// taken 32 at a time with every load of a chunk in flight together; lane
// (half, i4) accumulates float4 i4 of the chunk's splits of parity half.
__device__ inline void combine_splits(const DecodeArgs& a, int b, int h, float* obuf, int nthreads) {
  // every split has arrived (counter); its write-through partials are visible
  // once this workgroup drops stale lines from its own L2
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int G = a.group;
  const int64_t pstride = kPartialStride;
  const int lane = threadIdx.x & 63;
  const int i4 = lane & 31;
  const int half = lane >> 5;
  const int nwaves = nthreads >> 6;
  for (int g = threadIdx.x >> 6; g < G; g += nwaves) {
    const float* pp = a.partials + (static_cast<int64_t>(b) * a.n_q + h * G + g) * a.n_splits * pstride;
    float M = -INFINITY, L = 0.0f;
    float4 A = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int c0 = 0; c0 < a.n_splits; c0 += 32) {
      const int sm = c0 + i4;                       // split whose (m, l) this lane reads
      float2 ml = make_float2(-INFINITY, 0.0f);
      if (sm < a.n_splits) ml = *reinterpret_cast<const float2*>(pp + sm * pstride + kD);
      float4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int s = c0 + half + 2 * u;
        v[u] = (s < a.n_splits) ? *reinterpret_cast<const float4*>(pp + s * pstride + 4 * i4)
                                : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
      float mc = ml.x;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) mc = fmaxf(mc, __shfl_xor(mc, off, 64));
      const float Mn = fmaxf(M, mc);
      const float fo = (M == -INFINITY) ? 0.0f : __expf(M - Mn);
      M = Mn;
      const float wgt = (ml.x == -INFINITY) ? 0.0f : __expf(ml.x - M);   // weight of split c0 + i4
      float lw = ml.y * wgt;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) lw += __shfl_xor(lw, off, 64);
      L = L * fo + lw;
      A.x *= fo;
      A.y *= fo;
      A.z *= fo;
      A.w *= fo;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float ws = __shfl(wgt, half + 2 * u, 64);   // lane half + 2u holds split c0 + half + 2u
        A.x = fmaf(v[u].x, ws, A.x);
        A.y = fmaf(v[u].y, ws, A.y);
        A.z = fmaf(v[u].z, ws, A.z);
        A.w = fmaf(v[u].w, ws, A.w);
      }
    }
    A.x += __shfl_xor(A.x, 32, 64);
    A.y += __shfl_xor(A.y, 32, 64);
    A.z += __shfl_xor(A.z, 32, 64);
    A.w += __shfl_xor(A.w, 32, 64);
    if (half == 0) {
      const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
      obuf[g * kD + 4 * i4 + 0] = A.x * inv;
      obuf[g * kD + 4 * i4 + 1] = A.y * inv;
      obuf[g * kD + 4 * i4 + 2] = A.z * inv;
      obuf[g * kD + 4 * i4 + 3] = A.w * inv;
    }
  }
  const bool rotated = (a.v_codec == POLAR || a.v_codec == POLAR_TREE);
  if (rotated) block_fwht128(obuf, G, nthreads);   // H acc; D_V and 1/d below
  __syncthreads();
  for (int k = threadIdx.x; k < G * kD; k += nthreads) {
    const int g = k / kD, i = k % kD;
    float v = obuf[k];
    if (rotated) v = v * a.tb.dv[i] * (1.0f / static_cast<float>(kD));
    a.out[(static_cast<int64_t>(b) * a.n_q + h * G + g) * kD + i] = v;
  }
  if (threadIdx.x == 0) __hip_atomic_store(a.counters + b * a.n_kv + h, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace tq
