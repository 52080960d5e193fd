// tq_mfma_ops.h -- device helpers shared by the matrix-core decode kernels:
// bit words as fp4 matrix operands, the scaled fp8 x fp4 matrix instruction,
// buffer resources over a (sequence, KV head)'s blocks, waits and barriers,
// the split merge and the serving step's store of the new position.
#pragma once

#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_quant_unit.h"
// the quantiser above is exact-rounding code; what follows may contract
#pragma clang fp contract(fast)

namespace tq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int B>
struct NTerms {
  static constexpr int n = (B == 2) ? 2 : (B == 3 ? 4 : (B == 4 ? 8 : 1));
};

// Bits of term T: code planes for T < B, then XORs of three planes.
template <int B>
__device__ __forceinline__ uint32_t term_word(const uint32_t* w, int T) {
  if (T < B) return w[T];
  const int u = T - B;
  const int i0 = (u == 3) ? 1 : 0;
  const int i1 = (u <= 1) ? 1 : 2;
  const int i2 = (u == 0) ? 2 : 3;
  return __builtin_amdgcn_bitop3_b32(w[i0], w[i1], w[i2], 0x96);   // three-input XOR in one instruction
}

// 32 bits -> 32 fp4 elements with each bit used where it lies: element
// 8d + n is nibble n of dword d and takes bit 4n + d of w into nibble field d,
// the other fields fixed: d = 0 (mantissa) {4, 6}, d = 1 (low exponent bit)
// {2, 4}, d = 2 (high exponent bit) {0, 2}, d = 3 (sign) {+1, -1}.  With
// s = +1 for a set bit the element is 5 + s, 3 + s, 1 + s, -s: one AND(-OR) per
// dword.  The matrix operand on the other side carries -1 on the d = 3
// elements, and the offsets 5, 3, 1 are removed afterwards: for keys one
// constant per head, for values the product of the step's probabilities with
// a fixed operand (rows of all-one and all-zero words, whose mean is the
// offset row 5, 3, 1, 0).
// The masks (scalar registers) and fills (vector registers) of the
// expansion, made once per kernel so that each dword is one v_and_or_b32 (its
// three-operand form takes no literal; with literals the compiler splits it
// in two).  The empty asm statements only hide the values from constant
// folding and emit nothing: every instruction that writes an operand stays
// visible to the compiler, which pads the matrix instructions' operand
// hazards.
struct Fp4Fill {
  uint32_t m0, m1, m3;   // 0x11111111, 0x22222222, 0x88888888
  uint32_t c0, c1, c3;   // 0x66666666, 0x44444444, 0x22222222
};
__device__ __forceinline__ Fp4Fill fp4_fill() {
  Fp4Fill k{0x11111111u, 0x22222222u, 0x88888888u, 0x66666666u, 0x44444444u, 0x22222222u};
  asm volatile("" : "+s"(k.m0), "+s"(k.m1), "+s"(k.m3));
  asm volatile("" : "+v"(k.c0), "+v"(k.c1), "+v"(k.c3));
  return k;
}
__device__ __forceinline__ v8i expand_fp4_affine(uint32_t w, const Fp4Fill& k) {
  v8i r;
  r[0] = static_cast<int>((w & k.m0) | k.c0);
  r[1] = static_cast<int>((w & k.m1) | k.c1);
  r[2] = static_cast<int>(w & 0x44444444u);
  r[3] = static_cast<int>((w & k.m3) | k.c3);
  r[4] = r[5] = r[6] = r[7] = 0;
  return r;
}

// The same for the value operand, with the sign field taken from the
// complemented bit: element 8 * 3 + n is +s instead of -s, so the operand on
// the other side (the probability digits) needs no sign flip on those
// k-slots; fields 0..2 as above.
__device__ __forceinline__ v8i expand_fp4_affine_v(uint32_t w, const Fp4Fill& k) {
  v8i r;
  r[0] = static_cast<int>((w & k.m0) | k.c0);
  r[1] = static_cast<int>((w & k.m1) | k.c1);
  r[2] = static_cast<int>(w & 0x44444444u);
  r[3] = static_cast<int>((~w & k.m3) | k.c3);
  r[4] = r[5] = r[6] = r[7] = 0;
  return r;
}

__device__ __forceinline__ int exponent_of(float x) {   // floor(log2 x), x > 0 normal
  return static_cast<int>((__float_as_uint(x) >> 23) & 0xffu) - 127;
}

__device__ __forceinline__ float h2f(uint32_t bits16) { return __half2float(__ushort_as_half(static_cast<uint16_t>(bits16))); }

// fp6 (e2m3) digits x fp4 code operand: both at most 6 bits, the 4-pass rate
__device__ __forceinline__ v4f mfma_fp6_fp4(const v8i& a, const v8i& b, const v4f& c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 2, 4, 0, sa, 0, 127);
}
__device__ __forceinline__ v4f mfma_fp8_fp4(const v8i& a, const v8i& b, const v4f& c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, 127);
}
__device__ __forceinline__ v4f mfma_fp4_fp8(const v8i& a, const v8i& b, const v4f& c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, 127, 0, sb);
}

// Buffer resource over one (sequence, KV head)'s blocks [0, n_valid): reads at
// offsets past the end return zero without touching memory (raw buffer,
// stride 0; the range check covers the per-lane offset).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t* base, int64_t block_bytes, int n_valid) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), static_cast<short>(0),
                                           static_cast<int>(block_bytes * n_valid), 0x00020000);
}

// Workgroup barrier for shared-memory data only: waits for this wave's
// shared-memory operations, not for its copies in flight (a fenced barrier
// would drain those), and keeps the compiler from moving memory accesses
// across it.  Copies into the ring are covered by explicit waits.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Waits until at most n copies (or other vector memory operations) issued by
// this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Max / sum over the 32 lanes of each half-wave (rows via DPP, then the
// swizzle that swaps 16-lane halves within 32 lanes).
__device__ __forceinline__ float half_max32(float x) {
  x = row_max16(x);
  return fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F)));
}
__device__ __forceinline__ float half_sum32(float x) {
  x = row_sum16(x);
  return x + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}

// Merge of the split partials by the workgroup that arrives last: partial s
// of query head g holds o_s = D_V H acc_s / d (already in the original frame),
// its running max m_s (natural-log units) and denominator l_s; the output is
// sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M}.  Wave g merges head g; splits
// are taken 32 at a time with every load of a round in flight together; lane
// (half, i4) accumulates float4 i4 of the round's splits of parity half.
__device__ __forceinline__ void merge_splits(const DecodeArgs& a, int b, int hq0, int G, uint32_t* counter, int w,
                                             int lane) {
  // every split has arrived (counter); the partials were written through to
  // the device-coherent level and are read back with device-scope coherent
  // loads (sc1), so no cache invalidation is needed
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  constexpr int kCoherent = 16;   // sc1
  if (w < G) {
    const int pstride = kPartialStride;
    const int i4 = lane & 31;
    const int half = lane >> 5;
    const float* pp = a.partials + (static_cast<int64_t>(b) * a.n_q + hq0 + w) * a.n_splits * kPartialStride;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(pp), static_cast<short>(0), a.n_splits * pstride * 4, 0x00020000);
    float M = -INFINITY, L = 0.0f;
    float4 A = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int c0 = 0; c0 < a.n_splits; c0 += 32) {
      // splits past n_splits read as zero (out of the resource's range):
      // m = 0, l = 0, acc = 0, weight forced to zero below
      const int sm = c0 + i4;
      const v2u mlv = __builtin_amdgcn_raw_buffer_load_b64(rp, (sm * pstride + kD) * 4, 0, kCoherent);
      v4u v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rp, ((c0 + half + 2 * u) * pstride + 4 * i4) * 4, 0, kCoherent);
      const float mx = (sm < a.n_splits) ? __uint_as_float(mlv[0]) : -INFINITY;
      const float mc = half_max32(mx);
      const float Mn = fmaxf(M, mc);
      const float fo = (M == -INFINITY) ? 0.0f : __expf(M - Mn);
      M = Mn;
      const float wgt = (mx == -INFINITY) ? 0.0f : __expf(mx - M);
      const float lw = half_sum32(__uint_as_float(mlv[1]) * wgt);
      L = L * fo + lw;
      A.x *= fo;
      A.y *= fo;
      A.z *= fo;
      A.w *= fo;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float ws = __shfl(wgt, half + 2 * u, 64);   // lane half + 2u holds split c0 + half + 2u
        A.x = fmaf(__uint_as_float(v[u][0]), ws, A.x);
        A.y = fmaf(__uint_as_float(v[u][1]), ws, A.y);
        A.z = fmaf(__uint_as_float(v[u][2]), ws, A.z);
        A.w = fmaf(__uint_as_float(v[u][3]), ws, A.w);
      }
    }
    A.x += __shfl_xor(A.x, 32, 64);
    A.y += __shfl_xor(A.y, 32, 64);
    A.z += __shfl_xor(A.z, 32, 64);
    A.w += __shfl_xor(A.w, 32, 64);
    if (half == 0) {
      const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
      *reinterpret_cast<float4*>(a.out + (static_cast<int64_t>(b) * a.n_q + hq0 + w) * kD + 4 * i4) =
          make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Serving step (a launch with a new position per sequence): the workgroups
// whose split holds position len_in of (sequence b, KV head h) first store
// that position's record -- wavefront 0 its key, wavefront 1 its value, with
// the append path's one-position quantiser -- and start their copies of the
// cache only afterwards.  With several head groups per KV head each of them
// writes the same bytes.
template <int KB, bool QJL, int VB>
__device__ __forceinline__ void fused_append(const DecodeArgs& a, int b, int h, int len_in, int w, int lane,
                                             float* r_lds) {
  if (w < 2) {
    QuantArgs qa{};
    qa.tb = a.tb;
    qa.k_new = a.k_new;
    qa.v_new = a.v_new;
    qa.in_dtype = a.in_dtype;
    qa.k_codec = a.k_codec;
    qa.k_bits = a.k_bits;
    qa.v_codec = a.v_codec;
    qa.v_bits = a.v_bits;
    const int64_t cslot = (static_cast<int64_t>(b) * a.n_kv + h) * a.n_blocks + len_in / kBlock;
    const int64_t in_idx = (static_cast<int64_t>(b) * a.n_kv + h) * kD;   // [batch][1][n_kv][d]
    if (w == 0) {
      qunit::token_keys<(KB == 8 ? 0 : KB), QJL, kD>(qa, in_idx, const_cast<uint8_t*>(a.kc) + cslot * a.k_block_bytes,
                                                     len_in % kBlock, a.tb.s, r_lds, lane);
    } else {
      qunit::token_values<VB>(qa, in_idx, const_cast<uint8_t*>(a.vc) + cslot * a.v_block_bytes, len_in % kBlock, lane);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // the record's stores have completed
  }
  __syncthreads();
  // The record's stores went through this compute unit's write-through vector
  // cache; dropping that cache's lines as well (a workgroup-scope invalidate,
  // not the device-wide one an agent-scope acquire issues) leaves no stale
  // copy of the block that another workgroup on this unit fetched earlier.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  asm volatile("buffer_inv sc0\n\ts_waitcnt vmcnt(0)" ::: "memory");
}


}  // namespace
}  // namespace tq
