// tq_decode.hip -- single-query decode attention over the packed cache.
//
// What is computed (wis-web.com reader, TurboQuant article: the QJL
// paragraph's 1-bit corrector of the inner-product bias, and the
// llama-server example's flash attention): for every sequence b and query
// head h (KV head h / G), logits
//   l_t = (1/sqrt d) [ (n16_t / d) <q_raw, C_K[c_t]> + rho16_t sqrt(pi/2)/m <sq, sigma_t> ]
// with q_raw = H D_K q (the query rotated like the keys) and
// sq = S q_raw / sqrt(d) (the sketch of the rotated query), then a softmax
// over all stored positions and the weighted sum of values accumulated in the
// rotated frame: acc = sum_t p_t n16V_t C_V[c_t], out = D_V H acc / d (one
// inverse transform per head instead of one per position).  q8 keys use the
// unrotated query and per-block scales; RAW tensors are used as stored.
//
// Mapping: grid (split, KV head, sequence); a 256-thread workgroup serves
// all G query heads of its KV head over one chunk of 128-position blocks,
// keeping a running max and sum per head (online softmax).  Per block:
//   logits  thread = (position t, head parity); keys are token-major planes,
//           so a thread reads its position's words directly;
//   softmax one wavefront per head, wave-reduced max and sum;
//   PV      thread = (coordinate i, head parity); values are coordinate-major
//           planes, so a thread reads the 4 words of its coordinate and walks
//           the block's positions bit by bit.
// Partials (m, l, acc) go to the workspace; the last workgroup of each
// (sequence, KV head) (device-scope counter) merges them by log-sum-exp
// rescaling, applies the inverse rotation and writes the output.

#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return __half2float(__ushort_as_half(h)); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) v = fmaxf(v, __shfl_xor(v, w, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) v += __shfl_xor(v, w, 64);
  return v;
}

__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  __shared__ float qv[kMaxGroup * kD];   // q (or q_raw) per head
  __shared__ float sq[kMaxGroup * kM];   // S q_raw / sqrt(d) per head
  __shared__ float pt[kMaxGroup * kBlock];  // logits, then p * value radius
  __shared__ float kcb[16], vcb[16];
  __shared__ float m_run[kMaxGroup], l_run[kMaxGroup], scale[kMaxGroup];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.group;
  const int len = min(a.seq_lens[b], a.max_ctx);   // never read past the capacity
  const float inv_sqrt_d = 0.08838834764831845f;   // 1/sqrt(128)

  // ---------------------------------------------------------- prologue
  for (int k = tid; k < G * kD; k += kThreads) {
    const int g = k / kD, i = k % kD;
    float v = a.q[(static_cast<int64_t>(b) * a.n_q + h * G + g) * kD + i];
    if (a.k_codec == POLAR || a.k_codec == POLAR_QJL) v *= a.tb.dk[i];
    qv[k] = v;
  }
  if (tid < 16) {
    kcb[tid] = a.tb.ck[tid];
    vcb[tid] = a.tb.cv[tid];
  }
  if (tid < G) {
    m_run[tid] = -INFINITY;
    l_run[tid] = 0.0f;
  }
  if (a.k_codec == POLAR || a.k_codec == POLAR_QJL) block_fwht128(qv, G, kThreads);   // q_raw = H D_K q
  __syncthreads();
  if (a.k_codec == POLAR_QJL) {
    for (int k = tid; k < G * kM; k += kThreads) {
      const int g = k / kM, j = k % kM;
      const float* qg = qv + g * kD;
      float acc = 0.0f;
      for (int i = 0; i < kD; ++i) acc = fmaf(a.tb.st[i * kM + j], qg[i], acc);
      sq[k] = acc * inv_sqrt_d;
    }
  }
  __syncthreads();

  // accumulators: thread owns coordinate i = tid % 128 for heads g = tid/128 + 2u
  const int ci = tid & (kD - 1);
  const int hpar = tid >> 7;
  float acc[kMaxGroup / 2];
#pragma unroll
  for (int u = 0; u < kMaxGroup / 2; ++u) acc[u] = 0.0f;

  const int blk0 = split * a.chunk_blocks;
  const int nblk_seq = (len + kBlock - 1) / kBlock;
  const int blk1 = min(blk0 + a.chunk_blocks, nblk_seq);
  const int64_t slot0 = (static_cast<int64_t>(b) * a.n_kv + h) * a.n_blocks;
  const float alpha = inv_sqrt_d / static_cast<float>(kD);                       // (1/sqrt d)(1/d)
  const float beta = inv_sqrt_d * 1.2533141373155003f / static_cast<float>(kM);  // sqrt(pi/2)/m/sqrt d
  const int kbits = a.k_bits, vbits = a.v_bits;

  for (int blk = blk0; blk < blk1; ++blk) {
    const int n_t = min(kBlock, len - blk * kBlock);
    const uint8_t* kb = a.kc + (slot0 + blk) * a.k_block_bytes;
    const uint8_t* vb = a.vc + (slot0 + blk) * a.v_block_bytes;

    // ------------------------------------------------------- logits
    {
      const int t = tid & (kBlock - 1);
      float lg[kMaxGroup / 2];
#pragma unroll
      for (int u = 0; u < kMaxGroup / 2; ++u) lg[u] = 0.0f;
      if (t < n_t) {
        if (a.k_codec == POLAR || a.k_codec == POLAR_QJL) {
          const uint32_t* planes = reinterpret_cast<const uint32_t*>(kb);
          const int plane_words = (kD / 32) * kBlock;
          float cdot[kMaxGroup / 2], sdot[kMaxGroup / 2];
#pragma unroll
          for (int u = 0; u < kMaxGroup / 2; ++u) cdot[u] = sdot[u] = 0.0f;
          for (int j = 0; j < kD / 32; ++j) {
            uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
            for (int p = 0; p < 4; ++p)
              if (p < kbits) w[p] = planes[p * plane_words + j * kBlock + slot_of(t)];
            for (int e = 0; e < 32; ++e) {
              int c = 0;
#pragma unroll
              for (int p = 0; p < 4; ++p) c |= ((w[p] >> e) & 1u) << p;
              const float cv = kcb[c];
              const int i = j * 32 + e;
#pragma unroll
              for (int u = 0; u < kMaxGroup / 2; ++u) {
                const int g = hpar + 2 * u;
                if (g < G) cdot[u] = fmaf(qv[g * kD + i], cv, cdot[u]);
              }
            }
          }
          const uint8_t* after = kb + 4 * kbits * plane_words;
          float rho = 0.0f;
          if (a.k_codec == POLAR_QJL) {
            const uint32_t* sg = reinterpret_cast<const uint32_t*>(after);
            for (int j = 0; j < kM / 32; ++j) {
              const uint32_t w = sg[j * kBlock + slot_of(t)];
              for (int e = 0; e < 32; ++e) {
                const bool pos = (w >> e) & 1u;
                const int r = j * 32 + e;
#pragma unroll
                for (int u = 0; u < kMaxGroup / 2; ++u) {
                  const int g = hpar + 2 * u;
                  if (g < G) {
                    const float s = sq[g * kM + r];
                    sdot[u] += pos ? s : -s;
                  }
                }
              }
            }
            after += 4 * (kM / 32) * kBlock;
            rho = f16_to_f32(reinterpret_cast<const uint16_t*>(after + 2 * kBlock)[slot_of(t)]);
          }
          const float n16 = f16_to_f32(reinterpret_cast<const uint16_t*>(after)[slot_of(t)]);
#pragma unroll
          for (int u = 0; u < kMaxGroup / 2; ++u) lg[u] = alpha * n16 * cdot[u] + beta * rho * sdot[u];
        } else if (a.k_codec == Q8_BLOCK32) {
          const int8_t* row = reinterpret_cast<const int8_t*>(kb) + t * kD;
          const uint16_t* sc = reinterpret_cast<const uint16_t*>(kb + kBlock * kD) + t * (kD / 32);
          for (int blkq = 0; blkq < kD / 32; ++blkq) {
            float part[kMaxGroup / 2];
#pragma unroll
            for (int u = 0; u < kMaxGroup / 2; ++u) part[u] = 0.0f;
            for (int e = 0; e < 32; ++e) {
              const int i = blkq * 32 + e;
              const float kv = static_cast<float>(row[i]);
#pragma unroll
              for (int u = 0; u < kMaxGroup / 2; ++u) {
                const int g = hpar + 2 * u;
                if (g < G) part[u] = fmaf(qv[g * kD + i], kv, part[u]);
              }
            }
            const float s = f16_to_f32(sc[blkq]);
#pragma unroll
            for (int u = 0; u < kMaxGroup / 2; ++u) lg[u] = fmaf(s, part[u], lg[u]);
          }
#pragma unroll
          for (int u = 0; u < kMaxGroup / 2; ++u) lg[u] *= inv_sqrt_d;
        } else {
          const float* row = reinterpret_cast<const float*>(kb) + t * kD;
          for (int i = 0; i < kD; ++i) {
            const float kv = row[i];
#pragma unroll
            for (int u = 0; u < kMaxGroup / 2; ++u) {
              const int g = hpar + 2 * u;
              if (g < G) lg[u] = fmaf(qv[g * kD + i], kv, lg[u]);
            }
          }
#pragma unroll
          for (int u = 0; u < kMaxGroup / 2; ++u) lg[u] *= inv_sqrt_d;
        }
      }
#pragma unroll
      for (int u = 0; u < kMaxGroup / 2; ++u) {
        const int g = hpar + 2 * u;
        if (g < G) {
          pt[g * kBlock + t] = (t < n_t) ? lg[u] : -INFINITY;
          if (a.logits != nullptr && t < n_t) {
            a.logits[(static_cast<int64_t>(b) * a.n_q + h * G + g) * a.max_ctx + blk * kBlock + t] = lg[u];
          }
        }
      }
    }
    __syncthreads();

    // ------------------------------------------------------ softmax
    for (int g = wave; g < G; g += kThreads / 64) {
      const float l0 = pt[g * kBlock + lane];
      const float l1 = pt[g * kBlock + lane + 64];
      const float tmax = wave_max(fmaxf(l0, l1));
      const float mo = m_run[g];
      const float mn = fmaxf(mo, tmax);
      const float p0 = (lane < n_t) ? __expf(l0 - mn) : 0.0f;
      const float p1 = (lane + 64 < n_t) ? __expf(l1 - mn) : 0.0f;
      const float sum = wave_sum(p0 + p1);
      float vr0 = 1.0f, vr1 = 1.0f;
      if (a.v_codec == POLAR) {
        const uint16_t* vn = reinterpret_cast<const uint16_t*>(vb + 4 * vbits * 4 * kD);
        vr0 = (lane < n_t) ? f16_to_f32(vn[slot_of(lane)]) : 0.0f;
        vr1 = (lane + 64 < n_t) ? f16_to_f32(vn[slot_of(lane + 64)]) : 0.0f;
      }
      pt[g * kBlock + lane] = p0 * vr0;
      pt[g * kBlock + lane + 64] = p1 * vr1;
      if (lane == 0) {
        const float sc = (mo == -INFINITY) ? 0.0f : __expf(mo - mn);
        scale[g] = sc;
        l_run[g] = l_run[g] * sc + sum;
        m_run[g] = mn;
      }
    }
    __syncthreads();

    // ----------------------------------------------------------- PV
#pragma unroll
    for (int u = 0; u < kMaxGroup / 2; ++u) {
      const int g = hpar + 2 * u;
      if (g < G) acc[u] *= scale[g];
    }
    if (a.v_codec == POLAR) {
      const uint32_t* planes = reinterpret_cast<const uint32_t*>(vb);
      for (int j = 0; j * 32 < n_t; ++j) {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < 4; ++p)
          if (p < vbits) w[p] = planes[p * 4 * kD + j * kD + ci];
        const int e_end = min(32, n_t - j * 32);
        for (int e = 0; e < e_end; ++e) {
          int c = 0;
#pragma unroll
          for (int p = 0; p < 4; ++p) c |= ((w[p] >> e) & 1u) << p;
          const float cv = vcb[c];
          const int t = j * 32 + e;
#pragma unroll
          for (int u = 0; u < kMaxGroup / 2; ++u) {
            const int g = hpar + 2 * u;
            if (g < G) acc[u] = fmaf(pt[g * kBlock + t], cv, acc[u]);
          }
        }
      }
    } else {
      const float* rows = reinterpret_cast<const float*>(vb);
      for (int t = 0; t < n_t; ++t) {
        const float v = rows[t * kD + ci];
#pragma unroll
        for (int u = 0; u < kMaxGroup / 2; ++u) {
          const int g = hpar + 2 * u;
          if (g < G) acc[u] = fmaf(pt[g * kBlock + t], v, acc[u]);
        }
      }
    }
    __syncthreads();
  }

  // --------------------------------------------------------- partials
  const int64_t pstride = kPartialStride;
#pragma unroll
  for (int u = 0; u < kMaxGroup / 2; ++u) {
    const int g = hpar + 2 * u;
    if (g < G) {
      float* pp = a.partials + ((static_cast<int64_t>(b) * a.n_q + h * G + g) * a.n_splits + split) * pstride;
      store_coherent(pp + ci, acc[u]);
      if (ci == 0) {
        store_coherent(pp + kD, m_run[g]);
        store_coherent(pp + kD + 1, l_run[g]);
      }
    }
  }
  if (!arrive_last(a.counters + b * a.n_kv + h, a.n_splits, &s_last)) return;

  combine_splits(a, b, h, qv, kThreads);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.n_splits, a.n_kv, a.batch);
  hipLaunchKernelGGL(decode_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
