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
// Recursive polar tensors (the radius + angle step read as a pairwise tree)
// stand for y_hat = sqrt(d) n16 u, u the unit vector of the code angles: a
// key's logit is n16 <q_raw, u> / d with <q_raw, u> = sum over the 64
// level-1 pairs of (q_2i cos + q_2i+1 sin of the pair's angle) times the
// product of its ancestors' cos (left child) or sin (right child), walked
// top-down so that every node's angle is looked up once; a value coordinate
// u_i is the product over the 7 levels of the cos or sin of its ancestors'
// angles.
//
// Mapping: grid (split, KV head, sequence); a 256-thread workgroup serves
// all G query heads of its KV head over one chunk of 128-position blocks,
// keeping a running max and sum per head (online softmax).  Per block:
//   logits  thread = (position t, head parity); keys are token-major planes,
//           so a thread reads its position's words directly;
//   softmax one wavefront per head, wave-reduced max and sum;
//   PV      thread = (coordinate i, position parity) for every head: values
//           are coordinate-major planes, so a thread reads the words of its
//           coordinate and walks every other position of the block bit by
//           bit, decoding each value coordinate once; recursive polar values
//           take thread = (level-1 pair, quarter of the positions) instead,
//           one angle lookup per pair and position for both coordinates.
//           The partial sums meet in shared memory at the end of the split.
// Partials (m, l, acc) go to the workspace; the last workgroup of each
// (sequence, KV head) (device-scope counter) merges them by log-sum-exp
// rescaling, applies the inverse rotation and writes the output.

#include <hip/hip_fp16.h>

#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kThreads = 256;

// Recursive polar: (cos, sin) of the centroid angles, level 1 at [0][code],
// level l >= 2 at [l][code].
struct TreeLds {
  float2 l1[32];
  float2 up[8][8];
};

// code of an angle slot of one key from its word J (slot / 32, a constant
// at every call) and bit e: w[p][J] for the NB1 = b - 1 shared planes,
// x[k][J - 2] for the two extra level-1 planes
template <int NB1, int J>
__device__ __forceinline__ int tree_key_code(const uint32_t (&w)[3][4], const uint32_t (&x)[2][2], int e) {
  int c = 0;
#pragma unroll
  for (int p = 0; p < NB1; ++p) c |= ((w[p][J] >> e) & 1u) << p;
  if constexpr (J >= 2) {
    c |= ((x[0][J - 2] >> e) & 1u) << NB1;
    c |= ((x[1][J - 2] >> e) & 1u) << (NB1 + 1);
  }
  return c;
}

// dot[u] += <q_raw of head hb + HS u, u> over the subtree of level-6 node N6
// (coordinates 64 N6 .. 64 N6 + 63), its weight w6 being the root's cos or sin
template <int NB1, int N6, int NH, int HS>
__device__ __forceinline__ void tree_half_dot(float w6, const uint32_t (&w)[3][4], const uint32_t (&x)[2][2],
                                              const TreeLds& tab, const float* qv, int hb, float (&dot)[NH]) {
  const float2 c6 = tab.up[6][tree_key_code<NB1, 0>(w, x, 2 + N6)];
#pragma unroll 1
  for (int n5 = 2 * N6; n5 < 2 * N6 + 2; ++n5) {
    const float w5 = w6 * ((n5 & 1) ? c6.y : c6.x);
    const float2 c5 = tab.up[5][tree_key_code<NB1, 0>(w, x, 4 + n5)];
#pragma unroll 1
    for (int n4 = 2 * n5; n4 < 2 * n5 + 2; ++n4) {
      const float w4 = w5 * ((n4 & 1) ? c5.y : c5.x);
      const float2 c4 = tab.up[4][tree_key_code<NB1, 0>(w, x, 8 + n4)];
#pragma unroll 1
      for (int n3 = 2 * n4; n3 < 2 * n4 + 2; ++n3) {
        const float w3 = w4 * ((n3 & 1) ? c4.y : c4.x);
        const float2 c3 = tab.up[3][tree_key_code<NB1, 0>(w, x, 16 + n3)];
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
          const int n2 = 2 * n3 + b2;
          const float w2 = w3 * (b2 ? c3.y : c3.x);
          const float2 c2 = tab.up[2][tree_key_code<NB1, 1>(w, x, n2)];   // slot 32 + n2
#pragma unroll
          for (int b1 = 0; b1 < 2; ++b1) {
            const int i = 2 * n2 + b1;   // level-1 pair, slot 64 + i (word 2 + N6)
            const float w1 = w2 * (b1 ? c2.y : c2.x);
            const float2 cs = tab.l1[tree_key_code<NB1, 2 + N6>(w, x, i & 31)];
            const float a0 = w1 * cs.x, a1 = w1 * cs.y;
#pragma unroll
            for (int u = 0; u < NH; ++u) {
              const float2 q2 = *reinterpret_cast<const float2*>(qv + (hb + HS * u) * kD + 2 * i);
              dot[u] = fmaf(q2.x, a0, fmaf(q2.y, a1, dot[u]));
            }
          }
        }
      }
    }
  }
}

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

// HPT: query heads per thread, ceil(G / 2) rounded up to a power of two.  The
// inner loops run over all HPT heads without a test: rows past the group
// read shared memory that is allocated but holds no head, and their
// accumulators are never written out (a branch per head per element made
// every shared-memory read wait for its result).
// TVB: bits of recursive polar values (0: other value codecs); the path
// products of a word of positions are formed once per position in pp.
template <int HPT, int TVB>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  __shared__ float qv[kMaxGroup * kD];   // q (or q_raw) per head
  __shared__ float sq[kMaxGroup * kM];   // S q_raw / sqrt(d) per head
  __shared__ float pt[kMaxGroup * kBlock];  // logits, then p * value radius
  __shared__ float kcb[16], vcb[16];
  __shared__ TreeLds ktree, vtree;
  // recursive polar values: per position of a 32-position word, the product
  // of the level 2..7 factors on the path to each level-1 pair
  __shared__ float pp[TVB > 0 ? 32 : 1][TVB > 0 ? kD / 2 : 1];
  __shared__ float m_run[kMaxGroup], l_run[kMaxGroup], scale[kMaxGroup];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.group;
  const int len = min(a.seq_lens[b] + a.len_add, a.max_ctx);   // never read past the capacity
  const float inv_sqrt_d = 0.08838834764831845f;   // 1/sqrt(128)

  // ---------------------------------------------------------- prologue
  for (int k = tid; k < G * kD; k += kThreads) {
    const int g = k / kD, i = k % kD;
    float v = a.q[(static_cast<int64_t>(b) * a.n_q + h * G + g) * kD + i];
    if (a.k_codec == POLAR || a.k_codec == POLAR_QJL || a.k_codec == POLAR_TREE) v *= a.tb.dk[i];
    qv[k] = v;
  }
  if (tid < 32) {
    if (a.k_codec == POLAR_TREE) ktree.l1[tid] = a.tb.tk->cs1[tid];
    if (a.v_codec == POLAR_TREE) vtree.l1[tid] = a.tb.tv->cs1[tid];
  } else if (tid < 96) {
    const int l = (tid - 32) >> 3, c = (tid - 32) & 7;
    if (a.k_codec == POLAR_TREE) ktree.up[l][c] = a.tb.tk->cs[l][c];
    if (a.v_codec == POLAR_TREE) vtree.up[l][c] = a.tb.tv->cs[l][c];
  }
  if (tid < 16) {
    kcb[tid] = a.tb.ck[tid];
    vcb[tid] = a.tb.cv[tid];
  }
  if (tid < G) {
    m_run[tid] = -INFINITY;
    l_run[tid] = 0.0f;
  }
  if (a.k_codec == POLAR || a.k_codec == POLAR_QJL || a.k_codec == POLAR_TREE)
    block_fwht128(qv, G, kThreads);   // q_raw = H D_K q
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

  // accumulators: thread (coordinate ci = tid % 128, hpar = tid / 128) sums
  // the positions t = hpar (mod 2) of every block for every head g < 2 HPT
  // (each value coordinate formed once); the two halves are added at the end
  const int ci = tid & (kD - 1);
  const int hpar = tid >> 7;
  constexpr int NHA = 2 * HPT;
  // recursive polar values: thread (level-1 pair i = tid % 64, quarter
  // qq = tid / 64) sums coordinates 2 i, 2 i + 1 over the positions
  // t = qq (mod 4), acc[c NHA + g] for coordinate 2 i + c
  constexpr int NACC = TVB > 0 ? 2 * NHA : NHA;
  const int vpi = tid & 63, vqq = tid >> 6;
  float acc[NACC];
#pragma unroll
  for (int g = 0; g < NACC; ++g) acc[g] = 0.0f;


  const int blk0 = split_first_block(a, split);
  const int nblk_seq = (len + kBlock - 1) / kBlock;
  const int blk1 = min(blk0 + split_block_count(a, split), nblk_seq);
  const int64_t slot0 = (static_cast<int64_t>(b) * a.n_kv + h) * a.n_blocks;
  const float alpha = inv_sqrt_d / static_cast<float>(kD);                       // (1/sqrt d)(1/d)
  const float beta = inv_sqrt_d * 1.2533141373155003f / static_cast<float>(kM);  // sqrt(pi/2)/m/sqrt d
  const int kbits = a.k_bits, vbits = a.v_bits;

  for (int blk = blk0; blk < blk1; ++blk) {
    const int n_t = min(kBlock, len - blk * kBlock);
    const uint8_t* kb = a.kc + (slot0 + blk) * a.k_block_bytes;
    const uint8_t* vb = a.vc + (slot0 + blk) * a.v_block_bytes;

    // ------------------------------------------------------- logits
    if (a.k_codec == POLAR_TREE) {   // uniform
      // Groups of up to four heads: thread (t, half) walks the half `hpar`
      // of position t's tree (the root's left or right subtree) for every
      // head, once for all of them; the right halves' sums reach the left
      // halves through pt.  Larger groups: thread (t, hpar) walks the whole
      // tree for its heads hpar + 2u (fewer registers per thread).
      const int t = tid & (kBlock - 1);
      constexpr int NH = HPT <= 2 ? 2 * HPT : HPT;   // heads per thread's sums
      float dot[NH];
#pragma unroll
      for (int u = 0; u < NH; ++u) dot[u] = 0.0f;
      float n16 = 0.0f;
      if (t < n_t) {
        const uint32_t* planes = reinterpret_cast<const uint32_t*>(kb);
        const int sl = slot_of(t);
        // the walk with the plane count a constant (2-, 3- and 4-bit keys)
        auto walk = [&](auto nb1_c) __attribute__((always_inline)) {
          constexpr int NB1 = decltype(nb1_c)::value;
          uint32_t w[3][4] = {}, x[2][2];
#pragma unroll
          for (int p = 0; p < NB1; ++p)
#pragma unroll
            for (int j = 0; j < 4; ++j) w[p][j] = planes[(p * 4 + j) * kBlock + sl];
          const uint32_t* l1 = planes + NB1 * 4 * kBlock;
#pragma unroll
          for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int j = 0; j < 2; ++j) x[k][j] = l1[(k * 2 + j) * kBlock + sl];
          n16 = f16_to_f32(reinterpret_cast<const uint16_t*>(l1 + 4 * kBlock)[sl]);
          const float2 c7 = ktree.up[7][tree_key_code<NB1, 0>(w, x, 1)];
          if constexpr (HPT <= 2) {
            if (hpar == 0)
              tree_half_dot<NB1, 0, NH, 1>(c7.x, w, x, ktree, qv, 0, dot);
            else
              tree_half_dot<NB1, 1, NH, 1>(c7.y, w, x, ktree, qv, 0, dot);
          } else {
            tree_half_dot<NB1, 0, NH, 2>(c7.x, w, x, ktree, qv, hpar, dot);
            tree_half_dot<NB1, 1, NH, 2>(c7.y, w, x, ktree, qv, hpar, dot);
          }
        };
        switch (kbits) {   // uniform
          case 2: walk(std::integral_constant<int, 1>{}); break;
          case 3: walk(std::integral_constant<int, 2>{}); break;
          default: walk(std::integral_constant<int, 3>{}); break;
        }
      }
      if constexpr (HPT > 2) {
#pragma unroll
        for (int u = 0; u < NH; ++u) {
          const int g = hpar + 2 * u;
          if (g < G) {
            const float lgv = n16 * dot[u] * (1.0f / static_cast<float>(kD));
            pt[g * kBlock + t] = (t < n_t) ? lgv : -INFINITY;
            if (a.logits != nullptr && t < n_t)
              a.logits[(static_cast<int64_t>(b) * a.n_q + h * G + g) * a.max_ctx + blk * kBlock + t] = lgv;
          }
        }
      } else {
      if (hpar == 1) {
#pragma unroll
        for (int g = 0; g < NH; ++g)
          if (g < G) pt[g * kBlock + t] = dot[g];
      }
      __syncthreads();
      if (hpar == 0) {
#pragma unroll
        for (int g = 0; g < NH; ++g) {
          if (g < G) {
            const float lgv = n16 * (dot[g] + pt[g * kBlock + t]) * (1.0f / static_cast<float>(kD));
            pt[g * kBlock + t] = (t < n_t) ? lgv : -INFINITY;
            if (a.logits != nullptr && t < n_t)
              a.logits[(static_cast<int64_t>(b) * a.n_q + h * G + g) * a.max_ctx + blk * kBlock + t] = lgv;
          }
        }
      }
      }
    } else {
      const int t = tid & (kBlock - 1);
      float lg[HPT];
#pragma unroll
      for (int u = 0; u < HPT; ++u) lg[u] = 0.0f;
      if (t < n_t) {
        if (a.k_codec == POLAR || a.k_codec == POLAR_QJL) {
          const uint32_t* planes = reinterpret_cast<const uint32_t*>(kb);
          const int plane_words = (kD / 32) * kBlock;
          float cdot[HPT], sdot[HPT];
#pragma unroll
          for (int u = 0; u < HPT; ++u) cdot[u] = sdot[u] = 0.0f;
#pragma unroll 1
          for (int j = 0; j < kD / 32; ++j) {
            uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
            for (int p = 0; p < 4; ++p)
              if (p < kbits) w[p] = planes[p * plane_words + j * kBlock + slot_of(t)];
#pragma unroll 8
            for (int e = 0; e < 32; ++e) {
              int c = 0;
#pragma unroll
              for (int p = 0; p < 4; ++p) c |= ((w[p] >> e) & 1u) << p;
              const float cv = kcb[c];
              const int i = j * 32 + e;
#pragma unroll
              for (int u = 0; u < HPT; ++u) cdot[u] = fmaf(qv[(hpar + 2 * u) * kD + i], cv, cdot[u]);
            }
          }
          const uint8_t* after = kb + 4 * kbits * plane_words;
          float rho = 0.0f;
          if (a.k_codec == POLAR_QJL) {
            const uint32_t* sg = reinterpret_cast<const uint32_t*>(after);
#pragma unroll 1
            for (int j = 0; j < kM / 32; ++j) {
              const uint32_t w = sg[j * kBlock + slot_of(t)];
#pragma unroll 8
              for (int e = 0; e < 32; ++e) {
                const bool pos = (w >> e) & 1u;
                const int r = j * 32 + e;
#pragma unroll
                for (int u = 0; u < HPT; ++u) {
                  const float s = sq[(hpar + 2 * u) * kM + r];
                  sdot[u] += pos ? s : -s;
                }
              }
            }
            after += 4 * (kM / 32) * kBlock;
            rho = f16_to_f32(reinterpret_cast<const uint16_t*>(after + 2 * kBlock)[slot_of(t)]);
          }
          const float n16 = f16_to_f32(reinterpret_cast<const uint16_t*>(after)[slot_of(t)]);
#pragma unroll
          for (int u = 0; u < HPT; ++u) lg[u] = alpha * n16 * cdot[u] + beta * rho * sdot[u];
        } else if (a.k_codec == Q8_BLOCK32) {
          const int8_t* row = reinterpret_cast<const int8_t*>(kb) + t * kD;
          const uint16_t* sc = reinterpret_cast<const uint16_t*>(kb + kBlock * kD) + t * (kD / 32);
#pragma unroll 1
          for (int blkq = 0; blkq < kD / 32; ++blkq) {
            float part[HPT];
#pragma unroll
            for (int u = 0; u < HPT; ++u) part[u] = 0.0f;
#pragma unroll 8
            for (int e = 0; e < 32; ++e) {
              const int i = blkq * 32 + e;
              const float kv = static_cast<float>(row[i]);
#pragma unroll
              for (int u = 0; u < HPT; ++u) part[u] = fmaf(qv[(hpar + 2 * u) * kD + i], kv, part[u]);
            }
            const float s = f16_to_f32(sc[blkq]);
#pragma unroll
            for (int u = 0; u < HPT; ++u) lg[u] = fmaf(s, part[u], lg[u]);
          }
#pragma unroll
          for (int u = 0; u < HPT; ++u) lg[u] *= inv_sqrt_d;
        } else {
          const float* row = reinterpret_cast<const float*>(kb) + t * kD;
#pragma unroll 8
          for (int i = 0; i < kD; ++i) {
            const float kv = row[i];
#pragma unroll
            for (int u = 0; u < HPT; ++u) lg[u] = fmaf(qv[(hpar + 2 * u) * kD + i], kv, lg[u]);
          }
#pragma unroll
          for (int u = 0; u < HPT; ++u) lg[u] *= inv_sqrt_d;
        }
      }
#pragma unroll
      for (int u = 0; u < HPT; ++u) {
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
      if (a.v_codec == POLAR || a.v_codec == POLAR_TREE) {
        // the radius field sits after 4 b d bytes of code words in both layouts;
        // the recursive codec's y_hat is sqrt(d) n16 u
        const uint16_t* vn = reinterpret_cast<const uint16_t*>(vb + 4 * vbits * 4 * kD);
        const float sc = (a.v_codec == POLAR_TREE) ? 11.313708498984761f : 1.0f;
        vr0 = (lane < n_t) ? sc * f16_to_f32(vn[slot_of(lane)]) : 0.0f;
        vr1 = (lane + 64 < n_t) ? sc * f16_to_f32(vn[slot_of(lane + 64)]) : 0.0f;
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
    for (int g = 0; g < NACC; ++g) acc[g] *= scale[g % NHA];
    if constexpr (TVB > 0) {
      // coordinate ci: its level-1 pair is slot 64 + ci / 2, its level-l
      // ancestor slot 2^(7 - l) + ci / 2^l; the factor is the sin of an
      // ancestor's angle when ci lies in its right half, else the cos.  The
      // product of the level 2..7 factors depends on the pair only: per word
      // of 32 positions, thread (e, q) walks the level-4 subtree q of position
      // 32 j + e top-down and leaves the products of its 8 pairs in pp (each
      // node's angle looked up once per position), then thread (pair i,
      // quarter) looks up its pair's angle once per position and forms
      // u_2i = cos * pp[e][i], u_2i+1 = sin * pp[e][i].
      constexpr int nb1 = TVB - 1;
      const uint32_t* planes = reinterpret_cast<const uint32_t*>(vb);
      const uint32_t* l1 = planes + nb1 * 4 * kD;
      const int pe = tid & 31, pq = (tid >> 5) & 7;
#pragma unroll 1
      for (int j = 0; j * 32 < n_t; ++j) {
        // code of the upper slot sl for position 32 j + pe
        auto node_code = [&](int sl) __attribute__((always_inline)) {
          int c = 0;
#pragma unroll
          for (int p = 0; p < nb1; ++p) c |= ((planes[(p * 4 + j) * kD + sl] >> pe) & 1u) << p;
          return c;
        };
        __syncthreads();   // the previous word's pp has been read
        {
          const float2 c7 = vtree.up[7][node_code(1)];
          float f = (pq >> 2) ? c7.y : c7.x;
          const float2 c6 = vtree.up[6][node_code(2 + (pq >> 2))];
          f *= ((pq >> 1) & 1) ? c6.y : c6.x;
          const float2 c5 = vtree.up[5][node_code(4 + (pq >> 1))];
          f *= (pq & 1) ? c5.y : c5.x;
          const float2 c4 = vtree.up[4][node_code(8 + pq)];
#pragma unroll
          for (int a3 = 0; a3 < 2; ++a3) {
            const float f3 = f * (a3 ? c4.y : c4.x);
            const float2 c3 = vtree.up[3][node_code(16 + 2 * pq + a3)];
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2) {
              const float f2 = f3 * (a2 ? c3.y : c3.x);
              const int n2 = 4 * pq + 2 * a3 + a2;   // level-2 node
              const float2 c2 = vtree.up[2][node_code(32 + n2)];
              pp[pe][2 * n2] = f2 * c2.x;
              pp[pe][2 * n2 + 1] = f2 * c2.y;
            }
          }
        }
        __syncthreads();
        // pair vpi's code words; positions 32 j + e, e = vqq (mod 4)
        uint32_t w[nb1], x[2];
#pragma unroll
        for (int p = 0; p < nb1; ++p) w[p] = planes[(p * 4 + j) * kD + 64 + vpi];
#pragma unroll
        for (int k = 0; k < 2; ++k) x[k] = l1[(k * 4 + j) * (kD / 2) + vpi];
        const int e_end = min(32, n_t - j * 32);
#pragma unroll 2
        for (int e = vqq; e < e_end; e += 4) {
          int c = 0;
#pragma unroll
          for (int p = 0; p < nb1; ++p) c |= ((w[p] >> e) & 1u) << p;
          c |= ((x[0] >> e) & 1u) << nb1;
          c |= ((x[1] >> e) & 1u) << (nb1 + 1);
          const float2 cs1 = vtree.l1[c];
          const float pv = pp[e][vpi];
          const float u0 = cs1.x * pv, u1 = cs1.y * pv;
          const int t = j * 32 + e;
#pragma unroll
          for (int g = 0; g < NHA; ++g) {
            const float pg = pt[g * kBlock + t];
            acc[g] = fmaf(pg, u0, acc[g]);
            acc[NHA + g] = fmaf(pg, u1, acc[NHA + g]);
          }
        }
      }
    } else if (a.v_codec == POLAR) {
      const uint32_t* planes = reinterpret_cast<const uint32_t*>(vb);
#pragma unroll 1
      for (int j = 0; j * 32 < n_t; ++j) {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < 4; ++p)
          if (p < vbits) w[p] = planes[p * 4 * kD + j * kD + ci];
        const int e_end = min(32, n_t - j * 32);
#pragma unroll 4
        for (int e = hpar; e < e_end; e += 2) {
          int c = 0;
#pragma unroll
          for (int p = 0; p < 4; ++p) c |= ((w[p] >> e) & 1u) << p;
          const float cv = vcb[c];
          const int t = j * 32 + e;
#pragma unroll
          for (int g = 0; g < NHA; ++g) acc[g] = fmaf(pt[g * kBlock + t], cv, acc[g]);
        }
      }
    } else {
      const float* rows = reinterpret_cast<const float*>(vb);
#pragma unroll 8
      for (int t = hpar; t < n_t; t += 2) {
        const float v = rows[t * kD + ci];
#pragma unroll
        for (int g = 0; g < NHA; ++g) acc[g] = fmaf(pt[g * kBlock + t], v, acc[g]);
      }
    }
    __syncthreads();
  }

  // --------------------------------------------------------- partials
  // the sums per head and coordinate end in pt[g][coordinate] (free by now;
  // NHA <= kMaxGroup rows): the threads that hold parts of the positions add
  // theirs in turn, then thread (ci, hpar) stores heads hpar + 2 u
  static_assert(NHA <= kMaxGroup, "one row of pt per head");
  if constexpr (TVB > 0) {
#pragma unroll 1
    for (int q4 = 3; q4 >= 0; --q4) {   // quarter 3 writes, 2, 1, 0 add
      if (vqq == q4) {
#pragma unroll
        for (int g = 0; g < NHA; ++g) {
          float* r = &pt[g * kBlock + 2 * vpi];
          r[0] = (q4 == 3) ? acc[g] : r[0] + acc[g];
          r[1] = (q4 == 3) ? acc[NHA + g] : r[1] + acc[NHA + g];
        }
      }
      __syncthreads();
    }
  } else {
    if (hpar == 1) {
#pragma unroll
      for (int g = 0; g < NHA; ++g) pt[g * kBlock + ci] = acc[g];
    }
    __syncthreads();
    if (hpar == 0) {
#pragma unroll
      for (int g = 0; g < NHA; ++g) pt[g * kBlock + ci] += acc[g];
    }
    __syncthreads();
  }
  const int64_t pstride = kPartialStride;
#pragma unroll
  for (int u = 0; u < HPT; ++u) {
    const int g = hpar + 2 * u;
    if (g < G) {
      float* pp = a.partials + ((static_cast<int64_t>(b) * a.n_q + h * G + g) * a.n_splits + split) * pstride;
      store_coherent(pp + ci, pt[g * kBlock + ci]);
      if (ci == 0) {
        store_coherent(pp + kD, m_run[g]);
        store_coherent(pp + kD + 1, l_run[g]);
      }
    }
  }
  if (!arrive_last(a.counters + b * a.n_kv + h, a.n_splits, &s_last)) return;

  combine_splits(a, b, h, qv, kThreads);
}

template <int HPT>
hipError_t launch_h(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_splits, a.n_kv, a.batch);
  switch (a.v_codec == POLAR_TREE ? a.v_bits : 0) {
    case 0: hipLaunchKernelGGL((decode_kernel<HPT, 0>), grid, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<HPT, 2>), grid, dim3(kThreads), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((decode_kernel<HPT, 3>), grid, dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<HPT, 4>), grid, dim3(kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.group <= 2) return launch_h<1>(a, stream);
  if (a.group <= 4) return launch_h<2>(a, stream);
  if (a.group <= 8) return launch_h<4>(a, stream);
  return launch_h<8>(a, stream);
}

}  // namespace tq
