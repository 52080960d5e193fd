// tq_decode_mfma.hip -- decode attention on the gfx950 matrix cores, for
// POLAR / POLAR_QJL keys and POLAR values with up to 4 query heads per KV head.
//
// Same result as the VALU kernel (logits with the QJL-corrected estimator,
// softmax, rotated-frame weighted sum of values; wis-web.com reader,
// TurboQuant article, PolarQuant and QJL paragraphs), computed so that the
// packed bits feed the matrix cores directly:
//
//  * A symmetric sorted codebook of 2^b levels is an odd function of the
//    code bits read as signs s_k = +/-1, so C[c] = sum_T a_T prod_{k in T} s_k
//    over the odd subsets T (b = 2: 2 terms; 3: 4; 4: 8).  Each term is a
//    +/-1 vector whose bits are a code plane or the XOR of three planes, and
//    <q, C[c]> = sum_T a_T <q, s_T>.  The QJL term <Sq, sign> has the same form.
//  * A +/-1 bit vector becomes an fp4 (e2m1) matrix operand in two integer
//    operations per 8 elements; the query side (q_raw = H D_K q and
//    sq = S q_raw / sqrt d) is split into four fp8 (e4m3) limbs with one
//    E8M0 scale per 32 elements (about 16 significant bits), so
//    v_mfma_scale_f32_16x16x128_f8f6f4 computes 4 heads x 4 limbs x 16
//    positions x 128 coordinates per instruction with fp32 accumulation.
//  * The weighted sum is the same contraction over positions: value planes
//    (32 positions per word) are the fp4 operand, p * radius is split into
//    fp8 limbs per 32 positions (three limbs, about 12 significant bits).
//
// Operand layouts of the 16x16x128 instruction (lane l, element e): rows or
// columns are l % 16; an fp4 operand holds k = 32 (l / 16) + e; an fp8
// operand holds k = 64 (e / 16) + 16 (l / 16) + e % 16; the E8M0 scale of
// (row, k / 32) is taken from lane row + 16 (k / 32); lane l of the result
// holds rows 4 (l / 16) + i, column l % 16.  Element e of an fp4 operand built
// from a bit word is bit 4 (e % 8) + e / 8 of that word, so k-slot k stands for
// coordinate (or position) pos_of_slot(k) of its 32-group; the cache stores
// the per-position key fields and value radii at slot_of(position), which makes
// each lane's operands whole 8-byte loads.
//
// Mapping: grid (split, KV head, sequence); 4 waves per workgroup share each
// 128-position block.  Wave w computes the logits of the block's positions in
// k-slots [32w, 32w+32) (2 MFMA column groups), takes part in the block max
// (shared memory), writes its fp8 limbs of p * radius, then computes the
// weighted sum for coordinates [32w, 32w+32) over all 128 positions.  Loads
// of the block after next are issued before the current one is processed.

#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int B>
struct NTerms {
  static constexpr int n = (B == 2) ? 2 : (B == 3 ? 4 : 8);
};

// Bits of term T: code planes for T < B, then XORs of three planes.
template <int B>
__device__ __forceinline__ uint32_t term_word(const uint32_t* w, int T) {
  if (T < B) return w[T];
  const int u = T - B;
  const int i0 = (u == 3) ? 1 : 0;
  const int i1 = (u <= 1) ? 1 : 2;
  const int i2 = (u == 0) ? 2 : 3;
  return w[i0] ^ w[i1] ^ w[i2];
}

// 32 bits -> 32 fp4 elements of +/-1 (bit 1 -> +1.0 = 0x2, bit 0 -> -1.0 = 0xA);
// element 8d + n holds bit 4n + d.  Dword d keeps bits 4n+3 of ~(w << (3-d))
// (the sign bits) and ORs in 0x2 (magnitude 1): one shift and one v_bitop3
// ((~a & c) | b, table 0xCE) per dword.
__device__ __forceinline__ v8i expand_fp4(uint32_t w) {
  constexpr uint32_t kSign = 0x88888888u, kOne = 0x22222222u;
  v8i r;
  r[0] = static_cast<int>(__builtin_amdgcn_bitop3_b32(w << 3, kOne, kSign, 0xCE));
  r[1] = static_cast<int>(__builtin_amdgcn_bitop3_b32(w << 2, kOne, kSign, 0xCE));
  r[2] = static_cast<int>(__builtin_amdgcn_bitop3_b32(w << 1, kOne, kSign, 0xCE));
  r[3] = static_cast<int>(__builtin_amdgcn_bitop3_b32(w, kOne, kSign, 0xCE));
  r[4] = r[5] = r[6] = r[7] = 0;
  return r;
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

// Raw Sylvester FWHT of 128 values held as (lo = coord lane, hi = coord lane+64).
__device__ __forceinline__ void wave_fwht128(float& lo, float& hi, int lane) {
#pragma unroll
  for (int hh = 1; hh < 64; hh <<= 1) {
    const float plo = __shfl_xor(lo, hh, 64);
    const float phi = __shfl_xor(hi, hh, 64);
    if (lane & hh) {
      lo = plo - lo;
      hi = phi - hi;
    } else {
      lo = lo + plo;
      hi = hi + phi;
    }
  }
  const float x = lo, y = hi;
  lo = x + y;
  hi = x - y;
}

__device__ __forceinline__ int exponent_of(float x) {   // floor(log2 x), x > 0 normal
  return static_cast<int>((__float_as_uint(x) >> 23) & 0xffu) - 127;
}

__device__ __forceinline__ float h2f(uint32_t bits16) { return __half2float(__ushort_as_half(static_cast<uint16_t>(bits16))); }

__device__ __forceinline__ v4f mfma_fp8_fp4(const v8i& a, const v8i& b, const v4f& c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, 127);
}
__device__ __forceinline__ v4f mfma_fp4_fp8(const v8i& a, const v8i& b, const v4f& c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, 127, 0, sb);
}

template <int KB, int VB>
struct BlockRegs {
  uint2 kp[KB];       // key code words, slots 32w + 2t and +1, coordinate group g4
  uint2 ks;           // sign words
  uint32_t kn, kr, vn;  // two fp16 key radii, residual norms, value radii
  uint32_t vw[2][VB];   // value words for coordinates 32w + 16r + t, positions 32 g4 ..
};

template <int KB, bool QJL, int VB>
__device__ __forceinline__ void load_block(BlockRegs<KB, VB>& R, const uint8_t* kbp, const uint8_t* vbp, int w,
                                           int t, int g4) {
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(kbp);
  const int so = g4 * kBlock + 32 * w + 2 * t;
#pragma unroll
  for (int p = 0; p < KB; ++p) R.kp[p] = *reinterpret_cast<const uint2*>(kw + p * 4 * kBlock + so);
  const uint8_t* after = kbp + 4 * KB * 4 * kBlock;
  if (QJL) {
    R.ks = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint32_t*>(after) + so);
    after += 4 * 4 * kBlock;
    R.kr = *reinterpret_cast<const uint32_t*>(after + 2 * kBlock + 2 * (32 * w + 2 * t));
  } else {
    R.ks = make_uint2(0u, 0u);
    R.kr = 0u;
  }
  R.kn = *reinterpret_cast<const uint32_t*>(after + 2 * (32 * w + 2 * t));
  R.vn = *reinterpret_cast<const uint32_t*>(vbp + 4 * VB * 4 * kD + 2 * (32 * w + 2 * t));
  const uint32_t* vwp = reinterpret_cast<const uint32_t*>(vbp);
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int p = 0; p < VB; ++p) R.vw[r][p] = vwp[p * 4 * kD + g4 * kD + 32 * w + 16 * r + t];
}

template <int KB, bool QJL, int VB>
__global__ __launch_bounds__(kThreads, 2) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NTK = NTerms<KB>::n;
  constexpr int NTV = NTerms<VB>::n;
  __shared__ float qr[4 * kD];              // q_raw = H D_K q per head (zero rows past G)
  __shared__ float sqs[4 * kM];             // S q_raw / sqrt d
  __shared__ __attribute__((aligned(16))) uint8_t alimb[2][16 * 128];  // fp8 limbs [row = 4g + j][k]
  __shared__ uint8_t aexp[2][4][16];        // E8M0 scale [set][k / 32][row]
  __shared__ __attribute__((aligned(16))) uint8_t plimb[16 * 128];     // fp8 limbs of p * radius [col][k]
  __shared__ __attribute__((aligned(4))) uint8_t pexp[4][16];          // [k / 32][col]
  __shared__ float wred[kWaves][4];
  __shared__ float hmax[3][kWaves];         // per-head max |value| for the limb exponents
  __shared__ __attribute__((aligned(16))) float sred[8][4 * kM];   // partial sketch sums
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int t = lane & 15;
  const int g4 = lane >> 4;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.group;
  const int len = min(a.seq_lens[b], a.max_ctx);
  const int nblk_seq = (len + kBlock - 1) / kBlock;
  const int blk0 = split * a.chunk_blocks;
  const int blk1 = min(blk0 + a.chunk_blocks, nblk_seq);
  const int64_t slot0 = (static_cast<int64_t>(b) * a.n_kv + h) * a.n_blocks;

  // loads of the first two blocks, the query rows and the sketch rows go out
  // before any set-up arithmetic
  BlockRegs<KB, VB> cur, nx1;
  if (blk0 < blk1)
    load_block<KB, QJL, VB>(cur, a.kc + (slot0 + blk0) * a.k_block_bytes, a.vc + (slot0 + blk0) * a.v_block_bytes,
                            w, t, g4);
  if (blk0 + 1 < blk1)
    load_block<KB, QJL, VB>(nx1, a.kc + (slot0 + blk0 + 1) * a.k_block_bytes,
                            a.vc + (slot0 + blk0 + 1) * a.v_block_bytes, w, t, g4);
  const float inv_sqrt_d = 0.08838834764831845f;
  const int jq = tid & 31, ic = tid >> 5;   // sketch rows 4jq..4jq+3, coordinates 16ic..16ic+15
  float4 st4[16];
  if (QJL) {
#pragma unroll
    for (int u = 0; u < 16; ++u) st4[u] = *reinterpret_cast<const float4*>(a.tb.st + (16 * ic + u) * kM + 4 * jq);
  }
  float q_lo = 0.0f, q_hi = 0.0f;
  if (w < G) {
    const float* qp = a.q + (static_cast<int64_t>(b) * a.n_q + h * G + w) * kD;
    q_lo = qp[lane] * a.tb.dk[lane];
    q_hi = qp[lane + 64] * a.tb.dk[lane + 64];
  }

  // ------------------------------------------------------------- set-up
  // wave w rotates the query of head w in registers: q_raw = H D_K q
  wave_fwht128(q_lo, q_hi, lane);
  qr[w * kD + lane] = q_lo;
  qr[w * kD + lane + 64] = q_hi;
  {
    float qm = fmaxf(fabsf(q_lo), fabsf(q_hi));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) qm = fmaxf(qm, __shfl_xor(qm, off, 64));
    if (lane == 0) hmax[0][w] = qm;
  }
  __syncthreads();
  if (QJL) {
    // sq = S q_raw / sqrt d: partial sums over 16 coordinates per thread, then over the 8 partials
    float acc[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[g][jj] = 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float qv = qr[g * kD + 16 * ic + u];
        acc[g][0] = fmaf(st4[u].x, qv, acc[g][0]);
        acc[g][1] = fmaf(st4[u].y, qv, acc[g][1]);
        acc[g][2] = fmaf(st4[u].z, qv, acc[g][2]);
        acc[g][3] = fmaf(st4[u].w, qv, acc[g][3]);
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(&sred[ic][g * kM + 4 * jq]) = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
    __syncthreads();
    // thread tid owns outputs tid (head tid/128) and tid + 256 (head 2 + tid/128)
    float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int k = tid + 256 * r;
      float sum = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) sum += sred[c][k];
      sum *= inv_sqrt_d;
      sqs[k] = sum;
      if (r == 0) m0 = fabsf(sum); else m1 = fabsf(sum);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      m0 = fmaxf(m0, __shfl_xor(m0, off, 64));
      m1 = fmaxf(m1, __shfl_xor(m1, off, 64));
    }
    if (lane == 0) {
      hmax[1][w] = m0;   // waves 2g, 2g+1 cover head g (g < 2)
      hmax[2][w] = m1;   // ... and head g + 2
    }
    __syncthreads();
  }
  {
    // fp8 limbs of q_raw (set 0) and sq (set 1), one E8M0 exponent per (set,
    // head): item (set, head, k-slot), k-slot k holding coordinate pos_of_slot(k)
    const int n_items = (QJL ? 2 : 1) * 4 * 128;
    for (int it = tid; it < n_items; it += kThreads) {
      const int k = it & 127;
      const int g = (it >> 7) & 3;
      const int set = it >> 9;
      const int coord = pos_of_slot(k);
      const float u = set == 0 ? qr[g * kD + coord] : sqs[g * kM + coord];
      float m;
      if (set == 0) {
        m = hmax[0][g];
      } else {
        const int row = g < 2 ? 1 : 2;
        const int w0 = 2 * (g & 1);
        m = fmaxf(hmax[row][w0], hmax[row][w0 + 1]);
      }
      const int s0 = (m >= 1e-30f) ? exponent_of(m) - 7 : 0;
      float res = u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int sj = s0 - 4 * j;
        const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(res, -sj), 0.0f, 0, false);
        res -= __builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(pk, 0), sj);
        alimb[set][(4 * g + j) * 128 + k] = static_cast<uint8_t>(pk & 0xff);
        if ((k & 31) == 0) aexp[set][k >> 5][4 * g + j] = static_cast<uint8_t>(min(max(sj + 127, 1), 254));
      }
    }
  }
  __syncthreads();
  v8i Aq, Asq;
  int scq, scsq = 127;
  {
    const uint4 lo = *reinterpret_cast<const uint4*>(&alimb[0][t * 128 + 16 * g4]);
    const uint4 hi = *reinterpret_cast<const uint4*>(&alimb[0][t * 128 + 64 + 16 * g4]);
    Aq = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    scq = aexp[0][g4][t];
    if (QJL) {
      const uint4 l2 = *reinterpret_cast<const uint4*>(&alimb[1][t * 128 + 16 * g4]);
      const uint4 h2 = *reinterpret_cast<const uint4*>(&alimb[1][t * 128 + 64 + 16 * g4]);
      Asq = v8i{(int)l2.x, (int)l2.y, (int)l2.z, (int)l2.w, (int)h2.x, (int)h2.y, (int)h2.z, (int)h2.w};
      scsq = aexp[1][g4][t];
    } else {
      Asq = Aq;
    }
  }
  float ak[NTK], av[NTV];
#pragma unroll
  for (int T = 0; T < NTK; ++T) ak[T] = a.tb.ak[T];
#pragma unroll
  for (int T = 0; T < NTV; ++T) av[T] = a.tb.av[T];

  const float alpha2 = kLog2e * inv_sqrt_d / static_cast<float>(kD);
  const float beta2 = kLog2e * inv_sqrt_d * 1.2533141373155003f / static_cast<float>(kM);
  // running max (log2 units) of head g4 (this lane's logits row) and of head
  // t / 4 (this lane's result column); both follow the same block maxima
  float m_a = -INFINITY, m_b = -INFINITY;
  float lsum = 0.0f;   // this lane's share of the denominator of head g4
  v4f accV[2][NTV];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int T = 0; T < NTV; ++T) accV[r][T] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // the fourth limb column of each head stays zero (three limbs are written)
  for (int k = tid; k < 4 * 128; k += kThreads) plimb[(4 * (k >> 7) + 3) * 128 + (k & 127)] = 0;

  // ----------------------------------------------------------- main loop
  for (int blk = blk0; blk < blk1; ++blk) {
    const int n_t = min(kBlock, len - blk * kBlock);
    BlockRegs<KB, VB> nx2;
    if (blk + 2 < blk1)
      load_block<KB, QJL, VB>(nx2, a.kc + (slot0 + blk + 2) * a.k_block_bytes,
                              a.vc + (slot0 + blk + 2) * a.v_block_bytes, w, t, g4);

    // logits of k-slots 32w + 2t + c for head g4: every MFMA of the block is
    // issued before any result is read
    v4f dT[2][NTK];
    v4f dQ[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t wd[KB];
#pragma unroll
      for (int p = 0; p < KB; ++p) wd[p] = c ? cur.kp[p].y : cur.kp[p].x;
#pragma unroll
      for (int T = 0; T < NTK; ++T)
        dT[c][T] = mfma_fp8_fp4(Aq, expand_fp4(term_word<KB>(wd, T)), v4f{0.0f, 0.0f, 0.0f, 0.0f}, scq);
      if (QJL) dQ[c] = mfma_fp8_fp4(Asq, expand_fp4(c ? cur.ks.y : cur.ks.x), v4f{0.0f, 0.0f, 0.0f, 0.0f}, scsq);
    }
    float lg2[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float code = 0.0f;
#pragma unroll
      for (int T = 0; T < NTK; ++T) code = fmaf(ak[T], (dT[c][T][0] + dT[c][T][1]) + (dT[c][T][2] + dT[c][T][3]), code);
      const float qj = QJL ? (dQ[c][0] + dQ[c][1]) + (dQ[c][2] + dQ[c][3]) : 0.0f;
      const int tok = pos_of_slot(32 * w + 2 * t + c);
      const float nk = h2f(c ? (cur.kn >> 16) : cur.kn);
      const float rk = QJL ? h2f(c ? (cur.kr >> 16) : cur.kr) : 0.0f;
      const float l2 = alpha2 * nk * code + beta2 * rk * qj;
      const bool valid = (tok < n_t) && (g4 < G);
      if (a.logits != nullptr && valid)
        a.logits[(static_cast<int64_t>(b) * a.n_q + h * G + g4) * a.max_ctx + blk * kBlock + tok] = l2 * kLn2;
      lg2[c] = valid ? l2 : -INFINITY;
    }

    // block max per head (4 waves); the running max only moves when a block
    // exceeds it by 2^8, so rescaling is rare and p stays below 256
    const float mloc = row_max16(fmaxf(lg2[0], lg2[1]));
    if (t == 0) wred[w][g4] = mloc;
    __syncthreads();
    const int hb = t >> 2;
    const float bm_a = fmaxf(fmaxf(wred[0][g4], wred[1][g4]), fmaxf(wred[2][g4], wred[3][g4]));
    const float bm_b = fmaxf(fmaxf(wred[0][hb], wred[1][hb]), fmaxf(wred[2][hb], wred[3][hb]));
    const float mn_a = (bm_a > m_a + 8.0f) ? bm_a : m_a;
    const float mn_b = (bm_b > m_b + 8.0f) ? bm_b : m_b;
    const float fh = (m_a == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_a - mn_a);
    const float fv = (m_b == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_b - mn_b);
    m_a = mn_a;
    m_b = mn_b;

    // probabilities and fp8 limbs of p * value radius (3 limbs, ~12 bits)
    const float p0 = (lg2[0] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(lg2[0] - m_a);
    const float p1 = (lg2[1] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(lg2[1] - m_a);
    lsum = lsum * fh + (p0 + p1);
    float r0 = (p0 > 0.0f) ? p0 * h2f(cur.vn) : 0.0f;
    float r1 = (p1 > 0.0f) ? p1 * h2f(cur.vn >> 16) : 0.0f;
    const float pm = row_max16(fmaxf(r0, r1));
    const int s0 = (pm >= 1e-30f) ? exponent_of(pm) - 7 : 0;
    uint32_t ebytes = 127u << 24;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int sj = s0 - 4 * j;
      const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(r0, -sj),
                                                     __builtin_amdgcn_ldexpf(r1, -sj), 0, false);
      if (j < 2) {
        r0 -= __builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(pk, 0), sj);
        r1 -= __builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(pk, 1), sj);
      }
      *reinterpret_cast<uint16_t*>(&plimb[(4 * g4 + j) * 128 + 32 * w + 2 * t]) = static_cast<uint16_t>(pk & 0xffff);
      ebytes |= static_cast<uint32_t>(min(max(sj + 127, 1), 254)) << (8 * j);
    }
    if (t == 0) *reinterpret_cast<uint32_t*>(&pexp[w][4 * g4]) = ebytes;
    __syncthreads();

    // weighted sum of value terms for coordinates 32w + 16r + (row), columns (head, limb)
    if (__any(fv != 1.0f)) {   // rescale only when some head's max moved
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int T = 0; T < NTV; ++T) accV[r][T] *= fv;
    }
    v8i Pv;
    {
      const uint4 lo = *reinterpret_cast<const uint4*>(&plimb[t * 128 + 16 * g4]);
      const uint4 hi = *reinterpret_cast<const uint4*>(&plimb[t * 128 + 64 + 16 * g4]);
      Pv = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    const int scp = pexp[g4][t];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int T = 0; T < NTV; ++T) accV[r][T] = mfma_fp4_fp8(expand_fp4(term_word<VB>(cur.vw[r], T)), Pv, accV[r][T], scp);
    }
    __syncthreads();
    cur = nx1;
    nx1 = nx2;
  }

  // ----------------------------------------------------------- partials
  // denominator per head: lanes of row g4 in every wave
  const float ls = row_sum16(lsum);
  if (t == 0) wred[w][g4] = ls;
  __syncthreads();
  const int hc = t >> 2;   // head of this lane's result column
  const int64_t pstride = kPartialStride;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s = 0.0f;
#pragma unroll
      for (int T = 0; T < NTV; ++T) s = fmaf(av[T], accV[r][T][i], s);
      s += __shfl_xor(s, 1, 64);    // sum the 4 limb columns of head hc
      s += __shfl_xor(s, 2, 64);
      v[i] = s;
    }
    if (hc < G && (t & 3) == 0) {
      float* pp = a.partials + ((static_cast<int64_t>(b) * a.n_q + h * G + hc) * a.n_splits + split) * pstride;
#pragma unroll
      for (int i = 0; i < 4; ++i) store_coherent(pp + 32 * w + 16 * r + 4 * g4 + i, v[i]);
    }
  }
  if (w == 0 && g4 == 0 && (t & 3) == 0 && hc < G) {   // one lane per head: running max and denominator
    float* pp = a.partials + ((static_cast<int64_t>(b) * a.n_q + h * G + hc) * a.n_splits + split) * pstride;
    store_coherent(pp + kD, m_b * kLn2);
    store_coherent(pp + kD + 1, (wred[0][hc] + wred[1][hc]) + (wred[2][hc] + wred[3][hc]));
  }
  if (!arrive_last(a.counters + b * a.n_kv + h, a.n_splits, &s_last)) return;
  combine_splits(a, b, h, qr, kThreads);
}

template <int KB, bool QJL, int VB>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.n_splits, a.n_kv, a.batch);
  hipLaunchKernelGGL((decode_mfma_kernel<KB, QJL, VB>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int KB, bool QJL>
hipError_t launch_v(const DecodeArgs& a, hipStream_t stream) {
  switch (a.v_bits) {
    case 2: return launch_t<KB, QJL, 2>(a, stream);
    case 3: return launch_t<KB, QJL, 3>(a, stream);
    case 4: return launch_t<KB, QJL, 4>(a, stream);
  }
  return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  if (a.v_codec != POLAR || a.group > 4) return hipErrorNotSupported;
  if (a.k_codec == POLAR_QJL) {
    switch (a.k_bits) {
      case 2: return launch_v<2, true>(a, stream);
      case 3: return launch_v<3, true>(a, stream);
      case 4: return launch_v<4, true>(a, stream);
    }
  } else if (a.k_codec == POLAR) {
    switch (a.k_bits) {
      case 2: return launch_v<2, false>(a, stream);
      case 3: return launch_v<3, false>(a, stream);
      case 4: return launch_v<4, false>(a, stream);
    }
  }
  return hipErrorNotSupported;
}

}  // namespace tq
