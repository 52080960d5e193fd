// tq_decode_reg.hip -- decode attention on the gfx950 matrix cores with the
// packed cache streamed straight into registers, for POLAR or POLAR_QJL keys
// and POLAR values, up to 16 query heads per KV head (groups of four).
//
// The arithmetic is the matrix-core form of the estimator, softmax and
// rotated-frame weighted sum (wis-web.com reader, TurboQuant article, the
// PolarQuant and QJL paragraphs; see tq_decode_mfma.hip for the operand
// algebra): code planes become fp4 operands with one and-or per dword, the
// query and p * radius enter as exact base-32 fp8 digits with E8M0 scales.
// What differs is the data flow:
//
//  * No cache byte is read twice and none is staged: lane (t, g4) of wave w
//    needs exactly the key words of k-block g4 at slots 32w + 2t, 32w + 2t + 1
//    (one 8-byte load per plane) and the value words of k-block g4 for
//    coordinates 32w + 2t, 32w + 2t + 1 (row t of the value product stands
//    for coordinate 32w + 2t + rr in its pass rr, so that those two words are
//    one 8-byte load too).  Each block's loads are issued three steps before
//    the step that uses them, into one of three register sets.
//  * The query side is prepared once per (sequence, KV head, head group) by
//    qprep_kernel and read as ready-made operands: no sketch table, rotation
//    or digit formation in the decode workgroups.
//  * With at most four terms per key code (2- and 3-bit keys) the codebook
//    coefficients are folded into the query digits (one operand per term),
//    so a column's terms accumulate in one matrix instruction chain instead
//    of being summed and weighted afterwards.
//  * A workgroup is one group of four waves taking one 128-position block per
//    step (one barrier per step), and several workgroups share a compute
//    unit, so their steps interleave.

#include <algorithm>

#include "tq_mfma_ops.h"

namespace tq {
namespace {

constexpr int kRegThreads = 256;

template <int KB>
struct KeyOps {
  static constexpr int nt = NTerms<KB>::n;
  static constexpr bool chain = nt <= 4;      // one operand per code term
  static constexpr int code_sets = chain ? nt : 1;
};

// ------------------------------------------------------------- query prep
// One workgroup of eight waves per (sequence, KV head, head group) of four
// query heads (zero past the group).  Waves 0..3 rotate head w's query
// (q_raw = H D_K q); every wave loads its 16-coordinate slice of the sketch
// table and forms its share of (S H D_K / sqrt d) q for the four heads (the
// eight shares of a row are added in wave order), so the table's loads are
// in flight together and no wave walks all 128 coordinates.  Then base-32
// digits with one E8M0 exponent per 32 k-slots (the operand layout of
// v_mfma_scale_f32_16x16x128_f8f6f4: k-slot k stands for coordinate or sketch
// row pos_of_slot(k); the k-slots that meet the sign field of the affine key
// operand carry the value with its sign flipped), one (operand set, head)
// pair per wave at a time, written as each decode lane's 32 operand bytes
// and scale byte.
constexpr int kPrepThreads = 512;
// The logit's constant factors travel in the query digits: log2(e) / sqrt d
// (softmax in base 2, scale 1/sqrt d) times 1/d for the code term (the raw
// FWHT's d) and sqrt(pi/2)/m for the sketch term (the estimator's constant);
// a logit is then n16 * code + rho16 * sketch.
constexpr float kCodeScale = 1.4426950408889634f * 0.08838834764831845f / 128.0f;
constexpr float kSketchScale = 1.4426950408889634f * 0.08838834764831845f * 1.2533141373155003f / 128.0f;

template <int KB, bool QJL>
__global__ __launch_bounds__(kPrepThreads) void qprep_kernel(DecodeArgs a) {
  using KO = KeyOps<KB>;
  constexpr int NSETS = KO::code_sets + (QJL ? 1 : 0);
  constexpr int kWavesP = kPrepThreads / 64;
  constexpr int kCpw = kD / kWavesP;   // table coordinates per wave
  __shared__ __attribute__((aligned(16))) uint8_t alimb[NSETS][16 * 128];   // [set][row = 4g + j][k]
  __shared__ uint8_t aexp[NSETS][4][16];                                   // [set][k / 32][row]
  __shared__ float cconst[NSETS][4];
  __shared__ float qr[4][kD];     // rotated query per head
  __shared__ float qs[4][kD];     // the query per head (before rotation)
  __shared__ __attribute__((aligned(16))) float sred[kWavesP][4][kM];   // [wave][head][row]: partial sketch sums
  const int nhg = (a.group + 3) >> 2;
  const int u = blockIdx.x;                  // (b * n_kv + h) * nhg + hg
  const int hg = u % nhg;
  const int h = (u / nhg) % a.n_kv;
  const int b = u / (nhg * a.n_kv);
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int G = min(4, a.group - 4 * hg);
  const int hq0 = h * a.group + 4 * hg;
  float2 st2[kCpw];
  if constexpr (QJL) {
#pragma unroll
    for (int c = 0; c < kCpw; ++c) st2[c] = *reinterpret_cast<const float2*>(a.tb.shd + (kCpw * w + c) * kM + 2 * lane);
  }
  if (w < 4) {
    const float* qp = a.q + (static_cast<int64_t>(b) * a.n_q + hq0 + min(w, G - 1)) * kD;
    const float q0 = (w < G) ? qp[lane] : 0.0f, q1 = (w < G) ? qp[lane + 64] : 0.0f;
    float lo = q0 * a.tb.dk[lane], hi = q1 * a.tb.dk[lane + 64];
    qs[w][lane] = q0;
    qs[w][lane + 64] = q1;
    wave_fwht128(lo, hi, lane);
    qr[w][lane] = lo;
    qr[w][lane + 64] = hi;
  }
  __syncthreads();
  if constexpr (QJL) {
    float acc[4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[g][0] = acc[g][1] = 0.0f;
#pragma unroll
    for (int c = 0; c < kCpw; ++c) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float x = qs[g][kCpw * w + c];
        acc[g][0] = fmaf(st2[c].x, x, acc[g][0]);
        acc[g][1] = fmaf(st2[c].y, x, acc[g][1]);
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) *reinterpret_cast<float2*>(&sred[w][g][2 * lane]) = make_float2(acc[g][0], acc[g][1]);
  }

  // digits of u at k-slots 2 lane, 2 lane + 1 into operand set `set`, head g
  auto write_digits = [&](int set, int g, float u0, float u1) __attribute__((always_inline)) {
    const int k0 = 2 * lane;
    const int fld = (k0 & 31) >> 3;
    if (fld == 3) {
      u0 = -u0;
      u1 = -u1;
    }
    const float m = row_max16(fmaxf(fabsf(u0), fabsf(u1)));
    const int s0 = (m >= 1e-30f) ? exponent_of(m) - 3 : 0;   // |u| 2^-s0 < 16
    float r0 = __builtin_amdgcn_ldexpf(u0, -s0), r1 = __builtin_amdgcn_ldexpf(u1, -s0);
    float t0 = 0.0f, t1 = 0.0f;   // digit-exact values, in units of 2^s0
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float d0 = rintf(r0), d1 = rintf(r1);   // integers in [-16, 16]: exact in e4m3
      const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(d0, d1, 0, false);
      t0 = fmaf(d0, __builtin_amdgcn_ldexpf(1.0f, -5 * j), t0);
      t1 = fmaf(d1, __builtin_amdgcn_ldexpf(1.0f, -5 * j), t1);
      r0 = (r0 - d0) * 32.0f;
      r1 = (r1 - d1) * 32.0f;
      *reinterpret_cast<uint16_t*>(&alimb[set][(4 * g + j) * 128 + k0]) = static_cast<uint16_t>(pk & 0xffff);
      if ((k0 & 31) == 0) aexp[set][k0 >> 5][4 * g + j] = static_cast<uint8_t>(min(max(s0 - 5 * j + 127, 1), 254));
    }
    const float wf = (fld == 0) ? 5.0f : (fld == 1) ? 3.0f : (fld == 2) ? 1.0f : 0.0f;
    const float c = wave_sum64(__builtin_amdgcn_ldexpf(wf * (t0 + t1), s0));
    if (lane == 0) cconst[set][g] = c;
  };
  const int r0 = pos_of_slot(2 * lane), r1 = pos_of_slot(2 * lane + 1);
  // the code sets: (set, head) pairs spread over the waves
  for (int job = w; job < KO::code_sets * 4; job += kWavesP) {
    const int s = job >> 2, g = job & 3;
    const float coef = (KO::chain ? a.tb.ak[s] : 1.0f) * kCodeScale;
    write_digits(s, g, coef * qr[g][r0], coef * qr[g][r1]);
  }
  if constexpr (QJL) {
    __syncthreads();   // every wave's sketch shares are in shared memory
    // the sketch set: head w - 4 on waves 4..7
    if (w >= 4) {
      const int g = w - 4;
      float u0 = 0.0f, u1 = 0.0f;
#pragma unroll
      for (int c = 0; c < kWavesP; ++c) {
        u0 += sred[c][g][r0];
        u1 += sred[c][g][r1];
      }
      write_digits(KO::code_sets, g, kSketchScale * u0, kSketchScale * u1);
    }
  }
  __syncthreads();

  // lane L of the decode waves: row L % 16, k = 64 (e / 16) + 16 (L / 16) + e % 16
  uint32_t* out = a.qops + static_cast<int64_t>(u) * (kQopsStride / 4);
  for (int s = w; s < NSETS; s += kWavesP) {
    const int t = lane & 15, g4 = lane >> 4;
    const uint4 l4 = *reinterpret_cast<const uint4*>(&alimb[s][t * 128 + 16 * g4]);
    const uint4 h4 = *reinterpret_cast<const uint4*>(&alimb[s][t * 128 + 64 + 16 * g4]);
    *reinterpret_cast<uint4*>(out + (2 * s) * 256 + 4 * lane) = l4;
    *reinterpret_cast<uint4*>(out + (2 * s + 1) * 256 + 4 * lane) = h4;
    out[kQopsScaleWord + s * 64 + lane] = aexp[s][g4][t];
  }
  if (threadIdx.x < 4) {
    float cq = 0.0f;
    if constexpr (KO::chain) {
#pragma unroll
      for (int s = 0; s < KO::code_sets; ++s) cq += cconst[s][threadIdx.x];
    } else {
      float aksum = 0.0f;
#pragma unroll
      for (int T = 0; T < KO::nt; ++T) aksum += a.tb.ak[T];
      cq = cconst[0][threadIdx.x] * aksum;
    }
    reinterpret_cast<float*>(out)[kQopsConstWord + threadIdx.x] = cq;
    reinterpret_cast<float*>(out)[kQopsConstWord + 4 + threadIdx.x] = QJL ? cconst[NSETS - 1][threadIdx.x] : 0.0f;
  }
}

// ---------------------------------------------------------------- decode
// The words lane (t, g4) of one wave uses from one key block and one value
// block.
template <int KB, bool QJL, int VB>
struct StepRegs {
  uint2 kp[KB];    // key planes: slots 32w + 2t, + 1 of k-block g4
  uint2 ks;        // sign plane, same slots
  uint32_t kn;     // fp16 radii of the two slots
  uint32_t kr;     // fp16 residual norms
  uint2 vp[VB];    // value planes: coordinates 32w + 2t, + 1 of k-block g4
  uint32_t vn;     // fp16 value radii of the two slots
};

template <int KB, bool QJL, int VB>
struct RegFmt {
  static constexpr int kNorms = 2048 * KB + (QJL ? 2048 : 0);
  static constexpr int kBytes = kNorms + 256 + (QJL ? 256 : 0);
  static constexpr int vBytes = 2048 * VB + 256;
  static constexpr int loads = KB + (QJL ? 3 : 1) + VB + 1;   // vector loads per step and wave
};

template <int KB, bool QJL, int VB, bool FUSED>
__device__ __forceinline__ void decode_reg_body(const DecodeArgs& a) {
  // three register sets, except in the serving step with QJL keys and 4-bit
  // values, where the quantiser's registers leave room for two within 256
  constexpr int kSets = (FUSED && QJL && VB == 4) ? 2 : 3;
  using KO = KeyOps<KB>;
  using F = RegFmt<KB, QJL, VB>;
  using R = StepRegs<KB, QJL, VB>;
  constexpr int NTK = KO::nt;
  constexpr int NCS = KO::code_sets;
  constexpr int NTV = NTerms<VB>::n;
  constexpr int kWaves = kRegThreads / 64;
  __shared__ __attribute__((aligned(16))) uint8_t plimb[2][16 * 128];   // [parity][col][k]: digits of p * radius
  __shared__ __attribute__((aligned(4))) uint8_t pexp[2][4][16];        // [parity][k / 32][col]
  __shared__ float rwb[2][kWaves][4];       // [parity][wave][head]: each wave's step reference
  __shared__ float wred[kWaves][4];
  __shared__ float mrun[4];
  __shared__ __attribute__((aligned(16))) float obuf[4][kD];
  __shared__ __attribute__((aligned(16))) float r_lds[kD];   // the serving step's key residual
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane & 15;
  const int g4 = lane >> 4;
  // Workgroup -> (split, KV head, sequence, head group); the head groups of
  // one (split, KV head, sequence) get ids 8 apart (one XCD, one L2)
  const int nhg = (a.group + 3) >> 2;
  const int n_units = a.n_splits * a.n_kv * a.batch;
  const int id = blockIdx.x;
  const int kx = id >> 3;
  const int unit = (kx / nhg) * 8 + (id & 7);
  if (unit >= n_units) return;
  const int hg = kx - (kx / nhg) * nhg;
  const int split = unit % a.n_splits;
  const int h = (unit / a.n_splits) % a.n_kv;
  const int b = unit / (a.n_splits * a.n_kv);
  const int G = min(4, a.group - 4 * hg);
  const int hq0 = h * a.group + 4 * hg;
  uint32_t* const counter = a.counters + (static_cast<int64_t>(b) * a.n_kv + h) * nhg + hg;
  typedef __attribute__((address_space(4))) const int cint;
  const int len_in = min(*((cint*)(a.seq_lens) + b), a.max_ctx);
  if constexpr (FUSED) {
    if (len_in < a.max_ctx && (len_in / kBlock) / a.chunk_blocks == split)
      fused_append<KB, QJL, VB>(a, b, h, len_in, w, lane, r_lds);
  }

  // ------------------------------------------------ query operands (ready-made)
  const uint32_t* qo = a.qops + ((static_cast<int64_t>(b) * a.n_kv + h) * nhg + hg) * (kQopsStride / 4);
  v8i Aq[NCS];
  int scq[NCS];
#pragma unroll
  for (int s = 0; s < NCS; ++s) {
    const uint4 l4 = *reinterpret_cast<const uint4*>(qo + (2 * s) * 256 + 4 * lane);
    const uint4 h4 = *reinterpret_cast<const uint4*>(qo + (2 * s + 1) * 256 + 4 * lane);
    Aq[s] = v8i{(int)l4.x, (int)l4.y, (int)l4.z, (int)l4.w, (int)h4.x, (int)h4.y, (int)h4.z, (int)h4.w};
    scq[s] = static_cast<int>(qo[kQopsScaleWord + s * 64 + lane]);
  }
  v8i Asq = Aq[0];
  int scsq = 127;
  if constexpr (QJL) {
    const uint4 l4 = *reinterpret_cast<const uint4*>(qo + (2 * NCS) * 256 + 4 * lane);
    const uint4 h4 = *reinterpret_cast<const uint4*>(qo + (2 * NCS + 1) * 256 + 4 * lane);
    Asq = v8i{(int)l4.x, (int)l4.y, (int)l4.z, (int)l4.w, (int)h4.x, (int)h4.y, (int)h4.z, (int)h4.w};
    scsq = static_cast<int>(qo[kQopsScaleWord + NCS * 64 + lane]);
  }
  const float cq = reinterpret_cast<const float*>(qo)[kQopsConstWord + g4];
  const float csq = QJL ? reinterpret_cast<const float*>(qo)[kQopsConstWord + 4 + g4] : 0.0f;
  float ak[NTK], av[NTV];
#pragma unroll
  for (int T = 0; T < NTK; ++T) ak[T] = a.tb.ak[T];
#pragma unroll
  for (int T = 0; T < NTV; ++T) av[T] = a.tb.av[T];

  // ------------------------------------------------------------- streaming
  const int len = FUSED ? min(len_in + 1, a.max_ctx) : len_in;
  const int nblk_seq = (len + kBlock - 1) / kBlock;
  const int blk0 = split * a.chunk_blocks;
  const int blk1 = min(blk0 + a.chunk_blocks, nblk_seq);
  const int n_iter = max(0, blk1 - blk0);
  const int64_t slot0_idx = (static_cast<int64_t>(b) * a.n_kv + h) * a.n_blocks;
  const uint8_t* kbase = a.kc + slot0_idx * a.k_block_bytes;
  const uint8_t* vbase = a.vc + slot0_idx * a.v_block_bytes;
  // the first two blocks are requested before the length is known: over the
  // whole cache of this (sequence, KV head); later ones only within the split
  const __amdgpu_buffer_rsrc_t rk0 = block_rsrc(kbase, F::kBytes, a.n_blocks);
  const __amdgpu_buffer_rsrc_t rv0 = block_rsrc(vbase, F::vBytes, a.n_blocks);
  const __amdgpu_buffer_rsrc_t rk = block_rsrc(kbase, F::kBytes, blk1);
  const __amdgpu_buffer_rsrc_t rv = block_rsrc(vbase, F::vBytes, blk1);
  const int so = 4 * (g4 * kBlock + 32 * w + 2 * t);   // key words of this lane (and value words)
  const int sn = 2 * (32 * w + 2 * t);                 // its two fp16 per-slot fields
  constexpr int kNT = 2;   // streaming loads (read once)
  // The block index is clamped to the resource's last block (blocks past the
  // split re-read that block, unused), so every address lies inside the
  // (sequence, KV head)'s cache; the block's base travels in the scalar
  // offset and each lane's offset inside the block is a constant register.
  auto load = [&](R& B, int blk, int nvalid, __amdgpu_buffer_rsrc_t rsk, __amdgpu_buffer_rsrc_t rsv)
      __attribute__((always_inline)) {
    const int bc = __builtin_amdgcn_readfirstlane(min(blk, nvalid - 1));
    const int kb0 = bc * F::kBytes, vb0 = bc * F::vBytes;
#pragma unroll
    for (int p = 0; p < KB; ++p) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b64(rsk, so, kb0 + p * 2048, kNT);
      B.kp[p] = make_uint2(x[0], x[1]);
    }
    if constexpr (QJL) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b64(rsk, so, kb0 + KB * 2048, kNT);
      B.ks = make_uint2(x[0], x[1]);
      B.kr = __builtin_amdgcn_raw_buffer_load_b32(rsk, sn, kb0 + F::kNorms + 256, kNT);
    }
    B.kn = __builtin_amdgcn_raw_buffer_load_b32(rsk, sn, kb0 + F::kNorms, kNT);
#pragma unroll
    for (int p = 0; p < VB; ++p) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b64(rsv, so, vb0 + p * 2048, kNT);
      B.vp[p] = make_uint2(x[0], x[1]);
    }
    B.vn = __builtin_amdgcn_raw_buffer_load_b32(rsv, sn, vb0 + 2048 * VB, kNT);
  };
  // kSets register sets: blocks i + 1 .. i + kSets - 1 are in flight while
  // block i is worked on
  R buf0, buf1, buf2;
  load(buf0, blk0, a.n_blocks, rk0, rv0);
  load(buf1, blk0 + 1, a.n_blocks, rk0, rv0);
  if constexpr (kSets == 3) load(buf2, blk0 + 2, a.n_blocks, rk0, rv0);

  float m_a = -INFINITY, m_b = -INFINITY;   // running reference of head g4 (denominator) / head t / 4 (column)
  float m_top = -INFINITY;                  // Sparse-V: largest step reference of head t / 4 so far
  const bool sparse_v = a.sparse_v > 0;
  const float tau_v = static_cast<float>(a.sparse_v);
  float lsum = 0.0f;
  v4f accV[2][NTV];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int T = 0; T < NTV; ++T) accV[r][T] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  v4f accO = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const v8i aoff = expand_fp4_affine(t < 8 ? 0xffffffffu : 0u);

  // One step: logits of this wave's 32 positions for the four heads, its
  // reference and the digits of p * radius; one barrier; the running
  // references and the weighted sum of the block's values for this wave's 32
  // coordinates; then the register set is refilled kSets blocks ahead.
  auto step = [&](R& B, int i) __attribute__((always_inline)) {
    wait_vm<(kSets - 1) * F::loads>();   // this set has landed (the later sets' loads may still be in flight)
    const int blk = blk0 + i;
    const int n_t = min(kBlock, len - blk * kBlock);
    float lg2[2];
    // column group c = slots 32 w + 2 t + c: its matrix products, then its
    // logit (one column group at a time keeps the unchained sums' registers
    // to one group's)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t wd[KB];
#pragma unroll
      for (int p = 0; p < KB; ++p) wd[p] = c ? B.kp[p].y : B.kp[p].x;
      float code;
      if constexpr (KO::chain) {
        v4f acc = v4f{-cq, 0.0f, 0.0f, 0.0f};   // the affine operands' offset, removed up front
#pragma unroll
        for (int T = 0; T < NTK; ++T) acc = mfma_fp8_fp4(Aq[T], expand_fp4_affine(term_word<KB>(wd, T)), acc, scq[T]);
        code = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      } else {
        v4f dT[NTK];
#pragma unroll
        for (int T = 0; T < NTK; ++T)
          dT[T] = mfma_fp8_fp4(Aq[0], expand_fp4_affine(term_word<KB>(wd, T)), v4f{0.0f, 0.0f, 0.0f, 0.0f}, scq[0]);
        code = -cq;
#pragma unroll
        for (int T = 0; T < NTK; ++T) code = fmaf(ak[T], (dT[T][0] + dT[T][1]) + (dT[T][2] + dT[T][3]), code);
      }
      float qj = 0.0f;
      if constexpr (QJL) {
        const v4f dQ = mfma_fp8_fp4(Asq, expand_fp4_affine(c ? B.ks.y : B.ks.x), v4f{-csq, 0.0f, 0.0f, 0.0f}, scsq);
        qj = (dQ[0] + dQ[1]) + (dQ[2] + dQ[3]);
      }
      const int tok = pos_of_slot(32 * w + 2 * t + c);
      const float nk = h2f(c ? (B.kn >> 16) : B.kn);
      const float rho = QJL ? h2f(c ? (B.kr >> 16) : B.kr) : 0.0f;
      const float l2 = fmaf(nk, code, QJL ? __fmul_rn(rho, qj) : 0.0f);
      const bool valid = (tok < n_t) && (g4 < G);
      if (a.logits != nullptr && valid)
        a.logits[(static_cast<int64_t>(b) * a.n_q + hq0 + g4) * a.max_ctx + blk * kBlock + tok] = __fmul_rn(l2, kLn2);
      lg2[c] = valid ? l2 : -INFINITY;
    }
    // this wave's reference per head (row g4): the integer ceiling of its
    // step maximum; p <= 1 against it
    const int par = i & 1;
    uint8_t* const pl = &plimb[par][0];
    uint8_t* const pe = &pexp[par][0][0];
    const float mloc = row_max16(fmaxf(lg2[0], lg2[1]));
    const float rw = (mloc == -INFINITY) ? -INFINITY : ceilf(mloc);
    if (t == 0) rwb[par][w][g4] = rw;
    const float p0 = (lg2[0] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(lg2[0] - rw);
    const float p1 = (lg2[1] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(lg2[1] - rw);
    {
      float r0 = (p0 > 0.0f) ? p0 * h2f(B.vn) : 0.0f;
      float r1 = (p1 > 0.0f) ? p1 * h2f(B.vn >> 16) : 0.0f;
      const float pm = row_max16(fmaxf(r0, r1));
      const int s0 = (pm >= 1e-30f) ? exponent_of(pm) - 3 : 0;   // r 2^-s0 < 16
      const float sgn = (t >= 12) ? -1.0f : 1.0f;   // k-slots on the value operand's sign field
      r0 = sgn * __builtin_amdgcn_ldexpf(r0, -s0);
      r1 = sgn * __builtin_amdgcn_ldexpf(r1, -s0);
      uint32_t ebytes = 127u << 24;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int pk = 0;   // the fourth digit row stays zero
        if (j < 3) {
          const float d0 = rintf(r0), d1 = rintf(r1);
          pk = __builtin_amdgcn_cvt_pk_fp8_f32(d0, d1, 0, false);
          if (j < 2) {
            r0 = (r0 - d0) * 32.0f;
            r1 = (r1 - d1) * 32.0f;
          }
          ebytes |= static_cast<uint32_t>(min(max(s0 - 5 * j + 127, 1), 254)) << (8 * j);
        }
        *reinterpret_cast<uint16_t*>(&pl[(4 * g4 + j) * 128 + 32 * w + 2 * t]) = static_cast<uint16_t>(pk & 0xffff);
      }
      if (t == 0) *reinterpret_cast<uint32_t*>(&pe[16 * w + 4 * g4]) = ebytes;
    }
    const float ps = p0 + p1;
    lds_barrier();

    // running references of head g4 (denominator) and head t / 4 (column)
    const int hb = t >> 2;
    float ra = rwb[par][0][g4], rb = rwb[par][0][hb];
#pragma unroll
    for (int u = 1; u < kWaves; ++u) {
      ra = fmaxf(ra, rwb[par][u][g4]);
      rb = fmaxf(rb, rwb[par][u][hb]);
    }
    const float mn_a = (ra > m_a + 8.0f) ? ra : m_a;
    const float mn_b = (rb > m_b + 8.0f) ? rb : m_b;
    const float fh = (m_a == -INFINITY) ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, static_cast<int>(m_a - mn_a));
    const float fv = (m_b == -INFINITY) ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, static_cast<int>(m_b - mn_b));
    lsum = lsum * fh + ((rw == -INFINITY) ? 0.0f : __builtin_amdgcn_ldexpf(ps, static_cast<int>(rw - mn_a)));
    m_a = mn_a;
    m_b = mn_b;
    if (__any(fv != 1.0f)) {   // rescale only when some head's reference moved
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int T = 0; T < NTV; ++T) accV[rr][T] *= fv;
      accO *= fv;
    }
    bool skip = false;
    if (sparse_v) {
      // every weight of the block below 2^-tau of the largest one so far, for
      // every head of the group: the value work is skipped (the weights stay
      // in the denominator)
      m_top = fmaxf(m_top, rb);
      skip = __all((rb == -INFINITY) || (rb < m_top - tau_v));
    }
    if (!skip) {
      v8i Pv;
      {
        const uint4 lo = *reinterpret_cast<const uint4*>(&pl[t * 128 + 16 * g4]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&pl[t * 128 + 64 + 16 * g4]);
        Pv = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      // k-block g4 holds wave g4's positions: its digits carry 2^(its reference - the running one)
      const float rk_ = rwb[par][g4][hb];
      const int adj = (rk_ == -INFINITY) ? 0 : static_cast<int>(rk_ - m_b);
      const int scp = min(max(static_cast<int>(pe[16 * g4 + t]) + adj, 1), 254);
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        uint32_t vw[VB];
#pragma unroll
        for (int p = 0; p < VB; ++p) vw[p] = rr ? B.vp[p].y : B.vp[p].x;
#pragma unroll
        for (int T = 0; T < NTV; ++T)
          accV[rr][T] = mfma_fp4_fp8(expand_fp4_affine(term_word<VB>(vw, T)), Pv, accV[rr][T], scp);
      }
      accO = mfma_fp4_fp8(aoff, Pv, accO, scp);
    }
    // refill this register set kSets blocks ahead
    load(B, blk + kSets, blk1, rk, rv);
  };

  if (n_iter > 0) {   // uniform over the workgroup
    int i = 0;
    if constexpr (kSets == 3) {
      for (; i + 3 <= n_iter; i += 3) {
        step(buf0, i);
        step(buf1, i + 1);
        step(buf2, i + 2);
      }
      if (i < n_iter) step(buf0, i);
      if (i + 1 < n_iter) step(buf1, i + 1);
    } else {
      for (; i + 2 <= n_iter; i += 2) {
        step(buf0, i);
        step(buf1, i + 1);
      }
      if (i < n_iter) step(buf0, i);
    }
  }

  // ------------------------------------------------------------- partials
  const float dva = a.tb.dv[lane], dvb = a.tb.dv[lane + 64];
  {
    const float ls = row_sum16(lsum);
    if (t == 0) wred[w][g4] = ls;
    if (w == 0 && t == 0) mrun[g4] = m_a;
    const int hc = t >> 2;
    float avsum = 0.0f;
#pragma unroll
    for (int T = 0; T < NTV; ++T) avsum += av[T];
    const float voff = avsum * 0.5f * (accO[0] + __shfl_xor(accO[0], 32, 64));
    float v[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = -voff;
#pragma unroll
        for (int T = 0; T < NTV; ++T) s = fmaf(av[T], accV[r][T][i], s);
        s += __shfl_xor(s, 1, 64);   // the 4 digit columns of head hc
        s += __shfl_xor(s, 2, 64);
        v[r][i] = s;
      }
    // result row 4 g4 + i of pass r is coordinate 32 w + 8 g4 + 2 i + r
    if (hc < G && (t & 3) == 0) {
      float* o = &obuf[hc][32 * w + 8 * g4];
      *reinterpret_cast<float4*>(o) = make_float4(v[0][0], v[1][0], v[0][1], v[1][1]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(v[0][2], v[1][2], v[0][3], v[1][3]);
    }
  }
  __syncthreads();
  if (w < G) {
    float lo = obuf[w][lane], hi = obuf[w][lane + 64];
    wave_fwht128(lo, hi, lane);
    const float inv_d = 1.0f / static_cast<float>(kD);
    lo *= dva * inv_d;
    hi *= dvb * inv_d;
    float* pp = a.partials + ((static_cast<int64_t>(b) * a.n_q + hq0 + w) * a.n_splits + split) * kPartialStride;
    store_coherent(pp + lane, lo);
    store_coherent(pp + 64 + lane, hi);
    if (lane == 0) {
      float l = 0.0f;
#pragma unroll
      for (int u = 0; u < kWaves; ++u) l += wred[u][w];
      store_coherent(pp + kD, mrun[w] * kLn2);
      store_coherent(pp + kD + 1, l);
    }
  }
  if (!arrive_last(counter, a.n_splits, &s_last)) return;
  merge_splits(a, b, hq0, G, counter, w, lane);
}

template <int KB, bool QJL, int VB>
__global__ __launch_bounds__(kRegThreads, 2) void decode_reg_kernel(DecodeArgs a) {
  decode_reg_body<KB, QJL, VB, false>(a);
}

template <int KB, bool QJL, int VB>
__global__ __launch_bounds__(kRegThreads, 2) void decode_reg_append_kernel(DecodeArgs a) {
  decode_reg_body<KB, QJL, VB, true>(a);
}

template <int KB, bool QJL, int VB>
hipError_t launch_kv(const DecodeArgs& a, hipStream_t stream) {
  const int nhg = (a.group + 3) / 4;
  hipLaunchKernelGGL((qprep_kernel<KB, QJL>), dim3(a.batch * a.n_kv * nhg), dim3(kPrepThreads), 0, stream, a);
  const int n_units = a.n_splits * a.n_kv * a.batch;
  dim3 grid(((n_units + 7) / 8) * 8 * nhg);
  if (a.k_new != nullptr)
    hipLaunchKernelGGL((decode_reg_append_kernel<KB, QJL, VB>), grid, dim3(kRegThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_reg_kernel<KB, QJL, VB>), grid, dim3(kRegThreads), 0, stream, a);
  return hipGetLastError();
}

template <int KB, bool QJL>
hipError_t launch_k(const DecodeArgs& a, hipStream_t stream) {
  switch (a.v_bits) {
    case 2: return launch_kv<KB, QJL, 2>(a, stream);
    case 3: return launch_kv<KB, QJL, 3>(a, stream);
    case 4: return launch_kv<KB, QJL, 4>(a, stream);
  }
  return hipErrorNotSupported;
}

}  // namespace

bool decode_reg_applies(int k_codec, int v_codec, int group) {
  return v_codec == POLAR && group <= kMaxGroup && (k_codec == POLAR || k_codec == POLAR_QJL);
}

hipError_t launch_decode_reg(const DecodeArgs& a, hipStream_t stream) {
  if (!decode_reg_applies(a.k_codec, a.v_codec, a.group) || a.qops == nullptr) return hipErrorNotSupported;
  // block byte offsets (up to n_blocks + 2 blocks) are 32-bit buffer offsets
  const int64_t span = (static_cast<int64_t>(a.n_blocks) + 4) * std::max(a.k_block_bytes, a.v_block_bytes);
  if (span >= (int64_t{1} << 31) || static_cast<int64_t>(a.n_splits) * kPartialStride * 4 >= (int64_t{1} << 31))
    return hipErrorNotSupported;
  if (a.k_codec == POLAR_QJL) {
    switch (a.k_bits) {
      case 2: return launch_k<2, true>(a, stream);
      case 3: return launch_k<3, true>(a, stream);
      case 4: return launch_k<4, true>(a, stream);
    }
  } else {
    switch (a.k_bits) {
      case 2: return launch_k<2, false>(a, stream);
      case 3: return launch_k<3, false>(a, stream);
      case 4: return launch_k<4, false>(a, stream);
    }
  }
  return hipErrorNotSupported;
}

}  // namespace tq
