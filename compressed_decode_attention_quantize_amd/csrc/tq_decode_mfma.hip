// tq_decode_mfma.hip -- decode attention on the gfx950 matrix cores, for
// POLAR, POLAR_QJL or q8 keys and POLAR values, with up to 16 query heads per
// KV head served in head groups of four.
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
//  * A bit vector becomes an fp4 (e2m1) matrix operand in one integer
//    operation per 8 elements by leaving each bit where it lies and filling
//    the other fields of its nibble (see expand_fp4_affine): the elements are
//    affine in the signs, and the offset, one constant per head, is removed
//    after the product.  Value words take the same form; their offset
//    depends on the probabilities of the step and is itself a matrix product
//    (see the offset operand below).
//  * The query side (q_raw = H D_K q and sq = S q_raw / sqrt d) is written as
//    four base-32 fixed-point digits, integers in [-16, 16] that e4m3 holds
//    exactly, with one E8M0 scale per digit (about 19 significant bits).  The
//    products are then small integers, and the 128-term sums of
//    v_mfma_scale_f32_16x16x128_f8f6f4 are exact; with floating-point limbs
//    the instruction's accumulation loses low bits of the small products.
//    One instruction covers 4 heads x 4 digits x 16 positions x 128
//    coordinates.
//  * The weighted sum is the same contraction over positions: value planes
//    (32 positions per word) are the fp4 operand, p * radius is written as
//    three base-32 digits per 32 positions (about 14 significant bits).
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
// Mapping: grid (split, KV head, sequence, head group); a workgroup is NG
// groups of four waves (NG = 2: one workgroup per compute unit; NG = 1: two;
// the host picks NG per call).
// Each step takes NG 128-position blocks, one per group, from a ring of
// shared-memory slots that direct memory-to-shared-memory copies fill several
// steps ahead.  Within a group, wave w computes the logits of its block's
// positions in k-slots [32w, 32w+32) (2 MFMA column groups) and the digits of
// p * radius for them; after the step's one barrier the waves agree on the
// running reference and wave w computes its group's weighted sum for
// coordinates [32w, 32w+32).  The query set-up (rotation, sketch, digits) is
// done once per workgroup while the first copies are in flight.  The groups'
// sums are added in shared memory and rotated back (D_V H / d) before they
// leave the workgroup, so the workgroup that merges the splits only forms a
// weighted average.

#include <algorithm>

#include "tq_mfma_ops.h"

namespace tq {
namespace {

// read-only data at wave-uniform addresses: loads through the scalar cache
typedef __attribute__((address_space(4))) const v4f cv4f;
typedef __attribute__((address_space(4))) const float cfloat;

constexpr int kRing = 4;    // most ring slots in shared memory

// Byte layout of one cache block (128 positions) and of the shared-memory
// ring that stages NG blocks per step.
// NG block groups (four wavefronts each) per workgroup: with one group two
// workgroups share a compute unit and each may take half of its shared memory.
template <int KB, bool QJL, int VB, int NG>
struct Fmt {
  static constexpr int waves = 4 * NG;
  static constexpr int threads = 64 * waves;
  static constexpr int ldsBudget = (NG == 2 ? 160 : 80) * 1024;
  static constexpr bool q8 = KB == 8;   // q8 keys: int8[128][128], then fp16 scales [128][4]
  static constexpr int kNorms = q8 ? 0 : 2048 * KB + (QJL ? 2048 : 0);   // fp16 radii after planes (and signs)
  static constexpr int kBytes = q8 ? 128 * 128 + 128 * 8 : kNorms + 256 + (QJL ? 256 : 0);   // K block
  static constexpr int vBytes = 2048 * VB + 256;                       // V block: planes, fp16 radii
  static constexpr int kChunks = (NG * kBytes + 1023) / 1024;          // 1 KB copy units per step (NG blocks)
  static constexpr int vChunks = (NG * vBytes + 1023) / 1024;
  static constexpr int perWave = (kChunks + vChunks + waves - 1) / waves;   // copies per wave per step
  static constexpr int slotBytes = (kChunks + vChunks) * 1024;
  static constexpr int kOtherLds = (NG == 2 ? 31 : 20) * 1024;   // everything else the kernel keeps in shared memory
  static constexpr int slotsFit = (ldsBudget - kOtherLds) / slotBytes;
  static constexpr int nSlots = slotsFit < kRing ? slotsFit : kRing;
  static_assert(nSlots >= 2, "ring needs two slots");
};

typedef __attribute__((address_space(3))) void lds_void_t;

// q8 key rows (128 B per position) are stored in shared memory with their
// 16-byte granules permuted: granule j of position tok sits at granule
// j ^ q8_swizzle(tok) of its row.  The sixteen positions one matrix operand
// reads together then fall on distinct banks (plain rows share every bank).
__device__ __forceinline__ int q8_swizzle(int tok) { return ((tok >> 3) & 3) | ((tok & 2) << 1); }

template <int KB, bool QJL, int VB, int NG>
struct PairCopier {
  using F = Fmt<KB, QJL, VB, NG>;
  int lo[F::perWave];   // per-lane byte offset of each copy, less the block term
  // lane offsets and units of this wave's copies (q = w + 8 j)
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int j = 0; j < F::perWave; ++j) {
      const int q = w + F::waves * j;
      const bool isk = q < F::kChunks;
      const bool isv = !isk && q < F::kChunks + F::vChunks;
      int kgr = 64 * q + lane;   // granule of the step's K region this lane fills
      if constexpr (F::q8) {
        const int half = (kgr >= F::kBytes / 16) ? 1 : 0;
        const int g = kgr - half * (F::kBytes / 16);
        if (g < kBlock * kD / 16) kgr = half * (F::kBytes / 16) + (g & ~7) + ((g & 7) ^ q8_swizzle(g >> 3));
      }
      lo[j] = isk ? 16 * kgr : (isv ? 1024 * (q - F::kChunks) + 16 * lane : 0x7fff0000 + 16 * lane);
    }
  }
  // Copies the NG blocks from b0 (K region then V region) into a ring
  // slot straight from memory into shared memory, 1 KB per instruction (lane
  // l moves bytes 16l..16l+15 of its unit).  Every wave issues the same number
  // of copies; units past the data read zero into a junk buffer, so the count
  // of outstanding copies per wave is the same at every step.
  __device__ __forceinline__ void copy(uint8_t* slot, uint8_t* junk, __amdgpu_buffer_rsrc_t rk,
                                       __amdgpu_buffer_rsrc_t rv, int b0, int w) const {
#pragma unroll
    for (int j = 0; j < F::perWave; ++j) {
      const int q = w + F::waves * j;   // unit, uniform over the wave
      const bool isk = q < F::kChunks;
      const bool isv = !isk && q < F::kChunks + F::vChunks;
      const int stride = isk ? F::kBytes : (isv ? F::vBytes : 0);   // uniform
      uint8_t* dst = (isk || isv) ? slot + 1024 * q : junk;
      // (the block's base in the scalar offset: no per-lane add)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isk ? rk : rv, (lds_void_t*)(dst), 16, lo[j],
                                               __builtin_amdgcn_readfirstlane(b0 * stride), 0, 0);
    }
  }
};

template <int KB, bool QJL, int VB, int NG, bool FUSED>
__device__ __forceinline__ void decode_mfma_body(const DecodeArgs& a) {
  using F = Fmt<KB, QJL, VB, NG>;
  constexpr int kWaves = F::waves;
  constexpr bool KQ8 = F::q8;
  constexpr int NTK = NTerms<KB>::n;
  constexpr int NTV = NTerms<VB>::n;
  constexpr int NS = F::nSlots;
  // ring of step blocks: one array per slot, so that the compiler can tell
  // the slots' copies apart when it places its waits
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[F::slotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[F::slotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[NS > 2 ? F::slotBytes : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t slot3[NS > 3 ? F::slotBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t junk[1024];
  __shared__ float qr[4 * kD];              // q_raw = H D_K q per head (zero rows past G)
  __shared__ __attribute__((aligned(16))) uint8_t alimb[2][16 * 128];  // fp8 limbs [set][row = 4g + j][k]
  __shared__ uint8_t aexp[2][4][16];        // E8M0 scale [set][k / 32][row]
  __shared__ __attribute__((aligned(16))) uint8_t plimb[NG][16 * 128];  // per group: limbs of p * radius [col][k]
  __shared__ __attribute__((aligned(4))) uint8_t pexp[NG][4][16];       // per group: [k / 32][col]
  __shared__ float rwb[2][kWaves][4];       // per step parity: each wave's reference per head
  __shared__ float wred[kWaves][4];
  __shared__ float mrun[4];                 // running max per head at the end (log2 units)
  __shared__ float cconst[2][4];            // offsets of the affine key operand per (set, head)
  __shared__ __attribute__((aligned(8))) int8_t qdig[4][3][kD];   // q8 keys: base-128 digits of q per head
  __shared__ int qexp8[4];                  // q8 keys: leading exponent per head
  __shared__ __attribute__((aligned(16))) float sred[kWaves][4 * kM];   // partial sketch sums; later the group sums
  __shared__ int s_last;
  uint8_t* const slots[4] = {slot0, slot1, slot2, slot3};
  // digit buffers of odd steps: the query's digit buffers, free once the
  // operands are in registers
  uint8_t* const plimb0 = &plimb[0][0];
  uint8_t* const plimb1 = &alimb[0][0];
  uint8_t* const pexp0 = &pexp[0][0][0];
  uint8_t* const pexp1 = &aexp[0][0][0];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: buffer resources stay scalar
  const int gr = w >> 2;   // group: the first or second block of each step
  const int wl = w & 3;    // wave within the group
  const int t = lane & 15;
  const int g4 = lane >> 4;
  // Workgroup -> (split, KV head, sequence, head group).  Workgroups are
  // dispatched to the 8 XCDs round-robin by linear id, so the head groups of
  // one (split, KV head, sequence) unit get ids 8 apart: they run at the same
  // time on one XCD and read the unit's blocks through the same L2.
  const int nhg = (a.group + 3) >> 2;      // groups of up to four query heads per KV head
  const int n_units = a.n_splits * a.n_kv * a.batch;
  const int id = blockIdx.x;
  const int kx = id >> 3;
  const int unit = (kx / nhg) * 8 + (id & 7);
  if (unit >= n_units) return;             // padding of the grid to whole rounds of 8
  const int hg = kx - (kx / nhg) * nhg;    // head group of this workgroup
  const int split = unit % a.n_splits;
  const int h = (unit / a.n_splits) % a.n_kv;   // KV head
  const int b = unit / (a.n_splits * a.n_kv);
  const int G = min(4, a.group - 4 * hg);  // query heads served here
  const int hq0 = h * a.group + 4 * hg;    // the first of them
  uint32_t* const counter = a.counters + (static_cast<int64_t>(b) * a.n_kv + h) * nhg + hg;
  // a scalar load: a vector load here would make the first wait for it also
  // wait for every query and table load issued before it
  typedef __attribute__((address_space(4))) const int cint;
  const int len_in = min(*((cint*)(a.seq_lens) + b), a.max_ctx);
  if constexpr (FUSED) {
    // before anything else, so that nothing of the decode is live across it
    if (len_in < a.max_ctx && split_of_block(a, len_in / kBlock) == split)
      fused_append<KB, QJL, VB>(a, b, h, len_in, w, lane, reinterpret_cast<float*>(junk));
  }
  // loads the set-up needs are issued first, before the sequence length they
  // do not depend on: this wave's query rows, the rotation signs, its slice
  // of the sketch table, the codebook coefficients
  const float* qb0 = a.q + (static_cast<int64_t>(b) * a.n_q + hq0) * kD;
  const float* qp = qb0 + min(w & 3, G - 1) * kD;
  const float qa = qp[lane], qb = qp[lane + 64];
  const float da = a.tb.dk[lane], db = a.tb.dk[lane + 64];
  // the sketch's inputs: this wave takes coordinates [kCpw w, kCpw (w + 1));
  // lane l holds raw query coordinate kCpw w + 16 c + l % 16 of head l / 16
  // (zero past G) and sketch rows 2 (l % 64), 2 (l % 64) + 1 of the table
  constexpr int kCpw = kD / kWaves;
  float qsl[kCpw / 16];
#pragma unroll
  for (int c = 0; c < kCpw / 16; ++c) qsl[c] = qb0[min(lane >> 4, G - 1) * kD + kCpw * w + 16 * c + (lane & 15)];
  const int jq = threadIdx.x & 63;
  float2 st2[kCpw];
  if (QJL) {
#pragma unroll
    for (int u = 0; u < kCpw; ++u) st2[u] = *reinterpret_cast<const float2*>(a.tb.shd + (kCpw * w + u) * kM + 2 * jq);
  }
  float ak[NTK];
  {
    const cfloat* akp = (const cfloat*)(a.tb.ak);
#pragma unroll
    for (int T = 0; T < NTK; ++T) ak[T] = akp[T];
  }
  const int len = FUSED ? min(len_in + 1, a.max_ctx) : len_in;
  const int nblk_seq = (len + kBlock - 1) / kBlock;
  const int blk0 = split_first_block(a, split);
  const int blk1 = min(blk0 + split_block_count(a, split), nblk_seq);
  const int n_iter = max(0, (blk1 - blk0 + NG - 1) / NG);   // steps of NG blocks
  const int64_t slot0_idx = (static_cast<int64_t>(b) * a.n_kv + h) * a.n_blocks;
  const float inv_sqrt_d = 0.08838834764831845f;
  // The optional logits go through a buffer over this (sequence, head
  // group)'s rows, range-checked by the hardware: a lane with no logit to
  // store takes an offset past its end (no branch in the step)
  const __amdgpu_buffer_rsrc_t rlg = __builtin_amdgcn_make_buffer_rsrc(
      a.logits != nullptr ? a.logits + (static_cast<int64_t>(b) * a.n_q + hq0) * a.max_ctx : a.logits,
      static_cast<short>(0), a.logits != nullptr ? G * a.max_ctx * 4 : 0, 0x00020000);

  float av[NTV];
#pragma unroll
  for (int T = 0; T < NTV; ++T) av[T] = a.tb.av[T];
  // running max (log2 units) of head g4 (this lane's logits row) and of head
  // t / 4 (this lane's result column); both follow the same step maxima
  float m_a = -INFINITY, m_b = -INFINITY;
  // Sparse-V: the largest step reference of head t / 4 so far (not lazy), and
  // the skip distance in log2 units
  float m_top = -INFINITY;
  const bool sparse_v = a.sparse_v > 0;
  const float tau_v = static_cast<float>(a.sparse_v);
  float lsum = 0.0f;   // this lane's share of the denominator of head g4
  v4f accV[2][NTV];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int T = 0; T < NTV; ++T) accV[r][T] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  // Offset of the affine value operand: rows 0..7 of aoff are the all-one
  // word, rows 8..15 the all-zero word, so lanes 0..31 of accO gather the
  // all-one row's products and lanes 32..63 the all-zero row's; their mean
  // is what every value row carries on top of its signed sum.
  v4f accO = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const Fp4Fill kf = fp4_fill();
  const v8i aoff = expand_fp4_affine_v(t < 8 ? 0xffffffffu : 0u, kf);

  {
    // The query set-up and the ring's first copies do not wait for the
    // sequence length: the first copies range over the whole cache of this
    // (sequence, KV head) (blocks past the sequence are read but never
    // weighted), the loop's copies only over [0, blk1).
    float aksum = 0.0f;
    __builtin_amdgcn_sched_barrier(0);
    const __amdgpu_buffer_rsrc_t rk0 = block_rsrc(a.kc + slot0_idx * a.k_block_bytes, a.k_block_bytes, a.n_blocks);
    const __amdgpu_buffer_rsrc_t rv0 = block_rsrc(a.vc + slot0_idx * a.v_block_bytes, a.v_block_bytes, a.n_blocks);
    // the blocks of the first NS - 1 steps (at most three) are issued one per set-up phase
    // (step 0's here), so that the copies proceed while the waves compute
    PairCopier<KB, QJL, VB, NG> cp;
    cp.init(w, lane);
    cp.copy(slots[0], junk, rk0, rv0, blk0, w);

    // ------------------------------------------------------------- set-up
    // Waves 0..3 rotate the query of head w in registers (q_raw = H D_K q)
    // and write its digits; meanwhile every wave forms its share of the
    // sketch S q_raw / sqrt d as (S H D_K / sqrt d) q, which needs no rotated
    // query, and after one barrier waves 4..7 add the shares and write the
    // sketch's digits.
    //
    // Digits: base-32 fixed point of q' with one leading exponent per 32
    // k-slots (the E8M0 scales are per row and per 32 k-slots), k-slot k
    // holding coordinate (or sketch row) pos_of_slot(k); q' is the value with
    // its sign flipped on the k-slots that meet the sign field of the key
    // operand, (k mod 32) / 8 == 3.  The set's constant is the sum of 5, 3, 1,
    // 0 times the digit-exact q' over the k-slots of field 0..3.  Lane l of
    // the writing wave takes k-slots 2l, 2l + 1, so the 32 k-slots of an
    // exponent are the 16 lanes of a row.
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
    if constexpr (KQ8) {
      // q8 keys meet the query unrotated: three base-128 digits of q per head,
      // integers in [-64, 64], for the int8 matrix instruction
      if (w < 4) {
        const float x0 = (w < G) ? qa : 0.0f, x1 = (w < G) ? qb : 0.0f;
        const float m = wave_max64(fmaxf(fabsf(x0), fabsf(x1)));
        const int e = (m >= 1e-30f) ? exponent_of(m) - 5 : 0;   // |q| 2^-e < 64
        float r0 = __builtin_amdgcn_ldexpf(x0, -e), r1 = __builtin_amdgcn_ldexpf(x1, -e);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const float d0 = rintf(r0), d1 = rintf(r1);
          qdig[w][j][lane] = static_cast<int8_t>(d0);
          qdig[w][j][lane + 64] = static_cast<int8_t>(d1);
          r0 = (r0 - d0) * 128.0f;
          r1 = (r1 - d1) * 128.0f;
        }
        if (lane == 0) qexp8[w] = e;
      }
    } else if (w < 4) {
      float q_lo = (w < G) ? qa * da : 0.0f;
      float q_hi = (w < G) ? qb * db : 0.0f;
      wave_fwht128(q_lo, q_hi, lane);
      qr[w * kD + lane] = q_lo;
      qr[w * kD + lane + 64] = q_hi;
      // the same wave reads back its own rotated query in k-slot order (with a
      // sketch, after the barrier, beside the waves that write its digits)
      if constexpr (!QJL) write_digits(0, w, qr[w * kD + pos_of_slot(2 * lane)], qr[w * kD + pos_of_slot(2 * lane + 1)]);
    }
    if (QJL) {
      float acc[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[g][0] = acc[g][1] = 0.0f;
#pragma unroll
      for (int u = 0; u < kCpw; ++u) {
        const float qsv = ((lane >> 4) < G) ? qsl[u >> 4] : 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int x = __builtin_amdgcn_readlane(__float_as_int(qsv), 16 * g + (u & 15));
          acc[g][0] = fmaf(st2[u].x, __int_as_float(x), acc[g][0]);
          acc[g][1] = fmaf(st2[u].y, __int_as_float(x), acc[g][1]);
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) *reinterpret_cast<float2*>(&sred[w][g * kM + 2 * jq]) = make_float2(acc[g][0], acc[g][1]);
      lds_barrier();
      if constexpr (NS > 2) cp.copy(slots[1], junk, rk0, rv0, blk0 + NG, w);
      if (w < 4) write_digits(0, w, qr[w * kD + pos_of_slot(2 * lane)], qr[w * kD + pos_of_slot(2 * lane + 1)]);
      if (w >= kWaves - 4) {
        // sketch rows pos_of_slot(2 lane), pos_of_slot(2 lane + 1) of head g
        const int g = w - (kWaves - 4);
        const int r0 = pos_of_slot(2 * lane), r1 = pos_of_slot(2 * lane + 1);
        float u0 = 0.0f, u1 = 0.0f;
#pragma unroll
        for (int c = 0; c < kWaves; ++c) {
          u0 += sred[c][g * kM + r0];
          u1 += sred[c][g * kM + r1];
        }
        write_digits(1, g, u0, u1);
      }
    } else {
      if constexpr (NS > 2) cp.copy(slots[1], junk, rk0, rv0, blk0 + NG, w);
    }
    if constexpr (NS > 3) cp.copy(slots[2], junk, rk0, rv0, blk0 + 2 * NG, w);
    // the first step's blocks have landed (this wave's copies; the barrier covers the others')
    wait_vm<(NS - 2) * F::perWave>();
    lds_barrier();
    v8i Aq, Asq;
    int scq = 127, scsq = 127;
    long A8[4] = {0, 0, 0, 0};   // q8 keys: row t = (head t / 4, digit t % 4) over coordinates 32cb + 8g4 ..
    float qsc8 = 0.0f;           // q8 keys: 2^e log2(e) / sqrt d for this lane's head g4
    if constexpr (KQ8) {
      const int hh = t >> 2, dd = t & 3;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) A8[cb] = (dd < 3) ? *reinterpret_cast<const long*>(&qdig[hh][dd][32 * cb + 8 * g4]) : 0;
      qsc8 = __builtin_amdgcn_ldexpf(kLog2e * inv_sqrt_d, qexp8[g4] - 7);   // (the digit sums come in units of 2^-7)
    } else {
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
#pragma unroll
    for (int T = 0; T < NTK; ++T) aksum += ak[T];
    // offsets of the affine key operand for this lane's head g4: every term
    // carries the same per-head constant, the code sum carries it times sum a_T
    const float cq = KQ8 ? 0.0f : cconst[0][g4] * aksum;
    const float csq = QJL ? cconst[1][g4] : 0.0f;
    const float alpha2 = kLog2e * inv_sqrt_d / static_cast<float>(kD);
    const float beta2 = kLog2e * inv_sqrt_d * 1.2533141373155003f / static_cast<float>(kM);
    const int so = 4 * (g4 * kBlock + 32 * wl + 2 * t);   // this lane's key words in a block
    const int sn = 2 * (32 * wl + 2 * t);                 // its two fp16 per-position fields
    // the loop's copies: blocks past the split's sequence read zero
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(a.kc + slot0_idx * a.k_block_bytes, a.k_block_bytes, blk1);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(a.vc + slot0_idx * a.v_block_bytes, a.v_block_bytes, blk1);

    // --------------------------------------------------------- main loop
    // Step i processes blocks blk0 + 2i (group 0) and blk0 + 2i + 1 (group 1)
    // from ring slot i % NS, with one barrier, between the probability digits
    // and the weighted sum.  After it (every wave has then finished step
    // i - 1) the step refills slot (i - 1) % NS with the blocks of step
    // i + NS - 1; before it each wave waits for its copies of the blocks of step
    // i + 1 (issued in step i - 1), which the next step reads right after this
    // one's weighted sum.  With two slots the blocks of step i + 1 is only
    // issued in step i, and a second barrier ends the step.
    // Part A of step i: logits of the group's key block, this wave's
    // reference, the probability digits.  Carried to part B: the reference and
    // the sum of this lane's two probabilities.
    auto partA = [&](const uint8_t* cur, int i, float& rw_out, float& ps_out) __attribute__((always_inline)) {
      const int blk = blk0 + NG * i + gr;
      const int n_t = (blk < blk1) ? min(kBlock, len - blk * kBlock) : 0;
      const uint8_t* kb = cur + gr * F::kBytes;
      const uint8_t* vb = cur + F::kChunks * 1024 + gr * F::vBytes;

      // logits of k-slots 32wl + 2t + c for head g4: every MFMA of the block
      // is issued before any result is read
      float lg2[2];
      if constexpr (KQ8) {
        // q8: per 32-coordinate block cb, exact int32 sums of q digits times
        // k8, combined as (D0 2^7 + D1) + D2 2^-7 (the first two in integer
        // arithmetic: |D0|, |D1| <= 64 * 127 * 32 < 2^18, so the int32 is exact
        // and its conversion rounds below 2^-24 of it) and scaled by the
        // block's s16
        v4i dI[2][4];
        uint2 sc[2];
        int tok2[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          tok2[c] = pos_of_slot(32 * wl + 2 * t + c);
          const uint8_t* row = kb + tok2[c] * kD;
          sc[c] = *reinterpret_cast<const uint2*>(kb + kBlock * kD + tok2[c] * 8);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const int gran = (2 * cb + (g4 >> 1)) ^ q8_swizzle(tok2[c]);
            dI[c][cb] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                A8[cb], *reinterpret_cast<const long*>(row + 16 * gran + 8 * (g4 & 1)), v4i{0, 0, 0, 0}, 0, 0, 0);
          }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float code = 0.0f;
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const int d01 = dI[c][cb][0] * 128 + dI[c][cb][1];
            const float v = fmaf(static_cast<float>(dI[c][cb][2]), 0.0078125f, static_cast<float>(d01));
            const uint32_t sw = (cb < 2) ? sc[c].x : sc[c].y;
            code = fmaf(h2f((cb & 1) ? (sw >> 16) : sw), v, code);
          }
          const int tok = tok2[c];
          const float l2 = __fmul_rn(qsc8, code);
          const bool valid = (tok < n_t) && (g4 < G);
          // (no logits: an empty buffer, every store dropped; -1: past its end)
          const int lo = valid ? (g4 * a.max_ctx + blk * kBlock + tok) * 4 : -1;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(__fmul_rn(l2, kLn2)), rlg, lo, 0, 0);
          lg2[c] = valid ? l2 : -INFINITY;
        }
      } else {
      uint2 kp[KB];
#pragma unroll
      for (int p = 0; p < KB; ++p) kp[p] = *reinterpret_cast<const uint2*>(kb + p * 2048 + so);
      const uint2 ks = QJL ? *reinterpret_cast<const uint2*>(kb + 2048 * KB + so) : make_uint2(0u, 0u);
      const uint32_t kn = *reinterpret_cast<const uint32_t*>(kb + F::kNorms + sn);
      const uint32_t kr = QJL ? *reinterpret_cast<const uint32_t*>(kb + F::kNorms + 256 + sn) : 0u;
      v4f dT[2][NTK];
      v4f dQ[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint32_t wd[KB];
#pragma unroll
        for (int p = 0; p < KB; ++p) wd[p] = c ? kp[p].y : kp[p].x;
#pragma unroll
        for (int T = 0; T < NTK; ++T)
          dT[c][T] = mfma_fp8_fp4(Aq, expand_fp4_affine(term_word<KB>(wd, T), kf), v4f{0.0f, 0.0f, 0.0f, 0.0f}, scq);
        if (QJL) dQ[c] = mfma_fp8_fp4(Asq, expand_fp4_affine(c ? ks.y : ks.x, kf), v4f{0.0f, 0.0f, 0.0f, 0.0f}, scsq);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float code = -cq;
#pragma unroll
        for (int T = 0; T < NTK; ++T)
          code = fmaf(ak[T], (dT[c][T][0] + dT[c][T][1]) + (dT[c][T][2] + dT[c][T][3]), code);
        const float qj = QJL ? ((dQ[c][0] + dQ[c][1]) + (dQ[c][2] + dQ[c][3])) - csq : 0.0f;
        const int tok = pos_of_slot(32 * wl + 2 * t + c);
        const float nk = h2f(c ? (kn >> 16) : kn);
        const float rho = QJL ? h2f(c ? (kr >> 16) : kr) : 0.0f;
        // explicit roundings: every unrolled copy of the step computes the same bits
        const float l2 = fmaf(__fmul_rn(alpha2, nk), code, QJL ? __fmul_rn(__fmul_rn(beta2, rho), qj) : 0.0f);
        const bool valid = (tok < n_t) && (g4 < G);
        const int lo = valid ? (g4 * a.max_ctx + blk * kBlock + tok) * 4 : -1;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(__fmul_rn(l2, kLn2)), rlg, lo, 0, 0);
        lg2[c] = valid ? l2 : -INFINITY;
      }
      }

      // This wave's reference per head (row g4): the integer ceiling of its
      // step maximum, log2 units.  p <= 1 is formed against it without waiting
      // for the other waves; after the barrier every wave brings the eight
      // references to the common running one through exact powers of two (the
      // E8M0 scales of the probability digits and the denominators).  The
      // running reference only moves when a step exceeds it by 2^8.
      const int par = i & 1;   // the digit buffers alternate: one barrier per step
      uint8_t* const pl = (par ? plimb1 : plimb0) + gr * (16 * 128);
      uint8_t* const pe = (par ? pexp1 : pexp0) + gr * 64;
      const float mloc = row_max16(fmaxf(lg2[0], lg2[1]));
      const float rw = (mloc == -INFINITY) ? -INFINITY : ceilf(mloc);
      if (t == 0) rwb[par][w][g4] = rw;

      // probabilities and base-32 digits of p * value radius (3 digits, ~14 bits)
      const uint32_t vn = *reinterpret_cast<const uint32_t*>(vb + 2048 * VB + sn);
      const float p0 = (lg2[0] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(lg2[0] - rw);
      const float p1 = (lg2[1] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(lg2[1] - rw);
      float r0 = (p0 > 0.0f) ? p0 * h2f(vn) : 0.0f;
      float r1 = (p1 > 0.0f) ? p1 * h2f(vn >> 16) : 0.0f;
      const float pm = row_max16(fmaxf(r0, r1));
      const int s0 = (pm >= 1e-30f) ? exponent_of(pm) - 3 : 0;   // r 2^-s0 < 16
      // (the value operand's sign field takes the complemented bit: no sign flip here)
      r0 = __builtin_amdgcn_ldexpf(r0, -s0);
      r1 = __builtin_amdgcn_ldexpf(r1, -s0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int pk = 0;   // the fourth digit row stays zero
        if (j < 3) {
          const float d0 = rintf(r0), d1 = rintf(r1);   // integers in [-16, 16]: exact in e4m3
          pk = __builtin_amdgcn_cvt_pk_fp8_f32(d0, d1, 0, false);
          if (j < 2) {
            r0 = (r0 - d0) * 32.0f;
            r1 = (r1 - d1) * 32.0f;
          }
        }
        *reinterpret_cast<uint16_t*>(&pl[(4 * g4 + j) * 128 + 32 * wl + 2 * t]) = static_cast<uint16_t>(pk & 0xffff);
      }
      // bytes s0 + 127, s0 + 122, s0 + 117, 127: s0 lies in [-102, 125] (pm is
      // 0, a normal float of at least 1e-30 or at most +inf), so every byte
      // lies in [15, 252] and none carries into the next
      const uint32_t ebytes = static_cast<uint32_t>(s0 * 0x010101 + (0x7f000000 + 127 + (122 << 8) + (117 << 16)));
      if (t == 0) *reinterpret_cast<uint32_t*>(&pe[16 * wl + 4 * g4]) = ebytes;
      rw_out = rw;
      ps_out = p0 + p1;
    };

    // Part B of step i (after the barrier that follows every wave's part A):
    // the common running references, then the weighted sum of the group's
    // value block.
    auto partB = [&](const uint8_t* cur, int i, float rw, float ps) __attribute__((always_inline)) {
      const uint8_t* vb = cur + F::kChunks * 1024 + gr * F::vBytes;
      const int par = i & 1;
      const uint8_t* const pl = (par ? plimb1 : plimb0) + gr * (16 * 128);
      const uint8_t* const pe = (par ? pexp1 : pexp0) + gr * 64;
      // running references of head g4 (denominator) and head t / 4 (result column)
      const int hb = t >> 2;
      float rb = rwb[par][0][hb];
#pragma unroll
      for (int u = 1; u < kWaves; ++u) rb = fmaxf(rb, rwb[par][u][hb]);
      const float mn_b = (rb > m_b + 8.0f) ? rb : m_b;
      const float fv = (m_b == -INFINITY) ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, static_cast<int>(m_b - mn_b));
      // head g4's: every lane whose t / 4 is g4 holds them (the same recurrence
      // over the same wave references), lane 4 g4 among them
      const float mn_a = __int_as_float(__builtin_amdgcn_ds_bpermute(16 * g4, __float_as_int(mn_b)));
      const float fh = __int_as_float(__builtin_amdgcn_ds_bpermute(16 * g4, __float_as_int(fv)));
      lsum = lsum * fh + ((rw == -INFINITY) ? 0.0f : __builtin_amdgcn_ldexpf(ps, static_cast<int>(rw - mn_a)));
      m_a = mn_a;
      m_b = mn_b;

      // weighted sum of value terms for coordinates 32wl + 16r + (row), columns (head, limb)
      if (__any(fv != 1.0f)) {   // rescale only when some head's reference moved
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
          for (int T = 0; T < NTV; ++T) accV[rr][T] *= fv;
        accO *= fv;
      }
      // Sparse-V: a group block whose four wave references lie more than
      // tau_v below the running maximum for every head it serves holds only
      // weights below 2^-tau_v of the largest one (both sides are integer
      // ceilings); its value work is skipped, its weights stay in lsum
      if (sparse_v) {
        m_top = fmaxf(m_top, rb);
        float rblk = rwb[par][4 * gr][hb];
#pragma unroll
        for (int u = 1; u < 4; ++u) rblk = fmaxf(rblk, rwb[par][4 * gr + u][hb]);
        if (__all((rblk == -INFINITY) || (rblk < m_top - tau_v))) return;
      }
      v8i Pv;
      {
        const uint4 lo = *reinterpret_cast<const uint4*>(&pl[t * 128 + 16 * g4]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&pl[t * 128 + 64 + 16 * g4]);
        Pv = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      // k-block g4 holds the positions of wave g4 of this group: its digits
      // carry 2^(its reference - the running one)
      const float rk = rwb[par][4 * gr + g4][hb];
      const int adj = (rk == -INFINITY) ? 0 : static_cast<int>(rk - m_b);
      const int scp = min(max(static_cast<int>(pe[16 * g4 + t]) + adj, 1), 254);
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        uint32_t vw[VB];
#pragma unroll
        for (int p = 0; p < VB; ++p)
          vw[p] = *reinterpret_cast<const uint32_t*>(vb + 4 * (p * 4 * kD + g4 * kD + 32 * wl + 16 * rr + t));
#pragma unroll
        for (int T = 0; T < NTV; ++T)
          accV[rr][T] = mfma_fp4_fp8(expand_fp4_affine_v(term_word<VB>(vw, T), kf), Pv, accV[rr][T], scp);
      }
      accO = mfma_fp4_fp8(aoff, Pv, accO, scp);
    };

    // The barrier between part A of step i and part B: with three or more
    // slots the blocks of step i + 1 were issued a step ago, and this wave's
    // copies of them must have landed (everyone's, after the barrier).  Every
    // wave is then past part B of step i - 1: refill that slot with the
    // blocks of step i + NS - 1.
    auto sync = [&](uint8_t* refill, int i) __attribute__((always_inline)) {
      if constexpr (NS >= 3) wait_vm<(NS - 3) * F::perWave>();
      lds_barrier();
      cp.copy(refill, junk, rk, rv, blk0 + NG * (i + NS - 1), w);
    };
    // step i: A(i), barrier and refill, B(i); with two slots a second barrier
    // after waiting for the blocks of step i + 1
    auto step = [&](uint8_t* cur, uint8_t* refill, int i) __attribute__((always_inline)) {
      float rw, ps;
      partA(cur, i, rw, ps);
      sync(refill, i);
      partB(cur, i, rw, ps);
      if constexpr (NS == 2) {
        wait_vm<0>();
        lds_barrier();
      }
    };
    // whole rounds of the ring, then the last partial round; slot indices are
    // compile-time constants in every step
    if (n_iter > 0) {   // uniform over the workgroup
    int i0 = 0;
    for (; i0 + NS <= n_iter; i0 += NS) {
#pragma unroll
      for (int r = 0; r < NS; ++r) step(slots[r], slots[(r + NS - 1) % NS], i0 + r);
    }
    const int rem = n_iter - i0;   // 0 .. NS - 1, uniform
    if (rem > 0) {
      step(slots[0], slots[NS - 1], i0);
      if (rem > 1) {
        step(slots[1], slots[0], i0 + 1);
        if constexpr (NS > 3) {
          if (rem > 2) step(slots[2], slots[1], i0 + 2);
        }
      }
    }
    }   // n_iter > 0
  }

  // ------------------------------------------------------------- partials
  // denominator per (wave, head); running max per head; the two groups'
  // weighted sums per coordinate (in the sketch buffer, free by now)
  float (*obuf)[4][kD] = reinterpret_cast<float (*)[4][kD]>(&sred[0][0]);
  // the inverse rotation's signs, loaded before the exchange below so that
  // their latency overlaps it
  const float dva = a.tb.dv[lane], dvb = a.tb.dv[lane + 64];
  {
    const float ls = row_sum16(lsum);
    if (t == 0) wred[w][g4] = ls;
    if (w == 0 && t == 0) mrun[g4] = m_a;
    const int hc = t >> 2;   // head of this lane's result column
    // every term of column t carries the same offset, the code sum carries it
    // times sum a_T
    float avsum = 0.0f;
#pragma unroll
    for (int T = 0; T < NTV; ++T) avsum += av[T];
    const float voff = avsum * 0.5f * (accO[0] + __shfl_xor(accO[0], 32, 64));
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = -voff;
#pragma unroll
        for (int T = 0; T < NTV; ++T) s = fmaf(av[T], accV[r][T][i], s);
        s += __shfl_xor(s, 1, 64);   // sum the 4 limb columns of head hc
        s += __shfl_xor(s, 2, 64);
        v[i] = s;
      }
      if (hc < G && (t & 3) == 0)
        *reinterpret_cast<float4*>(&obuf[gr][hc][32 * wl + 16 * r + 4 * g4]) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
  __syncthreads();
  if (w < G) {
    // wave w: head w, o = D_V H (sum of both groups) / d
    float lo = obuf[0][w][lane], hi = obuf[0][w][lane + 64];
    if constexpr (NG == 2) {
      lo += obuf[1][w][lane];
      hi += obuf[1][w][lane + 64];
    }
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

template <int KB, bool QJL, int VB, int NG>
__global__ __launch_bounds__(256 * NG, 2) void decode_mfma_kernel(DecodeArgs a) {
  decode_mfma_body<KB, QJL, VB, NG, false>(a);
}

// the serving step: the same decode, after the new position is stored
template <int KB, bool QJL, int VB, int NG>
__global__ __launch_bounds__(256 * NG, 2) void decode_append_kernel(DecodeArgs a) {
  decode_mfma_body<KB, QJL, VB, NG, true>(a);
}

template <int KB, bool QJL, int VB, int NG>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  const int n_units = a.n_splits * a.n_kv * a.batch;
  dim3 grid(((n_units + 7) / 8) * 8 * ((a.group + 3) / 4));
  if (a.k_new != nullptr)
    hipLaunchKernelGGL((decode_append_kernel<KB, QJL, VB, NG>), grid, dim3(256 * NG), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<KB, QJL, VB, NG>), grid, dim3(256 * NG), 0, stream, a);
  return hipGetLastError();
}

// block groups per workgroup as the host chose them: one for q8 keys, one or
// two for four-bit values, two otherwise
template <int KB, bool QJL, int VB>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (KB == 8) {
    return a.groups == 1 ? launch_g<KB, QJL, VB, 1>(a, stream) : hipErrorInvalidValue;
  } else if constexpr (VB == 4) {
    if (a.groups == 1) return launch_g<KB, QJL, VB, 1>(a, stream);
    return a.groups == 2 ? launch_g<KB, QJL, VB, 2>(a, stream) : hipErrorInvalidValue;
  } else {
    return a.groups == 2 ? launch_g<KB, QJL, VB, 2>(a, stream) : hipErrorInvalidValue;
  }
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

bool decode_mfma_applies(int k_codec, int v_codec, int group) {
  return v_codec == POLAR && group <= kMaxGroup && (k_codec == POLAR || k_codec == POLAR_QJL || k_codec == Q8_BLOCK32);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  if (!decode_mfma_applies(a.k_codec, a.v_codec, a.group)) return hipErrorNotSupported;
  // block byte offsets (up to n_blocks + 2 kRing blocks) are 32-bit buffer offsets
  const int64_t span = (static_cast<int64_t>(a.n_blocks) + 2 * kRing + 4) * std::max(a.k_block_bytes, a.v_block_bytes);
  if (span >= (int64_t{1} << 31) || static_cast<int64_t>(a.n_splits) * kPartialStride * 4 >= (int64_t{1} << 31))
    return hipErrorNotSupported;
  // the logits of four heads of one sequence are addressed with 32-bit offsets
  if (a.logits != nullptr && int64_t{16} * a.max_ctx >= (int64_t{1} << 31)) return hipErrorNotSupported;
  if (a.k_codec == Q8_BLOCK32) return launch_v<8, false>(a, stream);
  if (a.k_codec == POLAR_QJL) {
    switch (a.k_bits) {
      case 2: return launch_v<2, true>(a, stream);
      case 3: return launch_v<3, true>(a, stream);
      case 4: return launch_v<4, true>(a, stream);
    }
  } else {
    switch (a.k_bits) {
      case 2: return launch_v<2, false>(a, stream);
      case 3: return launch_v<3, false>(a, stream);
      case 4: return launch_v<4, false>(a, stream);
    }
  }
  return hipErrorNotSupported;
}

}  // namespace tq
