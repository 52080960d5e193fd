// tq_decode_reg.hip -- decode attention on the gfx950 matrix cores with the
// packed cache streamed straight into registers, for POLAR or POLAR_QJL keys
// and POLAR values, up to 16 query heads per KV head (groups of four).
//
// The arithmetic is the matrix-core form of the estimator, softmax and
// rotated-frame weighted sum (wis-web.com reader, TurboQuant article, the
// PolarQuant and QJL paragraphs; see tq_decode_mfma.hip for the operand
// algebra): code planes become fp4 operands with one and-or per dword; the
// query enters as exact base-16 digits in fp6 (so that its products with the
// fp4 codes run at the matrix cores' 4-pass rate), p * radius as exact
// base-32 fp8 digits, both with E8M0 scales.
// What differs is the data flow:
//
//  * No cache byte is read twice and none is staged: lane (t, g4) of wave w
//    needs exactly the key words of k-block g4 at slots 32w + 2t, 32w + 2t + 1
//    (one 8-byte load per plane) and the value words of k-block g4 for
//    coordinates 32w + 2t, 32w + 2t + 1 (row t of the value product stands
//    for coordinate 32w + 2t + rr in its pass rr, so that those two words are
//    one 8-byte load too).  A block's key and value loads are issued about
//    three steps before the step that uses them, into one of three register
//    sets (two with 4-bit values).
//  * Each workgroup forms its query operands (rotation, sketch, digits) in
//    shared memory while its first blocks' loads are in flight, then keeps
//    them in registers through the loop: no separate launch for them.
//  * With at most four terms per key code (2- and 3-bit keys, values of 2 or
//    3 bits) the codebook coefficients are folded into the query digits (one
//    operand per term), so a column's terms accumulate in one matrix
//    instruction chain instead of being summed and weighted afterwards.
//  * A workgroup is one group of four waves taking one 128-position block per
//    step with one barrier per step, software-pipelined over two blocks: step
//    i forms the logits of block i and, around the barrier, the probability
//    digits, running references and weighted values of block i - 1.  Two
//    workgroups share a compute unit, so their steps interleave.
//  * Sparse-V (the wis-web.com article's third finding): the variant that
//    votes on blocks requests a block's value words only after its vote, so
//    the value bytes of a skipped block stay in HBM.

#include <algorithm>
#include <type_traits>

#include "tq_mfma_ops.h"

namespace tq {
namespace {

constexpr int kRegThreads = 256;
// A running or step reference with no valid position behind it: finite, so
// that differences and exponentials of it need no special case (it converts
// to a huge negative shift, 2^shift = 0).
constexpr float kNoRef = -1e30f;

// a * b for a >= 0 and b an fp16 radius, 0 for a = 0 whatever b (the cache
// words of slots past the length are arbitrary): 0 x inf and 0 x NaN give a
// quiet NaN, which the maximum with 0 drops (IEEE maxNum, the kernel's IEEE
// mode); negative garbage gives 0 as well.  Written as an fma with a zero
// addend (the same rounding as the product) so that one mixed-precision
// instruction takes the fp16 radius as it is.
__device__ __forceinline__ float mul_zero_wins(float a, float b) { return __builtin_fmaxf(fmaf(a, b, 0.0f), 0.0f); }
// float -> int of a shift that is at most a few units above zero, clamped
// below (an absent reference gives a large negative value)
__device__ __forceinline__ int shift_of(float x) { return static_cast<int>(fmaxf(x, -1073741824.0f)); }

// CHAIN: one query operand per code term (at most four terms); with 4-bit
// values the decode keeps one operand and weights the terms itself (the four
// operands would not fit in its registers).
template <int KB, int VB>
struct KeyOps {
  static constexpr int nt = NTerms<KB>::n;
  static constexpr bool chain = nt <= 4 && VB < 4;
  static constexpr int code_sets = chain ? nt : 1;
};

// ------------------------------------------------------------ query side
// The logit's constant factors travel in the query digits: log2(e) / sqrt d
// (softmax in base 2, scale 1/sqrt d) times 1/d for the code term (the raw
// FWHT's d) and sqrt(pi/2)/m for the sketch term (the estimator's constant);
// a logit is then n16 * code + rho16 * sketch.
constexpr float kCodeScale = 1.4426950408889634f * 0.08838834764831845f / 128.0f;
constexpr float kSketchScale = 1.4426950408889634f * 0.08838834764831845f * 1.2533141373155003f / 128.0f;
// Query operand rows in shared memory: 128 k-slots of fp6 (e2m3) digits,
// packed 6 bits per k-slot from bit 0 (96 bytes), padded to 104 bytes so
// that the 16 rows one 8-byte read instruction gathers fall on distinct banks.
// Lane (t, g4) of a product reads row t, k-slots 32 g4 .. 32 g4 + 31: the
// fp6 operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 (contiguous 32
// k-slots per group of 16 lanes, one E8M0 scale each).
constexpr int kARow = 104;

// Query digits of one (operand set, head) job, formed by a half-wave: lane l
// (0 .. 31) holds the values x (already divided by the job's coefficient
// coef) of k-slots 4 l .. 4 l + 3, which occupy 3 whole bytes of each operand
// row.  Digit j of value v = coef x is an integer n_j in [-8, 8] standing for
// n_j / 8 (exact in fp6 e2m3 as sign and magnitude: code |n_j|, sign in bit
// 5), with v = 2^s0 sum_j (n_j / 8) 16^-j; s0 is taken per 32 k-slots so that
// their largest |v| 2^-s0 lies in [0.5, 1), and each remainder again lies in
// [-1, 1].  Writes operand rows 4 g + j of `op` (kARow bytes each; each quad
// of lanes gathers its 12 bytes and stores them as 3 aligned words), their
// E8M0 bytes 2^(s0 - 4 j) into `ex` ([k / 32][row]) and, into cc[g], the
// operand's affine offset for head g (the sum of the digit-exact values
// times the fixed nibble-field offsets 5, 3, 1, 0 of the key operand).  The
// k-slots that meet the sign field of the affine key operand carry the value
// with its sign flipped (k-slot k stands for coordinate or sketch row
// pos_of_slot(k)).
struct DigitLane {
  uint32_t psel;   // byte selector of this lane's word (own 3 bytes, then the next lane's)
  int pofs;        // byte offset of that word inside a row
  int l;           // lane within the half-wave
};
__device__ __forceinline__ DigitLane digit_lane(int lane) {
  const int l = lane & 31, i = min(l & 3, 2);
  return DigitLane{(i == 0) ? 0x04020100u : (i == 1) ? 0x05040201u : 0x06050402u, 12 * (l >> 2) + 4 * i, l};
}
__device__ __forceinline__ void write_digits(uint8_t* op, uint8_t* ex, float* cc, int g, float4 x, float coef,
                                             const DigitLane& dl) {
  const int l = dl.l;
  const int fld = (l & 7) >> 1;
  float m = fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x141, 0xF, 0xF, false)));
  m *= fabsf(coef);   // the largest |v| of these 32 k-slots
  const int s0 = (m >= 1e-30f) ? exponent_of(m) + 1 : 0;
  float sc = __builtin_amdgcn_ldexpf(coef, 3 - s0);   // v 2^(3 - s0) = 8 v 2^-s0, in [-8, 8]
  if (fld == 3) sc = -sc;
  float r[4] = {x.x * sc, x.y * sc, x.z * sc, x.w * sc};
  const float r0[4] = {r[0], r[1], r[2], r[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t v = 0;   // fp6 codes of the 4 k-slots, k-slot 4 l + i at bits 6 i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float n = rintf(r[i]);
      r[i] = (r[i] - n) * 16.0f;   // exact
      const uint32_t c = static_cast<uint32_t>(fabsf(n)) | ((__float_as_uint(n) >> 26) & 0x20u);
      v |= c << (6 * i);
    }
    // lane i of a quad stores the word made of bytes 4 i' .. 4 i' + 3 of the
    // quad's 12 (i' = min(i, 2); lane 3 repeats lane 2's word)
    const uint32_t nxt = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xF9, 0xF, 0xF, false));
    const uint32_t slf = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xA4, 0xF, 0xF, false));
    *reinterpret_cast<uint32_t*>(&op[(4 * g + j) * kARow + dl.pofs]) = __builtin_amdgcn_perm(nxt, slf, dl.psel);
  }
  // the exponent of digit l & 3 of the 32 k-slots (lanes l and l + 4 store the same)
  ex[(l >> 3) * 16 + 4 * g + (l & 3)] = static_cast<uint8_t>(min(max(s0 - 4 * (l & 3) + 127, 1), 254));
  // digit-exact value of k-slot i in units of 2^(s0 - 3): r0 - r4 16^-4 (exact)
  float tv = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) tv += fmaf(r[i], -1.52587890625e-05f, r0[i]);
  const float wf = (fld == 0) ? 5.0f : (fld == 1) ? 3.0f : (fld == 2) ? 1.0f : 0.0f;
  float s = row_sum16(__builtin_amdgcn_ldexpf(wf * tv, s0 - 3));
  s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x142, 0xA, 0xF, false));   // rows 1, 3: + rows 0, 2
  if (l & 16) cc[g] = s;
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
  // with the value request after the vote: the probabilities of the two
  // slots of the block whose values the set holds, and whether they were
  // requested (its vote kept the block)
  float pp0, pp1;
  bool vreq;
};

template <int KB, bool QJL, int VB>
struct RegFmt {
  static constexpr int kNorms = 2048 * KB + (QJL ? 2048 : 0);
  static constexpr int kBytes = kNorms + 256 + (QJL ? 256 : 0);
  static constexpr int vBytes = 2048 * VB + 256;
  static constexpr int loads = KB + (QJL ? 3 : 1) + VB + 1;   // vector loads per step and wave
};

// AUX: the variant that also writes logits and skips the value work of
// blocks whose weights are negligible (Sparse-V; with 2- and 3-bit values it
// also never requests their value words); the plain variant has neither in
// its step.
// NG: block groups of four waves per workgroup.  With two, one workgroup of
// eight waves fills a compute unit: its groups take alternate blocks of the
// split (one block each per step, in lock step through the same barriers),
// share one query set-up and merge in shared memory before the split's
// partial leaves the workgroup (not with logits or Sparse-V).
template <int KB, bool QJL, int VB, bool FUSED, bool AUX, int NG>
__device__ __forceinline__ void decode_reg_body(const DecodeArgs& a) {
  static_assert(NG == 1 || (NG == 2 && !AUX), "two block groups: not with logits or Sparse-V");
  // three register sets, two with 4-bit values (three would not fit in 256)
  constexpr int kSets = (VB == 4) ? 2 : 3;
  // the logits / Sparse-V variant requests a block's values only after its
  // vote (three register sets needed)
  constexpr bool kLag = AUX && kSets == 3;
  using KO = KeyOps<KB, VB>;
  using F = RegFmt<KB, QJL, VB>;
  using R = StepRegs<KB, QJL, VB>;
  constexpr int NTK = KO::nt;
  constexpr int NCS = KO::code_sets;
  constexpr int NTV = NTerms<VB>::n;
  constexpr int kWaves = 4 * NG;
  // [parity][col][k]: digits of p * radius; rows padded to 144 bytes so that
  // the 16 rows one 16-byte read instruction gathers fall on distinct banks
  constexpr int kPRow = 144;
  // digit buffers: block j's digits go to buffer j mod kSets (the index of the
  // register set that holds its values), so every address in the unrolled
  // step is a constant offset; the voting variant uses j mod 2
  __shared__ __attribute__((aligned(16))) uint8_t plimb[NG][kSets][16 * kPRow];
  __shared__ __attribute__((aligned(4))) uint8_t pexp[NG][kSets][4][16];        // [group][buffer][k / 32][col]
  __shared__ float rwb[4][kWaves][4];       // [block mod kSets (voting: mod 4)][wave][head]: each wave's step reference
  __shared__ float wred[kWaves][4];
  __shared__ float mrun[NG][4];
  __shared__ __attribute__((aligned(16))) float obuf[NG][4][kD];
  __shared__ __attribute__((aligned(16))) float r_lds[kD];   // the serving step's key residual
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gr = w >> 2;   // block group
  const int wl = w & 3;    // wave within the group
  const int t = lane & 15;
  const int g4 = lane >> 4;
  // Workgroup -> (split, KV head, sequence, head group); the head groups of
  // one (split, KV head, sequence) get ids 8 apart (one XCD, one L2).  Units
  // are split-major, so the workgroups dispatched first are the low splits,
  // which the host may make longer (the first workgroup of a compute unit
  // runs ahead of the second).
  const int nhg = (a.group + 3) >> 2;
  const int pairs = a.n_kv * a.batch;
  const int n_units = a.n_splits * pairs;
  const int id = blockIdx.x;
  const int kx = id >> 3;
  const int unit = (kx / nhg) * 8 + (id & 7);
  if (unit >= n_units) return;
  const int hg = kx - (kx / nhg) * nhg;
  const int split = unit / pairs;
  const int pair = unit - split * pairs;
  const int h = pair % a.n_kv;
  const int b = pair / a.n_kv;
  const int G = min(4, a.group - 4 * hg);
  const int hq0 = h * a.group + 4 * hg;
  uint32_t* const counter = a.counters + (static_cast<int64_t>(b) * a.n_kv + h) * nhg + hg;
  typedef __attribute__((address_space(4))) const int cint;
  typedef __attribute__((address_space(4))) const float cfloat;
  const int len_in = min(*((cint*)(a.seq_lens) + b), a.max_ctx);
  if constexpr (FUSED) {
    if (len_in < a.max_ctx && split_of_block(a, len_in / kBlock) == split)
      fused_append<KB, QJL, VB>(a, b, h, len_in, w, lane, r_lds);
  }

  float ak[NTK], av[NTV];
#pragma unroll
  for (int T = 0; T < NTK; ++T) ak[T] = ((cfloat*)(a.tb.ak))[T];   // scalar loads
#pragma unroll
  for (int T = 0; T < NTV; ++T) av[T] = ((cfloat*)(a.tb.av))[T];

  // the query side's loads go first: waits for them then leave the cache
  // loads below in flight (vector memory counts complete in issue order)
  // (the rotation's operands first: its wait then leaves the table in flight)
  const float* qp = a.q + (static_cast<int64_t>(b) * a.n_q + hq0 + min(w, G - 1)) * kD;
  const float pq0 = (w < G) ? qp[lane] : 0.0f, pq1 = (w < G) ? qp[lane + 64] : 0.0f;
  const float pdk0 = a.tb.dk[lane], pdk1 = a.tb.dk[lane + 64];
  // Two block groups with a sketch: waves 0..3 rotate and form the code
  // digits while waves 4..7 form the sketch (32 table coordinates each); one
  // group: every wave takes 32 coordinates of the sketch.
  constexpr bool kPar = NG == 2 && QJL;
  constexpr int kCpw = kPar ? 32 : kD / kWaves;   // sketch-table coordinates per sketch wave
  const int cw = kPar ? w - 4 : w;                // this wave's coordinate slice (< 0: none)
  float2 st2[QJL ? kCpw : 1];
  if constexpr (QJL) {
    if (cw >= 0) {
#pragma unroll
      for (int c = 0; c < kCpw; ++c) st2[c] = *reinterpret_cast<const float2*>(a.tb.shd + (kCpw * cw + c) * kM + 2 * lane);
    }
  }

  // ------------------------------------------------------------- streaming
  const int len = FUSED ? min(len_in + 1, a.max_ctx) : len_in;
  const int nblk_seq = (len + kBlock - 1) / kBlock;
  const int blk0 = split_first_block(a, split);
  const int blk1 = min(blk0 + split_block_count(a, split), nblk_seq);
  const int n_iter = max(0, (blk1 - blk0 + NG - 1) / NG);   // steps; group gr takes blocks blk0 + NG i + gr
  auto bk = [&](int i) __attribute__((always_inline)) { return blk0 + NG * i + gr; };
  const int64_t slot0_idx = (static_cast<int64_t>(b) * a.n_kv + h) * a.n_blocks;
  const uint8_t* kbase = a.kc + slot0_idx * a.k_block_bytes;
  const uint8_t* vbase = a.vc + slot0_idx * a.v_block_bytes;
  // the first kSets blocks are requested before the length is known: over the
  // whole cache of this (sequence, KV head); later ones only within the split
  const __amdgpu_buffer_rsrc_t rk0 = block_rsrc(kbase, F::kBytes, a.n_blocks);
  const __amdgpu_buffer_rsrc_t rv0 = block_rsrc(vbase, F::vBytes, a.n_blocks);
  const __amdgpu_buffer_rsrc_t rk = block_rsrc(kbase, F::kBytes, blk1);
  const __amdgpu_buffer_rsrc_t rv = block_rsrc(vbase, F::vBytes, blk1);
  const int so = 4 * (g4 * kBlock + 32 * wl + 2 * t);   // key words of this lane (and value words)
  const int sn = 2 * (32 * wl + 2 * t);                 // its two fp16 per-slot fields
  constexpr int kNT = 2;   // streaming loads (read once)
  // The block index is clamped to the resource's last block (blocks past the
  // split re-read that block, unused), so every address lies inside the
  // (sequence, KV head)'s cache; the block's base travels in the scalar
  // offset and each lane's offset inside the block is a constant register.
  auto load_k = [&](R& B, int blk, int nvalid, __amdgpu_buffer_rsrc_t rsk) __attribute__((always_inline)) {
    const int kb0 = __builtin_amdgcn_readfirstlane(min(blk, nvalid - 1)) * F::kBytes;
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
  };
  auto load_v = [&](R& B, int blk, int nvalid, __amdgpu_buffer_rsrc_t rsv) __attribute__((always_inline)) {
    const int vb0 = __builtin_amdgcn_readfirstlane(min(blk, nvalid - 1)) * F::vBytes;
#pragma unroll
    for (int p = 0; p < VB; ++p) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b64(rsv, so, vb0 + p * 2048, kNT);
      B.vp[p] = make_uint2(x[0], x[1]);
    }
    B.vn = __builtin_amdgcn_raw_buffer_load_b32(rsv, sn, vb0 + 2048 * VB, kNT);
  };
  // Register set s holds the key words of block j and the value words of
  // block j' with j = j' = s (mod kSets): the keys of block i and the values
  // of block i - 1 are used in step i, then refilled with blocks i + kSets and
  // i - 1 + kSets.
  R buf0, buf1, buf2;
  load_k(buf0, bk(0), a.n_blocks, rk0);
  if constexpr (!kLag) load_v(buf0, bk(0), a.n_blocks, rv0);
  load_k(buf1, bk(1), a.n_blocks, rk0);
  if constexpr (!kLag) load_v(buf1, bk(1), a.n_blocks, rv0);
  if constexpr (kSets == 3) {
    load_k(buf2, bk(2), a.n_blocks, rk0);
    if constexpr (!kLag) load_v(buf2, bk(2), a.n_blocks, rv0);
  }
  __builtin_amdgcn_sched_barrier(0);   // (issued before the query-side work below)

  // ------------------------------------------------ query operands
  // Formed here while the first blocks' loads are in flight, in shared
  // memory, then read once into registers (6 words per set).  Wave w rotates
  // head w's query (q_raw = H D_K q) and takes a 32-coordinate slice of the
  // sketch table for its share of (S H D_K / sqrt d) q for the four heads;
  // then each half of wave w forms head w's digits for one operand set at a
  // time: the code sets two at a time (with the codebook coefficient folded
  // in when chained), then the sketch set.  Both vectors are kept in k-slot
  // order.
  constexpr int NQS = NCS + (QJL ? 1 : 0);
  __shared__ __attribute__((aligned(16))) uint8_t alimb[NQS][16 * kARow];   // [set][row = 4 g + j][k]
  __shared__ __attribute__((aligned(4))) uint8_t aexp[NQS][4 * 16];        // [set][k / 32][row]
  __shared__ float cconst[NQS][4];
  __shared__ __attribute__((aligned(16))) float qr[4][kD];                  // rotated query per head, by k-slot
  __shared__ __attribute__((aligned(16))) float qs[QJL ? 4 : 1][kD];       // the query per head
  __shared__ __attribute__((aligned(16))) float sred[QJL ? kWaves : 1][4][kM];   // partial sketch sums, by k-slot
  {
    // the fourth digit row of every digit buffer holds zeros throughout
    for (int o = tid; o < NG * kSets * 4 * (kPRow / 4); o += 64 * kWaves) {
      const int pb = o / (4 * (kPRow / 4)), rg = (o / (kPRow / 4)) % 4, dw = o % (kPRow / 4);
      reinterpret_cast<uint32_t*>(&plimb[pb / kSets][pb % kSets][(4 * rg + 3) * kPRow])[dw] = 0u;
    }
    const DigitLane dl = digit_lane(lane);
    const int half = lane >> 5;
    // the code sets' digits of head hw from its rotated query xr, set pairs
    // s2 = 2 p0, 2 p0 + 2, ... below 2 p1 (two sets at a time, one per half)
    auto code_digits = [&](int hw, const float4& xr, int p0, int p1) __attribute__((always_inline)) {
#pragma unroll
      for (int s2 = 0; s2 < NCS; s2 += 2) {
        if ((s2 >> 1) < p0 || (s2 >> 1) >= p1) continue;
        const int s = min(s2 + half, NCS - 1);   // (an odd last set is formed by both halves)
        const float coef = (KO::chain ? ((s == s2) ? ak[s2] : ak[min(s2 + 1, NCS - 1)]) : 1.0f) * kCodeScale;
        write_digits(&alimb[0][0] + s * (16 * kARow), &aexp[0][0] + s * 64, &cconst[0][0] + 4 * s, hw, xr, coef, dl);
      }
    };
    // this wave's share of (S H D_K / sqrt d) q for the four heads: table
    // coordinates kCpw cw .. kCpw cw + kCpw - 1, sketch rows 2 lane, 2 lane + 1
    auto sketch_share = [&]() __attribute__((always_inline)) {
      if constexpr (!QJL) return;
      else {
      float acc[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[g][0] = acc[g][1] = 0.0f;
#pragma unroll
      for (int c4 = 0; c4 < kCpw; c4 += 4) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 x = *reinterpret_cast<const float4*>(&qs[g][kCpw * cw + c4]);
          acc[g][0] = fmaf(st2[c4].x, x.x, acc[g][0]);
          acc[g][1] = fmaf(st2[c4].y, x.x, acc[g][1]);
          acc[g][0] = fmaf(st2[c4 + 1].x, x.y, acc[g][0]);
          acc[g][1] = fmaf(st2[c4 + 1].y, x.y, acc[g][1]);
          acc[g][0] = fmaf(st2[c4 + 2].x, x.z, acc[g][0]);
          acc[g][1] = fmaf(st2[c4 + 2].y, x.z, acc[g][1]);
          acc[g][0] = fmaf(st2[c4 + 3].x, x.w, acc[g][0]);
          acc[g][1] = fmaf(st2[c4 + 3].y, x.w, acc[g][1]);
        }
      }
      const int k0 = slot_of(2 * lane), k1 = slot_of(2 * lane + 1);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        sred[cw][g][k0] = acc[g][0];
        sred[cw][g][k1] = acc[g][1];
      }
      }
    };
    // head hd's sketch digits from the kD / kCpw shares
    auto sketch_digits = [&](int hd) __attribute__((always_inline)) {
      if constexpr (!QJL) return;
      else {
      float4 u = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int c = 0; c < kD / kCpw; ++c) {
        const float4 y = *reinterpret_cast<const float4*>(&sred[c][hd][4 * dl.l]);
        u.x += y.x;
        u.y += y.y;
        u.z += y.z;
        u.w += y.w;
      }
      write_digits(alimb[NCS], aexp[NCS], cconst[NCS], hd, u, kSketchScale, dl);   // (both halves: the same job)
      }
    };
    constexpr int kPairs = (NCS + 1) / 2;
    if constexpr (kPar) {
      // waves 0..3: head w's query into shared memory for the sketch waves;
      // after the barrier they rotate it and form the first code set pair
      // while waves 4..7 form the sketch shares; after the next barrier the
      // other code pairs and, on waves 4..7, the sketch digits
      if (w < 4) {
        qs[w][lane] = pq0;
        qs[w][lane + 64] = pq1;
      }
      lds_barrier();   // every head's query is in shared memory (the cache loads stay in flight)
      float4 xr = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (w < 4) {
        float lo = pq0 * pdk0, hi = pq1 * pdk1;
        wave_fwht128(lo, hi, lane);
        qr[w][slot_of(lane)] = lo;
        qr[w][slot_of(lane + 64)] = hi;
        // (this wave's own rotated query: no barrier)
        xr = *reinterpret_cast<const float4*>(&qr[w][4 * dl.l]);
        code_digits(w, xr, 0, 1);
      } else {
        sketch_share();
      }
      lds_barrier();   // the sketch shares are in shared memory
      if (w < 4) {
        code_digits(w, xr, 1, kPairs);
      } else {
        sketch_digits(w - 4);
      }
    } else {
      if (w < 4) {   // waves 0..3: head w
        float lo = pq0 * pdk0, hi = pq1 * pdk1;
        if constexpr (QJL) {
          qs[w][lane] = pq0;
          qs[w][lane + 64] = pq1;
        }
        wave_fwht128(lo, hi, lane);
        qr[w][slot_of(lane)] = lo;
        qr[w][slot_of(lane + 64)] = hi;
      }
      if constexpr (QJL) {
        lds_barrier();   // every head's query is in shared memory (the cache loads stay in flight)
        sketch_share();
      }
      if (w < 4) {
        // (head w's rotated query was written by this wave: no barrier)
        const float4 xr = *reinterpret_cast<const float4*>(&qr[w][4 * dl.l]);
        code_digits(w, xr, 0, kPairs);
      }
      if constexpr (QJL) {
        lds_barrier();   // every wave's sketch shares are in shared memory
        if (w < 4) sketch_digits(w);
      }
    }
  }
  lds_barrier();   // the operands are in shared memory (the cache loads above stay in flight)
  // the operands stay in registers through the loop (6 words per set)
  v8i qreg[NQS];
#pragma unroll
  for (int set = 0; set < NQS; ++set) {
    const uint2* rp = reinterpret_cast<const uint2*>(&alimb[set][t * kARow + 24 * g4]);
    const uint2 x = rp[0], y = rp[1], z = rp[2];
    qreg[set] = v8i{(int)x.x, (int)x.y, (int)y.x, (int)y.y, (int)z.x, (int)z.y, 0, 0};
  }
  auto qop = [&](int set) __attribute__((always_inline)) { return qreg[set]; };
  int scq[NCS];
#pragma unroll
  for (int s = 0; s < NCS; ++s) scq[s] = aexp[s][16 * g4 + t];
  const int scsq = QJL ? static_cast<int>(aexp[NQS - 1][16 * g4 + t]) : 127;
  float cq = 0.0f;
  if constexpr (KO::chain) {
#pragma unroll
    for (int s = 0; s < NCS; ++s) cq += cconst[s][g4];
  } else {
    float aksum = 0.0f;
#pragma unroll
    for (int T = 0; T < NTK; ++T) aksum += ak[T];
    cq = cconst[0][g4] * aksum;
  }
  const float csq = QJL ? cconst[NQS - 1][g4] : 0.0f;

  // The optional logits go through a buffer over this (sequence, head
  // group)'s rows: a lane with no logit to store takes an offset past its end
  // and the store is dropped (no branch in the step).
  const __amdgpu_buffer_rsrc_t rlg = __builtin_amdgcn_make_buffer_rsrc(
      a.logits != nullptr ? a.logits + (static_cast<int64_t>(b) * a.n_q + hq0) * a.max_ctx : a.logits,
      static_cast<short>(0), a.logits != nullptr ? G * a.max_ctx * 4 : 0, 0x00020000);

  float m_a = kNoRef, m_b = kNoRef;   // running reference of head g4 (denominator) / head t / 4 (column)
  const int ref_src = 16 * g4;         // byte address of lane 4 g4 (whose t / 4 is g4) for a lane permute
  float m_top = -INFINITY;                  // Sparse-V: largest step reference of head t / 4 so far
  const float tau_v = static_cast<float>(a.sparse_v);
  float lsum = 0.0f;
  v4f accV[2][NTV];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int T = 0; T < NTV; ++T) accV[r][T] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  v4f accO = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const Fp4Fill kf = fp4_fill();
  const v8i aoff = expand_fp4_affine_v(t < 8 ? 0xffffffffu : 0u, kf);
  float lgp[2] = {-INFINITY, -INFINITY};   // this lane's two logits of the block before

  // ---- the pieces of a step
  // (1a) key products of the block in Bk: column group c = slots 32 w + 2 t + c
  auto key_products = [&](R& Bk, float (&code2)[2], float (&qj2)[2]) __attribute__((always_inline)) {
    if constexpr (KO::chain && VB < 4) {   // both column groups' chains side by side
      uint32_t wd0[KB], wd1[KB];
#pragma unroll
      for (int p = 0; p < KB; ++p) {
        wd0[p] = Bk.kp[p].x;
        wd1[p] = Bk.kp[p].y;
      }
      v4f acc0 = v4f{-cq, 0.0f, 0.0f, 0.0f}, acc1 = acc0;   // the affine operands' offset, removed up front
#pragma unroll
      for (int T = 0; T < NTK; ++T) {
        const v8i A = qop(T);
        acc0 = mfma_fp6_fp4(A, expand_fp4_affine(term_word<KB>(wd0, T), kf), acc0, scq[T]);
        acc1 = mfma_fp6_fp4(A, expand_fp4_affine(term_word<KB>(wd1, T), kf), acc1, scq[T]);
      }
      code2[0] = (acc0[0] + acc0[1]) + (acc0[2] + acc0[3]);
      code2[1] = (acc1[0] + acc1[1]) + (acc1[2] + acc1[3]);
    } else {
      // one column group at a time (fewer live registers)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint32_t wd[KB];
#pragma unroll
        for (int p = 0; p < KB; ++p) wd[p] = c ? Bk.kp[p].y : Bk.kp[p].x;
        if constexpr (KO::chain) {
          v4f acc = v4f{-cq, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int T = 0; T < NTK; ++T) acc = mfma_fp6_fp4(qop(T), expand_fp4_affine(term_word<KB>(wd, T), kf), acc, scq[T]);
          code2[c] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        } else {
          v4f dT[NTK];
          const v8i A = qop(0);
#pragma unroll
          for (int T = 0; T < NTK; ++T)
            dT[T] = mfma_fp6_fp4(A, expand_fp4_affine(term_word<KB>(wd, T), kf), v4f{0.0f, 0.0f, 0.0f, 0.0f}, scq[0]);
          float code = -cq;
#pragma unroll
          for (int T = 0; T < NTK; ++T) code = fmaf(ak[T], (dT[T][0] + dT[T][1]) + (dT[T][2] + dT[T][3]), code);
          code2[c] = code;
        }
      }
    }
    if constexpr (QJL) {
      const v8i As = qop(NCS);
      const v4f dQ0 = mfma_fp6_fp4(As, expand_fp4_affine(Bk.ks.x, kf), v4f{-csq, 0.0f, 0.0f, 0.0f}, scsq);
      const v4f dQ1 = mfma_fp6_fp4(As, expand_fp4_affine(Bk.ks.y, kf), v4f{-csq, 0.0f, 0.0f, 0.0f}, scsq);
      qj2[0] = (dQ0[0] + dQ0[1]) + (dQ0[2] + dQ0[3]);
      qj2[1] = (dQ1[0] + dQ1[1]) + (dQ1[2] + dQ1[3]);
    }
  };
  // (1b) this wave's reference per head (row g4) for the logits in lgp: the
  // integer ceiling of its step maximum (p <= 1 against it), and the
  // probabilities of its two slots
  auto wave_ref = [&](float& rw, float& p0, float& p1) __attribute__((always_inline)) {
    const float mloc = row_max16(fmaxf(lgp[0], lgp[1]));
    rw = fmaxf(ceilf(mloc), kNoRef);
    p0 = __builtin_amdgcn_exp2f(lgp[0] - rw);   // exp2(-inf) = 0 for slots without a logit
    p1 = __builtin_amdgcn_exp2f(lgp[1] - rw);
  };
  // digits of p * radius (radii in vn) to shared memory
  auto p_digits = [&](uint8_t* pl, uint8_t* pe, float p0, float p1, uint32_t vn) __attribute__((always_inline)) {
    float r0 = mul_zero_wins(p0, h2f(vn));
    float r1 = mul_zero_wins(p1, h2f(vn >> 16));
    const float pm = row_max16(fmaxf(r0, r1));
    // r 2^-s0 < 16; s0 in [-103, 124] (pm < 2^128; pm below 2^-100 is taken
    // as 2^-100), so every digit's E8M0 byte s0 - 5 j + 127 lies in [14, 251]
    const int s0 = max(exponent_of(pm), -100) - 3;
    // (the value operand's sign field takes the complemented bit: no sign flip here)
    r0 = __builtin_amdgcn_ldexpf(r0, -s0);
    r1 = __builtin_amdgcn_ldexpf(r1, -s0);
    int pk = static_cast<int>(vn);   // (the high half of each packed word is not stored)
#pragma unroll
    for (int j = 0; j < 3; ++j) {   // (the fourth digit row is zero from the start)
      const float d0 = rintf(r0), d1 = rintf(r1);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(d0, d1, pk, false);
      if (j < 2) {
        r0 = (r0 - d0) * 32.0f;
        r1 = (r1 - d1) * 32.0f;
      }
      *reinterpret_cast<uint16_t*>(&pl[(4 * g4 + j) * kPRow + 32 * wl + 2 * t]) = static_cast<uint16_t>(pk & 0xffff);
    }
    // bytes s0 + 127, s0 + 122, s0 + 117, 127 (no byte carries into the next)
    const uint32_t ebytes = static_cast<uint32_t>(s0 * 0x010101 + (0x7f000000 + 127 + (122 << 8) + (117 << 16)));
    *reinterpret_cast<uint32_t*>(&pe[16 * wl + 4 * g4]) = ebytes;   // the same from every lane of the row
  };
  // (2a) logits of block i
  auto logits = [&](R& Bk, int i, const float (&code2)[2], const float (&qj2)[2]) __attribute__((always_inline)) {
    const int blk = bk(i);
    const int n_t = (blk < blk1) ? min(kBlock, len - blk * kBlock) : 0;   // (a group's block past the split: none)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int tok = pos_of_slot(32 * wl + 2 * t + c);
      const float nk = h2f(c ? (Bk.kn >> 16) : Bk.kn);
      const float rho = QJL ? h2f(c ? (Bk.kr >> 16) : Bk.kr) : 0.0f;
      // (rho * qj as an fma with a zero addend: one mixed-precision instruction
      // takes the fp16 rho as it is)
      float l2 = fmaf(nk, code2[c], QJL ? fmaf(rho, qj2[c], 0.0f) : 0.0f);
      // computed on every lane: used only where valid, the products feeding it
      // would otherwise be sunk into a divergent branch
      asm volatile("" : "+v"(l2));
      const bool valid = (tok < n_t) && (g4 < G);
      if constexpr (AUX) {   // (no logits: an empty buffer, every store dropped)
        const int lo = valid ? (g4 * a.max_ctx + blk * kBlock + tok) * 4 : -1;   // -1: past the buffer's end
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(__fmul_rn(l2, kLn2)), rlg, lo, 0, 0);
      }
      lgp[c] = valid ? l2 : -INFINITY;
    }
  };
  // (2b) the block's running references: head g4 (denominator) and head t / 4
  // (column) from the references of the group's waves in rwr (indexed by
  // wave within the group); returns the block's reference of head t / 4
  auto merge_refs = [&](const float (*rwr)[4], float rw, float ps) __attribute__((always_inline)) {
    const int hb = t >> 2;
    float rb = rwr[0][hb];
#pragma unroll
    for (int u = 1; u < 4; ++u) rb = fmaxf(rb, rwr[u][hb]);
    const float mn_b = (rb > m_b + 8.0f) ? rb : m_b;
    const float fv = __builtin_amdgcn_ldexpf(1.0f, shift_of(m_b - mn_b));
    // head g4's reference and factor: every lane whose t / 4 is g4 holds them
    // (the same recurrence over the same wave references), lane 4 g4 among them
    const float mn_a = __int_as_float(__builtin_amdgcn_ds_bpermute(ref_src, __float_as_int(mn_b)));
    const float fh = __int_as_float(__builtin_amdgcn_ds_bpermute(ref_src, __float_as_int(fv)));
    lsum = fmaf(lsum, fh, __builtin_amdgcn_ldexpf(ps, shift_of(rw - mn_a)));
    m_a = mn_a;
    m_b = mn_b;
    if (__any(fv != 1.0f)) {   // rescale only when some head's reference moved
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int T = 0; T < NTV; ++T) accV[rr][T] *= fv;
      accO *= fv;
    }
    return rb;
  };
  // Sparse-V: every weight of the block below 2^-tau of the largest one so
  // far, for every head of the group (the same verdict in every wave: they
  // merge the same references); its value work is skipped, its weights stay
  // in the denominator
  auto sparse_skip = [&](float rb) __attribute__((always_inline)) {
    if (!AUX || a.sparse_v <= 0) return false;
    m_top = fmaxf(m_top, rb);
    return static_cast<bool>(__all(rb < m_top - tau_v));   // a block with no position has rb = kNoRef
  };
  // value products of the block whose digits are in pl / pe and whose value
  // words are in Bv; rwr: every wave's reference of that block
  auto value_products = [&](const uint8_t* pl, const uint8_t* pe, const float (*rwr)[4], R& Bv)
      __attribute__((always_inline)) {
    const uint4 lo = *reinterpret_cast<const uint4*>(&pl[t * kPRow + 16 * g4]);
    const uint4 hi = *reinterpret_cast<const uint4*>(&pl[t * kPRow + 64 + 16 * g4]);
    const v8i Pv = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    // k-block g4 holds wave g4's positions: its digits carry 2^(its reference - the running one)
    const int adj = shift_of(rwr[g4][t >> 2] - m_b);   // an empty k-block gives the smallest scale (its digits are 0)
    const int scp = min(max(static_cast<int>(pe[16 * g4 + t]) + adj, 1), 254);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      uint32_t vw[VB];
#pragma unroll
      for (int p = 0; p < VB; ++p) vw[p] = rr ? Bv.vp[p].y : Bv.vp[p].x;
#pragma unroll
      for (int T = 0; T < NTV; ++T)
        accV[rr][T] = mfma_fp4_fp8(expand_fp4_affine_v(term_word<VB>(vw, T), kf), Pv, accV[rr][T], scp);
    }
    accO = mfma_fp4_fp8(aoff, Pv, accO, scp);
  };
  // each matrix instruction of a step's first half issued with a few vector
  // ones after it
  auto interleave = [&](auto n_mat) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < decltype(n_mat)::value; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix instruction
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // six vector ones
    }
  };
  using KMat = std::integral_constant<int, 2 * NTK + (QJL ? 2 : 0)>;

  // Step i is two halves around one barrier, each pairing matrix work with
  // independent vector work: (1) the key products of block i with the
  // probability digits of block i - 1 (written to shared memory); (2) after
  // the barrier, the logits of block i, then block i - 1's running references
  // and value products.  CUR: block i exists; PREV: block i - 1 does.
  auto step = [&](R& Bk, R& Bv, int i, auto cur_c, auto prev_c, auto set_c) __attribute__((always_inline)) {
    constexpr bool CUR = decltype(cur_c)::value;
    constexpr bool PREV = decltype(prev_c)::value;
    constexpr int pj = decltype(set_c)::value;   // Bv's register set = block (i - 1) mod kSets
    // no instruction moves across a step boundary (hoisting the next step's
    // products into this one's runs out of registers)
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<(kSets - 1) * F::loads>();   // block i's keys and block i - 1's values have landed
    float code2[2] = {0.0f, 0.0f}, qj2[2] = {0.0f, 0.0f};
    if constexpr (CUR) key_products(Bk, code2, qj2);
    float rw = -INFINITY, ps = 0.0f;
    if constexpr (PREV) {
      float p0, p1;
      wave_ref(rw, p0, p1);
      rwb[pj][w][g4] = rw;   // every lane of the row stores the same value
      p_digits(&plimb[gr][pj][0], &pexp[gr][pj][0][0], p0, p1, Bv.vn);
      ps = p0 + p1;
    }
    if constexpr (CUR && PREV) interleave(KMat{});
    if constexpr (PREV) lds_barrier();
    if constexpr (CUR) logits(Bk, i, code2, qj2);
    if constexpr (PREV) {
      const float rb = merge_refs(rwb[pj] + 4 * gr, rw, ps);
      if (!sparse_skip(rb)) value_products(&plimb[gr][pj][0], &pexp[gr][pj][0][0], rwb[pj] + 4 * gr, Bv);
    }
    // ---- refills: keys kSets blocks past block i, values kSets past block i - 1
    if constexpr (CUR) load_k(Bk, bk(i + kSets), blk1, rk);
    if constexpr (PREV) load_v(Bv, bk(i - 1 + kSets), blk1, rv);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Sparse-V that skips the value bytes too (the logits / Sparse-V variant
  // with three register sets): a block's value words are requested only once
  // its vote is known and used two steps later.  Step i: the key products of
  // block i and the reference of block i - 1; the digits of block i - 3;
  // barrier; the logits of block i; the vote on block i - 1 and its value
  // request; the value products of block i - 3.  Set s = i mod 3 holds the
  // keys of block i and the values, probabilities and vote of block i - 3.
  // CUR: block i exists; PREV: block i - 1 does; OLD: block i - 3 does.
  auto step_lag = [&](R& Bc, R& Bn, R& Bm, int i, auto cur_c, auto prev_c, auto old_c) __attribute__((always_inline)) {
    constexpr bool CUR = decltype(cur_c)::value;
    constexpr bool PREV = decltype(prev_c)::value;
    constexpr bool OLD = decltype(old_c)::value;
    __builtin_amdgcn_sched_barrier(0);
    // block i's keys (and block i - 3's values) have landed: issued after
    // them are the keys of blocks i + 1 and i + 2 and, unless its vote
    // skipped it, the values of block i - 2 (in set Bm); in the last steps
    // every load is waited for
    if (CUR || PREV) {
      if (Bm.vreq) wait_vm<2 * (F::loads - VB - 1) + VB + 1>();
      else wait_vm<2 * (F::loads - VB - 1)>();
    } else {
      wait_vm<0>();
    }
    float code2[2] = {0.0f, 0.0f}, qj2[2] = {0.0f, 0.0f};
    if constexpr (CUR) key_products(Bc, code2, qj2);
    float rw = -INFINITY, ps = 0.0f;
    if constexpr (PREV) {
      wave_ref(rw, Bn.pp0, Bn.pp1);
      rwb[(i - 1) & 3][w][g4] = rw;
      ps = Bn.pp0 + Bn.pp1;
    }
    const int pj = i & 1;
    if constexpr (OLD) {
      if (Bc.vreq) p_digits(&plimb[0][pj][0], &pexp[0][pj][0][0], Bc.pp0, Bc.pp1, Bc.vn);
    }
    if constexpr (CUR && PREV) interleave(KMat{});
    if constexpr (PREV || OLD) lds_barrier();
    if constexpr (CUR) logits(Bc, i, code2, qj2);
    if constexpr (PREV) {
      const float rb = merge_refs(rwb[(i - 1) & 3], rw, ps);
      Bn.vreq = !sparse_skip(rb);
      if (Bn.vreq) load_v(Bn, bk(i - 1), blk1, rv);
    }
    if constexpr (OLD) {
      if (Bc.vreq) value_products(&plimb[0][pj][0], &pexp[0][pj][0][0], rwb[(i - 3) & 3], Bc);
    }
    if constexpr (CUR) load_k(Bc, bk(i + kSets), blk1, rk);
    __builtin_amdgcn_sched_barrier(0);
  };

  using Y = std::true_type;
  using N = std::false_type;
  if (n_iter > 0) {   // uniform over the workgroup
    if constexpr (kLag) {
      buf0.vreq = buf1.vreq = buf2.vreq = false;
      // steps 0 .. n_iter + 2; set i mod 3 is (keys of i, values of i - 3)
      step_lag(buf0, buf2, buf1, 0, Y{}, N{}, N{});
      if (n_iter > 1) step_lag(buf1, buf0, buf2, 1, Y{}, Y{}, N{});
      else step_lag(buf1, buf0, buf2, 1, N{}, Y{}, N{});
      if (n_iter > 2) step_lag(buf2, buf1, buf0, 2, Y{}, Y{}, N{});
      else if (n_iter == 2) step_lag(buf2, buf1, buf0, 2, N{}, Y{}, N{});
      int i = 3;
      for (; i + 3 <= n_iter; i += 3) {
        step_lag(buf0, buf2, buf1, i, Y{}, Y{}, Y{});
        step_lag(buf1, buf0, buf2, i + 1, Y{}, Y{}, Y{});
        step_lag(buf2, buf1, buf0, i + 2, Y{}, Y{}, Y{});
      }
      // the rest: steps i .. n_iter + 2 (i = 0 mod 3, i >= 3; at most 5 steps)
      auto tail = [&](R& Bc, R& Bn, R& Bm, int j) __attribute__((always_inline)) {
        if (j < n_iter) {
          step_lag(Bc, Bn, Bm, j, Y{}, Y{}, Y{});
        } else if (j == n_iter) {
          step_lag(Bc, Bn, Bm, j, N{}, Y{}, Y{});
        } else if (j <= n_iter + 2) {
          step_lag(Bc, Bn, Bm, j, N{}, N{}, Y{});
        }
      };
      tail(buf0, buf2, buf1, i);
      tail(buf1, buf0, buf2, i + 1);
      tail(buf2, buf1, buf0, i + 2);
      tail(buf0, buf2, buf1, i + 3);
      tail(buf1, buf0, buf2, i + 4);
    } else {
      using S0 = std::integral_constant<int, 0>;
      using S1 = std::integral_constant<int, 1>;
      using S2 = std::integral_constant<int, 2>;
      step(buf0, buf1, 0, Y{}, N{}, S1{});   // (no block -1: its buffer is not used)
      int i = 1;
      if constexpr (kSets == 3) {
        for (; i + 3 <= n_iter; i += 3) {
          step(buf1, buf0, i, Y{}, Y{}, S0{});
          step(buf2, buf1, i + 1, Y{}, Y{}, S1{});
          step(buf0, buf2, i + 2, Y{}, Y{}, S2{});
        }
        // i = 1 (mod 3); the last step has no block i
        if (i < n_iter) {
          step(buf1, buf0, i, Y{}, Y{}, S0{});
          if (i + 1 < n_iter) {
            step(buf2, buf1, i + 1, Y{}, Y{}, S1{});
            step(buf0, buf2, i + 2, N{}, Y{}, S2{});
          } else {
            step(buf2, buf1, i + 1, N{}, Y{}, S1{});
          }
        } else {
          step(buf1, buf0, i, N{}, Y{}, S0{});
        }
      } else {
        for (; i + 2 <= n_iter; i += 2) {
          step(buf1, buf0, i, Y{}, Y{}, S0{});
          step(buf0, buf1, i + 1, Y{}, Y{}, S1{});
        }
        // i odd
        if (i < n_iter) {
          step(buf1, buf0, i, Y{}, Y{}, S0{});
          step(buf0, buf1, i + 1, N{}, Y{}, S1{});
        } else {
          step(buf1, buf0, i, N{}, Y{}, S0{});
        }
      }
    }
  }

  // ------------------------------------------------------------- partials
  const float dva = a.tb.dv[lane], dvb = a.tb.dv[lane + 64];
  {
    const float ls = row_sum16(lsum);
    if (t == 0) wred[w][g4] = ls;
    if (wl == 0 && t == 0) mrun[gr][g4] = (m_a == kNoRef) ? -INFINITY : m_a;
    const int hc = t >> 2;
    float avsum = 0.0f;
#pragma unroll
    for (int T = 0; T < NTV; ++T) avsum += av[T];
    const float voff = avsum * 0.5f * (accO[0] + lane_xor<32>(accO[0]));
    float v[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = -voff;
#pragma unroll
        for (int T = 0; T < NTV; ++T) s = fmaf(av[T], accV[r][T][i], s);
        s += lane_xor<1>(s);   // the 4 digit columns of head hc
        s += lane_xor<2>(s);
        v[r][i] = s;
      }
    // result row 4 g4 + i of pass r is coordinate 32 wl + 8 g4 + 2 i + r
    if (hc < G && (t & 3) == 0) {
      float* o = &obuf[gr][hc][32 * wl + 8 * g4];
      *reinterpret_cast<float4*>(o) = make_float4(v[0][0], v[1][0], v[0][1], v[1][1]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(v[0][2], v[1][2], v[0][3], v[1][3]);
    }
  }
  __syncthreads();
  if (w < G) {
    float lo = obuf[0][w][lane], hi = obuf[0][w][lane + 64];
    float mh = mrun[0][w], lh = 0.0f;   // the split's reference (log2 units) and denominator of head w
#pragma unroll
    for (int u = 0; u < 4; ++u) lh += wred[u][w];
    if constexpr (NG == 2) {
      // the two groups' sums, each against its own running reference, brought
      // to the larger one (powers of two)
      const float m1 = mrun[1][w];
      float l1 = 0.0f;
#pragma unroll
      for (int u = 4; u < 8; ++u) l1 += wred[u][w];
      const float mx = fmaxf(mh, m1);
      const float f0 = (mh == -INFINITY) ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, shift_of(mh - mx));
      const float f1 = (m1 == -INFINITY) ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, shift_of(m1 - mx));
      lo = fmaf(obuf[1][w][lane], f1, lo * f0);
      hi = fmaf(obuf[1][w][lane + 64], f1, hi * f0);
      lh = fmaf(l1, f1, lh * f0);
      mh = mx;
    }
    wave_fwht128(lo, hi, lane);
    const float inv_d = 1.0f / static_cast<float>(kD);
    lo *= dva * inv_d;
    hi *= dvb * inv_d;
    float* pp = a.partials + ((static_cast<int64_t>(b) * a.n_q + hq0 + w) * a.n_splits + split) * kPartialStride;
    store_coherent(pp + lane, lo);
    store_coherent(pp + 64 + lane, hi);
    if (lane == 0) {
      store_coherent(pp + kD, mh * kLn2);
      store_coherent(pp + kD + 1, lh);
    }
  }
  if (!arrive_last(counter, a.n_splits, &s_last)) return;
  merge_splits(a, b, hq0, G, counter, w, lane);
}

template <int KB, bool QJL, int VB, bool AUX, int NG>
__global__ __launch_bounds__(kRegThreads * NG, 2) void decode_reg_kernel(DecodeArgs a) {
  decode_reg_body<KB, QJL, VB, false, AUX, NG>(a);
}

template <int KB, bool QJL, int VB, bool AUX, int NG>
__global__ __launch_bounds__(kRegThreads * NG, 2) void decode_reg_append_kernel(DecodeArgs a) {
  decode_reg_body<KB, QJL, VB, true, AUX, NG>(a);
}

template <int KB, bool QJL, int VB>
hipError_t launch_kv(const DecodeArgs& a, hipStream_t stream) {
  const int nhg = (a.group + 3) / 4;
  const int n_units = a.n_splits * a.n_kv * a.batch;
  dim3 grid(((n_units + 7) / 8) * 8 * nhg);
  const bool aux = a.sparse_v > 0 || a.logits != nullptr;
  if (a.k_new != nullptr) {
    if (aux)
      hipLaunchKernelGGL((decode_reg_append_kernel<KB, QJL, VB, true, 1>), grid, dim3(kRegThreads), 0, stream, a);
    else if (a.groups == 2)
      hipLaunchKernelGGL((decode_reg_append_kernel<KB, QJL, VB, false, 2>), grid, dim3(2 * kRegThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_reg_append_kernel<KB, QJL, VB, false, 1>), grid, dim3(kRegThreads), 0, stream, a);
  } else {
    if (aux)
      hipLaunchKernelGGL((decode_reg_kernel<KB, QJL, VB, true, 1>), grid, dim3(kRegThreads), 0, stream, a);
    else if (a.groups == 2)   // one eight-wave workgroup per compute unit
      hipLaunchKernelGGL((decode_reg_kernel<KB, QJL, VB, false, 2>), grid, dim3(2 * kRegThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_reg_kernel<KB, QJL, VB, false, 1>), grid, dim3(kRegThreads), 0, stream, a);
  }
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
  if (!decode_reg_applies(a.k_codec, a.v_codec, a.group)) return hipErrorNotSupported;
  // block byte offsets (up to n_blocks + 2 blocks) are 32-bit buffer offsets
  const int64_t span = (static_cast<int64_t>(a.n_blocks) + 4) * std::max(a.k_block_bytes, a.v_block_bytes);
  if (span >= (int64_t{1} << 31) || static_cast<int64_t>(a.n_splits) * kPartialStride * 4 >= (int64_t{1} << 31))
    return hipErrorNotSupported;
  // the logits of four heads of one sequence are addressed with 32-bit offsets
  if (a.logits != nullptr && int64_t{16} * a.max_ctx >= (int64_t{1} << 31)) return hipErrorNotSupported;
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
