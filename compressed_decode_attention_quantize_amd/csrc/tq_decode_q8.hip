// tq_decode_q8.hip -- decode attention for q8 keys (the "K in q8_0" configuration
// of the wis-web.com reader article on TurboQuant in a llama.cpp fork: int8 rows
// with one fp16 scale per 32 coordinates) and POLAR values, when more than four
// query heads share a KV head.
//
// One workgroup serves every query head of its (split, KV head, sequence):
// HG groups of four waves, group g taking query heads 4 g .. 4 g + 3.  All
// groups read the same 128-position block from one ring of shared-memory
// slots, so a block crosses from L2 into shared memory once, not once per
// head group; with one eight-to-sixteen-wave workgroup per compute unit the
// ring holds four slots (three blocks in flight).  The arithmetic is that of
// the ring kernel in tq_decode_mfma.hip: per 32-coordinate block, exact int32
// sums of three base-128 int8 digits of the query against the key rows on
// v_mfma_i32_16x16x32_i8, weighted by the block's fp16 scale; softmax with
// power-of-two references; values as fp4 bit-plane operands against three
// base-32 fp8 digits of p * radius on v_mfma_scale_f32_16x16x128_f8f6f4; each
// split's sums rotated back (D_V H / d) and merged by the last split to
// arrive.

#include <algorithm>

#include "tq_mfma_ops.h"

namespace tq {
namespace {

// Block and ring layout: a key block is int8[128][128] then fp16 scales
// [128][4]; a value block is VB bit planes then fp16 radii.
template <int VB, int HG>
struct Q8Fmt {
  static constexpr int waves = 4 * HG;
  static constexpr int threads = 64 * waves;
  static constexpr int kBytes = kBlock * kD + kBlock * 8;
  static constexpr int vBytes = 2048 * VB + 256;
  static constexpr int kChunks = (kBytes + 1023) / 1024;   // 1 KB copy units per block
  static constexpr int vChunks = (vBytes + 1023) / 1024;
  static constexpr int perWave = (kChunks + vChunks + waves - 1) / waves;   // copies per wave per step
  static constexpr int slotBytes = (kChunks + vChunks) * 1024;
  // everything else the kernel keeps in shared memory, per head group and shared
  static constexpr int otherBytes = HG * (2 * 16 * 128 + 2 * 64 + 3 * 4 * kD + 4 * kD * 4 + 64) + 2 * 1024 + 4096;
  static constexpr int slotsFit = (160 * 1024 - otherBytes) / slotBytes;
  static constexpr int nSlots = slotsFit < 4 ? slotsFit : 4;
  static_assert(nSlots >= 3, "ring needs three slots");
};

// q8 key rows are stored in shared memory with their 16-byte granules
// permuted: granule j of position tok sits at granule j ^ swz(tok) of its row,
// so that the sixteen positions one matrix operand reads together fall on
// distinct banks.
__device__ __forceinline__ int q8_swz(int tok) { return ((tok >> 3) & 3) | ((tok & 2) << 1); }

// Copies of one block (K region, then V region) into a ring slot, straight
// from memory into shared memory, 1 KB per instruction (lane l moves bytes
// 16 l .. 16 l + 15 of its unit); every wave issues the same number of copies
// (units past the block read into a junk buffer).
template <int VB, int HG>
struct Q8Copier {
  using F = Q8Fmt<VB, HG>;
  int lo[F::perWave];
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int j = 0; j < F::perWave; ++j) {
      const int q = w + F::waves * j;
      const bool isk = q < F::kChunks;
      const bool isv = !isk && q < F::kChunks + F::vChunks;
      int g = 64 * q + lane;   // granule of the block's K region this lane fills
      if (isk && g < kBlock * kD / 16) g = (g & ~7) + ((g & 7) ^ q8_swz(g >> 3));
      lo[j] = isk ? 16 * g : (isv ? 1024 * (q - F::kChunks) + 16 * lane : 0x7fff0000 + 16 * lane);
    }
  }
  __device__ __forceinline__ void copy(uint8_t* slot, uint8_t* junk, __amdgpu_buffer_rsrc_t rk,
                                       __amdgpu_buffer_rsrc_t rv, int blk, int w) const {
#pragma unroll
    for (int j = 0; j < F::perWave; ++j) {
      const int q = w + F::waves * j;   // uniform over the wave
      const bool isk = q < F::kChunks;
      const bool isv = !isk && q < F::kChunks + F::vChunks;
      const int stride = isk ? F::kBytes : (isv ? F::vBytes : 0);
      uint8_t* dst = (isk || isv) ? slot + 1024 * q : junk;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isk ? rk : rv, (__attribute__((address_space(3))) void*)(dst), 16,
                                               lo[j], __builtin_amdgcn_readfirstlane(blk * stride), 0, 0);
    }
  }
};

// A running or step reference with no valid position behind it: finite, so
// that differences and exponentials of it need no special case (it converts
// to a huge negative shift, 2^shift = 0).
constexpr float kQ8NoRef = -1e30f;
// float -> int of a shift that is at most a few units above zero, clamped
// below (an absent reference gives a large negative value)
__device__ __forceinline__ int q8_shift(float x) { return static_cast<int>(fmaxf(x, -1073741824.0f)); }

// LG: logits requested (each step stores them through a range-checked
// buffer); the plain variant stores nothing in its loop.
template <int VB, int HG, bool FUSED, bool LG>
__device__ __forceinline__ void decode_q8_body(const DecodeArgs& a) {
  using F = Q8Fmt<VB, HG>;
  constexpr int kWaves = F::waves;
  constexpr int NTV = NTerms<VB>::n;
  constexpr int NS = F::nSlots;
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[F::slotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[F::slotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[F::slotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t slot3[NS > 3 ? F::slotBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t junk[1024];
  __shared__ __attribute__((aligned(16))) uint8_t plimb[HG][2][16 * 128];   // [group][parity][col][k]: digits of p * radius
  __shared__ __attribute__((aligned(4))) uint8_t pexp[HG][2][4][16];        // [group][parity][k / 32][col]
  __shared__ __attribute__((aligned(8))) int8_t qdig[HG][4][3][kD];         // base-128 digits of q per head
  __shared__ int qexp8[HG][4];
  __shared__ float rwb[2][kWaves][4];       // [parity][wave][head of its group]: each wave's step reference
  __shared__ float wred[kWaves][4];
  __shared__ float mrun[HG][4];
  __shared__ __attribute__((aligned(16))) float obuf[HG][4][kD];
  __shared__ __attribute__((aligned(16))) float r_lds[kD];   // the serving step's key residual (unused for q8)
  __shared__ int s_last;
  uint8_t* const slots[4] = {slot0, slot1, slot2, slot3};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hgl = w >> 2;   // head group of this wave
  const int wl = w & 3;     // wave within the group: positions 32 wl .. 32 wl + 31 of a block
  const int t = lane & 15;
  const int g4 = lane >> 4;
  // workgroup -> (split, KV head, sequence), split-major
  const int pairs = a.n_kv * a.batch;
  const int unit = blockIdx.x;
  if (unit >= a.n_splits * pairs) return;
  const int split = unit / pairs;
  const int pair = unit - split * pairs;
  const int h = pair % a.n_kv;
  const int b = pair / a.n_kv;
  const int G = min(4, a.group - 4 * hgl);   // query heads of this wave's group
  const int hq0 = h * a.group + 4 * hgl;     // the first of them
  uint32_t* const counter = a.counters + (static_cast<int64_t>(b) * a.n_kv + h) * (kMaxGroup / 4);
  typedef __attribute__((address_space(4))) const int cint;
  const int len_in = min(*((cint*)(a.seq_lens) + b), a.max_ctx);
  if constexpr (FUSED) {
    if (len_in < a.max_ctx && split_of_block(a, len_in / kBlock) == split)
      fused_append<8, false, VB>(a, b, h, len_in, w, lane, r_lds);
  }
  // this wave's query head (rows past G: zero digits)
  const float* qp = a.q + (static_cast<int64_t>(b) * a.n_q + hq0 + min(wl, G - 1)) * kD;
  const float qa = (wl < G) ? qp[lane] : 0.0f, qb = (wl < G) ? qp[lane + 64] : 0.0f;
  const float inv_sqrt_d = 0.08838834764831845f;
  float av[NTV];
#pragma unroll
  for (int T = 0; T < NTV; ++T) av[T] = a.tb.av[T];

  const int len = FUSED ? min(len_in + 1, a.max_ctx) : len_in;
  const int nblk_seq = (len + kBlock - 1) / kBlock;
  const int blk0 = split_first_block(a, split);
  const int blk1 = min(blk0 + split_block_count(a, split), nblk_seq);
  const int n_iter = max(0, blk1 - blk0);
  const int64_t slot0_idx = (static_cast<int64_t>(b) * a.n_kv + h) * a.n_blocks;
  const __amdgpu_buffer_rsrc_t rlg = __builtin_amdgcn_make_buffer_rsrc(
      LG ? a.logits + (static_cast<int64_t>(b) * a.n_q + hq0) * a.max_ctx : a.logits, static_cast<short>(0),
      LG ? G * a.max_ctx * 4 : 0, 0x00020000);

  float m_a = kQ8NoRef, m_b = kQ8NoRef;   // running reference (log2) of head g4 / head t / 4
  const int ref_src = 16 * g4;             // byte address of lane 4 g4 (whose t / 4 is g4) for a lane permute
  float m_top = -INFINITY;                  // Sparse-V: largest step reference of head t / 4 so far
  const bool sparse_v = a.sparse_v > 0;
  const float tau_v = static_cast<float>(a.sparse_v);
  float lsum = 0.0f;
  v4f accV[2][NTV];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int T = 0; T < NTV; ++T) accV[r][T] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  v4f accO = v4f{0.0f, 0.0f, 0.0f, 0.0f};   // the affine value operand's offset (see tq_decode_mfma.hip)
  const Fp4Fill kf = fp4_fill();
  const v8i aoff = expand_fp4_affine_v(t < 8 ? 0xffffffffu : 0u, kf);

  {
    __builtin_amdgcn_sched_barrier(0);
    // the first blocks range over the whole cache of this (sequence, KV head)
    // (blocks past the sequence are read but never weighted)
    const __amdgpu_buffer_rsrc_t rk0 = block_rsrc(a.kc + slot0_idx * a.k_block_bytes, a.k_block_bytes, a.n_blocks);
    const __amdgpu_buffer_rsrc_t rv0 = block_rsrc(a.vc + slot0_idx * a.v_block_bytes, a.v_block_bytes, a.n_blocks);
    Q8Copier<VB, HG> cp;
    cp.init(w, lane);
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) cp.copy(slots[s], junk, rk0, rv0, min(blk0 + s, a.n_blocks - 1), w);

    // ---- set-up: three base-128 digits of this wave's query head, integers
    // in [-64, 64], with one leading exponent per head
    {
      const float m = wave_max64(fmaxf(fabsf(qa), fabsf(qb)));
      const int e = (m >= 1e-30f) ? exponent_of(m) - 5 : 0;   // |q| 2^-e < 64
      float r0 = __builtin_amdgcn_ldexpf(qa, -e), r1 = __builtin_amdgcn_ldexpf(qb, -e);
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const float d0 = rintf(r0), d1 = rintf(r1);
        qdig[hgl][wl][j][lane] = static_cast<int8_t>(d0);
        qdig[hgl][wl][j][lane + 64] = static_cast<int8_t>(d1);
        r0 = (r0 - d0) * 128.0f;
        r1 = (r1 - d1) * 128.0f;
      }
      if (lane == 0) qexp8[hgl][wl] = e;
    }
    // the fourth digit row of every digit buffer holds zeros throughout
    for (int o = tid; o < HG * 2 * 4 * 32; o += F::threads) {
      const int gg = o / 256, par = (o / 128) & 1, rg = (o / 32) & 3, dw = o & 31;
      reinterpret_cast<uint32_t*>(&plimb[gg][par][(4 * rg + 3) * 128])[dw] = 0u;
    }
    // block blk0 has landed (this wave's copies of it; the barrier covers the
    // other waves'): the first step reads it before any wait of the loop
    wait_vm<(NS - 2) * F::perWave>();
    lds_barrier();
    // row t of the query operand = (head t / 4, digit t % 4) of this group
    long A8[4];
    {
      const int hh = t >> 2, dd = t & 3;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) A8[cb] = (dd < 3) ? *reinterpret_cast<const long*>(&qdig[hgl][hh][dd][32 * cb + 8 * g4]) : 0;
    }
    // 2^(e - 7) log2(e) / sqrt d for head g4: the digit sums come in units of 2^-7
    const float qsc8 = __builtin_amdgcn_ldexpf(kLog2e * inv_sqrt_d, qexp8[hgl][g4] - 7);
    const int sn = 2 * (32 * wl + 2 * t);   // this lane's two fp16 per-position fields
    // the loop's copies: blocks past the split's sequence are clamped to its last block (unused)
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(a.kc + slot0_idx * a.k_block_bytes, a.k_block_bytes, a.n_blocks);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(a.vc + slot0_idx * a.v_block_bytes, a.v_block_bytes, a.n_blocks);

    // Part A of step i: this wave's logits (positions 32 wl + 2 t + c of the
    // block for head g4 of its group), its reference per head, the digits of
    // p * radius.  Carried to part B: the reference and the sum of the lane's
    // two probabilities.
    auto partA = [&](const uint8_t* cur, int i, float& rw_out, float& ps_out) __attribute__((always_inline)) {
      const int blk = blk0 + i;
      const int n_t = min(kBlock, len - blk * kBlock);
      const uint8_t* kb = cur;
      const uint8_t* vb = cur + F::kChunks * 1024;
      float lg2[2];
      {
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
            const int gran = (2 * cb + (g4 >> 1)) ^ q8_swz(tok2[c]);
            dI[c][cb] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                A8[cb], *reinterpret_cast<const long*>(row + 16 * gran + 8 * (g4 & 1)), v4i{0, 0, 0, 0}, 0, 0, 0);
          }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float code = 0.0f;
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            // (D0 2^7 + D1) + D2 2^-7: |D0|, |D1| <= 64 * 127 * 32 < 2^18, so the
            // int32 is exact and its conversion rounds below 2^-24 of it
            const int d01 = dI[c][cb][0] * 128 + dI[c][cb][1];
            const float v = fmaf(static_cast<float>(dI[c][cb][2]), 0.0078125f, static_cast<float>(d01));
            const uint32_t sw = (cb < 2) ? sc[c].x : sc[c].y;
            code = fmaf(h2f((cb & 1) ? (sw >> 16) : sw), v, code);
          }
          const int tok = tok2[c];
          float l2 = __fmul_rn(qsc8, code);
          // computed on every lane: used only where valid, the arithmetic
          // feeding it would otherwise be sunk into a divergent branch
          asm volatile("" : "+v"(l2));
          const bool valid = (tok < n_t) && (g4 < G);
          if constexpr (LG) {   // -1: past the buffer's end, the store is dropped
            const int lo = valid ? (g4 * a.max_ctx + blk * kBlock + tok) * 4 : -1;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(__fmul_rn(l2, kLn2)), rlg, lo, 0, 0);
          }
          lg2[c] = valid ? l2 : -INFINITY;
        }
      }
      const int par = i & 1;
      uint8_t* const pl = &plimb[hgl][par][0];
      uint8_t* const pe = &pexp[hgl][par][0][0];
      const float mloc = row_max16(fmaxf(lg2[0], lg2[1]));
      const float rw = fmaxf(ceilf(mloc), kQ8NoRef);   // (no valid position: the finite no-reference)
      rwb[par][w][g4] = rw;   // every lane of the row stores the same value (no branch)
      // probabilities and base-32 digits of p * value radius (3 digits, ~14 bits)
      const uint32_t vn = *reinterpret_cast<const uint32_t*>(vb + 2048 * VB + sn);
      const float p0 = __builtin_amdgcn_exp2f(lg2[0] - rw);   // exp2(-inf) = 0 for slots without a logit
      const float p1 = __builtin_amdgcn_exp2f(lg2[1] - rw);
      // p * radius, 0 for p = 0 whatever the radius bits (slots past the length
      // hold arbitrary bytes): 0 x inf and 0 x NaN give a quiet NaN, which the
      // maximum with 0 drops (IEEE maxNum, the kernel's IEEE mode)
      // (an fma with a zero addend: one mixed-precision instruction takes the fp16 radius)
      float r0 = __builtin_fmaxf(fmaf(p0, h2f(vn), 0.0f), 0.0f);
      float r1 = __builtin_fmaxf(fmaf(p1, h2f(vn >> 16), 0.0f), 0.0f);
      const float pm = row_max16(fmaxf(r0, r1));
      // r 2^-s0 < 16; pm below 2^-100 (0 included) is taken as 2^-100
      const int s0 = max(exponent_of(pm), -100) - 3;
      // (the value operand's sign field takes the complemented bit: no sign flip here)
      r0 = __builtin_amdgcn_ldexpf(r0, -s0);
      r1 = __builtin_amdgcn_ldexpf(r1, -s0);
      int pk = static_cast<int>(vn);   // (the high half of each packed word is not stored)
#pragma unroll
      for (int j = 0; j < 3; ++j) {   // (the fourth digit row is zero from the start)
        const float d0 = rintf(r0), d1 = rintf(r1);   // integers in [-16, 16]: exact in e4m3
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(d0, d1, pk, false);
        if (j < 2) {
          r0 = (r0 - d0) * 32.0f;
          r1 = (r1 - d1) * 32.0f;
        }
        *reinterpret_cast<uint16_t*>(&pl[(4 * g4 + j) * 128 + 32 * wl + 2 * t]) = static_cast<uint16_t>(pk & 0xffff);
      }
      // bytes s0 + 127, s0 + 122, s0 + 117, 127: s0 lies in [-103, 124] (pm is
      // a finite float), so every byte lies in [14, 251] and none carries into
      // the next
      const uint32_t ebytes = static_cast<uint32_t>(s0 * 0x010101 + (0x7f000000 + 127 + (122 << 8) + (117 << 16)));
      *reinterpret_cast<uint32_t*>(&pe[16 * wl + 4 * g4]) = ebytes;   // the same from every lane of the row
      rw_out = rw;
      ps_out = p0 + p1;
    };

    // Part B of step i (after the barrier that follows every wave's part A):
    // the group's common running references, then the weighted sum of the
    // block's values for coordinates 32 wl .. 32 wl + 31 and the group's heads.
    auto partB = [&](const uint8_t* cur, int i, float rw, float ps) __attribute__((always_inline)) {
      const uint8_t* vb = cur + F::kChunks * 1024;
      const int par = i & 1;
      const uint8_t* const pl = &plimb[hgl][par][0];
      const uint8_t* const pe = &pexp[hgl][par][0][0];
      const int hb = t >> 2;
      const float(*rg)[4] = &rwb[par][4 * hgl];   // the group's four waves
      float rb = rg[0][hb];
#pragma unroll
      for (int u = 1; u < 4; ++u) rb = fmaxf(rb, rg[u][hb]);
      const float mn_b = (rb > m_b + 8.0f) ? rb : m_b;
      const float fv = __builtin_amdgcn_ldexpf(1.0f, q8_shift(m_b - mn_b));
      // head g4's reference and factor: every lane whose t / 4 is g4 holds them
      // (the same recurrence over the same wave references), lane 4 g4 among them
      const float mn_a = __int_as_float(__builtin_amdgcn_ds_bpermute(ref_src, __float_as_int(mn_b)));
      const float fh = __int_as_float(__builtin_amdgcn_ds_bpermute(ref_src, __float_as_int(fv)));
      lsum = fmaf(lsum, fh, __builtin_amdgcn_ldexpf(ps, q8_shift(rw - mn_a)));
      m_a = mn_a;
      m_b = mn_b;
      if (__any(fv != 1.0f)) {   // rescale only when some head's reference moved
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
          for (int T = 0; T < NTV; ++T) accV[rr][T] *= fv;
        accO *= fv;
      }
      // Sparse-V: every weight of the block below 2^-tau_v of the largest so
      // far for every head of the group: its value work is skipped
      if (sparse_v) {
        m_top = fmaxf(m_top, rb);
        if (__all(rb < m_top - tau_v)) return;   // (a block with no position: rb = kQ8NoRef, not skipped, p = 0)
      }
      v8i Pv;
      {
        const uint4 lo = *reinterpret_cast<const uint4*>(&pl[t * 128 + 16 * g4]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&pl[t * 128 + 64 + 16 * g4]);
        Pv = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      // k-block g4 holds the positions of wave g4 of the group: its digits
      // carry 2^(its reference - the running one)
      const float rk_ = rg[g4][hb];
      const int adj = q8_shift(rk_ - m_b);   // an empty k-block gives the smallest scale (its digits are 0)
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

    // Step i: part A, then a wait for this wave's copies of block i + 1
    // (issued NS - 2 steps ago; the barrier covers the other waves'), the
    // barrier, the refill of slot (i - 1) mod NS with block i + NS - 1 (every
    // wave is past part B of step i - 1), part B.  Exactly NS - 3 blocks of
    // copies were issued after block i + 1's; the logits' stores, when
    // requested, add to the count after them, which only makes the wait
    // stricter.
    auto step = [&](uint8_t* cur, uint8_t* refill, int i) __attribute__((always_inline)) {
      float rw, ps;
      partA(cur, i, rw, ps);
      wait_vm<(NS - 3) * F::perWave>();
      lds_barrier();
      cp.copy(refill, junk, rk, rv, min(blk0 + i + NS - 1, blk1 - 1), w);
      partB(cur, i, rw, ps);
    };
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
    }
    wait_vm<0>();   // (copies of blocks past the split may still be in flight)
  }

  // ------------------------------------------------------------- partials
  const float dva = a.tb.dv[lane], dvb = a.tb.dv[lane + 64];
  {
    const float ls = row_sum16(lsum);
    if (t == 0) wred[w][g4] = ls;
    if (wl == 0 && t == 0) mrun[hgl][g4] = (m_a == kQ8NoRef) ? -INFINITY : m_a;
    const int hc = t >> 2;
    float avsum = 0.0f;
#pragma unroll
    for (int T = 0; T < NTV; ++T) avsum += av[T];
    const float voff = avsum * 0.5f * (accO[0] + lane_xor<32>(accO[0]));
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = -voff;
#pragma unroll
        for (int T = 0; T < NTV; ++T) s = fmaf(av[T], accV[r][T][i], s);
        s += lane_xor<1>(s);   // the 3 digit columns of head hc (the fourth is zero)
        s += lane_xor<2>(s);
        v[i] = s;
      }
      if (hc < G && (t & 3) == 0)
        *reinterpret_cast<float4*>(&obuf[hgl][hc][32 * wl + 16 * r + 4 * g4]) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
  __syncthreads();
  if (wl < G) {
    // wave (group, wl): head hq0 + wl, o = D_V H (its sum) / d
    float lo = obuf[hgl][wl][lane], hi = obuf[hgl][wl][lane + 64];
    wave_fwht128(lo, hi, lane);
    const float inv_d = 1.0f / static_cast<float>(kD);
    lo *= dva * inv_d;
    hi *= dvb * inv_d;
    float* pp = a.partials + ((static_cast<int64_t>(b) * a.n_q + hq0 + wl) * a.n_splits + split) * kPartialStride;
    store_coherent(pp + lane, lo);
    store_coherent(pp + 64 + lane, hi);
    if (lane == 0) {
      float l = 0.0f;
#pragma unroll
      for (int u = 0; u < 4; ++u) l += wred[4 * hgl + u][wl];
      store_coherent(pp + kD, mrun[hgl][wl] * kLn2);
      store_coherent(pp + kD + 1, l);
    }
  }
  if (!arrive_last(counter, a.n_splits, &s_last)) return;
  merge_splits(a, b, h * a.group, a.group, counter, w, lane);
}

template <int VB, int HG, bool LG>
__global__ __launch_bounds__(256 * HG, HG) void decode_q8_kernel(DecodeArgs a) {
  decode_q8_body<VB, HG, false, LG>(a);
}
template <int VB, int HG, bool LG>
__global__ __launch_bounds__(256 * HG, HG) void decode_q8_append_kernel(DecodeArgs a) {
  decode_q8_body<VB, HG, true, LG>(a);
}

template <int VB, int HG>
hipError_t launch_q8(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_splits * a.n_kv * a.batch), block(256 * HG);
  const bool lg = a.logits != nullptr;
  if (a.k_new != nullptr) {
    if (lg) hipLaunchKernelGGL((decode_q8_append_kernel<VB, HG, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_q8_append_kernel<VB, HG, false>), grid, block, 0, stream, a);
  } else {
    if (lg) hipLaunchKernelGGL((decode_q8_kernel<VB, HG, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_q8_kernel<VB, HG, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

// The instantiations that fit their registers without spilling: with three
// waves per SIMD (three head groups) only 2-bit values; 3- and 4-bit values
// with two head groups.  Other shapes take the per-head-group ring kernel.
bool decode_q8_applies(int k_codec, int v_codec, int group, int v_bits) {
  if (k_codec != Q8_BLOCK32 || v_codec != POLAR || group <= 4) return false;
  const int hg = (group + 3) / 4;
  return hg == 2 ? (v_bits >= 2 && v_bits <= 4) : (hg == 3 && v_bits == 2);
}

hipError_t launch_decode_q8(const DecodeArgs& a, hipStream_t stream) {
  if (!decode_q8_applies(a.k_codec, a.v_codec, a.group, a.v_bits)) return hipErrorNotSupported;
  // block byte offsets are 32-bit buffer offsets
  const int64_t span = (static_cast<int64_t>(a.n_blocks) + 4) * std::max(a.k_block_bytes, a.v_block_bytes);
  if (span >= (int64_t{1} << 31) || static_cast<int64_t>(a.n_splits) * kPartialStride * 4 >= (int64_t{1} << 31))
    return hipErrorNotSupported;
  // the logits of four heads of one sequence are addressed with 32-bit offsets
  if (a.logits != nullptr && int64_t{16} * a.max_ctx >= (int64_t{1} << 31)) return hipErrorNotSupported;
  const int hg = (a.group + 3) / 4;
  if (hg == 3) return launch_q8<2, 3>(a, stream);
  switch (a.v_bits) {
    case 2: return launch_q8<2, 2>(a, stream);
    case 3: return launch_q8<3, 2>(a, stream);
    case 4: return launch_q8<4, 2>(a, stream);
  }
  return hipErrorNotSupported;
}

}  // namespace tq
