// tq_internal.h -- shared declarations between the host part of the library
// (tq_host.cpp) and its HIP kernels.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

constexpr int kD = 128;        // head_dim served by the kernels
constexpr int kM = 128;        // QJL sketch rows served by the kernels
constexpr int kBlock = 128;    // positions per cache block
constexpr int kMaxGroup = 16;  // largest GQA group
constexpr int kPartialStride = kD + 4;  // floats per split partial: acc[128], m, l, 2 pad (16-byte rows)
// Slot of position t inside its 128-position block for the per-position
// fields of POLAR keys (code words, sign words, radius, residual norm) and
// for the radius of POLAR values: a fixed permutation inside each group of
// 32 positions, chosen so that the decode kernel's fp4 matrix operands and
// its probability tiles line up with whole 8-byte loads.
__host__ __device__ inline int slot_of(int t) { return 32 * (t >> 5) + 8 * (t & 3) + ((t & 31) >> 2); }
// Inverse: the position stored in slot s.
__host__ __device__ inline int pos_of_slot(int s) { return 32 * (s >> 5) + 4 * (s & 7) + ((s & 31) >> 3); }

// Recursive polar codec ("radius + angle" tree) tables of one tensor with b
// bits: level-1 angles take b + 1 bits (uniform on the circle), the angles of
// levels 2..7 take b - 1 bits (Lloyd-Max for their law).  Decisions compare
// squared radii against cos^2 / sin^2 of the boundary angles in fp64.
struct TreeTab {
  float2 cs1[32];              // level 1: (cos, sin) of the centroid angle of each code
  float2 cs[8][8];             // level l = 2..7 at [l]: (cos, sin) of each code's centroid angle
  double c2_1[8], s2_1[8];     // level 1: cos^2, sin^2 of the boundaries inside a quadrant
  double c2[8][8], s2[8][8];   // level l = 2..7 at [l]: cos^2, sin^2 of its boundaries
};

// Byte offsets inside the parameter image (all fp32 arrays).
struct ParamsLayout {
  uint64_t dk, dv;   // float[d] rotation signs (+/-1) for K and V
  uint64_t s;        // float[m][d] Gaussian sketch (row j = sketch row)
  uint64_t st;       // float[d][m] its transpose
  uint64_t ck, kb;   // float[16] K centroids, float[16] K boundaries (2^b-1 used)
  uint64_t cv, vb;   // same for V
  uint64_t ak, av;   // float[8] odd multilinear coefficients of the K / V codebooks
  uint64_t shd;      // float[d][m]: (S H D_K / sqrt d)^T, the sketch of a query before rotation
  uint64_t tk, tv;   // TreeTab of K and of V (recursive polar codec)
  uint64_t total;
};

inline ParamsLayout params_layout(int d, int m) {
  ParamsLayout L{};
  uint64_t o = 0;
  L.dk = o; o += 4ull * d;
  L.dv = o; o += 4ull * d;
  L.s = o;  o += 4ull * m * d;
  L.st = o; o += 4ull * m * d;
  L.ck = o; o += 64;
  L.kb = o; o += 64;
  L.cv = o; o += 64;
  L.vb = o; o += 64;
  L.ak = o; o += 32;
  L.av = o; o += 32;
  L.shd = o; o += 4ull * m * d;
  o = (o + 255) & ~255ull;
  L.tk = o; o += (sizeof(TreeTab) + 255) & ~static_cast<uint64_t>(255);
  L.tv = o; o += (sizeof(TreeTab) + 255) & ~static_cast<uint64_t>(255);
  L.total = (o + 255) & ~255ull;
  return L;
}

// Codec ids (mirror tq.h; kernels are compiled without it).
enum { RAW_F32 = 0, POLAR = 1, POLAR_QJL = 2, Q8_BLOCK32 = 3, POLAR_TREE = 4 };
enum { IN_F32 = 0, IN_BF16 = 1, IN_F16 = 2 };

struct Tables {
  const float* dk;
  const float* dv;
  const float* s;    // [m][d]
  const float* st;   // [d][m]
  const float* ck;
  const float* kb;
  const float* cv;
  const float* vb;
  const float* ak;
  const float* av;
  const float* shd;  // [d][m]
  const TreeTab* tk;
  const TreeTab* tv;
};

struct QuantArgs {
  Tables tb;
  uint8_t* kc;
  uint8_t* vc;
  const int32_t* seq_lens;
  const void* k_new;
  const void* v_new;
  int32_t in_dtype;
  int32_t batch, n_kv, max_ctx, n_blocks, n_new;
  int32_t groups_per_seq;   // 32-position groups a sequence's append can touch
  int32_t k_codec, k_bits, v_codec, v_bits;
  int64_t k_block_bytes, v_block_bytes;
};

struct DecodeArgs {
  Tables tb;
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* seq_lens;
  const float* q;
  float* out;
  float* logits;      // may be null
  float* partials;    // [batch][n_q][n_splits][kPartialStride]
  uint32_t* counters; // [batch][n_kv][kMaxGroup / 4]
  int32_t batch, n_q, n_kv, group, max_ctx, n_blocks;
  int32_t chunk_blocks, n_splits;
  // splits [0, n_long) take long_blocks blocks each, the later ones
  // chunk_blocks (n_long = 0: every split takes chunk_blocks)
  int32_t long_blocks, n_long;
  int32_t k_codec, k_bits, v_codec, v_bits;
  int32_t sparse_v;   // 0, or skip value work of blocks below 2^-sparse_v of the running maximum
  int64_t k_block_bytes, v_block_bytes;
  // serving step: one new position per sequence at seq_lens[b], [batch][1][n_kv][d]
  // in in_dtype, stored before it is attended to (null: plain decode)
  const void* k_new;
  const void* v_new;
  int32_t in_dtype;
  int32_t len_add;    // positions attended = min(seq_lens[b] + len_add, max_ctx)
  int32_t groups;     // matrix-core kernel: block groups of four wavefronts per workgroup (1 or 2)
};

struct DequantArgs {
  Tables tb;
  const uint8_t* kc;
  const uint8_t* vc;
  float* k_out;
  float* v_out;
  int32_t b, start, count, n_kv, n_blocks;
  int32_t k_codec, k_bits, v_codec, v_bits;
  int32_t qjl;
  int64_t k_block_bytes, v_block_bytes;
};

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// Matrix-core decode for POLAR / POLAR_QJL keys with POLAR values and G <= 4;
// returns hipErrorNotSupported for other configurations.
bool decode_mfma_applies(int k_codec, int v_codec, int group);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);
// Register-streamed matrix-core decode for POLAR / POLAR_QJL keys with POLAR
// values and G <= 16; hipErrorNotSupported otherwise.
bool decode_reg_applies(int k_codec, int v_codec, int group);
hipError_t launch_decode_reg(const DecodeArgs& a, hipStream_t stream);
// q8 keys with POLAR values and more than four query heads per KV head: one
// workgroup per (split, KV head, sequence) serving every head group from one
// shared-memory ring; hipErrorNotSupported for other configurations.
bool decode_q8_applies(int k_codec, int v_codec, int group, int v_bits);
hipError_t launch_decode_q8(const DecodeArgs& a, hipStream_t stream);
// Block groups (of four wavefronts) per workgroup of the matrix-core decode
// kernel for a key codec: with one group two independent workgroups share a
// compute unit, with two groups one workgroup of eight wavefronts fills it.
// Workgroups the automatic split count aims for: the matrix-core kernel fills
// the 256 compute units of the target chip (512 / groups workgroups), the
// VALU kernel runs about four 256-thread workgroups per compute unit (it is
// latency-bound: more resident wavefronts hide more of it).
constexpr int kMfmaUnitWorkgroups = 512;
// register-streamed decode: 256-thread workgroups, two per compute unit
constexpr int kRegWorkgroups = 512;
constexpr int kRegMinChunkBlocks = 8;   // fewest blocks per split it is given
// With two register-streamed workgroups per compute unit, the one dispatched
// first runs ahead of the other (it wins issue arbitration): the splits whose
// workgroups go out in the first dispatch round (one per compute unit) are
// given about this many times the blocks of the later ones, so that both
// finish together.  Per mille.
#ifndef TQ_REG_LONG_SPLIT_PERMILLE
#define TQ_REG_LONG_SPLIT_PERMILLE 1400
#endif
constexpr int kRegLongSplitPermille = TQ_REG_LONG_SPLIT_PERMILLE;
constexpr int kComputeUnits = 256;   // workgroups of the first dispatch round
constexpr int kValuWorkgroups = 1024;
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t stream);
// The library's own decode workspace (tq_decode_attention_noalloc): counters
// in the first kScratchCounterBytes (zero between calls), the partials after
// them.  Device address of the current device's copy; set up on first use.
constexpr uint64_t kScratchBytes = 8ull << 20;
constexpr uint64_t kScratchCounterBytes = 64ull << 10;
hipError_t scratch_workspace(void** out, hipStream_t stream);
// Append for tensors stored with the recursive polar codec (the other kernel
// skips them).
hipError_t launch_quantize_tree(const QuantArgs& a, hipStream_t stream);
hipError_t launch_stream_read(const void* src, uint64_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace tq
