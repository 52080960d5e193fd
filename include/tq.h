/*
 * tq.h -- C ABI of the TurboQuant KV-cache library for MI355X (gfx950).
 *
 * The library implements the two data-parallel halves of the method the
 * pages describe (wis-web.com reader, article on TurboQuant in a llama.cpp
 * fork: the PolarQuant paragraph -- Walsh-Hadamard rotation, then radius +
 * angle with the angle's law known in advance -- and the QJL paragraph -- a
 * 1-bit corrector of the residual bias; leviatan.io, "TurboQuant : 6x moins
 * de cache, jusqu'a 8x plus rapide", section "Principe de quantification
 * sans calibration" -- a fixed, calibration-free transform):
 *
 *   tq_quantize_append   compress new K/V vectors into a packed block cache
 *   tq_decode_attention  one-query-per-sequence attention read straight
 *                        from the packed cache (flash-attention style,
 *                        the article's "-fa on")
 *   tq_dequantize        packed records back to fp32 (tests, inspection)
 *
 * Conventions
 *  - Plain C types only.  "device" pointers are HIP device memory owned by
 *    the caller; "host" pointers are ordinary host memory.  `stream` is a
 *    hipStream_t (NULL = the default stream) passed as void*.
 *  - The library never allocates, frees or synchronises device memory, with
 *    one exception: tq_init_params copies a host image to the device and
 *    waits for that copy.  It keeps no mutable global state apart from a
 *    process-wide cache of codebooks, so calls on different streams may run
 *    concurrently as long as they do not write the same buffers.
 *  - Every argument check runs on the host before any HIP call and returns
 *    a status; nothing aborts.  A failed kernel launch returns TQ_EDEVICE.
 *    Non-finite inputs are not checked and give unspecified codes.
 *  - Kernels exist for head_dim 128 and sketch size 128 (the shapes of the
 *    model families the pages name); other powers of two are rejected with
 *    TQ_EUNSUPPORTED.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 1u
/* Version of the packed cache and parameter-image format described at
 * tq_cache_bytes and tq_params_host.  A cache written under one format
 * version is read back (decode, dequantize, a resumed append) only by a
 * library of the same version. */
#define TQ_FORMAT_VERSION 1u
#define TQ_BLOCK_TOKENS 128   /* positions per cache block */

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = 1,        /* malformed argument (null, misaligned, out of range) */
  TQ_EUNSUPPORTED = 2,  /* well formed but no kernel for it (e.g. head_dim != 128) */
  TQ_ECAPACITY = 3,     /* append would pass max_ctx */
  TQ_EWORKSPACE = 4,    /* workspace or params buffer too small */
  TQ_EDEVICE = 5        /* a HIP call or kernel launch failed */
} tq_status;

/* Per-tensor cache codecs.  K and V are chosen separately, as the article's
 * llama-server example does with -ctk / -ctv. */
typedef enum {
  TQ_CODEC_RAW_F32 = 0,     /* bypass: fp32 copy (exact attention) */
  TQ_CODEC_POLAR = 1,       /* rotation + fp16 radius + b-bit angle codes */
  TQ_CODEC_POLAR_QJL = 2,   /* POLAR + 1-bit QJL sketch of the residual (K only) */
  TQ_CODEC_Q8_BLOCK32 = 3,  /* 8-bit symmetric per-32 block, fp16 scale, unrotated
                               (the article's "K in q8_0"; K only) */
  TQ_CODEC_POLAR_TREE = 4   /* the PolarQuant paragraph's Cartesian-to-polar step
                               taken literally: rotation + fp16 radius + 127
                               angles of a pairwise tree (K or V, b = 2..4 bits
                               per coordinate on average, no QJL) */
} tq_codec;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

/* dequantize flags */
#define TQ_DEQ_QJL 1u   /* keys: add the QJL correction (x_tilde) */

typedef struct tq_config {
  uint32_t abi_version;   /* must equal TQ_ABI_VERSION */
  int32_t head_dim;       /* d: 128 */
  int32_t n_q_heads;      /* query heads; a multiple of n_kv_heads (GQA group G = n_q/n_kv <= 16) */
  int32_t n_kv_heads;     /* query head h reads KV head h / G */
  int32_t batch;          /* sequences */
  int32_t max_ctx;        /* capacity per sequence, in positions */
  int32_t k_codec;        /* tq_codec */
  int32_t k_bits;         /* POLAR*: 2..4; Q8: 8; RAW: 32 */
  int32_t qjl_m;          /* POLAR_QJL: sketch rows (128); otherwise 0 */
  int32_t v_codec;        /* TQ_CODEC_RAW_F32, TQ_CODEC_POLAR or TQ_CODEC_POLAR_TREE */
  int32_t v_bits;         /* POLAR*: 2..4; RAW: 32 */
  int32_t decode_chunk;   /* positions per split-K workgroup, a multiple of 128; 0 = automatic */
  uint64_t seed;          /* rotation signs and sketch are drawn from (seed, layer) */
  int32_t layer;
  int32_t sparse_v;       /* decode: 0 = dense; t in 1..60 = Sparse-V (the
                           * wis-web.com reader article on the llama.cpp fork,
                           * its third finding): a 128-position block skips
                           * its value work when, for every query head it
                           * serves, the ceiling of its largest log2-logit is
                           * more than t below the ceiling of the running
                           * maximum of its split; every weight it leaves out
                           * is then below 2^-t of the largest weight.  Its
                           * weights still count in the softmax denominator.
                           * Which blocks are skipped depends on the split
                           * schedule.  Honoured by the matrix-core path
                           * (POLAR, POLAR_QJL or Q8 keys with POLAR values,
                           * G <= 16); other codecs decode densely. */
} tq_config;

/* Text for a status code (static storage). */
const char* tq_status_string(tq_status s);

/* Sizes in bytes of the K and V caches for cfg (host, pure); the memory
 * figures of the leviatan.io page's "Benchmarks de memoire" section are these
 * sizes in closed form.  Layout of one
 * cache: [batch][n_kv][ceil(max_ctx/128)][block]; block = 128 positions of one
 * (sequence, KV head):
 *   K POLAR / POLAR_QJL (b bits, m rows): b code planes u32[d/32][128] (bit e
 *     of word [j][s(t)] = bit p of the code of coordinate 32j+e of position t),
 *     then (QJL) the sign plane u32[m/32][128] (same slots), then fp16
 *     radius[128], then (QJL) fp16 residual norm[128], both at slot s(t);
 *   K Q8: int8[128][d] then fp16 scale[128][d/32] (natural order);
 *   V POLAR (b bits): b planes u32[4][d] (bit e of word [j][i] = bit p of the
 *     code of coordinate i of position 32j+e), then fp16 radius[128] at s(t);
 *   RAW: fp32[128][d].
 *   POLAR_TREE (b bits): 127 angle codes per position in heap slots a = 1..d-1
 *     (slot d/2 + i = level-1 pair i, slot 2^(L-l) + k = node k of level l,
 *     L = log2 d; slot 0 unused); level-1 codes have b + 1 bits, the others
 *     b - 1.  K: b - 1 planes u32[d/32][128] (bit e of word [j][s(t)] = bit p
 *     of slot 32j+e's code), then 2 planes u32[d/64][128] for bits b - 1 and
 *     b of slots d/2 + 32j + e, then fp16 radius[128] at s(t).  V: b - 1 planes
 *     u32[4][d] (bit e of word [j][a] = bit p of slot a's code of position
 *     32j+e), then 2 planes u32[4][d/2] (word [j][a - d/2]), then fp16
 *     radius[128] at s(t).  Same record size as POLAR with b bits.
 * Here t is the position inside its block and s(t) = 32(t/32) + 8(t%4) +
 * (t%32)/4, a fixed permutation inside each group of 32 positions.
 * Per position and head: K 3b+QJL 68 B, 4b+QJL 84 B, q8 136 B; V b bits
 * 16b+2 B (d = 128). */
tq_status tq_cache_bytes(const tq_config* cfg, uint64_t* k_bytes, uint64_t* v_bytes);

/* Size of the per-layer parameter image (rotation signs, sketch, codebooks). */
tq_status tq_params_bytes(const tq_config* cfg, uint64_t* bytes);

/* Build the parameter image in host memory `host_params` (>= tq_params_bytes).
 * Contents: signs D_K, D_V (+/-1, fp32[d]) drawn from counter-form SplitMix64
 * keyed by (seed, layer); the Gaussian sketch S (fp32[m][d], Box-Muller) and
 * its transpose; Lloyd-Max codebooks for the law of a rotated unit vector's
 * coordinate (fp16-exact centroids, fp32 midpoint boundaries); and, for
 * QJL keys, (S H D_K / sqrt d)^T (fp32[d][m], from fp64 products), which maps
 * a query before rotation straight to its sketch.  This is the
 * "distribution known in advance" of the PolarQuant paragraph and the fixed
 * transform of "Principe de quantification sans calibration".  Pure host. */
tq_status tq_params_host(const tq_config* cfg, void* host_params, uint64_t bytes);

/* Same image, copied to device memory `params` (>= tq_params_bytes) on
 * `stream`; returns after the copy has completed. */
tq_status tq_init_params(const tq_config* cfg, void* params, uint64_t bytes, void* stream);

/* Quantise n_new new positions per sequence and store them at positions
 * seq_lens[b] .. seq_lens[b]+n_new-1 of every sequence b.
 * The operation is the compression step of the wis-web.com reader article on
 * TurboQuant in a llama.cpp fork (its three-step description: Walsh-Hadamard
 * rotation, radius + angle with the angle's law known in advance, then the
 * 1-bit QJL corrector of the residual), with the problem statement's fp16
 * norms, fixed codebooks and m = 128 sign rows; the "K in q8_0" codec is the
 * same article's asymmetric configuration.
 *   params    device, from tq_init_params for the same cfg
 *   k_cache, v_cache  device, tq_cache_bytes each, 16-byte aligned
 *   seq_lens  device int32[batch]; read only (the caller advances it)
 *   max_seq_len  host bound: every seq_lens[b] <= max_seq_len; the call
 *             fails with TQ_ECAPACITY if max_seq_len + n_new > max_ctx
 *   k_new, v_new  device [batch][n_new][n_kv][d] in in_dtype (tq_dtype)
 * Per vector: y = H (D . x) (raw Walsh-Hadamard, fixed stage order), radius
 * n = |x| -> fp16, angle codes = nearest codebook centroid of y/n (bit
 * planes); keys with QJL add r = y - n16 C[code], its norm |r|/sqrt(d) ->
 * fp16 and the m sign bits of S r.  Q8 keys and RAW tensors are stored as
 * described at tq_cache_bytes.  POLAR_TREE: the same y and radius, then the
 * pairwise tree of y (level 1: angle of (y_2i, y_2i+1) on the circle, b + 1
 * bits, uniform cells; level l >= 2: atan2 of the two child radii in
 * [0, pi/2], b - 1 bits, Lloyd-Max for the law sin(2t)^(2^(l-1) - 1)); a code
 * counts the boundaries below its angle.  Positions of a 32-position group that this
 * call does not write keep their bits.  n_new == 0 is a no-op that does not
 * examine the buffer pointers. */
tq_status tq_quantize_append(const tq_config* cfg, const void* params, void* k_cache,
                             void* v_cache, const int32_t* seq_lens, int32_t max_seq_len,
                             const void* k_new, const void* v_new, int32_t in_dtype,
                             int32_t n_new, void* stream);

/* Workspace for tq_decode_attention with sequences up to max_seq_len (host,
 * pure): completion counters at a fixed offset, then the split partials.
 * A workspace sized for max_seq_len serves every call with a shorter bound,
 * in any order. */
tq_status tq_decode_workspace_bytes(const tq_config* cfg, int32_t max_seq_len, uint64_t* bytes);

/* Decode attention: one query per sequence over positions [0, seq_lens[b]).
 * The operation is the attention read straight from the compressed cache
 * that the leviatan.io page ("TurboQuant : 6x moins de cache, jusqu'a 8x plus
 * rapide", sections "Acceleration jusqu'a 8x du calcul d'attention" and
 * "Comparaison 4-bit vs 32-bit") times against a 32-bit cache, and that the
 * wis-web.com article runs as flash attention ("-fa on"); its logit is the
 * problem statement's QJL-corrected inner-product estimator.
 *   q        device fp32 [batch][n_q][d]
 *   out      device fp32 [batch][n_q][d]
 *   logits   device fp32 [batch][n_q][max_ctx] or NULL: pre-softmax scaled
 *            logits of positions [0, seq_lens[b]) (others untouched)
 *   workspace device, >= tq_decode_workspace_bytes(cfg, max_seq_len), and
 *            zero-filled before its first use; every call leaves its
 *            completion counters at zero again.
 * Logit of position t (scale 1/sqrt(d)), for POLAR_QJL keys the
 * QJL-corrected estimator <q, x_hat> + rho sqrt(pi/2)/m <S R q, sign(S r)>;
 * softmax over all stored positions; output sum_t p_t v_hat_t.  An empty
 * sequence gives a zero output.  Calls sharing a workspace must not overlap. */
tq_status tq_decode_attention(const tq_config* cfg, const void* params, const void* k_cache,
                              const void* v_cache, const int32_t* seq_lens, int32_t max_seq_len,
                              const float* q, float* out, float* logits, void* workspace,
                              uint64_t workspace_bytes, void* stream);

/* tq_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The library uses its own file-scope
 * device array instead: 8 MiB per GPU, held until the process ends, found
 * once per device on the first call (which also clears its completion
 * counters with a small kernel on `stream`).  The first 64 KiB hold the
 * counters (batch * n_kv_heads <= 4096), the rest the split partials; a call
 * that needs more returns TQ_EWORKSPACE before any launch.  No allocation,
 * free or allocating library routine is called.  `stream` must belong to the
 * current device.  Every call on one GPU shares that GPU's array: calls that
 * may overlap on one GPU (different streams, different threads) race and
 * must be serialised by the caller.  Arguments and results otherwise as
 * tq_decode_attention. */
tq_status tq_decode_attention_noalloc(const tq_config* cfg, const void* params, const void* k_cache,
                                      const void* v_cache, const int32_t* seq_lens, int32_t max_seq_len,
                                      const float* q, float* out, float* logits, void* stream);

/* Serving step in one launch (the batched-serving workload's step: one new
 * position per sequence appended, then one decode query per sequence, as the
 * wis-web.com article's llama-server runs it).  Append one new position per sequence (at
 * seq_lens[b], as tq_quantize_append with n_new = 1) and decode q over the
 * seq_lens[b] + 1 positions that then exist (as tq_decode_attention).  The
 * cache bytes and the outputs equal those of the two calls in that order.
 *   seq_lens     device int32[batch], lengths before the append; read only
 *                (the caller advances them)
 *   max_seq_len  host bound on seq_lens[b]; TQ_ECAPACITY if max_seq_len + 1
 *                passes max_ctx
 *   k_new, v_new device [batch][1][n_kv][d] in in_dtype
 *   workspace    >= tq_decode_workspace_bytes(cfg, max_seq_len + 1)
 * The matrix-core decode (the codecs tq_config.sparse_v names) stores the new
 * record from inside the decode launch: the workgroups whose split holds the
 * new position quantise and store it before they read the cache.  Other
 * codecs run the append and the decode as two launches on the stream. */
tq_status tq_append_decode(const tq_config* cfg, const void* params, void* k_cache, void* v_cache,
                           const int32_t* seq_lens, int32_t max_seq_len, const void* k_new, const void* v_new,
                           int32_t in_dtype, const float* q, float* out, float* logits, void* workspace,
                           uint64_t workspace_bytes, void* stream);

/* Dequantise positions [start, start+count) of sequence b: the inverse of
 * the append's steps (codebook centroid times radius, inverse rotation; the
 * wis-web.com article's PolarQuant paragraph), optionally with the QJL
 * correction of the problem statement's estimator, written out as a vector.
 *   k_out, v_out  device fp32 [count][n_kv][d]; either may be NULL
 *   flags         TQ_DEQ_QJL: keys return x_tilde = x_hat + rho sqrt(pi/2)/m
 *                 R^T S^T sign, whose inner product with q is the estimator
 * Fails with TQ_EINVAL when start + count > max_ctx. */
tq_status tq_dequantize(const tq_config* cfg, const void* params, const void* k_cache,
                        const void* v_cache, int32_t b, int32_t start, int32_t count,
                        float* k_out, float* v_out, uint32_t flags, void* stream);

/* Measurement helper, not part of the method: a plain streaming read of
 * `bytes` of device memory (16-byte non-temporal loads over the whole grid),
 * the practical HBM read ceiling that decode throughput is reported against
 * beside the published peak.  XORs every 32-bit word of the range into *sink
 * (XOR, so the result is exact whatever the schedule; the caller sets *sink
 * first, e.g. to 0).
 *   src    device, 16-byte aligned, read only
 *   bytes  a multiple of 16 (0: nothing is launched)
 *   sink   device uint32, 4-byte aligned
 * Fails with TQ_EINVAL on a null pointer, misalignment or a ragged length;
 * TQ_EDEVICE if the launch fails.  Asynchronous on `stream`. */
tq_status tq_stream_read(const void* src, uint64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
