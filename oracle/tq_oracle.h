/*
 * tq_oracle.h -- CPU oracle for the TurboQuant KV-cache path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this code.  The product library
 * never links it and shares no code, header, table or constant generator
 * with it.
 *
 * Plain, single-threaded C99.  Floating point is fp64 except where the
 * stored format fixes a narrower precision (the fp32 rotation, the fp32
 * decision products, the fp16 norm fields), and then the oracle performs
 * exactly the operations the format defines.
 *
 * Sources (web pages, cited by title and passage):
 *  [P1] wis-web.com reader, article on TurboQuant in a llama.cpp fork:
 *       the "D'abord PolarQuant" paragraph (Walsh-Hadamard rotation that
 *       gaussianises the vectors), the paragraph on the Cartesian-to-polar
 *       step (radius + angle, the angle's distribution known in advance),
 *       the QJL paragraph (a 1-bit corrector that removes the residual bias
 *       with no stored quantisation constants), the llama-server example
 *       (separate K and V cache types, flash attention on) and the finding
 *       that keeps K in q8_0.
 *  [P2] leviatan.io, "TurboQuant : 6x moins de cache, jusqu'a 8x plus
 *       rapide": section "Principe de quantification sans calibration"
 *       (fixed, data-oblivious transform, no calibration).
 * Where the pages are silent the oracle takes the plainest reading; each
 * reading is restated at the function that applies it.  The QJL estimator
 * follows from the identity E[sign(<s,r>) <s,q>] = sqrt(2/pi) <q,r>/|r|
 * for s ~ N(0, I): <q,r> ~ |r| sqrt(pi/2)/m sum_j sign(<S_j,r>) <S_j,q>.
 */
#ifndef TQ_ORACLE_H
#define TQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- codec identifiers (same numbering as the public ABI, restated) ---- */
enum { OR_RAW_F32 = 0, OR_POLAR = 1, OR_POLAR_QJL = 2, OR_Q8_BLOCK32 = 3, OR_POLAR_TREE = 4 };
enum { OR_BLOCK = 128 };   /* tokens per cache block */

/* ---- fp16 ---- */
uint16_t or_f32_to_f16(float f);       /* IEEE binary16, round to nearest even */
float    or_f16_to_f32(uint16_t h);
uint16_t or_norm_to_f16(float n);      /* min(n, 65504) then RNE (norm fields saturate) */

/* ---- counter-based SplitMix64 (Steele, Lea, Flood, OOPSLA 2014) ---- */
uint64_t or_splitmix64_mix(uint64_t z);
/* element k (0-based) of the SplitMix64 sequence whose state starts at s0 */
uint64_t or_splitmix64_at(uint64_t s0, uint64_t k);
/* random stream `stream` of layer `layer`: key = element (layer*256+stream)
 * of the sequence seeded with `seed`; value k = element k of the sequence
 * seeded with key. */
uint64_t or_stream_u64(uint64_t seed, int32_t layer, uint32_t stream, uint64_t k);
/* D (+/-1 as float) for stream 0 (K) or 1 (V); S (m x d, row-major fp32)
 * from stream 2 by Box-Muller on 53-bit uniforms. */
void or_make_signs(uint64_t seed, int32_t layer, uint32_t stream, int d, float* D);
void or_make_sketch(uint64_t seed, int32_t layer, int m, int d, float* S);

/* ---- codebook: Lloyd-Max for the standardised coordinate of a rotated
 *      vector, density prop. to (1 - t^2/d)^((d-3)/2) on |t| < sqrt(d) ---- */
/* cent64[2^b]: fp64 optimum; c16[2^b]: fp16 bits; bounds[2^b-1]: fp32
 * midpoints of adjacent fp16 centroids; *mse: E[(t - Q(t))^2] with the fp64
 * optimum.  Returns the number of Lloyd iterations, or -1 on bad args. */
int or_codebook(int d, int b, double* cent64, uint16_t* c16, float* bounds, double* mse);
/* density integrals on [a, c] (composite Simpson), exposed for the tests */
double or_marginal_mass(int d, double a, double c);
double or_marginal_moment1(int d, double a, double c);

/* ---- rotation ---- */
void or_fwht_f32(float* x, int d);     /* raw Sylvester H_d, stages h = 1,2,..,d/2 */
void or_fwht_f64(double* x, int d);
double or_tree_sumsq_f32(const float* x, int d);  /* fp64 pairwise tree, see .c */

/* ---- per-vector quantisers ---- */
/* POLAR / POLAR_QJL on one fp32 vector.  For POLAR pass m = 0, S = NULL.
 * Outputs: codes[d] (0..2^b-1), *n16, and for QJL signs[m] (0/1), *rho16.
 * Optional diagnostics (may be NULL): tmargin[d] = min_j |y_i/n - B_j|,
 * z[m] = fp64 sketch values, *rrot = |r| in the rotated frame. */
void or_quantize_polar(const float* x, int d, int b, const float* D,
                       const uint16_t* c16, const float* bounds,
                       int m, const float* S,
                       uint8_t* codes, uint16_t* n16, uint8_t* signs, uint16_t* rho16,
                       double* tmargin, double* z, double* rrot);
/* 8-bit symmetric per-32 block: s16[d/32], k8[d]; optional qmargin[d] =
 * |x/s - (k + 1/2)| distance of x/s to the nearest rounding tie. */
void or_quantize_q8(const float* x, int d, int8_t* k8, uint16_t* s16, double* qmargin);

/* ---- per-vector dequantisers (fp64) ---- */
void or_dequant_polar(int d, const float* D, const uint16_t* c16,
                      const uint8_t* codes, uint16_t n16, double* out);
/* QJL-corrected key: x_hat + rho sqrt(pi/2)/m * D.H.(S^T sigma)/sqrt(d) */
void or_dequant_polar_qjl(int d, int m, const float* D, const uint16_t* c16, const float* S,
                          const uint8_t* codes, uint16_t n16, const uint8_t* signs,
                          uint16_t rho16, double* out);
void or_dequant_q8(int d, const int8_t* k8, const uint16_t* s16, double* out);

/* ---- recursive polar codec (POLAR_TREE): one radius and d - 1 angles in
 *      heap slots 1..d-1 (slot d/2 + i = level-1 pair i, slot 2^(L-l) + k =
 *      node k of level l); see the .c file for the reading ---- */
typedef struct {
  int d, b, levels;
  int bits[13];            /* per level 1..levels */
  double cent[13][256];    /* centroids per level, increasing */
  double bnd[13][255];     /* decision boundaries per level */
} or_tree_tab;
/* angle law of level l >= 2: density prop. to sin(2 theta)^(2^(l-1)-1) on [0, pi/2] */
double or_angle_mass(int level, double a, double c);
double or_angle_moment1(int level, double a, double c);
int or_angle_codebook(int level, int bits, double* cent, double* bounds, double* mse);
double or_tree_angles(const double* y, int d, double* ang);
void or_tree_from_angles(const double* ang, double r, int d, double* y);
void or_tree_tables(int d, int b, or_tree_tab* T);
void or_quantize_tree(const float* x, int d, const float* D, const or_tree_tab* T,
                      uint8_t* codes, uint16_t* n16, double* amargin);
void or_dequant_tree(int d, const float* D, const or_tree_tab* T, const uint8_t* codes,
                     uint16_t n16, double* out);
/* tables for b = 2..4 at d = 128 used by the whole-cache helpers; prepare
 * once before any other call (not thread-safe), then read-only */
void or_tree_prepare(void);
const or_tree_tab* or_tree_table(int b);

/* ---- whole-cache helpers ---------------------------------------------
 * A "layer spec" describes one layer's cache: the codecs and sizes.  All
 * arrays are host memory.  Unpacked record arrays are indexed
 * [batch][pos][kv_head][...]. */
typedef struct {
  int32_t d, n_q, n_kv, batch, max_ctx;
  int32_t k_codec, k_bits, m;
  int32_t v_codec, v_bits;
} or_spec;

int64_t or_k_record_bytes(const or_spec* s);
int64_t or_v_record_bytes(const or_spec* s);
int64_t or_k_block_bytes(const or_spec* s);
int64_t or_v_block_bytes(const or_spec* s);
int64_t or_k_cache_bytes(const or_spec* s);
int64_t or_v_cache_bytes(const or_spec* s);

/* Unpacked K record store (host).  Fields used depend on k_codec. */
typedef struct {
  uint8_t*  codes;   /* [n][d]   POLAR, POLAR_QJL */
  uint16_t* n16;     /* [n]      */
  uint8_t*  signs;   /* [n][m]   POLAR_QJL */
  uint16_t* rho16;   /* [n]      POLAR_QJL */
  int8_t*   k8;      /* [n][d]   Q8 */
  uint16_t* s16;     /* [n][d/32] Q8 */
  float*    raw;     /* [n][d]   RAW_F32 */
} or_krec;
typedef struct {
  uint8_t*  codes;   /* [n][d]   POLAR */
  uint16_t* n16;     /* [n] */
  float*    raw;     /* [n][d]   RAW_F32 */
} or_vrec;

/* Quantise n vectors x[n][d] into unpacked K (or V) records. */
void or_quantize_k_many(const or_spec* s, const float* DK, const uint16_t* c16,
                        const float* bounds, const float* S, int64_t n,
                        const float* x, or_krec* out, int64_t out_off);
void or_quantize_v_many(const or_spec* s, const float* DV, const uint16_t* c16,
                        const float* bounds, int64_t n, const float* x,
                        or_vrec* out, int64_t out_off);

/* Pack / unpack one record (index rec = (b*max_ctx + pos)*n_kv + h) into / from
 * the cache byte image. */
void or_pack_k(const or_spec* s, int b, int pos, int h, const or_krec* r, int64_t rec, uint8_t* kc);
void or_unpack_k(const or_spec* s, int b, int pos, int h, const uint8_t* kc, or_krec* r, int64_t rec);
void or_pack_v(const or_spec* s, int b, int pos, int h, const or_vrec* r, int64_t rec, uint8_t* vc);
void or_unpack_v(const or_spec* s, int b, int pos, int h, const uint8_t* vc, or_vrec* r, int64_t rec);

/* Decode attention for one sequence b and one query head hq, in fp64, from
 * unpacked records: dequantise every key and value, logits =
 * (<q, x_hat> + rho sqrt(pi/2)/m <S R q, sigma>)/sqrt(d), softmax, weighted
 * sum.  q[d] fp32; out[d] fp64; logits_out[len] fp64 or NULL. */
void or_decode_head(const or_spec* s, const float* DK, const float* DV, const uint16_t* ck16,
                    const uint16_t* cv16, const float* S, const or_krec* kr, const or_vrec* vr,
                    int b, int hq, int len, const float* q, double* out, double* logits_out);

/* array forms of the fp16 conversions (for the tests) */
void or_f32_to_f16_array(const float* x, uint16_t* out, int64_t n);
void or_f16_to_f32_array(const uint16_t* x, float* out, int64_t n);

/* Whole-cache helpers: pack / unpack positions [0, lens[b]) of every
 * sequence and kv head; decode the listed (b, hq) pairs (n_pairs of them,
 * pairs[2k] = b, pairs[2k+1] = hq) with out[k][d] and logits[k][max_ctx]. */
void or_pack_cache(const or_spec* s, const int32_t* lens, const or_krec* kr, const or_vrec* vr,
                   uint8_t* kc, uint8_t* vc);
void or_unpack_cache(const or_spec* s, const int32_t* lens, const uint8_t* kc, const uint8_t* vc,
                     or_krec* kr, or_vrec* vr);
void or_decode_pairs(const or_spec* s, const float* DK, const float* DV, const uint16_t* ck16,
                     const uint16_t* cv16, const float* S, const or_krec* kr, const or_vrec* vr,
                     const int32_t* lens, const float* q /* [batch][n_q][d] */,
                     int n_pairs, const int32_t* pairs, double* out, double* logits);

#ifdef __cplusplus
}
#endif
#endif
