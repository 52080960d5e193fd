// tq_host.cpp -- host side of the C ABI declared in include/tq.h:
// argument checks, sizes, per-layer parameter generation and kernel launches.
//
// Parameters (wis-web.com reader, TurboQuant article: the PolarQuant
// paragraph's rotation "pour gaussianiser" and the angle law "connue a
// l'avance"; leviatan.io, "Principe de quantification sans calibration": a
// fixed, data-independent transform):
//   * rotation signs D_K, D_V and the Gaussian sketch S come from
//     counter-form SplitMix64 (Steele, Lea & Flood, OOPSLA 2014) keyed by
//     (seed, layer, stream), with Box-Muller for the Gaussians;
//   * the codebook is the Lloyd-Max quantiser of the coordinate law of a
//     uniformly random unit vector scaled by sqrt(d), density proportional to
//     (1 - t^2/d)^((d-3)/2); centroids are stored as fp16-exact values and
//     the decision boundaries as the fp32 midpoints of adjacent centroids;
//   * the recursive polar codec (the article's radius + angle step taken
//     literally, pairwise and level by level) quantises level-1 angles
//     uniformly on the circle and the angles of level l >= 2, whose law is
//     proportional to sin(2 theta)^(2^(l-1) - 1) on [0, pi/2], with their
//     Lloyd-Max codebooks.
// Integrals use composite 16-point Gauss-Legendre quadrature.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/tq.h"
#include "tq_internal.h"

namespace {

using tq::kBlock;
using tq::kD;
using tq::kM;

// ------------------------------------------------------------- checks

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

tq_status check_cfg(const tq_config* c) {
  if (c == nullptr) return TQ_EINVAL;
  if (c->abi_version != TQ_ABI_VERSION || c->sparse_v < 0 || c->sparse_v > 60) return TQ_EINVAL;
  if (!is_pow2(c->head_dim) || c->head_dim < 16 || c->head_dim > 256) return TQ_EINVAL;
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads != 0) return TQ_EINVAL;
  if (c->batch < 1 || c->max_ctx < 1) return TQ_EINVAL;
  if (c->decode_chunk < 0 || c->decode_chunk % kBlock != 0) return TQ_EINVAL;
  switch (c->k_codec) {
    case TQ_CODEC_RAW_F32:
      if (c->k_bits != 32 || c->qjl_m != 0) return TQ_EINVAL;
      break;
    case TQ_CODEC_POLAR:
    case TQ_CODEC_POLAR_QJL:
      if (c->k_bits < 1 || c->k_bits > 8) return TQ_EINVAL;
      if (c->k_codec == TQ_CODEC_POLAR_QJL) {
        if (c->qjl_m <= 0 || c->qjl_m % 64 != 0) return TQ_EINVAL;
      } else if (c->qjl_m != 0) {
        return TQ_EINVAL;
      }
      break;
    case TQ_CODEC_Q8_BLOCK32:
      if (c->k_bits != 8 || c->qjl_m != 0) return TQ_EINVAL;
      break;
    case TQ_CODEC_POLAR_TREE:
      if (c->k_bits < 2 || c->k_bits > 8 || c->qjl_m != 0) return TQ_EINVAL;
      break;
    default:
      return TQ_EINVAL;
  }
  switch (c->v_codec) {
    case TQ_CODEC_RAW_F32:
      if (c->v_bits != 32) return TQ_EINVAL;
      break;
    case TQ_CODEC_POLAR:
      if (c->v_bits < 1 || c->v_bits > 8) return TQ_EINVAL;
      break;
    case TQ_CODEC_POLAR_TREE:
      if (c->v_bits < 2 || c->v_bits > 8) return TQ_EINVAL;
      break;
    case TQ_CODEC_POLAR_QJL:
    case TQ_CODEC_Q8_BLOCK32:
      return TQ_EUNSUPPORTED;   // QJL corrects inner products: keys only; q8 is a key format
    default:
      return TQ_EINVAL;
  }
  // well formed; now what the kernels serve
  if (c->head_dim != kD) return TQ_EUNSUPPORTED;
  if (c->n_q_heads / c->n_kv_heads > tq::kMaxGroup) return TQ_EUNSUPPORTED;
  if ((c->k_codec == TQ_CODEC_POLAR || c->k_codec == TQ_CODEC_POLAR_QJL) &&
      (c->k_bits < 2 || c->k_bits > 4))
    return TQ_EUNSUPPORTED;
  if (c->k_codec == TQ_CODEC_POLAR_QJL && c->qjl_m != kM) return TQ_EUNSUPPORTED;
  if (c->v_codec == TQ_CODEC_POLAR && (c->v_bits < 2 || c->v_bits > 4)) return TQ_EUNSUPPORTED;
  if (c->k_codec == TQ_CODEC_POLAR_TREE && c->k_bits > 4) return TQ_EUNSUPPORTED;
  if (c->v_codec == TQ_CODEC_POLAR_TREE && c->v_bits > 4) return TQ_EUNSUPPORTED;
  return TQ_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int n_blocks(const tq_config* c) { return (c->max_ctx + kBlock - 1) / kBlock; }

int64_t k_record_bytes(const tq_config* c) {
  const int64_t d = c->head_dim;
  switch (c->k_codec) {
    case TQ_CODEC_RAW_F32: return 4 * d;
    case TQ_CODEC_POLAR:
    case TQ_CODEC_POLAR_TREE: return c->k_bits * d / 8 + 2;
    case TQ_CODEC_POLAR_QJL: return c->k_bits * d / 8 + c->qjl_m / 8 + 4;
    default: return d + 2 * (d / 32);
  }
}
int64_t v_record_bytes(const tq_config* c) {
  const int64_t d = c->head_dim;
  return c->v_codec == TQ_CODEC_RAW_F32 ? 4 * d : c->v_bits * d / 8 + 2;
}

int qjl_rows(const tq_config* c) { return c->k_codec == TQ_CODEC_POLAR_QJL ? c->qjl_m : 0; }

// --------------------------------------------------------------- PRNG

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

// Output k (0-based) of a SplitMix64 generator whose state starts at s.
uint64_t splitmix_nth(uint64_t s, uint64_t k) { return mix64(s + (k + 1) * kGamma); }

struct Stream {
  uint64_t key;
  Stream(uint64_t seed, int32_t layer, uint32_t id)
      : key(splitmix_nth(seed, (static_cast<uint64_t>(static_cast<uint32_t>(layer)) << 8) + id)) {}
  uint64_t operator()(uint64_t k) const { return splitmix_nth(key, k); }
};

void fill_signs(const Stream& st, int d, float* out) {
  for (int i = 0; i < d; ++i) out[i] = (st(i) >> 63) ? -1.0f : 1.0f;
}

void fill_sketch(const Stream& st, int m, int d, float* S) {
  const double two_pi = 6.283185307179586;
  const double scale53 = 1.0 / 9007199254740992.0;
  for (int j = 0; j < m; ++j) {
    for (int i = 0; i < d; ++i) {
      const uint64_t e = static_cast<uint64_t>(j) * d + i;
      const double u1 = static_cast<double>((st(2 * e) >> 11) + 1) * scale53;
      const double u2 = static_cast<double>(st(2 * e + 1) >> 11) * scale53;
      S[static_cast<size_t>(j) * d + i] = static_cast<float>(std::sqrt(-2.0 * std::log(u1)) * std::cos(two_pi * u2));
    }
  }
}

// ------------------------------------------------------------ codebook

struct GaussLegendre16 {
  double x[16], w[16];
  GaussLegendre16() {
    const int n = 16;
    for (int k = 0; k < n / 2; ++k) {
      double z = std::cos(M_PI * (k + 0.75) / (n + 0.5));
      double dp = 0.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int j = 2; j <= n; ++j) {
          const double p2 = ((2.0 * j - 1.0) * z * p1 - (j - 1.0) * p0) / j;
          p0 = p1;
          p1 = p2;
        }
        dp = n * (z * p1 - p0) / (z * z - 1.0);
        const double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) break;
      }
      x[k] = -z;
      x[n - 1 - k] = z;
      w[k] = w[n - 1 - k] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

struct Codebook {
  float centroids[16];
  float bounds[16];
  float coeffs[8];   // odd multilinear coefficients, see multilinear_coeffs
};

// A symmetric sorted codebook is an odd function of the code's bits read as
// signs s_k = 2 bit_k - 1, so C[c] = sum_T a_T prod_{k in T} s_k over the odd
// subsets T of the bit positions.  Order: singletons {0}..{b-1}, then (b = 3)
// {0,1,2}, (b = 4) {0,1,2}, {0,1,3}, {0,2,3}, {1,2,3}.  a_T = 2^-b sum_c C[c]
// prod_T s_k(c); with fp16-exact centroids these are exact in fp32.
void multilinear_coeffs(int bits, const float* centroids, float* out) {
  static const int triples[4][3] = {{0, 1, 2}, {0, 1, 3}, {0, 2, 3}, {1, 2, 3}};
  const int levels = 1 << bits;
  int n_terms = bits + (bits == 3 ? 1 : (bits == 4 ? 4 : 0));
  for (int T = 0; T < 8; ++T) out[T] = 0.0f;
  for (int T = 0; T < n_terms; ++T) {
    double acc = 0.0;
    for (int c = 0; c < levels; ++c) {
      auto s = [&](int k) { return ((c >> k) & 1) ? 1.0 : -1.0; };
      const double prod = (T < bits) ? s(T) : s(triples[T - bits][0]) * s(triples[T - bits][1]) * s(triples[T - bits][2]);
      acc += centroids[c] * prod;
    }
    out[T] = static_cast<float>(acc / levels);
  }
}

// int_a^c t^moment (1 - t^2/d)^((d-3)/2) dt, 48 panels of 16-point Gauss-Legendre
double law_integral(int d, double a, double c, int moment) {
  static const GaussLegendre16 gl;
  const int panels = 48;
  const double hw = (c - a) / panels;
  const double ex = 0.5 * (d - 3);
  double total = 0.0;
  for (int p = 0; p < panels; ++p) {
    const double mid = a + (p + 0.5) * hw;
    double s = 0.0;
    for (int k = 0; k < 16; ++k) {
      const double t = mid + 0.5 * hw * gl.x[k];
      const double base = 1.0 - t * t / d;
      if (base <= 0.0) continue;
      double f = std::pow(base, ex);
      if (moment == 1) f *= t;
      s += gl.w[k] * f;
    }
    total += 0.5 * hw * s;
  }
  return total;
}

Codebook make_codebook(int d, int bits) {
  static std::mutex mu;
  static std::map<std::pair<int, int>, Codebook> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({d, bits});
  if (it != cache.end()) return it->second;

  const int half = 1 << (bits - 1);
  const double top = std::min(std::sqrt(static_cast<double>(d)), 16.0);
  std::vector<double> c(half), edge(half + 1);
  for (int k = 0; k < half; ++k) c[k] = 3.0 * (k + 0.5) / half;   // positive half; symmetric law
  for (int round = 0; round < 100000; ++round) {
    edge[0] = 0.0;
    for (int k = 1; k < half; ++k) edge[k] = 0.5 * (c[k - 1] + c[k]);
    edge[half] = top;
    double moved = 0.0;
    for (int k = 0; k < half; ++k) {
      const double nc = law_integral(d, edge[k], edge[k + 1], 1) / law_integral(d, edge[k], edge[k + 1], 0);
      moved = std::max(moved, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    if (moved <= 1e-13) break;
  }
  Codebook cb{};
  const int levels = 2 * half;
  for (int k = 0; k < half; ++k) {
    const float pos = static_cast<float>(static_cast<_Float16>(c[k]));   // one RNE rounding to fp16
    cb.centroids[half + k] = pos;
    cb.centroids[half - 1 - k] = -pos;
  }
  for (int j = 0; j + 1 < levels; ++j) cb.bounds[j] = 0.5f * (cb.centroids[j] + cb.centroids[j + 1]);
  if (bits >= 2 && bits <= 4) multilinear_coeffs(bits, cb.centroids, cb.coeffs);
  cache[{d, bits}] = cb;
  return cb;
}

// ------------------------------------------- recursive polar codebooks

// int_a^c t^moment sin(2t)^(2^(level-1) - 1) dt, 32 panels of 16-point Gauss-Legendre
double angle_integral(int level, double a, double c, int moment) {
  static const GaussLegendre16 gl;
  const int panels = 32;
  const double hw = (c - a) / panels;
  const int ex = (1 << (level - 1)) - 1;
  double total = 0.0;
  for (int p = 0; p < panels; ++p) {
    const double mid = a + (p + 0.5) * hw;
    double s = 0.0;
    for (int k = 0; k < 16; ++k) {
      const double t = mid + 0.5 * hw * gl.x[k];
      double f = 1.0;
      const double sv = std::sin(2.0 * t);
      for (int e = 0; e < ex; ++e) f *= sv;
      if (moment == 1) f *= t;
      s += gl.w[k] * f;
    }
    total += 0.5 * hw * s;
  }
  return total;
}

// Lloyd-Max centroids (increasing) and boundaries of the level-l angle law
// on [0, pi/2] with 2^bits codes; the law is symmetric about pi/4, so the
// lower half is iterated and mirrored.
void angle_lloyd(int level, int bits, double* cent, double* bnd) {
  const int n = 1 << bits, half = n / 2;
  const double q = 0.25 * M_PI;
  std::vector<double> c(half), e(half + 1);
  for (int k = 0; k < half; ++k) c[k] = q * (k + 0.5) / half;
  for (int round = 0; round < 100000; ++round) {
    e[0] = 0.0;
    for (int k = 1; k < half; ++k) e[k] = 0.5 * (c[k - 1] + c[k]);
    e[half] = q;
    double moved = 0.0;
    for (int k = 0; k < half; ++k) {
      const double nc = angle_integral(level, e[k], e[k + 1], 1) / angle_integral(level, e[k], e[k + 1], 0);
      moved = std::max(moved, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    if (moved <= 1e-13) break;
  }
  for (int k = 0; k < half; ++k) {
    cent[k] = c[k];
    cent[n - 1 - k] = 2.0 * q - c[k];
  }
  for (int j = 0; j + 1 < n; ++j) bnd[j] = (j == half - 1) ? q : 0.5 * (cent[j] + cent[j + 1]);
}

tq::TreeTab make_tree_tab(int bits) {
  static std::mutex mu;
  static std::map<int, tq::TreeTab> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(bits);
  if (it != cache.end()) return it->second;
  tq::TreeTab t{};
  // level 1: 2^(bits+1) cells of the circle; a quadrant holds 2^(bits-1)
  const int n1 = 1 << (bits + 1), per_q = n1 / 4;
  for (int c = 0; c < n1; ++c) {
    const double th = (c + 0.5) * 2.0 * M_PI / n1;
    t.cs1[c] = make_float2(static_cast<float>(std::cos(th)), static_cast<float>(std::sin(th)));
  }
  // a boundary at pi/4 gets cos^2 = sin^2 = 1/2 exactly, so that an angle on
  // it (equal radii) goes to the lower cell like any other tie
  for (int j = 0; j + 1 < per_q; ++j) {
    const double beta = (j + 1) * 0.5 * M_PI / per_q;
    const bool mid = 2 * (j + 1) == per_q;
    t.c2_1[j] = mid ? 0.5 : std::cos(beta) * std::cos(beta);
    t.s2_1[j] = mid ? 0.5 : std::sin(beta) * std::sin(beta);
  }
  // levels 2..7: 2^(bits-1) codes each
  const int nl = 1 << (bits - 1);
  for (int l = 2; l <= 7; ++l) {
    double cent[8], bnd[7];
    angle_lloyd(l, bits - 1, cent, bnd);
    for (int c = 0; c < nl; ++c) t.cs[l][c] = make_float2(static_cast<float>(std::cos(cent[c])), static_cast<float>(std::sin(cent[c])));
    for (int j = 0; j + 1 < nl; ++j) {
      const bool mid = 2 * (j + 1) == nl;   // the symmetric codebook's middle boundary is pi/4
      t.c2[l][j] = mid ? 0.5 : std::cos(bnd[j]) * std::cos(bnd[j]);
      t.s2[l][j] = mid ? 0.5 : std::sin(bnd[j]) * std::sin(bnd[j]);
    }
  }
  cache[bits] = t;
  return t;
}

// ------------------------------------------------------- params image

void build_params(const tq_config* c, uint8_t* img) {
  const int d = c->head_dim;
  const int m = qjl_rows(c);
  const tq::ParamsLayout L = tq::params_layout(d, m);
  std::memset(img, 0, L.total);
  fill_signs(Stream(c->seed, c->layer, 0), d, reinterpret_cast<float*>(img + L.dk));
  fill_signs(Stream(c->seed, c->layer, 1), d, reinterpret_cast<float*>(img + L.dv));
  if (m > 0) {
    float* S = reinterpret_cast<float*>(img + L.s);
    float* ST = reinterpret_cast<float*>(img + L.st);
    fill_sketch(Stream(c->seed, c->layer, 2), m, d, S);
    for (int j = 0; j < m; ++j)
      for (int i = 0; i < d; ++i) ST[static_cast<size_t>(i) * m + j] = S[static_cast<size_t>(j) * d + i];
    // S q_raw / sqrt d = (S H D_K / sqrt d) q: row j of S H is the raw FWHT of
    // row j of S (H is symmetric); fp64 throughout, one rounding to fp32
    const float* DK = reinterpret_cast<const float*>(img + L.dk);
    float* SHD = reinterpret_cast<float*>(img + L.shd);
    std::vector<double> row(d);
    const double inv_sqrt_d = 1.0 / std::sqrt(static_cast<double>(d));
    for (int j = 0; j < m; ++j) {
      for (int i = 0; i < d; ++i) row[i] = S[static_cast<size_t>(j) * d + i];
      for (int h = 1; h < d; h <<= 1)
        for (int i = 0; i < d; i += 2 * h)
          for (int k = i; k < i + h; ++k) {
            const double x = row[k], y = row[k + h];
            row[k] = x + y;
            row[k + h] = x - y;
          }
      for (int i = 0; i < d; ++i)
        SHD[static_cast<size_t>(i) * m + j] = static_cast<float>(row[i] * DK[i] * inv_sqrt_d);
    }
  }
  if (c->k_codec == TQ_CODEC_POLAR || c->k_codec == TQ_CODEC_POLAR_QJL) {
    const Codebook cb = make_codebook(d, c->k_bits);
    std::memcpy(img + L.ck, cb.centroids, 64);
    std::memcpy(img + L.kb, cb.bounds, 64);
    std::memcpy(img + L.ak, cb.coeffs, 32);
  }
  if (c->v_codec == TQ_CODEC_POLAR) {
    const Codebook cb = make_codebook(d, c->v_bits);
    std::memcpy(img + L.cv, cb.centroids, 64);
    std::memcpy(img + L.vb, cb.bounds, 64);
    std::memcpy(img + L.av, cb.coeffs, 32);
  }
  if (c->k_codec == TQ_CODEC_POLAR_TREE) {
    const tq::TreeTab t = make_tree_tab(c->k_bits);
    std::memcpy(img + L.tk, &t, sizeof t);
  }
  if (c->v_codec == TQ_CODEC_POLAR_TREE) {
    const tq::TreeTab t = make_tree_tab(c->v_bits);
    std::memcpy(img + L.tv, &t, sizeof t);
  }
}

tq::Tables tables(const tq_config* c, const void* params) {
  const tq::ParamsLayout L = tq::params_layout(c->head_dim, qjl_rows(c));
  const uint8_t* p = static_cast<const uint8_t*>(params);
  tq::Tables t;
  t.dk = reinterpret_cast<const float*>(p + L.dk);
  t.dv = reinterpret_cast<const float*>(p + L.dv);
  t.s = reinterpret_cast<const float*>(p + L.s);
  t.st = reinterpret_cast<const float*>(p + L.st);
  t.ck = reinterpret_cast<const float*>(p + L.ck);
  t.kb = reinterpret_cast<const float*>(p + L.kb);
  t.cv = reinterpret_cast<const float*>(p + L.cv);
  t.vb = reinterpret_cast<const float*>(p + L.vb);
  t.ak = reinterpret_cast<const float*>(p + L.ak);
  t.av = reinterpret_cast<const float*>(p + L.av);
  t.shd = reinterpret_cast<const float*>(p + L.shd);
  t.tk = reinterpret_cast<const tq::TreeTab*>(p + L.tk);
  t.tv = reinterpret_cast<const tq::TreeTab*>(p + L.tv);
  return t;
}

// Register-streamed matrix-core decode (POLAR / POLAR_QJL keys, POLAR values).
bool reg_path(const tq_config* c) {
  return tq::decode_reg_applies(c->k_codec, c->v_codec, c->n_q_heads / c->n_kv_heads);
}

// q8 keys with more than four query heads per KV head: one workgroup serves
// every head group of its KV head from one shared-memory ring.
bool q8_path(const tq_config* c) {
  return tq::decode_q8_applies(c->k_codec, c->v_codec, c->n_q_heads / c->n_kv_heads, c->v_bits);
}

// Ring-staged matrix-core decode: the other codecs it serves (q8 keys).
bool mfma_path(const tq_config* c) {
  return !reg_path(c) && !q8_path(c) && tq::decode_mfma_applies(c->k_codec, c->v_codec, c->n_q_heads / c->n_kv_heads);
}

// Independent (sequence, KV head, head group) units the splits multiply: the
// matrix-core kernel serves up to four query heads per workgroup.
int64_t split_units(const tq_config* c) {
  const int64_t groups = (mfma_path(c) || reg_path(c)) ? (c->n_q_heads / c->n_kv_heads + 3) / 4 : 1;
  return static_cast<int64_t>(c->batch) * c->n_kv_heads * groups;
}

// Blocks per split when the grid aims at `target` workgroups, the number the
// chip holds at once: the split count rounds down, so that a grid never has a
// few workgroups left for a second round (with three head groups per KV head,
// 22 splits x 24 units would be 528 workgroups of the same length for 512
// places: the last 16 would start when the first finish, doubling the launch).
int chunk_blocks_for(const tq_config* c, int32_t max_seq_len, int64_t target) {
  const int blocks = std::max(1, (max_seq_len + kBlock - 1) / kBlock);
  if (c->decode_chunk > 0) return c->decode_chunk / kBlock;
  const int64_t pairs = split_units(c);
  const int64_t want_splits = std::max<int64_t>(1, target / pairs);
  const int64_t chunk = std::max<int64_t>(1, (blocks + want_splits - 1) / want_splits);
  // the register-streamed kernel's per-split costs (query operands, the
  // first loads' latency, partials, merge) want a few steps to spread over
  return static_cast<int>(reg_path(c) ? std::max<int64_t>(chunk, tq::kRegMinChunkBlocks) : chunk);
}

// Block groups (of four wavefronts, one block each per step) per workgroup
// of the matrix-core kernel.  q8 keys take one group: their large blocks leave
// a two-group ring too shallow.  Four-bit values take one group once a
// two-group workgroup would run 8 or more steps (two workgroups per compute
// unit then hide each other's stalls; with fewer steps the doubled set-up and
// merge cost more).  Measured with 4-bit keys and values, us per launch with
// two groups / one group: 32K Llama shape 24.2 / 26.2, 16 x 8K 60.3 / 57.8,
// 1M 394 / 356.  The choice only moves
// to one group as the length grows, so the splits of a shorter call never
// exceed those of a longer one.
int mfma_groups(const tq_config* c, int32_t max_seq_len) {
  if (c->k_codec == TQ_CODEC_Q8_BLOCK32) return 1;
  if (c->v_bits != 4) return 2;
  const int cb = chunk_blocks_for(c, max_seq_len, tq::kMfmaUnitWorkgroups / 2);
  return (cb + 1) / 2 >= 8 ? 1 : 2;
}

int64_t target_workgroups(const tq_config* c, int32_t max_seq_len) {
  if (reg_path(c)) return tq::kRegWorkgroups;
  if (q8_path(c)) return tq::kComputeUnits;   // one eight- or twelve-wave workgroup per compute unit
  return mfma_path(c) ? tq::kMfmaUnitWorkgroups / mfma_groups(c, max_seq_len) : tq::kValuWorkgroups;
}

int decode_chunk_blocks(const tq_config* c, int32_t max_seq_len) {
  // aim for the kernel's workgroup count over the whole grid
  return chunk_blocks_for(c, max_seq_len, target_workgroups(c, max_seq_len));
}

int decode_splits(const tq_config* c, int32_t max_seq_len) {
  const int blocks = std::max(1, (max_seq_len + kBlock - 1) / kBlock);
  const int cb = decode_chunk_blocks(c, max_seq_len);
  return (blocks + cb - 1) / cb;
}

// Register-streamed decode with two workgroups per compute unit: the first
// dispatch round (one workgroup per unit) holds the low splits (the kernel
// numbers its units split-major), and a unit's first workgroup runs ahead of
// its second, so those splits take about kRegLongSplitPermille / 1000 times
// the blocks of the later ones and both finish together.  Sets a's split
// ranges; the split count and so the workspace stay as decode_splits says.
void set_split_ranges(const tq_config* c, int32_t max_seq_len, tq::DecodeArgs* a) {
  a->long_blocks = 0;
  a->n_long = 0;
  if (!reg_path(c) || c->decode_chunk > 0) return;
  const int64_t units = split_units(c);
  const int64_t S = a->n_splits;
  const int64_t n_long = tq::kComputeUnits / units;
  if (n_long < 1 || n_long >= S) return;   // one round: every split equal
  const int64_t B = std::max(1, (max_seq_len + kBlock - 1) / kBlock);
  const int64_t P = tq::kRegLongSplitPermille;
  const int64_t shrt = std::max<int64_t>(1, B * 1000 / (n_long * P + (S - n_long) * 1000));
  const int64_t lng = std::max<int64_t>(shrt, (B - (S - n_long) * shrt + n_long - 1) / n_long);
  a->chunk_blocks = static_cast<int32_t>(shrt);
  a->long_blocks = static_cast<int32_t>(lng);
  a->n_long = static_cast<int32_t>(n_long);
}

// Block groups per workgroup of the register-streamed decode: when the grid
// holds at most one workgroup per compute unit, each workgroup takes eight
// waves in two block groups (alternate blocks of its split, one query set-up),
// so that two waves share each SIMD; otherwise two four-wave workgroups do.
int reg_groups(const tq_config* c, int splits) {
  return static_cast<int64_t>(splits) * split_units(c) <= tq::kComputeUnits ? 2 : 1;
}

// Largest split count of any call with lengths up to max_seq_len (the
// automatic chunking is not monotonic in the length), for workspace sizing.
int decode_splits_bound(const tq_config* c, int32_t max_seq_len) {
  const int blocks = std::max(1, (max_seq_len + kBlock - 1) / kBlock);
  if (c->decode_chunk > 0) return (blocks + c->decode_chunk / kBlock - 1) / (c->decode_chunk / kBlock);
  const int64_t pairs = split_units(c);
  const int64_t target = target_workgroups(c, max_seq_len);   // no shorter call aims higher
  const int64_t want_splits = std::max<int64_t>(1, (target + pairs - 1) / pairs);
  return static_cast<int>(std::min<int64_t>(blocks, want_splits));
}

// ------------------------------------------------------ entry helpers

// The completion counters [batch][n_kv][kMaxGroup / 4] u32 come first, at a
// fixed offset (they must stay where the previous call left them at zero,
// whatever length this call decodes), then the partials
// [batch][n_q][splits][kPartialStride] fp32; each part 256-byte aligned.
uint64_t counters_bytes(const tq_config* cfg) {
  const uint64_t counters = static_cast<uint64_t>(cfg->batch) * cfg->n_kv_heads * (tq::kMaxGroup / 4) * 4;
  return (counters + 255) & ~255ull;
}

uint64_t partials_bytes(const tq_config* cfg, int32_t max_seq_len) {
  const uint64_t splits = decode_splits_bound(cfg, max_seq_len);
  const uint64_t partial = static_cast<uint64_t>(cfg->batch) * cfg->n_q_heads * splits * tq::kPartialStride * 4;
  return (partial + 255) & ~255ull;
}

uint64_t workspace_need(const tq_config* cfg, int32_t max_seq_len) {
  return counters_bytes(cfg) + partials_bytes(cfg, max_seq_len);
}

tq_status check_append(const tq_config* cfg, const void* params, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, int32_t max_seq_len, const void* k_new, const void* v_new,
                       int32_t in_dtype, int32_t n_new) {
  const tq_status st = check_cfg(cfg);
  if (st != TQ_OK) return st;
  if (n_new < 0 || max_seq_len < 0) return TQ_EINVAL;
  if (in_dtype != TQ_F32 && in_dtype != TQ_BF16 && in_dtype != TQ_F16) return TQ_EINVAL;
  if (static_cast<int64_t>(max_seq_len) + n_new > cfg->max_ctx) return TQ_ECAPACITY;
  if (n_new == 0) return TQ_OK;
  if (params == nullptr || k_cache == nullptr || v_cache == nullptr || seq_lens == nullptr ||
      k_new == nullptr || v_new == nullptr)
    return TQ_EINVAL;
  if (!aligned(params, 256) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(seq_lens, 4) ||
      !aligned(k_new, in_dtype == TQ_F32 ? 4 : 2) || !aligned(v_new, in_dtype == TQ_F32 ? 4 : 2))
    return TQ_EINVAL;
  return TQ_OK;
}

hipError_t launch_append(const tq_config* cfg, const void* params, void* k_cache, void* v_cache,
                         const int32_t* seq_lens, const void* k_new, const void* v_new, int32_t in_dtype,
                         int32_t n_new, hipStream_t stream) {
  tq::QuantArgs a{};
  a.tb = tables(cfg, params);
  a.kc = static_cast<uint8_t*>(k_cache);
  a.vc = static_cast<uint8_t*>(v_cache);
  a.seq_lens = seq_lens;
  a.k_new = k_new;
  a.v_new = v_new;
  a.in_dtype = in_dtype;
  a.batch = cfg->batch;
  a.n_kv = cfg->n_kv_heads;
  a.max_ctx = cfg->max_ctx;
  a.n_blocks = n_blocks(cfg);
  a.n_new = n_new;
  a.groups_per_seq = (n_new + 31) / 32 + 1;
  a.k_codec = cfg->k_codec;
  a.k_bits = cfg->k_bits;
  a.v_codec = cfg->v_codec;
  a.v_bits = cfg->v_bits;
  a.k_block_bytes = kBlock * k_record_bytes(cfg);
  a.v_block_bytes = kBlock * v_record_bytes(cfg);
  hipError_t e = tq::launch_quantize(a, stream);
  if (e == hipSuccess && (cfg->k_codec == TQ_CODEC_POLAR_TREE || cfg->v_codec == TQ_CODEC_POLAR_TREE))
    e = tq::launch_quantize_tree(a, stream);
  return e;
}

// Checks and kernel arguments of a decode over lengths up to max_seq_len.
// Argument checks of a decode (no workspace involved).
tq_status check_decode(const tq_config* cfg, const void* params, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, int32_t max_seq_len, const float* q, float* out, float* logits) {
  const tq_status st = check_cfg(cfg);
  if (st != TQ_OK) return st;
  if (params == nullptr || k_cache == nullptr || v_cache == nullptr || seq_lens == nullptr || q == nullptr ||
      out == nullptr)
    return TQ_EINVAL;
  if (!aligned(params, 256) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(seq_lens, 4) ||
      !aligned(q, 16) || !aligned(out, 16) || (logits && !aligned(logits, 4)))
    return TQ_EINVAL;
  if (max_seq_len < 0 || max_seq_len > cfg->max_ctx) return TQ_EINVAL;
  return TQ_OK;
}

// Kernel arguments of a decode over lengths up to max_seq_len (arguments
// already checked): the completion counters at `counters` (counters_bytes
// of them, zero between calls), the rest of the workspace at `rest`.
void fill_decode_args(const tq_config* cfg, const void* params, const void* k_cache, const void* v_cache,
                      const int32_t* seq_lens, int32_t max_seq_len, const float* q, float* out, float* logits,
                      uint32_t* counters, uint8_t* rest, tq::DecodeArgs* out_args) {
  const int splits = decode_splits(cfg, max_seq_len);
  tq::DecodeArgs& a = *out_args;
  a = tq::DecodeArgs{};
  a.tb = tables(cfg, params);
  a.kc = static_cast<const uint8_t*>(k_cache);
  a.vc = static_cast<const uint8_t*>(v_cache);
  a.seq_lens = seq_lens;
  a.q = q;
  a.out = out;
  a.logits = logits;
  a.counters = counters;
  a.partials = reinterpret_cast<float*>(rest);
  a.batch = cfg->batch;
  a.n_q = cfg->n_q_heads;
  a.n_kv = cfg->n_kv_heads;
  a.group = cfg->n_q_heads / cfg->n_kv_heads;
  a.max_ctx = cfg->max_ctx;
  a.n_blocks = n_blocks(cfg);
  a.chunk_blocks = decode_chunk_blocks(cfg, max_seq_len);
  a.n_splits = splits;
  set_split_ranges(cfg, max_seq_len, &a);
  a.groups = mfma_path(cfg) ? mfma_groups(cfg, max_seq_len) : (reg_path(cfg) ? reg_groups(cfg, splits) : 1);
  a.k_codec = cfg->k_codec;
  a.k_bits = cfg->k_bits;
  a.v_codec = cfg->v_codec;
  a.v_bits = cfg->v_bits;
  a.sparse_v = cfg->sparse_v;
  a.k_block_bytes = kBlock * k_record_bytes(cfg);
  a.v_block_bytes = kBlock * v_record_bytes(cfg);
}

// Checks and kernel arguments of a decode on a caller's workspace: counters
// at offset 0, the partials after them.
tq_status prepare_decode(const tq_config* cfg, const void* params, const void* k_cache, const void* v_cache,
                         const int32_t* seq_lens, int32_t max_seq_len, const float* q, float* out, float* logits,
                         void* workspace, uint64_t workspace_bytes, tq::DecodeArgs* out_args) {
  const tq_status st = check_decode(cfg, params, k_cache, v_cache, seq_lens, max_seq_len, q, out, logits);
  if (st != TQ_OK) return st;
  if (workspace == nullptr || !aligned(workspace, 256)) return TQ_EINVAL;
  if (workspace_bytes < workspace_need(cfg, max_seq_len)) return TQ_EWORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  fill_decode_args(cfg, params, k_cache, v_cache, seq_lens, max_seq_len, q, out, logits,
                   reinterpret_cast<uint32_t*>(ws), ws + counters_bytes(cfg), out_args);
  return TQ_OK;
}

}  // namespace

extern "C" {

const char* tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument";
    case TQ_EUNSUPPORTED: return "unsupported configuration";
    case TQ_ECAPACITY: return "append exceeds cache capacity";
    case TQ_EWORKSPACE: return "buffer too small";
    case TQ_EDEVICE: return "device error";
  }
  return "unknown status";
}

tq_status tq_cache_bytes(const tq_config* cfg, uint64_t* k_bytes, uint64_t* v_bytes) {
  const tq_status st = check_cfg(cfg);
  if (st != TQ_OK) return st;
  if (k_bytes == nullptr || v_bytes == nullptr) return TQ_EINVAL;
  const uint64_t slots = static_cast<uint64_t>(cfg->batch) * cfg->n_kv_heads * n_blocks(cfg);
  *k_bytes = slots * kBlock * k_record_bytes(cfg);
  *v_bytes = slots * kBlock * v_record_bytes(cfg);
  return TQ_OK;
}

tq_status tq_params_bytes(const tq_config* cfg, uint64_t* bytes) {
  const tq_status st = check_cfg(cfg);
  if (st != TQ_OK) return st;
  if (bytes == nullptr) return TQ_EINVAL;
  *bytes = tq::params_layout(cfg->head_dim, qjl_rows(cfg)).total;
  return TQ_OK;
}

tq_status tq_params_host(const tq_config* cfg, void* host_params, uint64_t bytes) {
  const tq_status st = check_cfg(cfg);
  if (st != TQ_OK) return st;
  if (host_params == nullptr || !aligned(host_params, 4)) return TQ_EINVAL;
  if (bytes < tq::params_layout(cfg->head_dim, qjl_rows(cfg)).total) return TQ_EWORKSPACE;
  build_params(cfg, static_cast<uint8_t*>(host_params));
  return TQ_OK;
}

tq_status tq_init_params(const tq_config* cfg, void* params, uint64_t bytes, void* stream) {
  const tq_status st = check_cfg(cfg);
  if (st != TQ_OK) return st;
  if (params == nullptr || !aligned(params, 256)) return TQ_EINVAL;
  const uint64_t need = tq::params_layout(cfg->head_dim, qjl_rows(cfg)).total;
  if (bytes < need) return TQ_EWORKSPACE;
  std::vector<uint8_t> img(need);
  build_params(cfg, img.data());
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(params, img.data(), need, hipMemcpyHostToDevice, s) != hipSuccess) return TQ_EDEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return TQ_EDEVICE;
  return TQ_OK;
}

tq_status tq_quantize_append(const tq_config* cfg, const void* params, void* k_cache, void* v_cache,
                             const int32_t* seq_lens, int32_t max_seq_len, const void* k_new,
                             const void* v_new, int32_t in_dtype, int32_t n_new, void* stream) {
  const tq_status st = check_append(cfg, params, k_cache, v_cache, seq_lens, max_seq_len, k_new, v_new, in_dtype,
                                    n_new);
  if (st != TQ_OK || n_new == 0) return st;   // n_new == 0: nothing to write, buffers not examined
  const hipError_t e = launch_append(cfg, params, k_cache, v_cache, seq_lens, k_new, v_new, in_dtype, n_new,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : TQ_EDEVICE;
}

tq_status tq_decode_workspace_bytes(const tq_config* cfg, int32_t max_seq_len, uint64_t* bytes) {
  const tq_status st = check_cfg(cfg);
  if (st != TQ_OK) return st;
  if (bytes == nullptr || max_seq_len < 0 || max_seq_len > cfg->max_ctx) return TQ_EINVAL;
  *bytes = workspace_need(cfg, max_seq_len);
  return TQ_OK;
}

tq_status tq_decode_attention(const tq_config* cfg, const void* params, const void* k_cache,
                              const void* v_cache, const int32_t* seq_lens, int32_t max_seq_len,
                              const float* q, float* out, float* logits, void* workspace,
                              uint64_t workspace_bytes, void* stream) {
  tq::DecodeArgs a{};
  const tq_status st = prepare_decode(cfg, params, k_cache, v_cache, seq_lens, max_seq_len, q, out, logits, workspace,
                                      workspace_bytes, &a);
  if (st != TQ_OK) return st;
  hipError_t e = tq::launch_decode_reg(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) e = tq::launch_decode_q8(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) e = tq::launch_decode_mfma(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) e = tq::launch_decode(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : TQ_EDEVICE;
}

tq_status tq_decode_attention_noalloc(const tq_config* cfg, const void* params, const void* k_cache,
                                      const void* v_cache, const int32_t* seq_lens, int32_t max_seq_len,
                                      const float* q, float* out, float* logits, void* stream) {
  tq_status st = check_decode(cfg, params, k_cache, v_cache, seq_lens, max_seq_len, q, out, logits);
  if (st != TQ_OK) return st;
  // the same layout as a caller's workspace, with the counters in a region of
  // fixed size that calls of every configuration share
  if (counters_bytes(cfg) > tq::kScratchCounterBytes ||
      workspace_need(cfg, max_seq_len) - counters_bytes(cfg) > tq::kScratchBytes - tq::kScratchCounterBytes)
    return TQ_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ptr = nullptr;
  if (tq::scratch_workspace(&ptr, s) != hipSuccess) return TQ_EDEVICE;
  uint8_t* base = static_cast<uint8_t*>(ptr);
  tq::DecodeArgs a{};
  fill_decode_args(cfg, params, k_cache, v_cache, seq_lens, max_seq_len, q, out, logits,
                   reinterpret_cast<uint32_t*>(base), base + tq::kScratchCounterBytes, &a);
  hipError_t e = tq::launch_decode_reg(a, s);
  if (e == hipErrorNotSupported) e = tq::launch_decode_q8(a, s);
  if (e == hipErrorNotSupported) e = tq::launch_decode_mfma(a, s);
  if (e == hipErrorNotSupported) e = tq::launch_decode(a, s);
  return e == hipSuccess ? TQ_OK : TQ_EDEVICE;
}

tq_status tq_append_decode(const tq_config* cfg, const void* params, void* k_cache, void* v_cache,
                           const int32_t* seq_lens, int32_t max_seq_len, const void* k_new, const void* v_new,
                           int32_t in_dtype, const float* q, float* out, float* logits, void* workspace,
                           uint64_t workspace_bytes, void* stream) {
  tq_status st = check_append(cfg, params, k_cache, v_cache, seq_lens, max_seq_len, k_new, v_new, in_dtype, 1);
  if (st != TQ_OK) return st;
  tq::DecodeArgs a{};
  st = prepare_decode(cfg, params, k_cache, v_cache, seq_lens, max_seq_len + 1, q, out, logits, workspace,
                      workspace_bytes, &a);
  if (st != TQ_OK) return st;
  a.len_add = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (reg_path(cfg) || q8_path(cfg) || mfma_path(cfg)) {
    a.k_new = k_new;
    a.v_new = v_new;
    a.in_dtype = in_dtype;
    hipError_t e = reg_path(cfg) ? tq::launch_decode_reg(a, s) : hipErrorNotSupported;
    if (e == hipErrorNotSupported) e = tq::launch_decode_q8(a, s);
    if (e == hipErrorNotSupported) e = tq::launch_decode_mfma(a, s);
    if (e != hipErrorNotSupported) return e == hipSuccess ? TQ_OK : TQ_EDEVICE;
    a.k_new = a.v_new = nullptr;
  }
  // codecs the matrix-core kernel does not serve: the two launches in order
  hipError_t e = launch_append(cfg, params, k_cache, v_cache, seq_lens, k_new, v_new, in_dtype, 1, s);
  if (e == hipSuccess) e = tq::launch_decode(a, s);
  return e == hipSuccess ? TQ_OK : TQ_EDEVICE;
}

tq_status tq_dequantize(const tq_config* cfg, const void* params, const void* k_cache, const void* v_cache,
                        int32_t b, int32_t start, int32_t count, float* k_out, float* v_out, uint32_t flags,
                        void* stream) {
  const tq_status st = check_cfg(cfg);
  if (st != TQ_OK) return st;
  if (params == nullptr || !aligned(params, 256)) return TQ_EINVAL;
  if (b < 0 || b >= cfg->batch || start < 0 || count < 0 ||
      static_cast<int64_t>(start) + count > cfg->max_ctx)
    return TQ_EINVAL;
  if ((flags & ~TQ_DEQ_QJL) != 0) return TQ_EINVAL;
  if (k_out != nullptr && (k_cache == nullptr || !aligned(k_cache, 16) || !aligned(k_out, 4))) return TQ_EINVAL;
  if (v_out != nullptr && (v_cache == nullptr || !aligned(v_cache, 16) || !aligned(v_out, 4))) return TQ_EINVAL;
  if (count == 0 || (k_out == nullptr && v_out == nullptr)) return TQ_OK;
  tq::DequantArgs a{};
  a.tb = tables(cfg, params);
  a.kc = static_cast<const uint8_t*>(k_cache);
  a.vc = static_cast<const uint8_t*>(v_cache);
  a.k_out = k_out;
  a.v_out = v_out;
  a.b = b;
  a.start = start;
  a.count = count;
  a.n_kv = cfg->n_kv_heads;
  a.n_blocks = n_blocks(cfg);
  a.k_codec = cfg->k_codec;
  a.k_bits = cfg->k_bits;
  a.v_codec = cfg->v_codec;
  a.v_bits = cfg->v_bits;
  a.qjl = (flags & TQ_DEQ_QJL) ? 1 : 0;
  a.k_block_bytes = kBlock * k_record_bytes(cfg);
  a.v_block_bytes = kBlock * v_record_bytes(cfg);
  return tq::launch_dequantize(a, static_cast<hipStream_t>(stream)) == hipSuccess ? TQ_OK : TQ_EDEVICE;
}

tq_status tq_stream_read(const void* src, uint64_t bytes, uint32_t* sink, void* stream) {
  if (src == nullptr || sink == nullptr || !aligned(src, 16) || !aligned(sink, 4) || bytes % 16 != 0)
    return TQ_EINVAL;
  if (bytes == 0) return TQ_OK;
  return tq::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)) == hipSuccess ? TQ_OK
                                                                                                   : TQ_EDEVICE;
}

}  // extern "C"
