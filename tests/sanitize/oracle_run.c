/* Drives the oracle (oracle/tq_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer on the CPU: parameter generation, every
 * codebook, the per-vector quantisers on ordinary and edge-case vectors,
 * whole-cache pack / unpack round trips for every codec pair, and the fp64
 * decode.  Exit status 0 when every round trip holds. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tq_oracle.h"

enum { RAW = 0, POLAR = 1, QJL = 2, Q8 = 3, TREE = 4 };

static uint64_t rng_state = 12345;
static double urand(void) {
  rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}
static float nrand(void) {
  double u1 = urand() + 1e-300, u2 = urand();
  return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

static int run_pair(int kc, int kb, int vc, int vb) {
  or_spec s = {128, 8, 2, 2, 300, kc, kb, kc == QJL ? 128 : 0, vc, vb};
  const int d = s.d, m = s.m;
  const int64_t n = (int64_t)s.batch * s.max_ctx * s.n_kv;
  float DK[128], DV[128];
  or_make_signs(42, 1, 0, d, DK);
  or_make_signs(42, 1, 1, d, DV);
  float* S = m ? (float*)malloc(sizeof(float) * m * d) : NULL;
  if (S) or_make_sketch(42, 1, m, d, S);
  double cent[256], mse;
  uint16_t ck16[256], cv16[256];
  float kbnd[256], vbnd[256];
  memset(ck16, 0, sizeof ck16);
  memset(cv16, 0, sizeof cv16);
  memset(kbnd, 0, sizeof kbnd);
  memset(vbnd, 0, sizeof vbnd);
  if (kc == POLAR || kc == QJL) or_codebook(d, kb, cent, ck16, kbnd, &mse);
  if (vc == POLAR) or_codebook(d, vb, cent, cv16, vbnd, &mse);
  float* x = (float*)malloc(sizeof(float) * n * d);
  float* y = (float*)malloc(sizeof(float) * n * d);
  for (int64_t i = 0; i < n * d; i++) {
    x[i] = nrand();
    y[i] = nrand();
  }
  /* edge cases in the first records: zero, signed zero, huge, tiny */
  for (int i = 0; i < d; i++) {
    x[i] = 0.0f;
    x[d + i] = -0.0f;
    x[2 * d + i] *= 1e5f;
    x[3 * d + i] *= 1e-30f;
  }
  or_krec kr = {0}, kr2 = {0};
  or_vrec vr = {0}, vr2 = {0};
  kr.codes = calloc(n * d, 1); kr.n16 = calloc(n, 2); kr.signs = calloc(n * (m ? m : 1), 1);
  kr.rho16 = calloc(n, 2); kr.k8 = calloc(n * d, 1); kr.s16 = calloc(n * d / 32, 2); kr.raw = calloc(n * d, 4);
  vr.codes = calloc(n * d, 1); vr.n16 = calloc(n, 2); vr.raw = calloc(n * d, 4);
  kr2.codes = calloc(n * d, 1); kr2.n16 = calloc(n, 2); kr2.signs = calloc(n * (m ? m : 1), 1);
  kr2.rho16 = calloc(n, 2); kr2.k8 = calloc(n * d, 1); kr2.s16 = calloc(n * d / 32, 2); kr2.raw = calloc(n * d, 4);
  vr2.codes = calloc(n * d, 1); vr2.n16 = calloc(n, 2); vr2.raw = calloc(n * d, 4);
  or_quantize_k_many(&s, DK, ck16, kbnd, S, n, x, &kr, 0);
  or_quantize_v_many(&s, DV, cv16, vbnd, n, y, &vr, 0);
  int32_t lens[2] = {300, 171};
  int64_t kbytes = or_k_cache_bytes(&s), vbytes = or_v_cache_bytes(&s);
  uint8_t* kcache = calloc(kbytes, 1);
  uint8_t* vcache = calloc(vbytes, 1);
  or_pack_cache(&s, lens, &kr, &vr, kcache, vcache);
  or_unpack_cache(&s, lens, kcache, vcache, &kr2, &vr2);
  int bad = 0;
  for (int b = 0; b < s.batch; b++)
    for (int p = 0; p < lens[b]; p++)
      for (int h = 0; h < s.n_kv; h++) {
        int64_t r = ((int64_t)b * s.max_ctx + p) * s.n_kv + h;
        if (kc == POLAR || kc == QJL || kc == TREE) {
          bad |= memcmp(kr.codes + r * d, kr2.codes + r * d, d) != 0;
          bad |= kr.n16[r] != kr2.n16[r];
        }
        if (kc == QJL) bad |= memcmp(kr.signs + r * m, kr2.signs + r * m, m) != 0 || kr.rho16[r] != kr2.rho16[r];
        if (kc == Q8) bad |= memcmp(kr.k8 + r * d, kr2.k8 + r * d, d) != 0;
        if (kc == RAW) bad |= memcmp(kr.raw + r * d, kr2.raw + r * d, 4 * d) != 0;
        if (vc == POLAR || vc == TREE) bad |= memcmp(vr.codes + r * d, vr2.codes + r * d, d) != 0 || vr.n16[r] != vr2.n16[r];
        if (vc == RAW) bad |= memcmp(vr.raw + r * d, vr2.raw + r * d, 4 * d) != 0;
      }
  float* q = (float*)malloc(sizeof(float) * s.batch * s.n_q * d);
  for (int i = 0; i < s.batch * s.n_q * d; i++) q[i] = nrand();
  int32_t pairs[6] = {0, 0, 0, 7, 1, 3};
  double out[3 * 128];
  double* lg = (double*)malloc(sizeof(double) * 3 * s.max_ctx);
  or_decode_pairs(&s, DK, DV, ck16, cv16, S, &kr2, &vr2, lens, q, 3, pairs, out, lg);
  for (int i = 0; i < 3 * d; i++) bad |= !isfinite(out[i]);
  free(lg); free(q); free(kcache); free(vcache);
  free(kr.codes); free(kr.n16); free(kr.signs); free(kr.rho16); free(kr.k8); free(kr.s16); free(kr.raw);
  free(vr.codes); free(vr.n16); free(vr.raw);
  free(kr2.codes); free(kr2.n16); free(kr2.signs); free(kr2.rho16); free(kr2.k8); free(kr2.s16); free(kr2.raw);
  free(vr2.codes); free(vr2.n16); free(vr2.raw);
  free(x); free(y); free(S);
  if (bad) fprintf(stderr, "round trip failed for %d/%d %d/%d\n", kc, kb, vc, vb);
  return bad;
}

int main(void) {
  or_tree_prepare();
  int bad = 0;
  for (int b = 1; b <= 4; b++) {
    double cent[16], mse;
    uint16_t c16[16];
    float bnd[16];
    bad |= or_codebook(128, b, cent, c16, bnd, &mse) < 0;
  }
  const int pairs[][4] = {{QJL, 3, POLAR, 2}, {QJL, 4, POLAR, 4}, {QJL, 2, RAW, 32}, {POLAR, 3, POLAR, 3},
                          {Q8, 8, POLAR, 2}, {RAW, 32, RAW, 32}, {TREE, 3, TREE, 2}, {TREE, 4, POLAR, 3}};
  for (size_t i = 0; i < sizeof pairs / sizeof pairs[0]; i++)
    bad |= run_pair(pairs[i][0], pairs[i][1], pairs[i][2], pairs[i][3]);
  if (bad) return 1;
  printf("oracle run clean\n");
  return 0;
}
