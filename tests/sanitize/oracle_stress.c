/* Drives every oracle entry point over small random shapes, edge cases and
 * invalid arguments, for a build under AddressSanitizer and UndefinedBehavior-
 * Sanitizer (host code only).  Prints "ok" and exits 0 when every call returned
 * what its contract says; any sanitizer report aborts the run. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64* */
  rs ^= rs >> 12; rs ^= rs << 25; rs ^= rs >> 27;
  return (uint32_t)((rs * 0x2545F4914F6CDD1Dull) >> 32);
}
static int rint_in(int lo, int hi) { return lo + (int)(rnd() % (uint32_t)(hi - lo + 1)); }
static double runif(void) { return (rnd() + 0.5) / 4294967296.0; }
static float rnorm(void) { return (float)(sqrt(-2.0 * log(runif())) * cos(6.283185307179586 * runif())); }
static uint16_t bf16_of(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)(u >> 16); }

#define CHECK(cond) do { if (!(cond)) { fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); exit(1); } } while (0)

static void *xmalloc(size_t n) { void *p = malloc(n ? n : 1); CHECK(p); return p; }

/* A slot of valid-looking bytes: finite f32 / bf16 weights, MXFP4 codes random
 * with scales in a moderate range (an occasional 0xFF, NaN, included). */
static void fill_slot(int dtype, uint8_t *slot, size_t bytes, int H, int I) {
  if (dtype == ORA_F32) {
    for (size_t i = 0; i < bytes / 4; ++i) { float f = 0.05f * rnorm(); memcpy(slot + 4 * i, &f, 4); }
  } else if (dtype == ORA_BF16) {
    for (size_t i = 0; i < bytes / 2; ++i) { uint16_t b = bf16_of(0.05f * rnorm()); memcpy(slot + 2 * i, &b, 2); }
  } else {
    const size_t codes = (size_t)2 * I * H / 2 + (size_t)H * I / 2;
    for (size_t i = 0; i < bytes; ++i)
      slot[i] = i < codes ? (uint8_t)rnd() : (uint8_t)(rnd() % 97 == 0 ? 0xFF : 120 + rnd() % 8);
  }
}

static void layer_case(int dtype, int T, int H, int I, int E, int k, int shared) {
  const size_t eb = ora_expert_bytes(dtype, H, I);
  CHECK(eb > 0);
  uint8_t **ptr = xmalloc(sizeof(uint8_t *) * E);
  for (int e = 0; e < E; ++e) { ptr[e] = xmalloc(eb); fill_slot(dtype, ptr[e], eb, H, I); }
  const int Is = 32;
  uint8_t *sh = NULL;
  if (shared) { size_t sb = ora_expert_bytes(dtype, H, Is); sh = xmalloc(sb); fill_slot(dtype, sh, sb, H, Is); }
  void *x;
  if (dtype == ORA_F32) {
    float *f = xmalloc(sizeof(float) * (size_t)T * H);
    for (size_t i = 0; i < (size_t)T * H; ++i) f[i] = rnorm();
    x = f;
  } else {
    uint16_t *b = xmalloc(2 * (size_t)T * H);
    for (size_t i = 0; i < (size_t)T * H; ++i) b[i] = bf16_of(rnorm() * (rnd() % 5 == 0 ? 1e-30f : 1.0f));
    x = b;
  }
  float *logits = xmalloc(sizeof(float) * (size_t)T * E);
  for (size_t i = 0; i < (size_t)T * E; ++i) logits[i] = (rnd() % 4 == 0) ? 0.5f : rnorm();  /* ties */
  double *y = xmalloc(sizeof(double) * (size_t)T * H), *w = xmalloc(sizeof(double) * (size_t)T * k);
  double *rows = xmalloc(sizeof(double) * (size_t)T * k * H), *so = xmalloc(sizeof(double) * (size_t)T * H);
  int32_t *ids = xmalloc(sizeof(int32_t) * (size_t)T * k);
  CHECK(ora_layer(dtype, (const uint8_t *const *)ptr, sh, shared ? Is : 0, x, logits, T, H, I, E, k, y, ids, w,
                  rows, shared ? so : NULL) == 0);
  for (int t = 0; t < T; ++t) for (int j = 0; j < k; ++j) CHECK(ids[t * k + j] >= 0 && ids[t * k + j] < E);
  /* the same experts' rows, token lists of every length up to T */
  int32_t *toks = xmalloc(sizeof(int32_t) * (T ? T : 1));
  for (int n = 0; n <= T; ++n) {
    for (int i = 0; i < n; ++i) toks[i] = rint_in(0, T - 1);
    double *o = xmalloc(sizeof(double) * (size_t)(n ? n : 1) * H);
    CHECK(ora_expert_rows(dtype, ptr[rint_in(0, E - 1)], H, I, x, T, toks, n, o) == 0);
    free(o);
  }
  /* decode paths on their own */
  double *wg = xmalloc(sizeof(double) * (size_t)I * H), *wu = xmalloc(sizeof(double) * (size_t)I * H);
  double *wd = xmalloc(sizeof(double) * (size_t)H * I), *xd = xmalloc(sizeof(double) * (size_t)(T ? T : 1) * H);
  CHECK(ora_decode_expert(dtype, ptr[0], H, I, wg, wu, wd) == 0);
  CHECK(ora_decode_x(dtype, x, T, H, xd) == 0);
  if (dtype != ORA_F32 && T > 0) {
    uint8_t *codes = xmalloc((size_t)T * H), *scales = xmalloc((size_t)T * H / 32);
    CHECK(ora_mx8_quantize(x, T, H, codes, scales) == 0);
    free(codes); free(scales);
  }
  free(wg); free(wu); free(wd); free(xd); free(toks);
  for (int e = 0; e < E; ++e) free(ptr[e]);
  free(ptr); free(sh); free(x); free(logits); free(y); free(w); free(rows); free(so); free(ids);
}

static void lru_case(int S, int L, int E, int steps) {
  ora_lru *c = ora_lru_new(S, L, E);
  CHECK(c);
  int32_t *counts = xmalloc(sizeof(int32_t) * E), *ae = xmalloc(sizeof(int32_t) * E), *ah = xmalloc(sizeof(int32_t) * E);
  int32_t *as = xmalloc(sizeof(int32_t) * E), *aw = xmalloc(sizeof(int32_t) * E), *ac = xmalloc(sizeof(int32_t) * E);
  int32_t *ie = xmalloc(sizeof(int32_t) * E), *ic = xmalloc(sizeof(int32_t) * E);
  int64_t *ev = xmalloc(sizeof(int64_t) * E);
  for (int s = 0; s < steps; ++s) {
    const int dens = rint_in(0, 3);
    for (int e = 0; e < E; ++e) counts[e] = (int)(rnd() % 4) < dens ? rint_in(1, 9) : 0;
    int na = -1, ni = -1;
    const int layer = rint_in(0, L - 1);
    int nw;
    if (rnd() % 2) {
      nw = ora_lru_step(c, layer, counts, &na, ae, ah, as, aw, ac, ev);
    } else {
      const int den = rint_in(1, 5);
      nw = ora_lru_step_split(c, layer, counts, rint_in(0, den), den, &na, ae, ah, as, aw, ac, ev, &ni, ie, ic);
    }
    CHECK(nw >= 0 && na >= 0);
    for (int i = 0; i < na; ++i) CHECK(as[i] >= 0 && as[i] < S);
    if (rnd() % 8 == 0) {
      const int nS = rint_in(1, 2 * S);
      int32_t *mf = xmalloc(sizeof(int32_t) * nS);
      CHECK(ora_lru_resize(c, nS, mf) == 0);
      for (int i = 0; i < nS; ++i) CHECK(mf[i] >= -1 && mf[i] < S);
      free(mf);
      S = nS;
    }
    int64_t *ks = xmalloc(sizeof(int64_t) * S), *ts = xmalloc(sizeof(int64_t) * S);
    ora_lru_state(c, ks, ts);
    for (int i = 0; i < S; ++i) CHECK(ks[i] >= -1 && ks[i] < (int64_t)L * E);
    free(ks); free(ts);
  }
  /* invalid arguments are refused */
  int na, ni;
  CHECK(ora_lru_step(c, L, counts, &na, ae, ah, as, aw, ac, ev) < 0);
  CHECK(ora_lru_step_split(c, 0, counts, 2, 1, &na, ae, ah, as, aw, ac, ev, &ni, ie, ic) < 0);
  CHECK(ora_lru_resize(c, 0, ae) < 0);
  ora_lru_free(c);
  free(counts); free(ae); free(ah); free(as); free(aw); free(ac); free(ie); free(ic); free(ev);
}

int main(void) {
  const int dts[4] = {ORA_F32, ORA_BF16, ORA_MXFP4, ORA_MXFP4_A8};
  for (int rep = 0; rep < 6; ++rep)
    for (int d = 0; d < 4; ++d) {
      const int H = 32 * rint_in(1, 5), I = 32 * rint_in(1, 3), E = rint_in(1, 6);
      layer_case(dts[d], rint_in(0, 5), H, I, E, rint_in(1, E), rnd() % 2);
    }
  layer_case(ORA_MXFP4, 3, 256, 128, 4, 4, 1);   /* several 128-column steps */
  for (int rep = 0; rep < 6; ++rep) lru_case(rint_in(1, 12), rint_in(1, 3), rint_in(1, 20), 60);
  /* routing and permutation edge cases and refusals */
  {
    float lg[6] = {1.f, 1.f, -0.f, 0.f, 2.f, NAN};
    int32_t ids[6], cnt[6], off[7], srt[6], inv[6];
    float w32[6];
    double w64[6];
    CHECK(ora_route_topk(lg, 1, 5, 5, ids, w32, w64) == 0);
    CHECK(ora_route_topk(lg, 1, 6, 2, ids, w32, w64) == -2);
    CHECK(ora_route_topk(lg, 1, 5, 6, ids, NULL, NULL) < 0);
    CHECK(ora_route_topk(lg, 0, 5, 2, ids, NULL, NULL) == 0);
    int32_t bad[2] = {0, 7};
    CHECK(ora_permute(bad, 1, 2, 5, cnt, off, srt, inv) < 0);
    CHECK(ora_permute(ids, 0, 2, 5, cnt, off, srt, inv) == 0);
    uint16_t xb[64], wr[96];
    double z[6];
    for (int i = 0; i < 64; ++i) xb[i] = bf16_of(rnorm());
    for (int i = 0; i < 96; ++i) wr[i] = bf16_of(rnorm());
    CHECK(ora_router_logits(xb, wr, 2, 32, 3, z) == 0);
    CHECK(ora_router_logits(xb, wr, 2, 0, 3, z) < 0);
    uint8_t codes[64], scales[2];
    CHECK(ora_mx8_quantize(xb, 2, 31, codes, scales) < 0);
    CHECK(ora_expert_bytes(ORA_MXFP4, 48, 32) == 0);
    for (int c = 0; c < 256; ++c) { (void)ora_e4m3_value((uint8_t)c); (void)ora_e8m0_value((uint8_t)c); }
    for (int c = 0; c < 16; ++c) (void)ora_e2m1_value((uint8_t)c);
  }
  printf("ok\n");
  return 0;
}
