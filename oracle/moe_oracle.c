/*
 * moe_oracle.c -- plain fp64 CPU oracle of one MoE layer's routed-expert forward
 * pass.  TEST INFRASTRUCTURE ONLY (tests, smoke check, bench CPU baseline).
 *
 * Pages: "Meet FreeToken: An Edge-Native MoE Serving Engine that Runs 753B GLM-5.2
 * on a Single Workstation GPU" (MarkTechPost).  The pages state the system's
 * policies (routing left as the model has it, one LRU cache of experts keyed over
 * every MoE layer, nothing cached at start, exact expert output) but print no layer
 * equation; every formula here is the textbook definition of the step, and each
 * reading the pages leave open is named where it is taken.
 *
 * Everything is written for obviousness, not speed: straight loops, fp64, no
 * blocking or reordering.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ===========================================================================
 * Stored formats
 * ======================================================================== */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
double ora_bf16_value(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* E2M1 element of OCP Microscaling Formats (MX) v1.0 (the pages name the MXFP4
 * build in the section "Results").  Bit 3 is the sign; codes 0..7 carry the
 * magnitudes of the spec's E2M1 table. */
double ora_e2m1_value(uint8_t code) {
  static const double magnitude[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double v = magnitude[code & 7u];
  return (code & 8u) ? -v : v;
}

/* E8M0 block scale of OCP MX v1.0: 2^(code - 127); code 0xFF encodes NaN. */
double ora_e8m0_value(uint8_t code) {
  if (code == 0xFFu) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* E4M3 element of OCP MX v1.0 (the activations of the native FP4 path): bit 7 the
 * sign, bits 6..3 the exponent (bias 7), bits 2..0 the mantissa; exponent field 0
 * holds the subnormals m/8 * 2^-6; S.1111.111 is NaN (no infinities). */
double ora_e4m3_value(uint8_t code) {
  const int e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return (code & 0x80u) ? -v : v;
}

/* MXFP8 quantization, written out: block scale from the block's largest
 * magnitude, then each scaled element to the nearest finite E4M3 value found by
 * trying every code (ties to the even code; anything beyond 448 lands on 448). */
int ora_mx8_quantize(const uint16_t* x, int T, int H, uint8_t* codes, uint8_t* scales) {
  if (T < 0 || H <= 0 || H % 32) return -1;
  for (int t = 0; t < T; ++t)
    for (int b = 0; b < H / 32; ++b) {
      const uint16_t* xb = x + (size_t)t * H + (size_t)b * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        const double a = fabs(ora_bf16_value(xb[i]));
        if (a > amax) amax = a;
      }
      int X = -127;
      if (amax > 0.0) {
        int e2;
        frexp(amax, &e2);  /* amax = f * 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
        X = e2 - 1 - 8;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
      }
      scales[(size_t)t * (H / 32) + b] = (uint8_t)(X + 127);
      for (int i = 0; i < 32; ++i) {
        const double v = ldexp(ora_bf16_value(xb[i]), -X), a = fabs(v);
        int best = 0;
        double best_d = INFINITY;
        for (int c = 0; c <= 0x7E; ++c) {
          const double d = fabs(ora_e4m3_value((uint8_t)c) - a);
          if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
          }
        }
        codes[(size_t)t * H + (size_t)b * 32 + i] = (uint8_t)(best | (signbit(v) ? 0x80 : 0));
      }
    }
  return 0;
}

/* Tiled slot layout (a reading: the pages say only that experts are stored in
 * pinned host memory in the layout they are computed from, "Three mechanisms",
 * elastic memory management).
 * A matrix of `rows` rows (a multiple of 16) and K columns is cut into tiles of
 * 16 rows by KS columns (KS = 32 for bf16, 128 for MXFP4); tiles are stored
 * row-tile major, then by column step.  Inside a tile the 64 fragments of 16
 * bytes are ordered by f = 16*g + (row % 16), where g = (k % KS) / (KS / 4) is
 * the column group: a bf16 fragment is 8 consecutive k, an MXFP4 fragment is
 * one 32-element block (element 2i in the low nibble of byte i).  An MXFP4 matrix
 * also has one E8M0 byte per fragment, stored apart from the codes: per row tile
 * the column steps are grouped 16 at a time into 1 KB scale blocks, in which
 * fragment f owns bytes 16f .. 16f+15, byte i holding its scale at step
 * 16*block + i (steps past the last one are padding).  If K is not a multiple of
 * 128 the last MXFP4 step is padded with zero fragments. */
static size_t ksteps(int dtype, int K) { return dtype == ORA_MXFP4 ? (size_t)(K + 127) / 128 : (size_t)K / 32; }

static size_t fragment_index(int dtype, int K, int r, int c) {
  const int KS = dtype == ORA_MXFP4 ? 128 : 32;
  const size_t tile = (size_t)(r / 16) * ksteps(dtype, K) + (size_t)(c / KS);
  const int g = (c % KS) / (KS / 4);
  return tile * 64 + (size_t)(16 * g + r % 16);
}

/* Byte offset of the scale of MXFP4 element (r, c) inside its matrix's scales. */
static size_t scale_index(int K, int r, int c) {
  const size_t nblocks = (ksteps(ORA_MXFP4, K) + 15) / 16;
  const size_t step = (size_t)(c / 128);
  const int f = 16 * ((c % 128) / 32) + r % 16;
  return ((size_t)(r / 16) * nblocks + step / 16) * 1024 + (size_t)(16 * f) + step % 16;
}

/* Element (r, c) of a rows x K matrix: f32 row-major; bf16 and MXFP4 tiled as
 * above (MXFP4 scales in the separate array `s`). */
static double element(int dtype, const uint8_t* p, const uint8_t* s, int K, int r, int c) {
  if (dtype == ORA_F32) {
    float f;
    memcpy(&f, p + 4 * ((size_t)r * (size_t)K + (size_t)c), sizeof f);
    return (double)f;
  }
  const size_t f = fragment_index(dtype, K, r, c);
  if (dtype == ORA_BF16) {
    uint16_t b;
    memcpy(&b, p + 16 * f + 2 * (size_t)(c % 8), sizeof b);
    return ora_bf16_value(b);
  }
  {
    const int e = c % 32; /* element inside its block */
    const uint8_t byte = p[16 * f + (size_t)(e / 2)];
    const uint8_t code = (e % 2 == 0) ? (uint8_t)(byte & 0x0Fu) : (uint8_t)(byte >> 4);
    return ora_e2m1_value(code) * ora_e8m0_value(s[scale_index(K, r, c)]);
  }
}

/* Bytes of one tiled matrix (codes, and for MXFP4 the scales). */
static size_t matrix_bytes(int dtype, int rows, int K) {
  if (dtype == ORA_F32) return (size_t)4 * rows * K;
  if (dtype == ORA_BF16) return (size_t)2 * rows * K;
  return (size_t)(rows / 16) * ksteps(dtype, K) * 1024;
}
static size_t scale_bytes(int rows, int K) {
  return (size_t)(rows / 16) * ((ksteps(ORA_MXFP4, K) + 15) / 16) * 1024;
}

size_t ora_expert_bytes(int dtype, int H, int I) {
  if (H <= 0 || I <= 0) return 0;
  if (dtype == ORA_MXFP4_A8) dtype = ORA_MXFP4;  /* same weights */
  if (dtype == ORA_F32 || dtype == ORA_BF16) return matrix_bytes(dtype, 2 * I, H) + matrix_bytes(dtype, H, I);
  if (dtype != ORA_MXFP4 || H % 32 || I % 32) return 0;
  return matrix_bytes(dtype, 2 * I, H) + matrix_bytes(dtype, H, I) + scale_bytes(2 * I, H) + scale_bytes(H, I);
}

/* Slot layout (the layout experts are kept in, host and device; one contiguous run per expert):
 *   W13 (2I rows, K = H) then W2 (H rows, K = I); MXFP4: codes of W13, codes of
 *   W2, scales of W13, scales of W2.
 * Row order of W13: f32 keeps gate rows 0..I-1 then up rows; bf16 and MXFP4
 * interleave per 16-row tile: stored row 16t + q holds gate row 8t + q for
 * q < 8 and up row 8t + q - 8 otherwise. */
int ora_decode_expert(int dtype, const uint8_t* slot, int H, int I, double* wg, double* wu, double* wd) {
  const uint8_t *w13, *w2, *s13 = NULL, *s2 = NULL;
  if (H <= 0 || I <= 0) return -1;
  if (dtype == ORA_MXFP4_A8) dtype = ORA_MXFP4;  /* same weights */
  if (dtype == ORA_F32) {
    w13 = slot;
    w2 = slot + matrix_bytes(dtype, 2 * I, H);
    for (int j = 0; j < I; ++j)
      for (int h = 0; h < H; ++h) {
        wg[(size_t)j * H + h] = element(dtype, w13, NULL, H, j, h);
        wu[(size_t)j * H + h] = element(dtype, w13, NULL, H, I + j, h);
      }
  } else {
    if (H % 32 || I % 32) return -1;
    if (dtype != ORA_BF16 && dtype != ORA_MXFP4) return -1;
    w13 = slot;
    w2 = w13 + matrix_bytes(dtype, 2 * I, H);
    if (dtype == ORA_MXFP4) {
      s13 = w2 + matrix_bytes(dtype, H, I);
      s2 = s13 + scale_bytes(2 * I, H);
    }
    for (int j = 0; j < I; ++j) {
      const int gate_row = 16 * (j / 8) + j % 8, up_row = gate_row + 8;
      for (int h = 0; h < H; ++h) {
        wg[(size_t)j * H + h] = element(dtype, w13, s13, H, gate_row, h);
        wu[(size_t)j * H + h] = element(dtype, w13, s13, H, up_row, h);
      }
    }
  }
  for (int h = 0; h < H; ++h)
    for (int j = 0; j < I; ++j) wd[(size_t)h * I + j] = element(dtype, w2, s2, I, h, j);
  return 0;
}

int ora_decode_x(int dtype, const void* x, int T, int H, double* out) {
  size_t n = (size_t)T * (size_t)H;
  if (dtype == ORA_F32) {
    const float* f = (const float*)x;
    for (size_t i = 0; i < n; ++i) out[i] = (double)f[i];
  } else if (dtype == ORA_BF16 || dtype == ORA_MXFP4) {
    const uint16_t* b = (const uint16_t*)x;
    for (size_t i = 0; i < n; ++i) out[i] = ora_bf16_value(b[i]);
  } else if (dtype == ORA_MXFP4_A8) {
    if (H % 32) return -1;
    uint8_t* codes = (uint8_t*)malloc(n ? n : 1);
    uint8_t* scales = (uint8_t*)malloc(n / 32 + 1);
    if (!codes || !scales) { free(codes); free(scales); return -3; }
    ora_mx8_quantize((const uint16_t*)x, T, H, codes, scales);
    for (size_t i = 0; i < n; ++i) out[i] = ora_e4m3_value(codes[i]) * ora_e8m0_value(scales[i / 32]);
    free(codes); free(scales);
  } else {
    return -1;
  }
  return 0;
}

/* ===========================================================================
 * Routing
 * ======================================================================== */

/* Does (va, a) rank before (vb, b)?  Larger logit first; equal logits (IEEE
 * equality, so -0.0 == +0.0) go to the lower expert index.  The pages require
 * routing to be left unmodified ("Three mechanisms", bandwidth-adaptive
 * execution; "Key Takeaways"); the tie-break is the lowest-index reading. */
static int ranks_before(float va, int a, float vb, int b) {
  if (va > vb) return 1;
  if (va < vb) return 0;
  return a < b;
}

/* Gate weights are the softmax over the k selected logits, which in exact
 * arithmetic equals a softmax over all E followed by renormalising the k
 * selected probabilities. */
int ora_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w32, double* w64) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
  char* taken = (char*)malloc((size_t)E);
  double* z = (double*)malloc(sizeof(double) * (size_t)k);
  if (!taken || !z) { free(taken); free(z); return -3; }
  for (int t = 0; t < T; ++t) {
    const float* row = logits + (size_t)t * E;
    for (int e = 0; e < E; ++e)
      if (!isfinite(row[e])) { free(taken); free(z); return -2; }
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || ranks_before(row[e], e, row[best], best)) best = e;
      }
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
      z[j] = (double)row[best];
    }
    double zmax = z[0];
    double denom = 0.0;
    for (int j = 0; j < k; ++j) denom += exp(z[j] - zmax);
    for (int j = 0; j < k; ++j) {
      double wj = exp(z[j] - zmax) / denom;
      if (w64) w64[(size_t)t * k + j] = wj;
      if (w32) w32[(size_t)t * k + j] = (float)wj;
    }
  }
  free(taken);
  free(z);
  return 0;
}

/* counts[e] = #{r : ids[r] == e}; offsets = exclusive prefix sum (E+1 entries);
 * sorted_rows lists r grouped by expert, ascending r within an expert;
 * inv_rows[r] is the position of r in sorted_rows. */
int ora_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                int32_t* sorted_rows, int32_t* inv_rows) {
  int n = T * k;
  if (T < 0 || k <= 0 || E <= 0) return -1;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int r = 0; r < n; ++r) {
    if (ids[r] < 0 || ids[r] >= E) return -1;
    counts[ids[r]]++;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  if (!next) return -3;
  for (int e = 0; e < E; ++e) next[e] = offsets[e];
  for (int r = 0; r < n; ++r) {
    int p = next[ids[r]]++;
    sorted_rows[p] = r;
    inv_rows[r] = p;
  }
  free(next);
  return 0;
}

/* ===========================================================================
 * Expert FFN (SwiGLU) and combine
 * ======================================================================== */

static double silu(double z) { return z / (1.0 + exp(-z)); }

void ora_expert_ffn(const double* wg, const double* wu, const double* wd, int H, int I,
                    const double* x, double* o) {
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  for (int j = 0; j < I; ++j) {
    double a = 0.0, b = 0.0;
    for (int c = 0; c < H; ++c) {
      a += wg[(size_t)j * H + c] * x[c];
      b += wu[(size_t)j * H + c] * x[c];
    }
    h[j] = silu(a) * b;
  }
  for (int r = 0; r < H; ++r) {
    double acc = 0.0;
    for (int j = 0; j < I; ++j) acc += wd[(size_t)r * I + j] * h[j];
    o[r] = acc;
  }
  free(h);
}

/* The pages say the routed experts' partial sums are added without approximation ("Three
 * mechanisms"); the merge is the gate-weighted sum, plus the shared expert with
 * weight 1 when the layer has one. */
void ora_combine(const double* rows, const double* w, const double* shared, int T, int k, int H, double* y) {
  for (int t = 0; t < T; ++t)
    for (int c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += w[(size_t)t * k + j] * rows[((size_t)t * k + j) * H + c];
      if (shared) acc += shared[(size_t)t * H + c];
      y[(size_t)t * H + c] = acc;
    }
}

int ora_expert_rows(int dtype, const uint8_t* slot, int H, int I, const void* x, int T,
                    const int32_t* tokens, int n, double* o) {
  double* wg = (double*)malloc(sizeof(double) * (size_t)I * H);
  double* wu = (double*)malloc(sizeof(double) * (size_t)I * H);
  double* wd = (double*)malloc(sizeof(double) * (size_t)H * I);
  double* xt = (double*)malloc(sizeof(double) * (size_t)H);
  int rc = 0;
  if (!wg || !wu || !wd || !xt) { rc = -3; goto done; }
  rc = ora_decode_expert(dtype, slot, H, I, wg, wu, wd);
  if (rc) goto done;
  for (int i = 0; i < n; ++i) {
    int t = tokens[i];
    if (t < 0 || t >= T) { rc = -1; goto done; }
    if (dtype == ORA_F32)
      ora_decode_x(dtype, (const float*)x + (size_t)t * H, 1, H, xt);
    else
      ora_decode_x(dtype, (const uint16_t*)x + (size_t)t * H, 1, H, xt);
    ora_expert_ffn(wg, wu, wd, H, I, xt, o + (size_t)i * H);
  }
done:
  free(wg); free(wu); free(wd); free(xt);
  return rc;
}

int ora_layer(int dtype, const uint8_t* const* expert_ptr, const uint8_t* shared, int I_shared,
              const void* x, const float* logits, int T, int H, int I, int E, int k,
              double* y, int32_t* ids, double* w, double* rows, double* shared_out) {
  int rc = ora_route_topk(logits, T, E, k, ids, NULL, w);
  if (rc) return rc;
  double* own_rows = rows ? rows : (double*)malloc(sizeof(double) * (size_t)T * k * H);
  double* sh = NULL;
  if (!own_rows) return -3;
  /* Each routed expert that any token selected, in expert order. */
  for (int e = 0; e < E && rc == 0; ++e) {
    int n = 0;
    for (int r = 0; r < T * k; ++r) n += ids[r] == e;
    if (!n) continue;
    int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t* pair = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    double* o = (double*)malloc(sizeof(double) * (size_t)n * H);
    int m = 0;
    for (int r = 0; r < T * k; ++r)
      if (ids[r] == e) { tok[m] = r / k; pair[m] = r; ++m; }
    rc = ora_expert_rows(dtype, expert_ptr[e], H, I, x, T, tok, n, o);
    for (int i = 0; i < n && rc == 0; ++i)
      memcpy(own_rows + (size_t)pair[i] * H, o + (size_t)i * H, sizeof(double) * (size_t)H);
    free(tok); free(pair); free(o);
  }
  if (rc == 0 && shared) {
    sh = shared_out ? shared_out : (double*)malloc(sizeof(double) * (size_t)T * H);
    int32_t* all = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    for (int t = 0; t < T; ++t) all[t] = t;
    rc = ora_expert_rows(dtype, shared, H, I_shared, x, T, all, T, sh);
    free(all);
  }
  if (rc == 0) ora_combine(own_rows, w, sh, T, k, H, y);
  if (!rows) free(own_rows);
  if (sh && !shared_out) free(sh);
  return rc;
}

/* ===========================================================================
 * Global LRU expert cache
 *
 * The pages: in decode, a single least-recently-used cache keyed over all MoE
 * layers holds the experts the router keeps selecting ("Three mechanisms",
 * semantic-aware caching), and nothing is cached when serving begins ("Three
 * mechanisms", elastic memory management).  Readings taken where they are silent:
 *  - keys are (layer, expert), key = layer*E + expert; the cache starts empty;
 *  - within one (step, layer) the active experts are accessed hits first, then
 *    misses, each group in ascending expert id, hit/miss judged against the state
 *    before the step (so no expert of the step evicts another when they fit);
 *  - a miss takes the lowest-index free slot, otherwise evicts the least recently
 *    used key;
 *  - when the active set exceeds the capacity S, the accesses run in consecutive
 *    waves of S.
 * ======================================================================== */

struct ora_lru {
  int S, L, E;
  int64_t clock;
  int64_t* key_of_slot;  /* [S] */
  int64_t* tick_of_slot; /* [S] */
  int32_t* slot_of_key;  /* [L*E], -1 if not resident */
  char* seen;            /* [L*E] */
};

ora_lru* ora_lru_new(int n_slots, int n_layers, int n_experts) {
  if (n_slots <= 0 || n_layers <= 0 || n_experts <= 0) return NULL;
  ora_lru* c = (ora_lru*)calloc(1, sizeof *c);
  size_t nk = (size_t)n_layers * (size_t)n_experts;
  c->S = n_slots; c->L = n_layers; c->E = n_experts; c->clock = 0;
  c->key_of_slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_slots);
  c->tick_of_slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_slots);
  c->slot_of_key = (int32_t*)malloc(sizeof(int32_t) * nk);
  c->seen = (char*)calloc(nk, 1);
  for (int s = 0; s < n_slots; ++s) { c->key_of_slot[s] = -1; c->tick_of_slot[s] = -1; }
  for (size_t q = 0; q < nk; ++q) c->slot_of_key[q] = -1;
  return c;
}

void ora_lru_free(ora_lru* c) {
  if (!c) return;
  free(c->key_of_slot); free(c->tick_of_slot); free(c->slot_of_key); free(c->seen); free(c);
}

/* One textbook LRU access.  Returns the slot; *hit, *evicted as outputs. */
static int lru_access(ora_lru* c, int64_t key, int* hit, int64_t* evicted) {
  int s = c->slot_of_key[key];
  *evicted = -1;
  if (s >= 0) {
    *hit = 1;
  } else {
    *hit = 0;
    for (int q = 0; q < c->S && s < 0; ++q)
      if (c->key_of_slot[q] < 0) s = q;
    if (s < 0) {
      s = 0;
      for (int q = 1; q < c->S; ++q)
        if (c->tick_of_slot[q] < c->tick_of_slot[s]) s = q;
      *evicted = c->key_of_slot[s];
      c->slot_of_key[*evicted] = -1;
    }
    c->key_of_slot[s] = key;
    c->slot_of_key[key] = s;
  }
  c->tick_of_slot[s] = ++c->clock;
  return s;
}

/* Misses of a step that are filled into slots when the step has m misses and the
 * fill fraction is num/den: q = floor(m * num / den + 1/2). */
static int filled_misses(int m, int num, int den) { return (int)((2LL * m * num + den) / (2LL * den)); }

int ora_lru_step(ora_lru* c, int layer, const int32_t* counts, int* n_access, int32_t* acc_expert,
                 int32_t* acc_hit, int32_t* acc_slot, int32_t* acc_wave, int32_t* acc_cold,
                 int64_t* acc_evicted) {
  int n_inplace = 0;
  return ora_lru_step_split(c, layer, counts, 1, 1, n_access, acc_expert, acc_hit, acc_slot, acc_wave, acc_cold,
                            acc_evicted, &n_inplace, NULL, NULL);
}

/* The step with a split of its misses (the pages: of a step's misses, a share
 * set by the host-link and host-memory bandwidths crosses the link into GPU
 * memory and the rest is computed where the weights already sit, the partial
 * sums merging exactly; "Three mechanisms", bandwidth-adaptive execution).  The
 * one-GPU reading: of the m misses (ascending expert id), the first
 * q = floor(m num / den + 1/2) are filled into slots as in ora_lru_step; the
 * other m - q are computed in place from host memory and are not accessed: they
 * take no slot, evict nothing and leave every tick as it was.  The cache sees the
 * hits and the q filled misses only.  Outputs as ora_lru_step, plus the in-place
 * experts (ascending id) and their cold flags (key never accessed before). */
int ora_lru_step_split(ora_lru* c, int layer, const int32_t* counts, int fill_num, int fill_den, int* n_access,
                       int32_t* acc_expert, int32_t* acc_hit, int32_t* acc_slot, int32_t* acc_wave,
                       int32_t* acc_cold, int64_t* acc_evicted, int* n_inplace, int32_t* inplace_expert,
                       int32_t* inplace_cold) {
  if (!c || layer < 0 || layer >= c->L || fill_den < 1 || fill_num < 0 || fill_num > fill_den) return -1;
  int n = 0, m = 0;
  /* hits first (state before the step), ascending expert id ... */
  for (int e = 0; e < c->E; ++e)
    if (counts[e] > 0 && c->slot_of_key[(int64_t)layer * c->E + e] >= 0) acc_expert[n++] = e;
  /* ... then the misses, ascending expert id: the first q are accessed, the rest
   * are computed in place */
  for (int e = 0; e < c->E; ++e)
    if (counts[e] > 0 && c->slot_of_key[(int64_t)layer * c->E + e] < 0) ++m;
  const int q = filled_misses(m, fill_num, fill_den);
  int seen_misses = 0, ni = 0;
  for (int e = 0; e < c->E; ++e)
    if (counts[e] > 0 && c->slot_of_key[(int64_t)layer * c->E + e] < 0) {
      if (seen_misses++ < q) {
        acc_expert[n++] = e;
      } else {
        if (inplace_expert) inplace_expert[ni] = e;
        if (inplace_cold) inplace_cold[ni] = !c->seen[(int64_t)layer * c->E + e];
        ++ni;
      }
    }
  *n_inplace = ni;
  for (int a = 0; a < n; ++a) {
    int64_t key = (int64_t)layer * c->E + acc_expert[a];
    int hit;
    int64_t ev;
    acc_cold[a] = !c->seen[key];
    c->seen[key] = 1;
    acc_slot[a] = lru_access(c, key, &hit, &ev);
    acc_hit[a] = hit;
    acc_evicted[a] = ev;
    acc_wave[a] = a / c->S;
  }
  *n_access = n;
  return n == 0 ? 0 : (n - 1) / c->S + 1;
}

void ora_lru_state(const ora_lru* c, int64_t* key_of_slot, int64_t* tick_of_slot) {
  for (int s = 0; s < c->S; ++s) {
    key_of_slot[s] = c->key_of_slot[s];
    tick_of_slot[s] = c->tick_of_slot[s];
  }
}

/* Elastic resize (the pages: the slot pool grows and shrinks with the memory the
 * GPU can spare, "Three mechanisms", elastic memory management).  Readings: the
 * resize happens between steps; the kept keys are the most recently used ones and
 * move to the front of the new pool, most recent first; ticks and the clock carry
 * over.  Written as a plain selection: repeatedly take the resident key with the
 * largest tick not yet taken. */
int ora_lru_resize(ora_lru* c, int new_S, int32_t* moved_from) {
  if (!c || new_S <= 0 || !moved_from) return -1;
  int64_t* key2 = (int64_t*)malloc(sizeof(int64_t) * (size_t)new_S);
  int64_t* tick2 = (int64_t*)malloc(sizeof(int64_t) * (size_t)new_S);
  char* taken = (char*)calloc((size_t)c->S, 1);
  if (!key2 || !tick2 || !taken) { free(key2); free(tick2); free(taken); return -2; }
  for (int s = 0; s < new_S; ++s) {
    int best = -1;
    for (int q = 0; q < c->S; ++q)
      if (!taken[q] && c->key_of_slot[q] >= 0 && (best < 0 || c->tick_of_slot[q] > c->tick_of_slot[best])) best = q;
    if (best < 0) {
      key2[s] = -1; tick2[s] = -1; moved_from[s] = -1;
    } else {
      taken[best] = 1;
      key2[s] = c->key_of_slot[best]; tick2[s] = c->tick_of_slot[best]; moved_from[s] = best;
    }
  }
  const size_t nk = (size_t)c->L * (size_t)c->E;
  for (size_t q = 0; q < nk; ++q) c->slot_of_key[q] = -1;
  for (int s = 0; s < new_S; ++s)
    if (key2[s] >= 0) c->slot_of_key[key2[s]] = s;
  free(c->key_of_slot); free(c->tick_of_slot); free(taken);
  c->key_of_slot = key2; c->tick_of_slot = tick2; c->S = new_S;
  return 0;
}

/* Router projection (a reading: the pages say the engine leaves the model's router
 * as it is, "Three mechanisms", bandwidth-adaptive execution, and do not give the
 * router; the plain linear gate of an MoE layer is used, logits = W_r x).  Each
 * logit is the exact products of the bf16 values summed in fp64 in h order. */
int ora_router_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E, double* logits) {
  if (T < 0 || H <= 0 || E <= 0 || (T > 0 && (!x || !wr || !logits))) return -1;
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += ora_bf16_value(x[(size_t)t * H + h]) * ora_bf16_value(wr[(size_t)e * H + h]);
      logits[(size_t)t * E + e] = acc;
    }
  return 0;
}
