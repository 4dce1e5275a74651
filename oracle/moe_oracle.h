/*
 * moe_oracle.h -- plain, slow, fp64 CPU oracle of one MoE layer's routed-expert
 * forward pass.  TEST INFRASTRUCTURE ONLY: it is used by the tests, by the smoke
 * check and by the bench's CPU-baseline leg, never by the product path.  It shares
 * no code, header, table or helper with the GPU library.
 *
 * Source pages: "Meet FreeToken: An Edge-Native MoE Serving Engine that Runs 753B
 * GLM-5.2 on a Single Workstation GPU" (MarkTechPost article, as republished on
 * youzum.net and dailyaifeed.com).  Citations below give the page's section.
 * The pages describe the serving system, not the layer's equations; where they
 * are silent the plainest textbook reading is taken, as each function states.
 *
 * All functions return 0 on success and a negative value on invalid input.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORA_F32 0
#define ORA_BF16 1
#define ORA_MXFP4 2
/* MXFP4 weights with the gate/up activations quantized to MXFP8 (E4M3 elements,
 * one E8M0 scale per 32 consecutive elements of a token row), OCP MX v1.0. */
#define ORA_MXFP4_A8 3

/* ---- stored formats -> exact fp64 ---------------------------------------- */
double ora_bf16_value(uint16_t bits);
double ora_e2m1_value(uint8_t code);   /* low 4 bits used */
double ora_e8m0_value(uint8_t code);   /* 0xFF is NaN */
double ora_e4m3_value(uint8_t code);   /* 0x7F and 0xFF are NaN */
/* MXFP8 (E4M3) quantization of bf16 activations x [T][H] (H a multiple of 32), OCP
 * MX v1.0: per block of 32 elements along a row the shared exponent is
 * X = floor(log2(max |x|)) - 8 (8 = the largest E4M3 exponent), clamped to
 * [-127, 127] (X = -127 for an all-zero block); scales [T][H/32] = X + 127; each
 * element x / 2^X becomes the nearest finite E4M3 value, ties to the even code,
 * magnitudes beyond 448 clamped to 448. codes [T][H]. */
int ora_mx8_quantize(const uint16_t* x, int T, int H, uint8_t* codes, uint8_t* scales);
size_t ora_expert_bytes(int dtype, int H, int I);
/* Decode one expert slot into fp64 Wg [I][H], Wu [I][H], Wd [H][I]. */
int ora_decode_expert(int dtype, const uint8_t* slot, int H, int I, double* wg, double* wu, double* wd);
/* Decode activations: f32 [T][H] for ORA_F32, bf16 bits [T][H] otherwise; for
 * ORA_MXFP4_A8 the bf16 values after their MXFP8 quantization (ora_mx8_quantize). */
int ora_decode_x(int dtype, const void* x, int T, int H, double* out);

/* ---- routing -------------------------------------------------------------- */
/* Top-k by logit (descending, ties to the lower expert index) and softmax over
 * the k selected logits.  ids [T][k]; w32 (nullable) the weights rounded to f32;
 * w64 (nullable) the weights in fp64.  Rejects non-finite logits (-2). */
int ora_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w32, double* w64);
/* Router projection ahead of top-k: logits[t][e] = sum_h x[t][h] * wr[e][h] with x
 * [T][H] and wr [E][H] bf16 bits, products and sum in fp64 (h ascending). */
int ora_router_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E, double* logits);

/* Stable counting sort of the T*k (token, choice) pairs r = t*k + j by expert. */
int ora_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                int32_t* sorted_rows, int32_t* inv_rows);

/* ---- expert FFN and combine ----------------------------------------------- */
/* o = Wd . (SiLU(Wg . x) * (Wu . x)), all fp64, no intermediate rounding. */
void ora_expert_ffn(const double* wg, const double* wu, const double* wd, int H, int I,
                    const double* x, double* o);
/* y[t] = sum_j w[t][j] * rows[t*k + j]  (+ shared[t] when non-null), fp64. */
void ora_combine(const double* rows, const double* w, const double* shared, int T, int k, int H, double* y);

/* Whole layer.  expert_ptr[e] points at expert e's slot bytes; shared (nullable)
 * at the always-on shared expert with intermediate size I_shared.  Outputs:
 * y [T][H]; ids [T][k]; w [T][k] (fp64); rows (nullable) [T*k][H], the routed
 * expert output of pair r = t*k + j before weighting; shared_out (nullable) [T][H]. */
int ora_layer(int dtype, const uint8_t* const* expert_ptr, const uint8_t* shared, int I_shared,
              const void* x, const float* logits, int T, int H, int I, int E, int k,
              double* y, int32_t* ids, double* w, double* rows, double* shared_out);

/* Expert FFN for a list of tokens of one expert: x rows decoded from `x` by
 * token index, outputs o [n][H].  Used for sampled checks at full sizes. */
int ora_expert_rows(int dtype, const uint8_t* slot, int H, int I, const void* x, int T,
                    const int32_t* tokens, int n, double* o);

/* ---- global LRU expert cache ---------------------------------------------- */
typedef struct ora_lru ora_lru;
ora_lru* ora_lru_new(int n_slots, int n_layers, int n_experts);
void ora_lru_free(ora_lru* c);
/* One (step, layer).  Active experts are those with counts[e] > 0.  Per access a
 * (in access order): expert, hit (0/1), slot, wave, cold (first ever access of
 * the key, 0/1), evicted key (-1 if none).  Arrays need room for E entries.
 * Returns the number of waves (>= 0) or a negative error. */
int ora_lru_step(ora_lru* c, int layer, const int32_t* counts, int* n_access, int32_t* acc_expert,
                 int32_t* acc_hit, int32_t* acc_slot, int32_t* acc_wave, int32_t* acc_cold,
                 int64_t* acc_evicted);
/* The same step with its misses split: of the m misses (ascending expert id) the
 * first floor(m * fill_num / fill_den + 1/2) are accessed (filled) as above; the
 * others are computed in place and not accessed: listed in inplace_expert
 * (nullable, room for E) with their cold flags (inplace_cold, nullable), count in
 * *n_inplace.  0 <= fill_num <= fill_den, fill_den >= 1. */
int ora_lru_step_split(ora_lru* c, int layer, const int32_t* counts, int fill_num, int fill_den, int* n_access,
                       int32_t* acc_expert, int32_t* acc_hit, int32_t* acc_slot, int32_t* acc_wave,
                       int32_t* acc_cold, int64_t* acc_evicted, int* n_inplace, int32_t* inplace_expert,
                       int32_t* inplace_cold);
/* key_of_slot [S] (layer*E + expert, -1 if empty) and last-use tick per slot. */
void ora_lru_state(const ora_lru* c, int64_t* key_of_slot, int64_t* tick_of_slot);
/* Elastic resize to new_S slots between steps: keeps the min(new_S, resident)
 * most recently used keys, in new slots 0, 1, ... by decreasing recency, with
 * their ticks; the others are dropped.  moved_from [new_S] receives the old slot
 * of each new slot's key (-1 for an empty slot).  Returns 0, or a negative error. */
int ora_lru_resize(ora_lru* c, int new_S, int32_t* moved_from);

#ifdef __cplusplus
}
#endif
#endif
