/*
 * moe.h -- C ABI of the MI355X (gfx950) routed-expert MoE layer library, libmoe.so.
 *
 * One MoE layer's routed-expert forward pass, as the hot path of the edge MoE
 * serving engine described in "Meet FreeToken: An Edge-Native MoE Serving Engine
 * that Runs 753B GLM-5.2 on a Single Workstation GPU" (MarkTechPost):
 *
 *   moe_route_topk         top-k gating over router logits
 *   moe_permute            stable permutation of (token, choice) pairs by expert
 *   moe_cache_lookup_fill  global-LRU expert-slot cache in HBM, filled from pinned host memory
 *                          (moe_cache_lookup_fill_split + moe_cache_wait_fills: hits computed during fills)
 *   moe_grouped_ffn        grouped SwiGLU expert FFN (f32, bf16 or MXFP4 weights)
 *   moe_combine            gate-weighted merge of the expert outputs
 *   moe_layer_stream_*     whole-layer double buffering for prefill
 *
 * Conventions
 *  - Pointers are device pointers unless the name ends in _host.
 *  - Every call returns a moe_status; nothing throws, aborts or exits.  On failure
 *    moe_last_error() holds a message for the calling thread.
 *  - Calls that take a hipStream_t are asynchronous on it, except
 *    moe_cache_lookup_fill(_split) for wave 0 (it waits for the step's expert counts).
 *  - The caller owns every buffer and stream.  The library owns only the opaque
 *    handles (host metadata and HIP events) and allocates no device memory on the
 *    hot path: scratch comes from the caller through moe_grouped_ffn_workspace().
 *  - Device buffers must be 16-byte aligned.
 *  - Shapes: 1 <= E <= 1024, 1 <= k <= min(E, 32), T >= 0, T*k < 2^31,
 *    H and I multiples of 32 for bf16/MXFP4 weights (multiples of 4 for f32).
 *  - Logits must be finite; a NaN logit makes the selection unspecified.
 *
 * Expert slot layout (one expert = one contiguous run of moe_expert_bytes(); the
 * host pool stores experts in this final layout so that a fill is one copy):
 *    f32   :  W13 [2I][H] then W2 [H][I], row-major (rows K-contiguous);
 *             W13 rows 0..I-1 are the gate projection, I..2I-1 the up projection
 *    bf16  :  W13 (2I rows, K = H) then W2 (H rows, K = I), both tiled
 *    MXFP4 :  W13 codes, W2 codes, W13 scales, W2 scales, all tiled
 *  Tiled matrix (R rows, K columns): tiles of 16 rows x KS columns (KS = 32 for
 *  bf16, 128 for MXFP4; K rounded up to a multiple of KS with zero padding),
 *  stored row-tile major then column step; each tile is 64 fragments of 16 bytes
 *  in the order f = 16*g + row%16 with g = (k % KS) / (KS/4): a bf16 fragment is 8
 *  consecutive k, an MXFP4 fragment one 32-element block (OCP MX v1.0 E2M1,
 *  element 2i in the low nibble of byte i).  This is the operand order of the
 *  bf16 MFMA, so a wave reads 1 KB of contiguous memory per load.  MXFP4 E8M0
 *  scales: per row tile the column steps are grouped 16 at a time into 1 KB scale
 *  blocks (the last one padded), row-tile major; in a block, fragment f owns bytes
 *  16f .. 16f+15, byte i being its scale at step 16*block + i, so one 16-byte load
 *  per lane brings its scales for 16 steps.  For bf16 and MXFP4, stored W13
 *  row 16t+q is gate row 8t+q for q < 8 and up row 8t+q-8 otherwise.  W2 is the
 *  down projection.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,         /* bad argument (shape, null or misaligned pointer, range) */
  MOE_EUNSUPPORTED = 2,   /* valid request this build does not implement */
  MOE_ECAPACITY = 3,      /* workspace or buffer too small */
  MOE_EHIP = 4,           /* a HIP runtime call or kernel launch failed */
  MOE_ENOMEM = 5,         /* host allocation failed */
  MOE_ESTATE = 6          /* call out of order (e.g. wave w before wave w-1) */
} moe_status;

/* MOE_MXFP4_A8: MXFP4 weights (the MOE_MXFP4 slot layout) with the gate/up
 * activations quantized to MXFP8 (OCP MX v1.0: E4M3 elements, one E8M0 scale per
 * 32 consecutive elements of a token row, X = floor(log2 max|x|) - 8, round to
 * nearest even, clamp to 448) and multiplied on the scaled FP4 x FP8 MFMA; the
 * down projection stays on the exact path (bf16 intermediate).  A precision
 * trade for prefill throughput (the pages' 8,192-token prefill chunks, "Data Check"
 * claim table, Fig 4a row); the other types never lower activation precision. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2, MOE_MXFP4_A8 = 3 } moe_dtype;

int moe_abi_version(void);
const char* moe_status_str(int status);
const char* moe_last_error(void);

/* Bytes of one expert slot of the given weight type (0 for invalid shapes). */
size_t moe_expert_bytes(int wdt, int H, int I);

/* ------------------------------------------------------------------------- */
/* Top-k gating.  The pages: the model's own routing decides which experts run
 * and the engine leaves it unchanged ("Three mechanisms": bandwidth-adaptive execution; "Key Takeaways").
 * For each token t: the k experts with the largest f32 logits, in descending
 * logit order, equal logits (IEEE equality, -0.0 == +0.0) going to the lower
 * expert index; gate weights are the softmax over the k selected logits (equal,
 * in exact arithmetic, to softmax over all E renormalised over the selection),
 * computed in f32.
 *   logits   [T][E] f32          (read)
 *   topk_ids [T][k] int32        (written)  expert ids, bit-exact
 *   topk_w   [T][k] f32          (written)  gate weights, sum to 1 within rounding */
int moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                   hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Permutation by expert (the grouping step between routing and the grouped FFN;
 * the pages route each token to its experts, "The gap it targets").  Stable
 * counting sort of the pairs r = t*k + j by topk_ids[r]:
 *   counts      [E]    pairs per expert
 *   offsets     [E+1]  exclusive prefix sum, offsets[E] = T*k
 *   sorted_rows [T*k]  r grouped by expert, ascending r within an expert
 *   inv_rows    [T*k]  position of r in sorted_rows
 * Deterministic, bit-exact.  topk_ids values must lie in [0, E). */
int moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                int32_t* sorted_rows, int32_t* inv_rows, hipStream_t stream);

/* moe_route_topk followed by moe_permute on the same buffers, with the same
 * arguments, requirements and results; batches of at most 8 tokens run as one
 * workgroup launch (one launch fewer per decode layer). */
int moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w, int32_t* counts,
              int32_t* offsets, int32_t* sorted_rows, int32_t* inv_rows, hipStream_t stream);

/* Router projection then moe_route: logits[t][e] = sum_h x[t][h] * w_router[e][h]
 * (x [T][H] and w_router [E][H] bf16, f32 accumulation in a fixed order, written
 * to logits [T][E] f32), then top-k gating and the permutation on those logits
 * exactly as moe_route.  H a positive multiple of 8.  The pages leave the model's
 * router as it is ("Three mechanisms", bandwidth-adaptive execution); the plain
 * linear gate of an MoE layer is computed.  Selections follow the f32 logits, so
 * they can differ from an exact-arithmetic selection only where two logits are
 * within the summation error of each other. */
int moe_route_project(const void* x, const void* w_router, int T, int H, int E, int k, float* logits,
                      int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_rows,
                      int32_t* inv_rows, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Expert-slot cache.  The pages: experts that are not in use are kept in host
 * memory and brought to the GPU only when a token is routed to them ("The gap it
 * targets"); in decode, one recency-ordered cache whose keys cover every MoE
 * layer decides which experts stay on the GPU, driven by what the router picks
 * ("Three mechanisms": semantic-aware caching); host copies of the experts are
 * pinned in the layout the GPU computes from, and serving begins with nothing
 * cached ("Three mechanisms": elastic memory management).
 *
 * Keys are (layer, expert), key = layer*n_experts + expert.  The cache starts
 * empty.  For one (step, layer) the active experts (counts > 0) are accessed
 * hits first, then misses, each group in ascending expert id, hit or miss judged
 * against the state before the step; a miss takes the lowest-index free slot,
 * else evicts the least recently used key.  If more experts are active than
 * there are slots, the accesses run in waves of n_slots: the caller runs the FFN
 * of wave w before asking for wave w+1.  The shared expert is never cached. */
typedef struct moe_cache moe_cache;

typedef struct {
  int n_layers;
  int n_experts;
  int n_slots;
  size_t expert_bytes;  /* bytes copied per fill */
  size_t slot_stride;   /* bytes between slots in slot_pool; >= expert_bytes, multiple of 256 */
  void* slot_pool;      /* device, n_slots*slot_stride bytes; NULL = host-only planning handle */
  const void* host_pool_host;               /* pinned, key-major, expert_bytes per key */
  const void* const* host_expert_ptrs_host; /* optional [n_layers*n_experts] pinned pointers; overrides host_pool_host */
  hipStream_t fill_stream;                  /* side stream the fills run on (device handles) */
} moe_cache_desc;

typedef struct {
  int64_t accesses;     /* distinct active experts of the step (all waves) */
  int64_t hits;
  int64_t misses;
  int64_t cold_misses;  /* misses of keys never accessed before */
  int64_t fill_bytes;   /* bytes copied by this call */
  int32_t n_waves;      /* waves this step needs */
  int32_t wave_accesses;/* accesses in the wave this call handled */
  int64_t inplace;      /* misses of the step computed in place (miss split), not filled */
} moe_cache_stats;

typedef struct {
  int32_t slot;
  int32_t layer;
  int32_t expert;
  int32_t wave;
} moe_fill;

int moe_cache_create(const moe_cache_desc* desc, moe_cache** out);
/* Waits for the handle's in-flight fills, then frees it. */
int moe_cache_destroy(moe_cache* c);

/* Device handle.  counts: device [n_experts] (moe_permute output).  For wave 0
 * the counts are copied to the host and the call waits for them (the only host
 * synchronisation of the layer); waves 1.. must follow in order, each after the
 * FFN of the previous wave has been enqueued on compute_stream.  Writes
 * slot_of_expert (device [n_experts]): the slot of each expert in this wave, -1
 * for the rest.  Fills run on the fill stream after all work enqueued on
 * compute_stream so far (write-after-read on victim slots); compute_stream then
 * waits for them (read-after-write).  stats_host (nullable) receives the
 * counters.  On error no key maps to a slot whose bytes may have been
 * overwritten; the rest of the state is as before the call. */
int moe_cache_lookup_fill(moe_cache* c, int layer, const int32_t* counts, int wave,
                          int32_t* slot_of_expert, moe_cache_stats* stats_host, hipStream_t compute_stream);

/* Split lookup, for computing the resident experts while the misses stream in
 * (the pages: the GPU keeps computing what it holds while missing experts are
 * transferred, "Three mechanisms", bandwidth-adaptive execution).  Same plan,
 * fills, ordering of waves and errors as moe_cache_lookup_fill, but two device
 * tables [n_experts] are written on compute_stream: slot_hits holds the slots of
 * the wave's hits (-1 elsewhere) and may be used at once, since hits are never
 * victims of the wave's misses; slot_misses holds the slots of the wave's filled
 * experts (-1 elsewhere) and may be used only after moe_cache_wait_fills.  The
 * caller runs the FFN over slot_hits, then moe_cache_wait_fills, then the FFN over
 * slot_misses (skipped when stats->fill_bytes is 0); the two FFNs write disjoint
 * output rows, so the layer equals the unsplit one bit for bit.  Both pointers
 * must be 16-byte aligned and distinct. */
int moe_cache_lookup_fill_split(moe_cache* c, int layer, const int32_t* counts, int wave, int32_t* slot_hits,
                                int32_t* slot_misses, moe_cache_stats* stats_host, hipStream_t compute_stream);
/* Miss split (the pages: of a step's misses, a share set by the host-link and
 * host-memory bandwidths crosses into GPU memory and the rest is computed where
 * the weights already are, the partial sums merging exactly; "Three mechanisms",
 * bandwidth-adaptive execution).  On one GPU "where the weights are" is pinned
 * host memory read by the GPU in place.  With fill fraction num/den, of a step's
 * m misses (ascending expert id) the first floor(m*num/den + 1/2) are filled as
 * usual and the others are computed in place: they take no slot, evict nothing
 * and leave the recency order as it is (hits are still refreshed).  Default 1/1
 * (every miss filled).  Between steps only (MOE_ESTATE otherwise);
 * 0 <= num <= den, den >= 1. */
int moe_cache_set_fill_fraction(moe_cache* c, int num, int den);
/* moe_cache_lookup_fill_split plus the step's in-place experts: addr_inplace
 * (device [n_experts] uint64, 16-byte aligned) receives, with wave 0, the
 * device-visible address of the pinned host copy of each in-place expert of the
 * step (0 for every other expert, and everywhere for later waves), for
 * moe_grouped_ffn_addr.  The host copies must be pinned memory the GPU can read
 * (hipHostMalloc).  Same ordering rules as the split lookup; the in-place FFN can
 * run while the fills are in flight (it reads only host memory). */
int moe_cache_lookup_fill_inplace(moe_cache* c, int layer, const int32_t* counts, int wave, int32_t* slot_hits,
                                  int32_t* slot_misses, uint64_t* addr_inplace, moe_cache_stats* stats_host,
                                  hipStream_t compute_stream);
/* The in-place experts of the last step begun (ascending id); experts_host has
 * room for n_experts.  Works on host-only and device handles. */
int moe_cache_step_inplace(const moe_cache* c, int32_t* experts_host, int* n_host);

/* Elastic resize of the slot pool (the pages: the expert pool grows and shrinks
 * with the memory the GPU can spare, "Three mechanisms", elastic memory
 * management).  Between steps only (MOE_ESTATE while a step's waves are open):
 * keeps the min(n_slots, resident) most recently used keys, most recent first in
 * new slots 0, 1, ..., with their recency; the others are dropped (later accesses
 * miss).  Nothing is read from the host pool.  Device handle: slot_pool is the new
 * pool (256-byte aligned, n_slots * slot_stride bytes, stride >= expert_bytes and a
 * multiple of 256, not overlapping the current pool); in-flight fills are waited
 * for, then each kept expert is copied from its old slot on `stream` (after the
 * work already on it); the next lookup makes its compute stream, and through it
 * its fills, wait for those copies, so `stream` may differ from the compute
 * stream; the caller may free the old pool once that work is done.  Host-only handle:
 * slot_pool must be NULL.  moved_from_host (nullable, [n_slots]) receives the old
 * slot of each new slot's expert, -1 for an empty slot.  On error the cache is
 * unchanged. */
int moe_cache_resize(moe_cache* c, int n_slots, void* slot_pool, size_t slot_stride, int32_t* moved_from_host,
                     hipStream_t stream);
/* Makes compute_stream wait for the fills of the last split lookup (no-op if it
 * had none or they were already waited for).  A later lookup on the handle
 * inserts this wait itself if the caller skipped it. */
int moe_cache_wait_fills(moe_cache* c, hipStream_t compute_stream);

/* Same policy without any device work: counts_host in, slot table and the list
 * of fills (slot, layer, expert, wave) out, for the caller to perform.  Works on
 * host-only and device handles.  max_fills >= n_slots is always enough. */
int moe_cache_lookup_host(moe_cache* c, int layer, const int32_t* counts_host, int wave,
                          int32_t* slot_of_expert_host, moe_fill* fills_host, int max_fills,
                          int* n_fills_host, moe_cache_stats* stats_host);

/* Snapshot: key held by each slot (-1 if empty) and its last-use tick. */
int moe_cache_state(const moe_cache* c, int64_t* key_of_slot_host, int64_t* tick_of_slot_host);

/* Test hook for failure handling: make the (n+1)-th fill from now fail with
 * MOE_EHIP without issuing it (n < 0 disables). */
int moe_cache_inject_fill_failure(moe_cache* c, int64_t n);

/* ------------------------------------------------------------------------- */
/* Grouped SwiGLU expert FFN.  The pages: GPU expert compute on cached and filled
 * experts, exact, with precision never lowered ("Three mechanisms";
 * "Key Takeaways").  For every expert e with counts > 0 and slot_of_expert[e] >= 0,
 * for each of its pairs p in [offsets[e], offsets[e+1]) with token t = sorted_rows[p]/k:
 *     out_rows[p] = W2 . ( SiLU(Wgate . x[t]) * (Wup . x[t]) ),   SiLU(z) = z/(1+e^-z)
 * with the expert's weights at slot_pool + slot*slot_stride.  Rows of experts
 * without a slot are not written.  If shared_w is non-null, the shared expert
 * (intermediate I_shared, same layout, always resident) is applied to every
 * token: shared_out[t] = FFN_shared(x[t]).
 *   wdt         weight type (moe_dtype)
 *   x           [T][H] f32 for MOE_F32, bf16 otherwise
 *   out_rows    [T*k][H] f32, indexed by sorted position
 *   shared_out  [T][H] f32 (required iff shared_w)
 *   workspace   >= moe_grouped_ffn_workspace() bytes of device memory
 * Arithmetic: f32 weights use f32 FMA; bf16 and MXFP4 weights use bf16 MFMA
 * with f32 accumulation (MXFP4 is expanded to bf16 exactly), and the SwiGLU
 * intermediate is rounded to bf16.  MOE_MXFP4_A8: gate/up multiply the E2M1
 * weights by the MXFP8 activations exactly (f32 accumulation), H, I and
 * I_shared multiples of 128 (MOE_EUNSUPPORTED otherwise). */
size_t moe_grouped_ffn_workspace(int T, int k, int E, int H, int I, int I_shared, int wdt);
int moe_grouped_ffn(int wdt, const void* slot_pool, size_t slot_stride, const int32_t* slot_of_expert,
                    const void* shared_w, int I_shared, const void* x, const int32_t* offsets,
                    const int32_t* sorted_rows, int T, int k, int E, int H, int I, float* out_rows,
                    float* shared_out, void* workspace, size_t ws_bytes, hipStream_t stream);
/* moe_grouped_ffn over experts addressed one by one instead of through slots:
 * expert_addr (device [E] uint64) holds the address of each expert's weights
 * (same layout as a slot; 16-byte aligned; device memory or pinned host memory
 * the GPU can read), 0 for experts not computed by this call.  Used for the
 * in-place half of the miss split; the results for an expert are bit for bit
 * those of moe_grouped_ffn on a slot holding the same bytes. */
int moe_grouped_ffn_addr(int wdt, const uint64_t* expert_addr, const void* shared_w, int I_shared, const void* x,
                         const int32_t* offsets, const int32_t* sorted_rows, int T, int k, int E, int H, int I,
                         float* out_rows, float* shared_out, void* workspace, size_t ws_bytes, hipStream_t stream);

/* moe_grouped_ffn for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops or harnesses that forbid hipMalloc): the same
 * arguments and results without the workspace.  The SwiGLU intermediate goes to a
 * fixed array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends; its device address is looked up on the first
 * call on each device (with that device current).  The call allocates nothing.
 * MOE_ECAPACITY if moe_grouped_ffn_workspace() for the shape exceeds the array
 * (32 MiB: e.g. up to 8192 token-expert pairs at I = 2048).  Every call on one GPU
 * uses the same array, so calls that overlap on one GPU (several streams or
 * threads) race; nothing in it needs clearing between calls. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int moe_grouped_ffn_noalloc(int wdt, const void* slot_pool, size_t slot_stride, const int32_t* slot_of_expert,
                            const void* shared_w, int I_shared, const void* x, const int32_t* offsets,
                            const int32_t* sorted_rows, int T, int k, int E, int H, int I, float* out_rows,
                            float* shared_out, hipStream_t stream);

/* MXFP8 quantization of activations, as MOE_MXFP4_A8 applies it before gate/up
 * (OCP Microscaling Formats v1.0, the format of the pages' MXFP4 build, "Results"):
 * x [T][H] bf16 (H a multiple of 32) -> codes [T][H] E4M3 bytes and scales
 * [T][H/32] E8M0 bytes; per 32-element block of a row X = floor(log2 max|x|) - 8
 * (X = -127 for an all-zero block), scale X + 127, each element x / 2^X rounded to
 * the nearest E4M3 value, ties to even, clamped to +-448.  Deterministic: the codes
 * depend on x alone.  codes 16-byte aligned. */
int moe_mx8_quantize(const void* x, int T, int H, uint8_t* codes, uint8_t* scales, hipStream_t stream);

/* Which kernel family moe_grouped_ffn runs for a shape (the results are the same
 * computation either way): MOE_FFN_WEIGHT_STREAM (decode-sized batches: each
 * expert's weights stream once past its few tokens) or MOE_FFN_GROUPED_GEMM
 * (32 or more (token, expert) pairs per expert on average, bf16 or MXFP4 weights
 * with H, I and I_shared multiples of 128; MOE_MXFP4_A8 always).  -1 for an
 * invalid shape. */
enum { MOE_FFN_WEIGHT_STREAM = 0, MOE_FFN_GROUPED_GEMM = 1 };
int moe_grouped_ffn_kind(int T, int k, int E, int H, int I, int I_shared, int wdt);
/* The two phases of moe_grouped_ffn, same arguments: gate_up writes the SwiGLU
 * intermediate into the workspace, down reads it.  moe_grouped_ffn is exactly
 * gate_up followed by down on the same stream. */
int moe_grouped_ffn_gate_up(int wdt, const void* slot_pool, size_t slot_stride, const int32_t* slot_of_expert,
                            const void* shared_w, int I_shared, const void* x, const int32_t* offsets,
                            const int32_t* sorted_rows, int T, int k, int E, int H, int I, float* out_rows,
                            float* shared_out, void* workspace, size_t ws_bytes, hipStream_t stream);
int moe_grouped_ffn_down(int wdt, const void* slot_pool, size_t slot_stride, const int32_t* slot_of_expert,
                         const void* shared_w, int I_shared, const void* x, const int32_t* offsets,
                         const int32_t* sorted_rows, int T, int k, int E, int H, int I, float* out_rows,
                         float* shared_out, void* workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Combine.  The pages: the partial sums are added without approximation ("Three mechanisms").
 *   y[t] = sum_{j=0..k-1} topk_w[t][j] * out_rows[inv_rows[t*k+j]]  (+ shared_out[t])
 * in f32, j in increasing order (fused multiply-add), then the shared term,
 * then one rounding to ydt (MOE_F32, or MOE_BF16 with round-to-nearest-even).
 * The fixed order makes the result independent of how experts were split into
 * cache waves.  y: [T][H] of ydt. */
int moe_combine(const float* out_rows, const float* topk_w, const int32_t* inv_rows, const float* shared_out,
                int T, int k, int H, void* y, int ydt, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Whole-layer streaming for prefill.  The pages: in prefill, whole layers are
 * copied into one of two device buffers, the next layer arriving while the
 * current one is computed from the other ("Three mechanisms": semantic-aware
 * caching).  Two device banks each hold one layer
 * (layer_bytes); a fill copies one layer from pinned host memory with one
 * hipMemcpyAsync on the fill stream.  Ordering: fill(bank) waits for the last
 * release(bank); acquire(bank) makes the compute stream wait for the last
 * fill(bank); release(bank) marks the compute work enqueued so far as the last
 * reader of the bank.  Typical loop: fill(0, b0); for l: fill(l+1, b(l+1));
 * acquire(b(l)); compute(l); release(b(l)). */
typedef struct moe_layer_stream moe_layer_stream;

typedef struct {
  int n_layers;
  size_t layer_bytes;
  const void* host_layers_host;            /* pinned [n_layers][layer_bytes] */
  const void* const* host_layer_ptrs_host; /* optional [n_layers] pinned pointers; overrides host_layers_host */
  void* banks[2];                          /* device, layer_bytes each */
  hipStream_t fill_stream;
} moe_layer_stream_desc;

int moe_layer_stream_create(const moe_layer_stream_desc* desc, moe_layer_stream** out);
int moe_layer_stream_destroy(moe_layer_stream* s);
int moe_layer_stream_fill(moe_layer_stream* s, int layer, int bank);
int moe_layer_stream_acquire(moe_layer_stream* s, int bank, hipStream_t compute_stream);
int moe_layer_stream_release(moe_layer_stream* s, int bank, hipStream_t compute_stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
