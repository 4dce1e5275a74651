// api.cpp -- the C ABI of libmoe (declared in include/moe.h): argument checks,
// error reporting, kernel dispatch, the device side of the expert-slot cache
// (fills on a side stream fenced by events) and the prefill layer streamer.
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "cache_core.hpp"
#include "common.hpp"
#include "kernels.hpp"

// A roctx range around every call of the C ABI, named by the entry point, for
// rocprofv3 --marker-trace (a no-op when no tool is attached).
struct CallRange {
  explicit CallRange(const char* name) { roctxRangePushA(name); }
  ~CallRange() { roctxRangePop(); }
  CallRange(const CallRange&) = delete;
  CallRange& operator=(const CallRange&) = delete;
};

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, ...)                          \
  do {                                              \
    if (!(cond)) return fail(MOE_EINVAL, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p)                                                              \
  do {                                                                              \
    if ((p) == nullptr) return fail(MOE_EINVAL, "%s must not be null", #p);         \
    if (!aligned16(p)) return fail(MOE_EINVAL, "%s must be 16-byte aligned", #p);   \
  } while (0)

int check_dims(int wdt, int H, int I, const char* what) {
  if (wdt < MOE_F32 || wdt > MOE_MXFP4_A8) return fail(MOE_EINVAL, "%s: unknown weight type %d", what, wdt);
  if (H <= 0 || I <= 0) return fail(MOE_EINVAL, "%s: H=%d and I=%d must be positive", what, H, I);
  const int q = wdt == MOE_F32 ? 4 : 32;
  if (H % q || I % q) return fail(MOE_EINVAL, "%s: H=%d and I=%d must be multiples of %d", what, H, I, q);
  return MOE_OK;
}

int check_routing(int T, int E, int k) {
  if (T < 0) return fail(MOE_EINVAL, "T=%d must be >= 0", T);
  if (E < 1 || E > 1024) return fail(MOE_EINVAL, "E=%d must be in [1, 1024]", E);
  if (k < 1 || k > 32 || k > E) return fail(MOE_EINVAL, "k=%d must be in [1, min(E, 32)]", k);
  if ((int64_t)T * k >= ((int64_t)1 << 31)) return fail(MOE_EINVAL, "T*k must be < 2^31");
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
  const CallRange range_(__func__);
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported";
    case MOE_ECAPACITY: return "capacity";
    case MOE_EHIP: return "HIP error";
    case MOE_ENOMEM: return "out of host memory";
    case MOE_ESTATE: return "call out of order";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_expert_bytes(int wdt, int H, int I) {
  const CallRange range_(__func__);
  if (H <= 0 || I <= 0) return 0;
  switch (wdt) {
    case MOE_F32: return (size_t)4 * 3 * H * I;
    case MOE_BF16: return (H % 32 || I % 32) ? 0 : (size_t)2 * 3 * H * I;
    case MOE_MXFP4:
    case MOE_MXFP4_A8: {
      if (H % 32 || I % 32) return 0;
      // tiled: 1 KB of codes per 16-row x 128-column tile (K padded to 128), and per
      // row tile one 1 KB scale block per 16 column steps
      const size_t k13 = (H + 127) / 128, k2 = (I + 127) / 128;
      const size_t r13 = 2 * I / 16, r2 = H / 16;
      return (r13 * k13 + r2 * k2) * 1024 + (r13 * ((k13 + 15) / 16) + r2 * ((k2 + 15) / 16)) * 1024;
    }
    default: return 0;
  }
}

// ---------------------------------------------------------------------------
int moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  const CallRange range_(__func__);
  if (int rc = check_routing(T, E, k)) return rc;
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(logits);
  REQUIRE_PTR(topk_ids);
  REQUIRE_PTR(topk_w);
  hipError_t e = moe::launch_topk(logits, T, E, k, topk_ids, topk_w, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route_topk launch");
}

int moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                int32_t* sorted_rows, int32_t* inv_rows, hipStream_t stream) {
  const CallRange range_(__func__);
  if (int rc = check_routing(T, E, k)) return rc;
  REQUIRE_PTR(counts);
  REQUIRE_PTR(offsets);
  if (T > 0) {
    REQUIRE_PTR(topk_ids);
    REQUIRE_PTR(sorted_rows);
    REQUIRE_PTR(inv_rows);
  }
  hipError_t e = moe::launch_permute(topk_ids, T, k, E, counts, offsets, sorted_rows, inv_rows, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_permute launch");
}

int moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w, int32_t* counts,
              int32_t* offsets, int32_t* sorted_rows, int32_t* inv_rows, hipStream_t stream) {
  const CallRange range_(__func__);
  if (int rc = check_routing(T, E, k)) return rc;
  REQUIRE_PTR(counts);
  REQUIRE_PTR(offsets);
  if (T > 0) {
    REQUIRE_PTR(logits);
    REQUIRE_PTR(topk_ids);
    REQUIRE_PTR(topk_w);
    REQUIRE_PTR(sorted_rows);
    REQUIRE_PTR(inv_rows);
  }
  hipError_t e = moe::launch_route(logits, T, E, k, topk_ids, topk_w, counts, offsets, sorted_rows, inv_rows, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route launch");
}

int moe_route_project(const void* x, const void* w_router, int T, int H, int E, int k, float* logits,
                      int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_rows,
                      int32_t* inv_rows, hipStream_t stream) {
  const CallRange range_(__func__);
  if (int rc = check_routing(T, E, k)) return rc;
  if (H <= 0 || H % 8) return fail(MOE_EINVAL, "moe_route_project: H=%d must be a positive multiple of 8", H);
  REQUIRE_PTR(counts);
  REQUIRE_PTR(offsets);
  if (T > 0) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(w_router);
    REQUIRE_PTR(logits);
    REQUIRE_PTR(topk_ids);
    REQUIRE_PTR(topk_w);
    REQUIRE_PTR(sorted_rows);
    REQUIRE_PTR(inv_rows);
  }
  hipError_t e = moe::launch_router_logits(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router), T,
                                           H, E, logits, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_route_project projection launch");
  e = moe::launch_route(logits, T, E, k, topk_ids, topk_w, counts, offsets, sorted_rows, inv_rows, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route_project route launch");
}

int moe_combine(const float* out_rows, const float* topk_w, const int32_t* inv_rows, const float* shared_out, int T,
                int k, int H, void* y, int ydt, hipStream_t stream) {
  const CallRange range_(__func__);
  if (T < 0 || k < 1 || k > 32 || H <= 0 || H % 4) return fail(MOE_EINVAL, "moe_combine: bad T=%d k=%d H=%d", T, k, H);
  if (ydt != MOE_F32 && ydt != MOE_BF16) return fail(MOE_EINVAL, "moe_combine: ydt must be MOE_F32 or MOE_BF16");
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(out_rows);
  REQUIRE_PTR(topk_w);
  REQUIRE_PTR(inv_rows);
  REQUIRE_PTR(y);
  if (shared_out && !aligned16(shared_out)) return fail(MOE_EINVAL, "shared_out must be 16-byte aligned");
  hipError_t e = moe::launch_combine(out_rows, topk_w, inv_rows, shared_out, T, k, H, y, ydt == MOE_BF16, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_combine launch");
}

// ---------------------------------------------------------------------------
size_t moe_grouped_ffn_workspace(int T, int k, int E, int H, int I, int I_shared, int wdt) {
  const CallRange range_(__func__);
  (void)E;
  if (T < 0 || k < 1 || H <= 0 || I <= 0 || I_shared < 0 || wdt < MOE_F32 || wdt > MOE_MXFP4_A8) return 0;
  return moe::ffn_workspace_bytes(wdt, T, k, H, I, I_shared);
}

namespace {

enum { PHASE_GATE_UP = 1, PHASE_DOWN = 2 };

// Prefill-sized batches (32 or more pairs per expert on average) take the grouped
// GEMM kernels, smaller ones the weight-streaming kernels; both compute the same
// thing.
constexpr int64_t kPrefillMinPairs = 32;
bool uses_prefill(int wdt, int T, int k, int E, int H, int I, int I_shared) {
  if (wdt == MOE_MXFP4_A8) return true;  // the native FP4 path has only the grouped GEMM
  return (int64_t)T * k >= kPrefillMinPairs * E && moe::prefill_supported(wdt, H, I, I_shared);
}

int grouped_ffn(int phases, int wdt, const void* slot_pool, size_t slot_stride, const int32_t* slot_of_expert,
                const void* shared_w, int I_shared, const void* x, const int32_t* offsets, const int32_t* sorted_rows,
                int T, int k, int E, int H, int I, float* out_rows, float* shared_out, void* workspace,
                size_t ws_bytes, hipStream_t stream, const uint64_t* expert_addr = nullptr) {
  if (int rc = check_routing(T, E, k)) return rc;
  if (int rc = check_dims(wdt, H, I, "moe_grouped_ffn")) return rc;
  if (shared_w) {
    if (int rc = check_dims(wdt, H, I_shared, "moe_grouped_ffn shared expert")) return rc;
    REQUIRE_PTR(shared_w);
    REQUIRE_PTR(shared_out);
  } else {
    I_shared = 0;
  }
  if (T == 0) return MOE_OK;
  if (expert_addr) {
    REQUIRE_PTR(expert_addr);
  } else {
    REQUIRE_PTR(slot_pool);
    REQUIRE_PTR(slot_of_expert);
  }
  REQUIRE_PTR(x);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(sorted_rows);
  REQUIRE_PTR(out_rows);
  REQUIRE_PTR(workspace);
  const size_t eb = moe_expert_bytes(wdt, H, I);
  if (!expert_addr)
    REQUIRE(slot_stride >= eb && slot_stride % 16 == 0,
            "slot_stride=%zu must be >= expert bytes %zu and a multiple of 16", slot_stride, eb);
  if (wdt == MOE_MXFP4_A8 && !moe::prefill_supported(MOE_MXFP4, H, I, I_shared))
    return fail(MOE_EUNSUPPORTED, "MXFP4 weights with MXFP8 activations need H, I and I_shared multiples of 128");
  const size_t need = moe::ffn_workspace_bytes(wdt, T, k, H, I, I_shared);
  if (ws_bytes < need) return fail(MOE_ECAPACITY, "workspace %zu bytes < %zu needed", ws_bytes, need);
  moe::FfnArgs a;
  a.slot_pool = static_cast<const uint8_t*>(slot_pool);
  a.slot_stride = slot_stride;
  a.slot_of_expert = expert_addr ? nullptr : slot_of_expert;
  a.expert_addr = expert_addr;
  a.shared_w = static_cast<const uint8_t*>(shared_w);
  a.x = x;
  a.offsets = offsets;
  a.sorted_rows = sorted_rows;
  a.out_rows = out_rows;
  a.shared_out = shared_out;
  a.h = workspace;
  a.T = T;
  a.k = k;
  a.E = E;
  a.H = H;
  a.I = I;
  a.I_shared = I_shared;
  a.h_ld = I > I_shared ? I : I_shared;
  a.routed_items = (int)((int64_t)T * k < E ? (int64_t)T * k : E);
  a.pass_rows = 0;  // one item per expert (the decode launchers split items into passes)
  a.lds_rows = 0;  // set per launch by the decode launchers
  a.xq = nullptr;
  a.xs = nullptr;
  const bool prefill = uses_prefill(wdt, T, k, E, H, I, I_shared);
  if (wdt == MOE_MXFP4_A8) {
    // native FP4 path: x -> MXFP8 in the workspace, gate_up on the scaled MFMA, down
    // as the MXFP4 grouped GEMM (bf16 intermediate)
    uint8_t* xq = static_cast<uint8_t*>(workspace) + moe::ffn_workspace_xq_offset(T, k, I, I_shared);
    a.xq = xq;
    a.xs = xq + (size_t)T * H;
    if (phases & PHASE_GATE_UP) {
      hipError_t e = moe::launch_mx8_quantize(static_cast<const uint16_t*>(x), T, H, xq, xq + (size_t)T * H, stream);
      if (e == hipSuccess) e = moe::launch_native_gate_up(a, stream);
      if (e != hipSuccess) return hip_fail(e, "moe_grouped_ffn native gate_up launch");
    }
    if (phases & PHASE_DOWN) {
      hipError_t e = moe::launch_prefill_down(MOE_MXFP4, a, stream);
      if (e != hipSuccess) return hip_fail(e, "moe_grouped_ffn down launch");
    }
    return MOE_OK;
  }
  if (phases & PHASE_GATE_UP) {
    hipError_t e = prefill ? moe::launch_prefill_gate_up(wdt, a, stream) : moe::launch_ffn_gate_up(wdt, a, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_grouped_ffn gate_up launch");
  }
  if (phases & PHASE_DOWN) {
    hipError_t e = prefill ? moe::launch_prefill_down(wdt, a, stream) : moe::launch_ffn_down(wdt, a, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_grouped_ffn down launch");
  }
  return MOE_OK;
}

}  // namespace

int moe_grouped_ffn_addr(int wdt, const uint64_t* expert_addr, const void* shared_w, int I_shared, const void* x,
                         const int32_t* offsets, const int32_t* sorted_rows, int T, int k, int E, int H, int I,
                         float* out_rows, float* shared_out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  const CallRange range_(__func__);
  return grouped_ffn(PHASE_GATE_UP | PHASE_DOWN, wdt, nullptr, 0, nullptr, shared_w, I_shared, x, offsets, sorted_rows,
                     T, k, E, H, I, out_rows, shared_out, workspace, ws_bytes, stream, expert_addr);
}

int moe_mx8_quantize(const void* x, int T, int H, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const CallRange range_(__func__);
  if (T < 0 || H <= 0 || H % 32) return fail(MOE_EINVAL, "moe_mx8_quantize: T=%d, H=%d (a multiple of 32)", T, H);
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(codes);
  if (!scales) return fail(MOE_EINVAL, "scales must not be null");
  hipError_t e = moe::launch_mx8_quantize(static_cast<const uint16_t*>(x), T, H, codes, scales, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_mx8_quantize launch");
}

int moe_grouped_ffn_kind(int T, int k, int E, int H, int I, int I_shared, int wdt) {
  const CallRange range_(__func__);
  if (check_routing(T, E, k) || check_dims(wdt, H, I, "moe_grouped_ffn_kind")) return -1;
  if (I_shared && check_dims(wdt, H, I_shared, "moe_grouped_ffn_kind shared expert")) return -1;
  if (wdt == MOE_MXFP4_A8 && !moe::prefill_supported(MOE_MXFP4, H, I, I_shared)) return -1;
  return uses_prefill(wdt, T, k, E, H, I, I_shared) ? MOE_FFN_GROUPED_GEMM : MOE_FFN_WEIGHT_STREAM;
}

int moe_grouped_ffn(int wdt, const void* slot_pool, size_t slot_stride, const int32_t* slot_of_expert,
                    const void* shared_w, int I_shared, const void* x, const int32_t* offsets,
                    const int32_t* sorted_rows, int T, int k, int E, int H, int I, float* out_rows,
                    float* shared_out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  const CallRange range_(__func__);
  return grouped_ffn(PHASE_GATE_UP | PHASE_DOWN, wdt, slot_pool, slot_stride, slot_of_expert, shared_w, I_shared, x,
                     offsets, sorted_rows, T, k, E, H, I, out_rows, shared_out, workspace, ws_bytes, stream);
}

int moe_grouped_ffn_gate_up(int wdt, const void* slot_pool, size_t slot_stride, const int32_t* slot_of_expert,
                            const void* shared_w, int I_shared, const void* x, const int32_t* offsets,
                            const int32_t* sorted_rows, int T, int k, int E, int H, int I, float* out_rows,
                            float* shared_out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  const CallRange range_(__func__);
  return grouped_ffn(PHASE_GATE_UP, wdt, slot_pool, slot_stride, slot_of_expert, shared_w, I_shared, x, offsets,
                     sorted_rows, T, k, E, H, I, out_rows, shared_out, workspace, ws_bytes, stream);
}

int moe_grouped_ffn_down(int wdt, const void* slot_pool, size_t slot_stride, const int32_t* slot_of_expert,
                         const void* shared_w, int I_shared, const void* x, const int32_t* offsets,
                         const int32_t* sorted_rows, int T, int k, int E, int H, int I, float* out_rows,
                         float* shared_out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  const CallRange range_(__func__);
  return grouped_ffn(PHASE_DOWN, wdt, slot_pool, slot_stride, slot_of_expert, shared_w, I_shared, x, offsets,
                     sorted_rows, T, k, E, H, I, out_rows, shared_out, workspace, ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free grouped FFN.  The SwiGLU intermediate goes to a fixed device
// array instead of a caller workspace.  Every GPU the library runs on holds its
// own copy of the array (MOE_NOALLOC_SCRATCH_BYTES) until the process ends; its
// address on a device is looked up once, with that device current, and kept.  In
// host code `scratch` names a host-side stand-in, never the device memory: only
// the looked-up pointer is handed to kernels.
namespace {

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "moe_grouped_ffn_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_EUNSUPPORTED, "moe_grouped_ffn_noalloc: device %d beyond the %d this build tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "moe_grouped_ffn_noalloc: hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_EHIP, "moe_grouped_ffn_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_grouped_ffn_noalloc(int wdt, const void* slot_pool, size_t slot_stride, const int32_t* slot_of_expert,
                            const void* shared_w, int I_shared, const void* x, const int32_t* offsets,
                            const int32_t* sorted_rows, int T, int k, int E, int H, int I, float* out_rows,
                            float* shared_out, hipStream_t stream) {
  const CallRange range_(__func__);
  if (int rc = check_routing(T, E, k)) return rc;
  if (int rc = check_dims(wdt, H, I, "moe_grouped_ffn_noalloc")) return rc;
  if (I_shared < 0) return fail(MOE_EINVAL, "moe_grouped_ffn_noalloc: I_shared=%d < 0", I_shared);
  const size_t need = moe::ffn_workspace_bytes(wdt, T, k, H, I, shared_w ? I_shared : 0);
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ECAPACITY, "moe_grouped_ffn_noalloc: the intermediate needs %zu bytes, more than the %zu of "
                "the fixed scratch array", need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int rc = scratch_of_current_device(&ws)) return rc;
  return grouped_ffn(PHASE_GATE_UP | PHASE_DOWN, wdt, slot_pool, slot_stride, slot_of_expert, shared_w, I_shared, x,
                     offsets, sorted_rows, T, k, E, H, I, out_rows, shared_out, ws, MOE_NOALLOC_SCRATCH_BYTES,
                     stream);
}

}  // extern "C"

// ===========================================================================
// Expert-slot cache
// ===========================================================================
struct moe_cache {
  moe::LruCore core;
  moe_cache_desc desc;
  bool device = false;
  int32_t* counts_pinned = nullptr;       // [E]
  int32_t* stage_pinned = nullptr;        // [kStages][2E] (a split lookup uploads two tables)
  uint64_t* stage_addr_pinned = nullptr;  // [kStages][E] (in-place expert addresses)
  std::vector<uint64_t> dev_addr;         // [L*E] device-visible address of each host copy (0: not looked up)
  hipEvent_t stage_ev[8] = {};
  bool stage_used[8] = {};
  int stage_next = 0;
  hipEvent_t ev_counts = nullptr, ev_compute = nullptr, ev_fill = nullptr;
  hipEvent_t ev_move = nullptr;           // end of the last resize's moves (on the caller's stream)
  bool fill_pending = false;              // a split lookup's fills not yet waited for
  bool move_pending = false;              // a resize's moves not yet ordered before the compute stream
  int64_t fail_after = -1;                // injected failure: fills left before one fails
  std::vector<moe::PlannedFill> fills;
  std::vector<int32_t> table;

  moe_cache(const moe_cache_desc& d)
      : core(d.n_slots, d.n_layers, d.n_experts),
        desc(d),
        dev_addr((size_t)d.n_layers * d.n_experts, 0),
        table(d.n_experts) {}
};

namespace {
constexpr int kStages = 8;

const void* host_src(const moe_cache* c, int layer, int expert) {
  const int64_t key = (int64_t)layer * c->desc.n_experts + expert;
  if (c->desc.host_expert_ptrs_host) return c->desc.host_expert_ptrs_host[key];
  return static_cast<const uint8_t*>(c->desc.host_pool_host) + (size_t)key * c->desc.expert_bytes;
}

void fill_stats(const moe_cache* c, int nacc, int64_t bytes, moe_cache_stats* st) {
  if (!st) return;
  const moe::StepStats& s = c->core.step_stats();
  st->accesses = s.accesses;
  st->hits = s.hits;
  st->misses = s.misses;
  st->cold_misses = s.cold_misses;
  st->fill_bytes = bytes;
  st->n_waves = s.n_waves;
  st->wave_accesses = nacc;
  st->inplace = s.inplace;
}

// Shared between the host and device lookups: open/validate the step and plan the wave.
int plan(moe_cache* c, int layer, const int32_t* counts_host, int wave, int* nacc) {
  if (layer < 0 || layer >= c->desc.n_layers) return fail(MOE_EINVAL, "layer %d out of range", layer);
  if (wave < 0) return fail(MOE_EINVAL, "wave %d < 0", wave);
  if (wave == 0) {
    c->core.begin_step(layer, counts_host);
  } else if (!c->core.step_open() || c->core.next_wave() != wave) {
    return fail(MOE_ESTATE, "wave %d requested, expected %d", wave,
                c->core.step_open() ? c->core.next_wave() : 0);
  }
  *nacc = c->core.plan_wave(wave, c->table.data(), c->fills);
  return MOE_OK;
}

// Returns true if the injected failure fires for the next fill.
bool injected_failure(moe_cache* c) {
  if (c->fail_after < 0) return false;
  if (c->fail_after == 0) {
    c->fail_after = -1;
    return true;
  }
  --c->fail_after;
  return false;
}

void invalidate_upto(moe_cache* c, size_t n_touched) {
  std::vector<int32_t> slots;
  for (size_t i = 0; i < n_touched && i < c->fills.size(); ++i) slots.push_back(c->fills[i].slot);
  c->core.invalidate(slots);
}

}  // namespace

extern "C" {

int moe_cache_create(const moe_cache_desc* d, moe_cache** out) {
  const CallRange range_(__func__);
  if (!d || !out) return fail(MOE_EINVAL, "moe_cache_create: null argument");
  *out = nullptr;
  if (d->n_layers < 1 || d->n_experts < 1 || d->n_experts > 1024 || d->n_slots < 1)
    return fail(MOE_EINVAL, "moe_cache_create: bad sizes layers=%d experts=%d slots=%d", d->n_layers, d->n_experts,
                d->n_slots);
  const bool device = d->slot_pool != nullptr;
  if (device) {
    if (d->expert_bytes == 0 || d->slot_stride < d->expert_bytes || d->slot_stride % 256)
      return fail(MOE_EINVAL, "moe_cache_create: slot_stride must be >= expert_bytes and a multiple of 256");
    if (((uintptr_t)d->slot_pool & 255u) != 0) return fail(MOE_EINVAL, "slot_pool must be 256-byte aligned");
    if (!d->host_pool_host && !d->host_expert_ptrs_host)
      return fail(MOE_EINVAL, "moe_cache_create: a host pool or host pointer table is required");
  }
  moe_cache* c = new (std::nothrow) moe_cache(*d);
  if (!c) return fail(MOE_ENOMEM, "moe_cache_create: out of memory");
  c->device = device;
  if (device) {
    hipError_t e = hipHostMalloc((void**)&c->counts_pinned, sizeof(int32_t) * d->n_experts, hipHostMallocDefault);
    if (e == hipSuccess)
      e = hipHostMalloc((void**)&c->stage_pinned, sizeof(int32_t) * 2 * d->n_experts * kStages, hipHostMallocDefault);
    if (e == hipSuccess)
      e = hipHostMalloc((void**)&c->stage_addr_pinned, sizeof(uint64_t) * d->n_experts * kStages,
                        hipHostMallocDefault);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_counts, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_compute, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_fill, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_move, hipEventDisableTiming);
    for (int i = 0; i < kStages && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&c->stage_ev[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      moe_cache_destroy(c);
      return hip_fail(e, "moe_cache_create");
    }
  }
  *out = c;
  return MOE_OK;
}

int moe_cache_destroy(moe_cache* c) {
  const CallRange range_(__func__);
  if (!c) return MOE_OK;
  int rc = MOE_OK;
  if (c->device) {
    if (c->ev_fill) {
      hipError_t e = hipEventSynchronize(c->ev_fill);
      if (e != hipSuccess) rc = hip_fail(e, "moe_cache_destroy: waiting for fills");
    }
    for (int i = 0; i < kStages; ++i)
      if (c->stage_ev[i]) {
        if (c->stage_used[i]) (void)hipEventSynchronize(c->stage_ev[i]);
        (void)hipEventDestroy(c->stage_ev[i]);
      }
    if (c->ev_counts) (void)hipEventDestroy(c->ev_counts);
    if (c->ev_compute) (void)hipEventDestroy(c->ev_compute);
    if (c->ev_fill) (void)hipEventDestroy(c->ev_fill);
    if (c->ev_move) {
      if (c->move_pending) (void)hipEventSynchronize(c->ev_move);
      (void)hipEventDestroy(c->ev_move);
    }
    if (c->counts_pinned) (void)hipHostFree(c->counts_pinned);
    if (c->stage_pinned) (void)hipHostFree(c->stage_pinned);
    if (c->stage_addr_pinned) (void)hipHostFree(c->stage_addr_pinned);
  }
  delete c;
  return rc;
}

int moe_cache_inject_fill_failure(moe_cache* c, int64_t n) {
  const CallRange range_(__func__);
  if (!c) return fail(MOE_EINVAL, "null cache");
  c->fail_after = n < 0 ? -1 : n;
  return MOE_OK;
}

int moe_cache_state(const moe_cache* c, int64_t* key_of_slot_host, int64_t* tick_of_slot_host) {
  const CallRange range_(__func__);
  if (!c || !key_of_slot_host || !tick_of_slot_host) return fail(MOE_EINVAL, "moe_cache_state: null argument");
  c->core.state(key_of_slot_host, tick_of_slot_host);
  return MOE_OK;
}

int moe_cache_lookup_host(moe_cache* c, int layer, const int32_t* counts_host, int wave, int32_t* slot_of_expert_host,
                          moe_fill* fills_host, int max_fills, int* n_fills_host, moe_cache_stats* stats_host) {
  const CallRange range_(__func__);
  if (!c || !slot_of_expert_host || !n_fills_host) return fail(MOE_EINVAL, "moe_cache_lookup_host: null argument");
  if (wave == 0 && !counts_host) return fail(MOE_EINVAL, "moe_cache_lookup_host: counts_host is required for wave 0");
  int nacc = 0;
  if (int rc = plan(c, layer, counts_host, wave, &nacc)) return rc;
  if ((int)c->fills.size() > max_fills || (!fills_host && !c->fills.empty())) {
    c->core.abort_step();
    return fail(MOE_ECAPACITY, "moe_cache_lookup_host: %zu fills, room for %d", c->fills.size(), max_fills);
  }
  for (size_t i = 0; i < c->fills.size(); ++i) {
    if (injected_failure(c)) {
      invalidate_upto(c, i + 1);
      return fail(MOE_EHIP, "moe_cache_lookup_host: injected fill failure at fill %zu", i);
    }
  }
  for (size_t i = 0; i < c->fills.size(); ++i) {
    fills_host[i].slot = c->fills[i].slot;
    fills_host[i].layer = layer;
    fills_host[i].expert = c->fills[i].expert;
    fills_host[i].wave = wave;
  }
  *n_fills_host = (int)c->fills.size();
  for (int e = 0; e < c->desc.n_experts; ++e) slot_of_expert_host[e] = c->table[e];
  c->core.commit_wave(wave);
  fill_stats(c, nacc, (int64_t)c->fills.size() * (int64_t)c->desc.expert_bytes, stats_host);
  return MOE_OK;
}

}  // extern "C"

namespace {

// Lookup of one wave on the device cache.  Without `slot_misses` the wave's
// fills are awaited on the compute stream and `slot_a` is the whole table; with
// it, `slot_a` holds the hits only (usable at once: hits are never victims of
// the wave's misses) and `slot_misses` the filled experts only, and the compute
// stream waits for the fills only at moe_cache_wait_fills.
int lookup_fill_device(moe_cache* c, int layer, const int32_t* counts, int wave, int32_t* slot_a,
                       int32_t* slot_misses, uint64_t* addr_inplace, moe_cache_stats* stats_host,
                       hipStream_t compute_stream, const char* what) {
  if (!c) return fail(MOE_EINVAL, "null cache");
  if (!c->device) return fail(MOE_EINVAL, "%s needs a device cache (slot_pool set)", what);
  if (!slot_a || !aligned16(slot_a)) return fail(MOE_EINVAL, "%s: slot table must be a 16-byte aligned pointer", what);
  if (slot_misses && !aligned16(slot_misses))
    return fail(MOE_EINVAL, "%s: slot_misses must be a 16-byte aligned pointer", what);
  if (addr_inplace && !aligned16(addr_inplace))
    return fail(MOE_EINVAL, "%s: addr_inplace must be a 16-byte aligned pointer", what);
  const bool split = slot_misses != nullptr;
  const int E = c->desc.n_experts;
  hipError_t e;
  if (c->fill_pending) {
    // a split wave whose fills were never awaited: order them before anything else
    e = hipStreamWaitEvent(compute_stream, c->ev_fill, 0);
    if (e != hipSuccess) return hip_fail(e, (std::string(what) + ": fencing earlier fills").c_str());
    c->fill_pending = false;
  }
  if (c->move_pending) {
    // experts moved by a resize on another stream: the compute stream (and, through
    // ev_compute, the fills of this lookup) come after the moves
    e = hipStreamWaitEvent(compute_stream, c->ev_move, 0);
    if (e != hipSuccess) return hip_fail(e, (std::string(what) + ": fencing a resize").c_str());
    c->move_pending = false;
  }
  if (wave == 0) {
    if (!counts) return fail(MOE_EINVAL, "%s: null counts", what);
    // The one host synchronisation of the layer: the step's counts.
    e = hipMemcpyAsync(c->counts_pinned, counts, sizeof(int32_t) * E, hipMemcpyDeviceToHost, compute_stream);
    if (e == hipSuccess) e = hipEventRecord(c->ev_counts, compute_stream);
    if (e == hipSuccess) e = hipEventSynchronize(c->ev_counts);
    if (e != hipSuccess) return hip_fail(e, (std::string(what) + ": reading counts").c_str());
  }
  int nacc = 0;
  if (int rc = plan(c, layer, c->counts_pinned, wave, &nacc)) return rc;
  // device-visible addresses of the step's in-place experts (reported with wave 0)
  const int q = c->stage_next;
  if (addr_inplace) {
    if (c->stage_used[q]) {
      e = hipEventSynchronize(c->stage_ev[q]);
      if (e != hipSuccess) {
        c->core.abort_step();
        return hip_fail(e, (std::string(what) + ": staging buffer").c_str());
      }
      c->stage_used[q] = false;
    }
    uint64_t* stage_addr = c->stage_addr_pinned + (size_t)q * E;
    for (int x = 0; x < E; ++x) stage_addr[x] = 0;
    if (wave == 0)
      for (int x : c->core.inplace()) {
        const int64_t key = (int64_t)layer * E + x;
        if (!c->dev_addr[key]) {
          void* d = nullptr;
          e = hipHostGetDevicePointer(&d, const_cast<void*>(host_src(c, layer, x)), 0);
          if (e != hipSuccess || !d) {
            c->core.abort_step();
            return hip_fail(e != hipSuccess ? e : hipErrorInvalidValue,
                            (std::string(what) + ": host copy of an in-place expert is not device-visible").c_str());
          }
          c->dev_addr[key] = (uint64_t)(uintptr_t)d;
        }
        stage_addr[x] = c->dev_addr[key];
      }
  }
  int64_t bytes = 0;
  if (!c->fills.empty()) {
    // write-after-read: victims may still be read by FFN work already enqueued
    e = hipEventRecord(c->ev_compute, compute_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(c->desc.fill_stream, c->ev_compute, 0);
    if (e != hipSuccess) {
      c->core.abort_step();
      return hip_fail(e, (std::string(what) + ": fencing fills").c_str());
    }
    for (size_t i = 0; i < c->fills.size(); ++i) {
      const moe::PlannedFill& f = c->fills[i];
      if (injected_failure(c)) {
        invalidate_upto(c, i + 1);
        return fail(MOE_EHIP, "%s: injected fill failure at fill %zu", what, i);
      }
      void* dst = static_cast<uint8_t*>(c->desc.slot_pool) + (size_t)f.slot * c->desc.slot_stride;
      e = hipMemcpyAsync(dst, host_src(c, layer, f.expert), c->desc.expert_bytes, hipMemcpyHostToDevice,
                         c->desc.fill_stream);
      if (e != hipSuccess) {
        invalidate_upto(c, i + 1);
        return hip_fail(e, (std::string(what) + ": fill copy").c_str());
      }
      bytes += (int64_t)c->desc.expert_bytes;
    }
    // read-after-write: the FFN over the filled experts waits for the fills
    e = hipEventRecord(c->ev_fill, c->desc.fill_stream);
    if (e == hipSuccess && !split) e = hipStreamWaitEvent(compute_stream, c->ev_fill, 0);
    if (e != hipSuccess) {
      invalidate_upto(c, c->fills.size());
      return hip_fail(e, (std::string(what) + ": fencing compute").c_str());
    }
    c->fill_pending = split;
  }
  c->core.commit_wave(wave);
  // slot table(s): the wave's (expert, slot) pairs as the arguments of one small
  // kernel when they fit (and no in-place address table is asked for), else an
  // upload through a ring of pinned staging buffers
  if (!addr_inplace) {
    moe::SlotPairs sp;
    sp.table_a = slot_a;
    sp.table_b = split ? slot_misses : nullptr;
    sp.E = E;
    sp.n = 0;
    bool fits = true;
    for (int x = 0; x < E && fits; ++x) {
      if (c->table[x] < 0) continue;
      if (sp.n == moe::kSlotPairsMax) {
        fits = false;
        break;
      }
      sp.key[sp.n] = x;
      sp.slot[sp.n] = c->table[x];
      ++sp.n;
    }
    if (fits) {
      if (split)
        for (const moe::PlannedFill& f : c->fills)
          for (int i = 0; i < sp.n; ++i)
            if (sp.key[i] == f.expert) sp.key[i] |= 1 << 16;  // a filled expert: the misses' table
      e = moe::launch_write_slot_tables(sp, compute_stream);
      if (e != hipSuccess) return hip_fail(e, (std::string(what) + ": slot tables").c_str());
      fill_stats(c, nacc, bytes, stats_host);
      return MOE_OK;
    }
  }
  c->stage_next = (q + 1) % kStages;
  if (c->stage_used[q]) {
    e = hipEventSynchronize(c->stage_ev[q]);
    if (e != hipSuccess) return hip_fail(e, (std::string(what) + ": staging buffer").c_str());
  }
  int32_t* stage = c->stage_pinned + (size_t)q * 2 * E;
  for (int x = 0; x < E; ++x) stage[x] = c->table[x];
  if (split) {
    int32_t* miss = stage + E;
    for (int x = 0; x < E; ++x) miss[x] = -1;
    for (const moe::PlannedFill& f : c->fills) {
      miss[f.expert] = stage[f.expert];
      stage[f.expert] = -1;
    }
  }
  e = hipMemcpyAsync(slot_a, stage, sizeof(int32_t) * E, hipMemcpyHostToDevice, compute_stream);
  if (e == hipSuccess && split)
    e = hipMemcpyAsync(slot_misses, stage + E, sizeof(int32_t) * E, hipMemcpyHostToDevice, compute_stream);
  if (e == hipSuccess && addr_inplace)
    e = hipMemcpyAsync(addr_inplace, c->stage_addr_pinned + (size_t)q * E, sizeof(uint64_t) * E,
                       hipMemcpyHostToDevice, compute_stream);
  if (e == hipSuccess) e = hipEventRecord(c->stage_ev[q], compute_stream);
  if (e != hipSuccess) return hip_fail(e, (std::string(what) + ": slot table upload").c_str());
  c->stage_used[q] = true;
  fill_stats(c, nacc, bytes, stats_host);
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_cache_lookup_fill(moe_cache* c, int layer, const int32_t* counts, int wave, int32_t* slot_of_expert,
                          moe_cache_stats* stats_host, hipStream_t compute_stream) {
  const CallRange range_(__func__);
  return lookup_fill_device(c, layer, counts, wave, slot_of_expert, nullptr, nullptr, stats_host, compute_stream,
                            "moe_cache_lookup_fill");
}

int moe_cache_lookup_fill_split(moe_cache* c, int layer, const int32_t* counts, int wave, int32_t* slot_hits,
                                int32_t* slot_misses, moe_cache_stats* stats_host, hipStream_t compute_stream) {
  const CallRange range_(__func__);
  if (!slot_misses) return fail(MOE_EINVAL, "moe_cache_lookup_fill_split: null slot_misses");
  return lookup_fill_device(c, layer, counts, wave, slot_hits, slot_misses, nullptr, stats_host, compute_stream,
                            "moe_cache_lookup_fill_split");
}

int moe_cache_lookup_fill_inplace(moe_cache* c, int layer, const int32_t* counts, int wave, int32_t* slot_hits,
                                  int32_t* slot_misses, uint64_t* addr_inplace, moe_cache_stats* stats_host,
                                  hipStream_t compute_stream) {
  const CallRange range_(__func__);
  if (!slot_misses || !addr_inplace) return fail(MOE_EINVAL, "moe_cache_lookup_fill_inplace: null table");
  return lookup_fill_device(c, layer, counts, wave, slot_hits, slot_misses, addr_inplace, stats_host,
                            compute_stream, "moe_cache_lookup_fill_inplace");
}

int moe_cache_set_fill_fraction(moe_cache* c, int num, int den) {
  const CallRange range_(__func__);
  if (!c) return fail(MOE_EINVAL, "null cache");
  if (den < 1 || num < 0 || num > den)
    return fail(MOE_EINVAL, "moe_cache_set_fill_fraction: need 0 <= num <= den and den >= 1 (got %d/%d)", num, den);
  if (c->core.step_open()) return fail(MOE_ESTATE, "moe_cache_set_fill_fraction: a step is still open");
  c->core.set_fill_fraction(num, den);
  return MOE_OK;
}

int moe_cache_step_inplace(const moe_cache* c, int32_t* experts_host, int* n_host) {
  const CallRange range_(__func__);
  if (!c || !experts_host || !n_host) return fail(MOE_EINVAL, "moe_cache_step_inplace: null argument");
  const std::vector<int32_t>& v = c->core.inplace();
  for (size_t i = 0; i < v.size(); ++i) experts_host[i] = v[i];
  *n_host = (int)v.size();
  return MOE_OK;
}

int moe_cache_resize(moe_cache* c, int n_slots, void* slot_pool, size_t slot_stride, int32_t* moved_from_host,
                     hipStream_t stream) {
  const CallRange range_(__func__);
  if (!c) return fail(MOE_EINVAL, "null cache");
  if (n_slots < 1) return fail(MOE_EINVAL, "moe_cache_resize: n_slots=%d must be >= 1", n_slots);
  if (c->core.step_open()) return fail(MOE_ESTATE, "moe_cache_resize: a step is still open (finish its waves first)");
  std::vector<int32_t> moved;
  c->core.plan_resize(n_slots, moved);
  if (c->device) {
    if (!slot_pool || ((uintptr_t)slot_pool & 255u) != 0)
      return fail(MOE_EINVAL, "moe_cache_resize: slot_pool must be a 256-byte aligned device pointer");
    if (slot_stride < c->desc.expert_bytes || slot_stride % 256)
      return fail(MOE_EINVAL, "moe_cache_resize: slot_stride must be >= expert_bytes and a multiple of 256");
    const uintptr_t a0 = (uintptr_t)slot_pool, a1 = a0 + (uintptr_t)n_slots * slot_stride;
    const uintptr_t b0 = (uintptr_t)c->desc.slot_pool, b1 = b0 + (uintptr_t)c->desc.n_slots * c->desc.slot_stride;
    if (a0 < b1 && b0 < a1) return fail(MOE_EINVAL, "moe_cache_resize: the new slot pool overlaps the current one");
    // in-flight fills write the current pool: let them land first
    hipError_t e = hipEventSynchronize(c->ev_fill);
    if (e != hipSuccess) return hip_fail(e, "moe_cache_resize: waiting for fills");
    c->fill_pending = false;
    // kept experts move device to device, after the work already on `stream`
    std::vector<int32_t> from, to;
    for (int q = 0; q < n_slots; ++q)
      if (moved[q] >= 0) {
        from.push_back(moved[q]);
        to.push_back(q);
      }
    if (c->desc.expert_bytes % 16 == 0 && aligned16(c->desc.slot_pool)) {
      e = moe::launch_move_slots(static_cast<const uint8_t*>(c->desc.slot_pool), c->desc.slot_stride,
                                 static_cast<uint8_t*>(slot_pool), slot_stride, c->desc.expert_bytes, from.data(),
                                 to.data(), (int)from.size(), stream);
      if (e != hipSuccess) return hip_fail(e, "moe_cache_resize: moving experts");
    } else {
      for (size_t q = 0; q < from.size(); ++q) {
        e = hipMemcpyAsync(static_cast<uint8_t*>(slot_pool) + (size_t)to[q] * slot_stride,
                           static_cast<const uint8_t*>(c->desc.slot_pool) + (size_t)from[q] * c->desc.slot_stride,
                           c->desc.expert_bytes, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, "moe_cache_resize: moving an expert");
      }
    }
    e = hipEventRecord(c->ev_move, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_cache_resize: recording the moves");
    c->move_pending = true;
    c->desc.slot_pool = slot_pool;
    c->desc.slot_stride = slot_stride;
  } else if (slot_pool) {
    return fail(MOE_EINVAL, "moe_cache_resize: a host-only handle takes no slot_pool");
  }
  c->core.commit_resize(n_slots, moved);
  c->desc.n_slots = n_slots;
  if (moved_from_host)
    for (int q = 0; q < n_slots; ++q) moved_from_host[q] = moved[q];
  return MOE_OK;
}

int moe_cache_wait_fills(moe_cache* c, hipStream_t compute_stream) {
  const CallRange range_(__func__);
  if (!c) return fail(MOE_EINVAL, "null cache");
  if (!c->device) return fail(MOE_EINVAL, "moe_cache_wait_fills needs a device cache (slot_pool set)");
  if (!c->fill_pending) return MOE_OK;
  const hipError_t e = hipStreamWaitEvent(compute_stream, c->ev_fill, 0);
  if (e != hipSuccess) return hip_fail(e, "moe_cache_wait_fills");
  c->fill_pending = false;
  return MOE_OK;
}

}  // extern "C"

// ===========================================================================
// Prefill layer streaming (two banks)
// ===========================================================================
struct moe_layer_stream {
  moe_layer_stream_desc desc;
  hipEvent_t ready[2] = {};    // last fill of the bank
  hipEvent_t released[2] = {}; // last reader of the bank
  bool filled[2] = {false, false};
  bool has_release[2] = {false, false};
};

extern "C" {

int moe_layer_stream_create(const moe_layer_stream_desc* d, moe_layer_stream** out) {
  const CallRange range_(__func__);
  if (!d || !out) return fail(MOE_EINVAL, "moe_layer_stream_create: null argument");
  *out = nullptr;
  if (d->n_layers < 1 || d->layer_bytes == 0) return fail(MOE_EINVAL, "moe_layer_stream_create: bad sizes");
  if (!d->banks[0] || !d->banks[1] || !aligned16(d->banks[0]) || !aligned16(d->banks[1]))
    return fail(MOE_EINVAL, "moe_layer_stream_create: two 16-byte aligned banks are required");
  if (!d->host_layers_host && !d->host_layer_ptrs_host)
    return fail(MOE_EINVAL, "moe_layer_stream_create: host layers are required");
  moe_layer_stream* s = new (std::nothrow) moe_layer_stream();
  if (!s) return fail(MOE_ENOMEM, "moe_layer_stream_create: out of memory");
  s->desc = *d;
  hipError_t e = hipSuccess;
  for (int b = 0; b < 2 && e == hipSuccess; ++b) {
    e = hipEventCreateWithFlags(&s->ready[b], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&s->released[b], hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    moe_layer_stream_destroy(s);
    return hip_fail(e, "moe_layer_stream_create");
  }
  *out = s;
  return MOE_OK;
}

int moe_layer_stream_destroy(moe_layer_stream* s) {
  const CallRange range_(__func__);
  if (!s) return MOE_OK;
  int rc = MOE_OK;
  for (int b = 0; b < 2; ++b) {
    if (s->ready[b]) {
      if (s->filled[b]) {
        hipError_t e = hipEventSynchronize(s->ready[b]);
        if (e != hipSuccess) rc = hip_fail(e, "moe_layer_stream_destroy");
      }
      (void)hipEventDestroy(s->ready[b]);
    }
    if (s->released[b]) (void)hipEventDestroy(s->released[b]);
  }
  delete s;
  return rc;
}

int moe_layer_stream_fill(moe_layer_stream* s, int layer, int bank) {
  const CallRange range_(__func__);
  if (!s) return fail(MOE_EINVAL, "null layer stream");
  if (layer < 0 || layer >= s->desc.n_layers || bank < 0 || bank > 1)
    return fail(MOE_EINVAL, "moe_layer_stream_fill: layer %d / bank %d out of range", layer, bank);
  hipError_t e = hipSuccess;
  if (s->has_release[bank]) e = hipStreamWaitEvent(s->desc.fill_stream, s->released[bank], 0);
  const void* src = s->desc.host_layer_ptrs_host
                        ? s->desc.host_layer_ptrs_host[layer]
                        : static_cast<const uint8_t*>(s->desc.host_layers_host) + (size_t)layer * s->desc.layer_bytes;
  if (e == hipSuccess)
    e = hipMemcpyAsync(s->desc.banks[bank], src, s->desc.layer_bytes, hipMemcpyHostToDevice, s->desc.fill_stream);
  if (e == hipSuccess) e = hipEventRecord(s->ready[bank], s->desc.fill_stream);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_stream_fill");
  s->filled[bank] = true;
  return MOE_OK;
}

int moe_layer_stream_acquire(moe_layer_stream* s, int bank, hipStream_t compute_stream) {
  const CallRange range_(__func__);
  if (!s || bank < 0 || bank > 1) return fail(MOE_EINVAL, "moe_layer_stream_acquire: bad argument");
  if (!s->filled[bank]) return fail(MOE_ESTATE, "moe_layer_stream_acquire: bank %d was never filled", bank);
  hipError_t e = hipStreamWaitEvent(compute_stream, s->ready[bank], 0);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_layer_stream_acquire");
}

int moe_layer_stream_release(moe_layer_stream* s, int bank, hipStream_t compute_stream) {
  const CallRange range_(__func__);
  if (!s || bank < 0 || bank > 1) return fail(MOE_EINVAL, "moe_layer_stream_release: bad argument");
  hipError_t e = hipEventRecord(s->released[bank], compute_stream);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_stream_release");
  s->has_release[bank] = true;
  return MOE_OK;
}

}  // extern "C"
