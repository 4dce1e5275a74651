// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to libmoe).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct FfnArgs;

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t st);
// Router projection: logits [T][E] = x [T][H] . wr [E][H]^T (bf16 in, f32 out).
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E, float* logits,
                                hipStream_t st);
// Top-k then permutation; one workgroup launch for small batches.
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_rows, int32_t* inv_rows, hipStream_t st);
hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_rows, int32_t* inv_rows, hipStream_t st);
hipError_t launch_combine(const float* rows, const float* w, const int32_t* inv, const float* shared, int T, int k,
                          int H, void* y, bool bf16_out, hipStream_t st);

// Elastic cache resize: copy `bytes` of each of n experts from slot from[i] of
// one pool to slot to[i] of another (batched launches, the table in the kernel
// arguments).  Expert bytes must be a multiple of 16 and the pools 16-byte aligned.
constexpr int kMoveBatch = 480;
// The slot tables of one cache wave from up to kSlotPairsMax (expert, slot) pairs
// passed by value: table_a (and table_b if non-null) [E] set to -1, then
// key = expert | (table << 16) (table 0: a, 1: b) gets slot.  E <= 65535.
constexpr int kSlotPairsMax = 240;
struct SlotPairs {
  int32_t* table_a;
  int32_t* table_b;
  int E, n;
  int32_t key[kSlotPairsMax];
  int32_t slot[kSlotPairsMax];
};
hipError_t launch_write_slot_tables(const SlotPairs& p, hipStream_t st);
hipError_t launch_move_slots(const uint8_t* src, uint64_t src_stride, uint8_t* dst, uint64_t dst_stride,
                             uint64_t bytes, const int32_t* from, const int32_t* to, int n, hipStream_t st);

// Grouped FFN phases.  wtype: 0 f32, 1 bf16, 2 mxfp4 (3, MXFP4 with MXFP8
// activations, runs the grouped GEMM only).
hipError_t launch_ffn_gate_up(int wtype, const FfnArgs& a, hipStream_t st);
hipError_t launch_ffn_down(int wtype, const FfnArgs& a, hipStream_t st);
// Prefill-sized batches (LDS-staged token tiles); same arguments and results.
bool prefill_supported(int wtype, int H, int I, int I_shared);
hipError_t launch_prefill_gate_up(int wtype, const FfnArgs& a, hipStream_t st);
hipError_t launch_prefill_down(int wtype, const FfnArgs& a, hipStream_t st);
// Native FP4 path: MXFP8 activations (E4M3 codes [T][H], E8M0 scales [T][H/32])
// from bf16 x, then gate_up on the scaled f8f6f4 MFMA (a.xq, a.xs); the down phase
// is launch_prefill_down with MXFP4 weights.
hipError_t launch_mx8_quantize(const uint16_t* x, int T, int H, uint8_t* codes, uint8_t* scales, hipStream_t st);
hipError_t launch_native_gate_up(const FfnArgs& a, hipStream_t st);
// Workspace bytes: the SwiGLU intermediate for T*k routed + T shared rows; for the
// native path (wtype 3) also the MXFP8 activations, at ffn_workspace_xq_offset.
size_t ffn_workspace_bytes(int wtype, int T, int k, int H, int I, int I_shared);
size_t ffn_workspace_xq_offset(int T, int k, int I, int I_shared);

}  // namespace moe
