// ffn_common.hpp -- device pieces shared by the grouped-FFN kernels (decode and
// prefill): work-item lookup, the tiled weight matrices and their buffer
// descriptors.
#pragma once

#include "common.hpp"

namespace moe {

struct Item {
  const uint8_t* w;  // expert slot
  int I;             // intermediate size
  int n;             // tokens of the item
  int p0;            // first pair of the item in sorted order (shared: first token)
  int hrow0;         // first row of the item in the intermediate workspace
  int tile;          // tile index inside the item
  bool shared;
  bool valid;
};

// Items of the shared expert: its T tokens in runs of up to P (one item if P = 0;
// P is 0 or a power of two).
__host__ __device__ inline int shared_items(int T, int P) { return P > 0 ? (T + P - 1) >> __builtin_ctz((unsigned)P) : 1; }

// Upper bound on the routed items of a call: N = T*k pairs over at most
// A = min(E, N) experts, each expert's ceil(n / P) <= (n + P - 1) / P, summed.
inline int routed_item_bound(int T, int k, int E, int P) {
  const int64_t N = (int64_t)T * k, A = N < E ? N : E;
  return (int)(P > 0 ? (N + A * (P - 1)) / P : A);
}

// Work item of logical block b: the shared expert's items come first (shared_tiles
// blocks each), then routed_tiles blocks of each routed item in ascending expert id
// (and, within an expert, ascending run).  An item covers pairs p0 .. p0+n-1 of the
// sorted order (the shared expert: tokens p0 .. p0+n-1).  Kernels that never split
// (SPLIT false: a.pass_rows is 0 for them) compile the one-item-per-expert lookup.
template <bool SPLIT = false>
__device__ __forceinline__ Item resolve_item_at(const FfnArgs& a, int b, int shared_tiles, int routed_tiles) {
  Item it;
  const int P = SPLIT ? a.pass_rows : 0;
  const int shared_total = SPLIT && a.shared_w ? shared_tiles * shared_items(a.T, P) : shared_tiles;
  if (b < shared_total) {
    it.shared = true;
    it.valid = true;
    it.w = a.shared_w;
    it.I = a.I_shared;
    if (SPLIT && P > 0) {
      const int run = b / shared_tiles;
      it.p0 = run * P;
      it.n = min(P, a.T - it.p0);
      it.tile = b - run * shared_tiles;
    } else {
      it.p0 = 0;
      it.n = a.T;
      it.tile = b;
    }
    it.hrow0 = a.T * a.k + it.p0;
    return it;
  }
  b -= shared_total;
  const int item = b / routed_tiles;
  it.tile = b - item * routed_tiles;
  it.shared = false;
  const ItemRef ref = nth_item<SPLIT>(a.offsets, a.slot_of_expert, a.expert_addr, a.E, item, P);
  it.valid = uniform(ref.expert) >= 0;
  if (!it.valid) return it;
  it.w = a.expert_addr ? uniform(reinterpret_cast<const uint8_t*>(ref.addr))
                       : uniform(a.slot_pool + (uint64_t)uniform(ref.slot) * a.slot_stride);
  it.I = a.I;
  it.p0 = uniform(ref.lo);
  it.n = uniform(ref.hi) - it.p0;
  if (SPLIT && P > 0) {
    const int skip = uniform(ref.run) * P;
    it.p0 += skip;
    it.n = min(P, it.n - skip);
  }
  it.hrow0 = it.p0;
  return it;
}

// Grouped-GEMM order (no shared expert): block b runs on XCD b % 8, in dispatch
// order; the routed experts ranked longest first (nth_longest) are dealt round
// robin over the XCDs, rank r to XCD r % 8 at item position r / 8 there, so every
// XCD gets an even share of the work and starts its longest items first (shortest
// last, so its CUs finish close together); the routed_tiles blocks of one item stay
// consecutive on one XCD.  The grid is 8 * ceil(items / 8) * routed_tiles blocks.
__device__ __forceinline__ Item resolve_item_longest(const FfnArgs& a, int routed_tiles) {
  Item it;
  const int x = blockIdx.x % 8, q = blockIdx.x / 8;
  const int pos = q / routed_tiles;
  it.tile = q - pos * routed_tiles;
  it.shared = false;
  const ItemRef ref = nth_longest(a.offsets, a.slot_of_expert, a.expert_addr, a.E, pos * 8 + x);
  it.valid = uniform(ref.expert) >= 0;
  if (!it.valid) return it;
  it.w = a.expert_addr ? uniform(reinterpret_cast<const uint8_t*>(ref.addr))
                       : uniform(a.slot_pool + (uint64_t)uniform(ref.slot) * a.slot_stride);
  it.I = a.I;
  it.p0 = uniform(ref.lo);
  it.n = uniform(ref.hi) - it.p0;
  it.hrow0 = it.p0;
  return it;
}

template <bool SPLIT = false>
__device__ __forceinline__ Item resolve_item(const FfnArgs& a, int shared_tiles, int routed_tiles) {
  return resolve_item_at<SPLIT>(a, blockIdx.x, shared_tiles, routed_tiles);
}

// Token of row i of an item (SPLIT as for the lookup: only then does a shared item
// start past token 0).
template <bool SPLIT = false>
__device__ __forceinline__ int item_token(const FfnArgs& a, const Item& it, int i) {
  return it.shared ? (SPLIT ? it.p0 + i : i) : a.sorted_rows[it.p0 + i] / a.k;
}

template <int WT>
struct KStep {
  static constexpr int value = WT == W_MXFP4 ? 128 : 32;
};

// One tiled weight matrix of an expert, addressed through buffer resources:
// the uniform part of every address (tile, step) is a scalar offset and the
// per-lane part (fragment `lane`) a fixed vector offset, so a load costs no
// vector ALU work.
struct Mat {
  __amdgpu_buffer_rsrc_t codes;   // 1 KB per (row tile, column step)
  __amdgpu_buffer_rsrc_t scales;  // MXFP4: 1 KB per (row tile, 16 column steps)
  int nK;                         // column steps
  int nKs;                        // MXFP4 scale blocks per row tile (16 steps each)
  int K;                          // columns
};

// Token rows of the B operand: a buffer and its row stride in elements; when the
// pass's rows are staged in LDS, row i of the pass sits at lds + i * lds_ld.
struct Rows {
  __amdgpu_buffer_rsrc_t buf;
  int ld;
  const uint8_t* lds;
  int lds_ld;
};

constexpr int kBufferFlags = 0x00020000;  // raw (untyped) 32-bit buffer access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0x7fffffffull ? bytes : 0x7fffffffull), kBufferFlags);
}

__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// MXFP4 block scales.  Per row tile the column steps form blocks of 16; in the
// 1 KB scale block of (row tile, step / 16) this lane's fragment owns bytes
// 16 * lane .. 16 * lane + 15, byte i being its scale at step 16 * block + i.
// A lane reads the whole 16 bytes at once (16 steps), or the word holding 4 of
// them; the byte is only picked out where the scale is used, so the wait for the
// load stays there too (a byte load is widened right after it is issued, which
// forces an early wait).
__device__ __forceinline__ int scale_block_offset(const Mat& w, int tile, int step) {
  return (tile * w.nKs + step / 16) * 1024;
}
__device__ __forceinline__ u32x4 load_scale_block(const Mat& w, int lane, int tile, int step) {
  return bld16(w.scales, lane * 16, scale_block_offset(w, tile, step));
}
__device__ __forceinline__ uint32_t load_scale_word(const Mat& w, int lane, int tile, int step) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(w.scales, lane * 16,
                                                         scale_block_offset(w, tile, step) + (step % 16) / 4 * 4, 0);
}
// The scale of step `step` from the word holding it.
__device__ __forceinline__ float scale_of_word(uint32_t word, int step) {
  return e8m0_to_f32((word >> (8 * (step & 3))) & 0xffu);
}

// Column steps of a K-wide matrix and byte offsets inside an expert slot.
template <int WT>
__device__ __forceinline__ int ksteps(int K) {
  return WT == W_MXFP4 ? (K + 127) / 128 : K / 32;
}
// Slot: codes of W13 (2*Ie rows, K = H), codes of W2 (H rows, K = Ie), then for
// MXFP4 the scale blocks of W13 and of W2.
template <int WT>
__device__ __forceinline__ Mat w13_mat(const uint8_t* slot, int H, int Ie) {
  const size_t r13 = 2 * Ie / 16, r2 = H / 16, k13 = ksteps<WT>(H), k2 = ksteps<WT>(Ie);
  const size_t c13 = r13 * k13 * 1024, c2 = r2 * k2 * 1024;
  Mat m;
  m.codes = make_rsrc(slot, c13);
  m.nKs = (int)((k13 + 15) / 16);
  m.scales = make_rsrc(WT == W_MXFP4 ? slot + c13 + c2 : slot, WT == W_MXFP4 ? r13 * m.nKs * 1024 : 0);
  m.nK = (int)k13;
  m.K = H;
  return m;
}
template <int WT>
__device__ __forceinline__ Mat w2_mat(const uint8_t* slot, int H, int Ie) {
  const size_t r13 = 2 * Ie / 16, r2 = H / 16, k13 = ksteps<WT>(H), k2 = ksteps<WT>(Ie);
  const size_t c13 = r13 * k13 * 1024, c2 = r2 * k2 * 1024;
  const size_t s13 = r13 * ((k13 + 15) / 16) * 1024;
  Mat m;
  m.codes = make_rsrc(slot + c13, c2);
  m.nKs = (int)((k2 + 15) / 16);
  m.scales = make_rsrc(WT == W_MXFP4 ? slot + c13 + c2 + s13 : slot, WT == W_MXFP4 ? r2 * m.nKs * 1024 : 0);
  m.nK = (int)k2;
  m.K = Ie;
  return m;
}

}  // namespace moe
