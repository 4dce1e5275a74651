// common.hpp -- device helpers shared by the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// W_MXFP4_A8: MXFP4 weights whose gate/up activations are MXFP8 (the native FP4 x
// FP8 path); the weights and their layout are W_MXFP4's.
enum WType { W_F32 = 0, W_BF16 = 1, W_MXFP4 = 2, W_MXFP4_A8 = 3 };

// Everything the grouped FFN kernels need, passed by value.
struct FfnArgs {
  const uint8_t* slot_pool;
  uint64_t slot_stride;
  const int32_t* slot_of_expert;  // [E] slot of each expert (-1: not computed), or null when expert_addr is set
  const uint64_t* expert_addr;    // [E] address of each expert's weights (0: not computed), or null
  const uint8_t* shared_w;        // nullable
  const void* x;                  // [T][H] f32 or bf16
  const uint8_t* xq;              // MXFP8 activations: [T][H] E4M3 codes of x (native FP4 path)
  const uint8_t* xs;              //                    [T][H/32] E8M0 block scales
  const int32_t* offsets;         // [E+1]
  const int32_t* sorted_rows;     // [T*k]
  float* out_rows;                // [T*k][H]
  float* shared_out;              // [T][H]
  void* h;                        // workspace: [T*k + T][I_max] bf16 or f32
  int T, k, E, H, I, I_shared;
  int h_ld;                       // row stride of h in elements (max(I, I_shared))
  int routed_items;               // grid slots for routed items (an upper bound on their number)
  int pass_rows;                  // a power of two: an item is a run of up to pass_rows pairs of one
                                  // expert (the shared expert: of its tokens); 0: one item per expert
  int lds_rows;                   // token rows the launch's dynamic LDS holds (0: none)
};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// f32 -> bf16, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// E8M0 code -> the f32 multiplier 2^(s-127) (s = 0 is the subnormal 2^-127; the
// code 0xFF is NaN in OCP MX v1.0, and a NaN scale makes its whole block NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s == 0 ? 0x00400000u : s == 255u ? 0x7fc00000u : (s << 23));
}

// 8 E2M1 codes (one 32-bit word, element 0 in the low nibble of byte 0) times the
// block scale -> 8 bf16 in element order.  The hardware convert is exact for every
// E8M0 scale (products beyond the bf16 range become inf).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float scale) {
  u32x4 v;
  v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return __builtin_bit_cast(bf16x8, v);
}


__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Values the whole wave agrees on, moved to scalar registers so that addresses
// built from them (buffer descriptors, tile offsets) stay scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const uint8_t* uniform(const uint8_t* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u), hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every global load still in flight, which would drain a software
// prefetch pipeline at each barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// SiLU z * sigmoid(z) = z / (1 + e^-z), from the hardware's base-2 exponential
// (e^-z = 2^(-z log2 e)) and reciprocal, each within about one f32 ulp: far below
// the bf16 rounding of the gate/up product that follows, and a few instructions
// instead of a range-reduced exponential and an IEEE division.  Large negative z
// gives 2^+inf = inf and z * 0 = -0, the limit.
__device__ __forceinline__ float silu_f32(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Item resolution for the grouped FFN.  Items are taken in ascending expert id over
// the experts that have pairs and a slot (or a non-zero weight address) in this call:
// one item per expert (RUNS false), or one item per run of up to P of its pairs (RUNS,
// P > 0, a power of two: an expert with n pairs gives ceil(n / P) items, so the passes
// of a busy expert run on different waves side by side).  Finds item a: its expert,
// the item's index among that expert's items, and the expert's first and end pair
// and slot or weight address, taken from the lane that loaded them (no second trip
// to memory).  Every lane of the wave gets the same answer; expert -1 if there are
// fewer than a+1 items.  All loads are issued before the scan, so the lookup costs
// one memory round trip.
struct ItemRef {
  int expert, run, lo, hi, slot;
  uint64_t addr;
};

template <int EPL, bool RUNS>
__device__ __forceinline__ ItemRef nth_item_t(const int32_t* __restrict__ offsets,
                                              const int32_t* __restrict__ slot_of_expert,
                                              const uint64_t* __restrict__ expert_addr, int E, int a, int P) {
  const int lane = threadIdx.x & 63;
  int lo[EPL], hi[EPL], sl[EPL];
  uint64_t ad[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * 64 + lane;
    const bool in = e < E;
    lo[i] = in ? offsets[e] : 0;
    hi[i] = in ? offsets[e + 1] : 0;
    ad[i] = 0;
    if (expert_addr) {
      ad[i] = in ? expert_addr[e] : 0;
      sl[i] = ad[i] != 0 ? 0 : -1;
    } else {
      sl[i] = in ? slot_of_expert[e] : -1;
    }
  }
  const int lp = RUNS && P > 0 ? __builtin_ctz((unsigned)P) : 0;
  ItemRef ref;
  int base = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int n = hi[i] - lo[i];
    const int cnt = (n > 0 && sl[i] >= 0) ? (RUNS && P > 0 ? (n + P - 1) >> lp : 1) : 0;
    const int incl = wave_incl_scan(cnt);
    const int total = __shfl(incl, 63, 64);
    if (a < base + total) {
      const int r = a - base;  // item r of this group of 64 experts
      int owner;
      if constexpr (RUNS) {
        owner = __builtin_ctzll(__ballot(cnt > 0 && incl > r && incl - cnt <= r));
        ref.run = r - __shfl(incl - cnt, owner, 64);
      } else {
        owner = __builtin_ctzll(__ballot(cnt && incl == r + 1));
        ref.run = 0;
      }
      ref.expert = i * 64 + owner;
      ref.lo = __shfl(lo[i], owner, 64);
      ref.hi = __shfl(hi[i], owner, 64);
      ref.slot = __shfl(sl[i], owner, 64);
      ref.addr = expert_addr ? ((uint64_t)(uint32_t)__shfl((int)(uint32_t)(ad[i] >> 32), owner, 64) << 32) |
                                   (uint32_t)__shfl((int)(uint32_t)ad[i], owner, 64)
                             : 0;
      return ref;
    }
    base += total;
  }
  ref.expert = -1;
  ref.run = ref.lo = ref.hi = ref.slot = 0;
  ref.addr = 0;
  return ref;
}

template <bool RUNS>
__device__ __forceinline__ ItemRef nth_item(const int32_t* __restrict__ offsets, const int32_t* __restrict__ slot_of_expert,
                                            const uint64_t* __restrict__ expert_addr, int E, int a, int P) {
  if (E <= 64) return nth_item_t<1, RUNS>(offsets, slot_of_expert, expert_addr, E, a, P);
  if (E <= 128) return nth_item_t<2, RUNS>(offsets, slot_of_expert, expert_addr, E, a, P);
  if (E <= 256) return nth_item_t<4, RUNS>(offsets, slot_of_expert, expert_addr, E, a, P);
  if (E <= 512) return nth_item_t<8, RUNS>(offsets, slot_of_expert, expert_addr, E, a, P);
  return nth_item_t<16, RUNS>(offsets, slot_of_expert, expert_addr, E, a, P);
}

// Routed expert of rank r when the active experts are ordered longest first: by
// their number of 32-token tiles, ceil(n / 32), descending, then by ascending id
// (same loads and the same ItemRef as nth_item; expert -1 if fewer than r+1
// experts are active).  Each round takes the largest tile count left below the
// previous one, so the loop ends after at most as many rounds as there are
// distinct counts, and every active expert has exactly one rank.
template <int EPL>
__device__ __forceinline__ ItemRef nth_longest_t(const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ slot_of_expert,
                                                 const uint64_t* __restrict__ expert_addr, int E, int r) {
  const int lane = threadIdx.x & 63;
  int lo[EPL], hi[EPL], sl[EPL], c[EPL];
  uint64_t ad[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * 64 + lane;
    const bool in = e < E;
    lo[i] = in ? offsets[e] : 0;
    hi[i] = in ? offsets[e + 1] : 0;
    ad[i] = 0;
    if (expert_addr) {
      ad[i] = in ? expert_addr[e] : 0;
      sl[i] = ad[i] != 0 ? 0 : -1;
    } else {
      sl[i] = in ? slot_of_expert[e] : -1;
    }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) c[i] = (hi[i] > lo[i] && sl[i] >= 0) ? (hi[i] - lo[i] + 31) >> 5 : 0;
  ItemRef ref;
  int base = 0, bound = 0x7fffffff;
  for (;;) {
    int m = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) m = max(m, c[i] < bound ? c[i] : 0);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = max(m, __shfl_xor(m, d, 64));
    if (m == 0) break;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint64_t bits = __ballot(c[i] == m);
      const int cnt = __popcll(bits);
      if (r < base + cnt) {
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
        const int owner = __builtin_ctzll(__ballot(c[i] == m && below == r - base));
        ref.expert = i * 64 + owner;
        ref.run = 0;
        ref.lo = __shfl(lo[i], owner, 64);
        ref.hi = __shfl(hi[i], owner, 64);
        ref.slot = __shfl(sl[i], owner, 64);
        ref.addr = expert_addr ? ((uint64_t)(uint32_t)__shfl((int)(uint32_t)(ad[i] >> 32), owner, 64) << 32) |
                                     (uint32_t)__shfl((int)(uint32_t)ad[i], owner, 64)
                               : 0;
        return ref;
      }
      base += cnt;
    }
    bound = m;
  }
  ref.expert = -1;
  ref.run = ref.lo = ref.hi = ref.slot = 0;
  ref.addr = 0;
  return ref;
}

__device__ __forceinline__ ItemRef nth_longest(const int32_t* __restrict__ offsets,
                                               const int32_t* __restrict__ slot_of_expert,
                                               const uint64_t* __restrict__ expert_addr, int E, int r) {
  if (E <= 64) return nth_longest_t<1>(offsets, slot_of_expert, expert_addr, E, r);
  if (E <= 128) return nth_longest_t<2>(offsets, slot_of_expert, expert_addr, E, r);
  if (E <= 256) return nth_longest_t<4>(offsets, slot_of_expert, expert_addr, E, r);
  if (E <= 512) return nth_longest_t<8>(offsets, slot_of_expert, expert_addr, E, r);
  return nth_longest_t<16>(offsets, slot_of_expert, expert_addr, E, r);
}

}  // namespace moe
