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

enum WType { W_F32 = 0, W_BF16 = 1, W_MXFP4 = 2 };

// Everything the grouped FFN kernels need, passed by value.
struct FfnArgs {
  const uint8_t* slot_pool;
  uint64_t slot_stride;
  const int32_t* slot_of_expert;  // [E]
  const uint8_t* shared_w;        // nullable
  const void* x;                  // [T][H] f32 or bf16
  const int32_t* offsets;         // [E+1]
  const int32_t* sorted_rows;     // [T*k]
  float* out_rows;                // [T*k][H]
  float* shared_out;              // [T][H]
  void* h;                        // workspace: [T*k + T][I_max] bf16 or f32
  int T, k, E, H, I, I_shared;
  int h_ld;                       // row stride of h in elements (max(I, I_shared))
  int routed_items;               // grid slots for routed experts: min(E, T*k)
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

// E8M0 code -> the f32 multiplier 2^(s-127) (s = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s == 0 ? 0x00400000u : (s << 23));
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

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

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

// Item resolution for the grouped FFN.  The a-th expert (ascending id) that has
// pairs and a slot in this call.  Every lane of the wave gets the same answer.
// Returns -1 if fewer than a+1 experts are active.  All loads are issued before
// the scan, so the lookup costs one memory round trip.
template <int EPL>
__device__ __forceinline__ int nth_active_expert_t(const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ slot_of_expert, int E, int a) {
  const int lane = threadIdx.x & 63;
  int lo[EPL], hi[EPL], sl[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * 64 + lane;
    const bool in = e < E;
    lo[i] = in ? offsets[e] : 0;
    hi[i] = in ? offsets[e + 1] : 0;
    sl[i] = in ? slot_of_expert[e] : -1;
  }
  int base = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int act = (hi[i] > lo[i]) && (sl[i] >= 0);
    const int incl = wave_incl_scan(act);
    const int total = __shfl(incl, 63, 64);
    if (a < base + total) {
      const uint64_t hit = __ballot(act && (incl == a + 1 - base));
      return i * 64 + __builtin_ctzll(hit);
    }
    base += total;
  }
  return -1;
}

__device__ __forceinline__ int nth_active_expert(const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ slot_of_expert, int E, int a) {
  if (E <= 64) return nth_active_expert_t<1>(offsets, slot_of_expert, E, a);
  if (E <= 128) return nth_active_expert_t<2>(offsets, slot_of_expert, E, a);
  if (E <= 256) return nth_active_expert_t<4>(offsets, slot_of_expert, E, a);
  if (E <= 512) return nth_active_expert_t<8>(offsets, slot_of_expert, E, a);
  return nth_active_expert_t<16>(offsets, slot_of_expert, E, a);
}

}  // namespace moe
