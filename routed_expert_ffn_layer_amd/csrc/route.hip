// route.hip -- top-k gating, stable permutation by expert, and the weighted combine.
//
// Pages: "Meet FreeToken: An Edge-Native MoE Serving Engine that Runs 753B GLM-5.2
// on a Single Workstation GPU" (MarkTechPost).  Routing is left exactly as the
// router decides ("Three mechanisms": bandwidth-adaptive execution, no router
// modification; "Key Takeaways": bit-exact expert output) and the experts'
// partial sums are added without approximation ("Three mechanisms").
#include <climits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Top-k: one wave64 per token.  Lane l holds the logits of experts i*64 + l.
// k rounds of a wave-wide argmax (butterfly over __shfl_xor) under the order
// "larger logit first, equal logits to the lower index" (IEEE compare, so -0.0
// equals +0.0); the winner's owner lane marks it taken.  Lane j keeps the j-th
// winner; the gate weights are a max-subtracted softmax over those k values.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  if (ia == INT_MAX) return false;
  if (ib == INT_MAX) return true;
  return va > vb || (va == vb && ia < ib);
}

// Top-k of one token row (all 64 lanes of the wave take part); lane j < k writes
// the j-th winner and its gate weight to ids_out[j], w_out[j].
template <int EPL>
__device__ __forceinline__ void topk_row(const float* __restrict__ row, int E, int k, int32_t* __restrict__ ids_out,
                                         float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * 64 + lane;
    v[i] = e < E ? row[e] : 0.0f;
  }
  uint32_t taken = 0;
  float my_z = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = i * 64 + lane;
      if (e < E && !((taken >> i) & 1u) && ranks_before(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d, 64);
      const int oe = __shfl_xor(be, d, 64);
      if (ranks_before(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_z = bv;
      my_id = be;
    }
  }
  const float z0 = __shfl(my_z, 0, 64);
  const float ex = lane < k ? expf(my_z - z0) : 0.0f;
  float s = ex;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  if (lane < k) {
    ids_out[lane] = my_id;
    w_out[lane] = ex / s;
  }
}

template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int32_t* __restrict__ ids, float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  topk_row<EPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k);
}

// ---------------------------------------------------------------------------
// Router projection ahead of top-k: logits[t][e] = x[t] . Wr[e] (bf16 inputs,
// f32 accumulation).  A wave computes kRouterEPW experts of one token; lanes stride
// over H in 16-byte pieces (8 bf16), each piece a run of f32 fused multiply-adds of
// exact bf16 products, then a fixed butterfly sums the lanes, so the result is the
// same on every run.  Grid (T, E / (4 * kRouterEPW)) of 4-wave blocks.
// ---------------------------------------------------------------------------
constexpr int kRouterEPW = 4;

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr, int H, int E,
                                                            float* __restrict__ logits) {
  const int t = blockIdx.x, lane = threadIdx.x & 63;
  const int e0 = (blockIdx.y * 4 + (threadIdx.x >> 6)) * kRouterEPW;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (size_t)t * H);
  const int pieces = H / 8;
#pragma unroll
  for (int q = 0; q < kRouterEPW; ++q) {
    const int e = e0 + q;
    if (e >= E) break;  // uniform per wave
    const u32x4* wrow = reinterpret_cast<const u32x4*>(wr + (size_t)e * H);
    float acc = 0.0f;
    for (int c = lane; c < pieces; c += 64) {
      const u32x4 xv = xr[c], wv = wrow[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fmaf(__uint_as_float(xv[i] << 16), __uint_as_float(wv[i] << 16), acc);
        acc = fmaf(__uint_as_float(xv[i] & 0xffff0000u), __uint_as_float(wv[i] & 0xffff0000u), acc);
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
    if (lane == 0) logits[(size_t)t * E + e] = acc;
  }
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E, float* logits,
                                hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)T, (unsigned)((E + 4 * kRouterEPW - 1) / (4 * kRouterEPW))), block(256);
  hipLaunchKernelGGL(router_logits_kernel, grid, block, 0, st, x, wr, H, E, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64) hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, st, logits, T, E, k, ids, w);
  else if (E <= 128) hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, st, logits, T, E, k, ids, w);
  else if (E <= 256) hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, st, logits, T, E, k, ids, w);
  else if (E <= 512) hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, st, logits, T, E, k, ids, w);
  else hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, st, logits, T, E, k, ids, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Permutation: one workgroup of 1024 threads (16 waves), E <= 1024.
//  1. histogram of expert ids in LDS;
//  2. exclusive scan -> counts, offsets;
//  3. rounds of 1024 consecutive pairs: inside a wave, the lanes holding the same
//     expert are found with one ballot per bit of the id, and a pair's rank among
//     them is the popcount of the matching lower lanes; per-wave per-expert totals
//     in LDS give the offset of each wave's group, and a running count per expert
//     carries between rounds.  Pairs therefore land in ascending r within each
//     expert (stable) with no ordering atomics.  A pair whose id lies outside
//     [0, E) is dropped: not counted, not placed, inv_rows = -1.
// ---------------------------------------------------------------------------
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kRouteFusedMaxT = 8;  // batches routed by one workgroup launch (measured: wins up to 8)

// The whole permutation, run by one workgroup of kPermThreads threads.
__device__ __forceinline__ void permute_block(const int32_t* ids, int n, int E, int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_rows,
                                              int32_t* __restrict__ inv_rows) {
  __shared__ int s_base[1024];   // histogram, then exclusive offsets
  __shared__ int s_run[1024];    // pairs of each expert placed in earlier rounds
  __shared__ uint16_t s_wcnt[kPermWaves][1024];
  __shared__ int s_wsum[kPermWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < 1024; e += kPermThreads) {
    s_base[e] = 0;
    s_run[e] = 0;
  }
  for (int i = tid; i < kPermWaves * 1024; i += kPermThreads) (&s_wcnt[0][0])[i] = 0;
  __syncthreads();
  for (int r = tid; r < n; r += kPermThreads) {
    const int e = ids[r];
    if (e >= 0 && e < E) atomicAdd(&s_base[e], 1);
  }
  __syncthreads();
  const int c = tid < E ? s_base[tid] : 0;
  const int incl = wave_incl_scan(c);
  if (lane == 63) s_wsum[wv] = incl;
  __syncthreads();
  int wbase = 0;
  for (int q = 0; q < wv; ++q) wbase += s_wsum[q];
  const int excl = wbase + incl - c;
  __syncthreads();
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = excl;
    s_base[tid] = excl;
    if (tid == E - 1) offsets[E] = excl + c;
  }
  __syncthreads();
  const int nbits = 32 - __clz(E - 1);
  const uint64_t lanes_below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < n; base += kPermThreads) {
    const int r = base + tid;
    const int raw = r < n ? ids[r] : -1;
    const bool valid = raw >= 0 && raw < E;
    const int e = valid ? raw : 0;
    if (r < n && !valid) inv_rows[r] = -1;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(valid && bit);
      match &= bit ? m : ~m;
    }
    const int rank = __popcll(match & lanes_below);
    const int cnt = __popcll(match);
    if (valid && rank == 0) s_wcnt[wv][e] = (uint16_t)cnt;
    __syncthreads();
    if (valid) {
      int pos = s_run[e];
      for (int q = 0; q < wv; ++q) pos += s_wcnt[q][e];
      const int dest = s_base[e] + pos + rank;
      sorted_rows[dest] = r;
      inv_rows[r] = dest;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&s_run[e], cnt);
      s_wcnt[wv][e] = 0;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                               int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_rows,
                                                               int32_t* __restrict__ inv_rows) {
  permute_block(ids, n, E, counts, offsets, sorted_rows, inv_rows);
}

// Top-k and permutation in one workgroup launch (small batches): the 16 waves
// take the tokens in turn, the barrier makes every token's ids visible to the
// workgroup, then the permutation runs on them.  Same code as the two kernels,
// so the same results.
template <int EPL>
__global__ __launch_bounds__(kPermThreads) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                             int32_t* __restrict__ ids, float* __restrict__ w,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted_rows,
                                                             int32_t* __restrict__ inv_rows) {
  for (int t = threadIdx.x >> 6; t < T; t += kPermWaves)
    topk_row<EPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k);
  __syncthreads();
  permute_block(ids, T * k, E, counts, offsets, sorted_rows, inv_rows);
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_rows, int32_t* inv_rows, hipStream_t st) {
  if (T > kRouteFusedMaxT) {
    hipError_t e = launch_topk(logits, T, E, k, ids, w, st);
    if (e != hipSuccess) return e;
    return launch_permute(ids, T, k, E, counts, offsets, sorted_rows, inv_rows, st);
  }
  const dim3 grid(1), block(kPermThreads);
  if (E <= 64)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, st, logits, T, E, k, ids, w, counts, offsets, sorted_rows, inv_rows);
  else if (E <= 128)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, st, logits, T, E, k, ids, w, counts, offsets, sorted_rows, inv_rows);
  else if (E <= 256)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, st, logits, T, E, k, ids, w, counts, offsets, sorted_rows, inv_rows);
  else if (E <= 512)
    hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, st, logits, T, E, k, ids, w, counts, offsets, sorted_rows, inv_rows);
  else
    hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, st, logits, T, E, k, ids, w, counts, offsets, sorted_rows, inv_rows);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_rows, int32_t* inv_rows, hipStream_t st) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, st, ids, T * k, E, counts, offsets,
                     sorted_rows, inv_rows);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: y[t] = sum_j w[t][j] * rows[inv[t*k+j]] (+ shared[t]), f32 fused
// multiply-add in increasing j, then one rounding to the output type.  Each
// thread owns 4 consecutive columns of one token.
// ---------------------------------------------------------------------------
template <bool BF16OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ rows, const float* __restrict__ w,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ shared, int k, int H,
                                                      void* __restrict__ y) {
  const int cb = (H / 4 + 255) / 256;
  const int t = blockIdx.x / cb;
  const int c4 = (blockIdx.x % cb) * 256 + threadIdx.x;
  if (c4 * 4 >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int p = inv[(size_t)t * k + j];
    if (p < 0) continue;  // pair dropped by the permutation (expert id out of range)
    const float wj = w[(size_t)t * k + j];
    const float4 o = reinterpret_cast<const float4*>(rows + (size_t)p * H)[c4];
    acc.x = fmaf(wj, o.x, acc.x);
    acc.y = fmaf(wj, o.y, acc.y);
    acc.z = fmaf(wj, o.z, acc.z);
    acc.w = fmaf(wj, o.w, acc.w);
  }
  if (shared) {
    const float4 s = reinterpret_cast<const float4*>(shared + (size_t)t * H)[c4];
    acc.x += s.x;
    acc.y += s.y;
    acc.z += s.z;
    acc.w += s.w;
  }
  if (BF16OUT) {
    uint2 packed;
    packed.x = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
    packed.y = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
    reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + (size_t)t * H)[c4] = packed;
  } else {
    reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + (size_t)t * H)[c4] = acc;
  }
}

hipError_t launch_combine(const float* rows, const float* w, const int32_t* inv, const float* shared, int T, int k,
                          int H, void* y, bool bf16_out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)T * ((H / 4 + 255) / 256)), block(256);
  if (bf16_out)
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, st, rows, w, inv, shared, k, H, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, st, rows, w, inv, shared, k, H, y);
  return hipGetLastError();
}

}  // namespace moe
