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
// Top-k: one wave64 per token.  Lane l holds the logits of experts i*64 + l.  The
// order is "larger logit first, equal logits to the lower index" (IEEE compare, so
// -0.0 equals +0.0).  Logits become unsigned keys that order the same way; a radix
// select finds the k-th largest key bit by bit from the top (32 rounds of a compare
// and a ballot count, no cross-lane shuffles); the winners are every key above it
// plus the keys equal to it in ascending expert index until there are k.  They are
// compacted (ascending index) into a small per-wave LDS list, and each of the k
// lanes finds its winner's output position by counting the winners ranked before
// it.  The gate weights are a max-subtracted softmax over the k values.
// ---------------------------------------------------------------------------
// Orderable key of a finite logit: larger value -> larger key, -0.0 and +0.0 the
// same key; 0 lies below every finite value and marks lanes past E.
__device__ __forceinline__ uint32_t logit_key(float v) {
  const uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kTopkMaxWaves = 16;  // waves per block of the kernels that call topk_row
constexpr int kTopkMaxK = 32;

struct TopkLane {
  int id;   // lane j < k: a winner's expert id
  int pos;  // and its output position (rank among the winners)
};

// Top-k of one token row (all 64 lanes of the wave take part); writes the k winners
// and their gate weights to ids_out[0..k), w_out[0..k) in order.  Lane j < k
// returns one winner and its position (every position once).
template <int EPL>
__device__ __forceinline__ TopkLane topk_row(const float* __restrict__ row, int E, int k,
                                             int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  __shared__ uint32_t s_key[kTopkMaxWaves][kTopkMaxK];
  __shared__ int s_id[kTopkMaxWaves][kTopkMaxK];
  __shared__ float s_val[kTopkMaxWaves][kTopkMaxK];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t lanes_below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  float v[EPL];
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * 64 + lane;
    v[i] = e < E ? row[e] : 0.0f;
    key[i] = e < E ? logit_key(v[i]) : 0u;
  }
  // the k-th largest key: the largest t with at least k keys >= t
  uint32_t thr = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = thr | (1u << b);
    int c = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) c += __popcll(__ballot(key[i] >= cand));
    if (c >= k) thr = cand;
  }
  int gt = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) gt += __popcll(__ballot(key[i] > thr));
  // winners in ascending expert index: keys above thr, and the first k - gt keys equal to it
  int ties = 0, before = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const bool eq = key[i] == thr;
    const uint64_t eqm = __ballot(eq);
    const bool win = key[i] > thr || (eq && ties + __popcll(eqm & lanes_below) < k - gt);
    const uint64_t wm = __ballot(win);
    if (win) {
      const int at = before + __popcll(wm & lanes_below);
      s_key[wv][at] = key[i];
      s_id[wv][at] = i * 64 + lane;
      s_val[wv][at] = v[i];
    }
    ties += __popcll(eqm);
    before += __popcll(wm);
  }
  __builtin_amdgcn_wave_barrier();  // a wave's LDS accesses complete in order
  uint32_t my_key = 0;
  int my_id = 0;
  float my_v = 0.0f;
  if (lane < k) {
    my_key = s_key[wv][lane];
    my_id = s_id[wv][lane];
    my_v = s_val[wv][lane];
  }
  // position: winners with a larger key, or the same key and a lower index (the
  // list is in ascending index)
  int pos = 0;
  for (int q = 0; q < k; ++q) {
    const uint32_t kq = (uint32_t)__builtin_amdgcn_readlane((int)my_key, q);
    pos += kq > my_key || (kq == my_key && q < lane);
  }
  const int top = __builtin_ctzll(__ballot(lane < k && pos == 0));
  const float z0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), top));
  const float ex = lane < k ? expf(my_v - z0) : 0.0f;
  float s = ex;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  if (lane < k) {
    ids_out[pos] = my_id;
    w_out[pos] = ex / s;
  }
  return TopkLane{my_id, pos};
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

// Router projection for batches of 32 tokens or more, as one bf16 MFMA GEMM
// (v_mfma_f32_32x32x16_bf16): a wave computes a 32-expert x 32-token tile, the
// router rows as the A operand (lane l: expert l % 32) and the tokens as B (lane
// l: token l % 32); lane half l / 32 takes k = 8 (l / 32) .. +7 of every 16-wide
// step for both operands, so A and B agree on the k order whatever it is inside
// the instruction.  The K loop runs in order, so results are deterministic.
// D: lane l, element v holds expert 8 (v / 4) + 4 (l / 32) + v % 4 of the tile,
// token l % 32.  Tiles past E or T clamp their loads to the last row and are not
// stored.  Grid (ceil(T / 32), ceil(E / 128)) of 4-wave blocks, wave w taking
// expert tile 4 * blockIdx.y + w.  H must be a multiple of 16.
constexpr int kRouterUnroll = 16;

__global__ __launch_bounds__(256) void router_logits_mfma(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr, int T, int H, int E,
                                                          float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, hh = lane >> 5, j = lane & 31;
  const int t0 = blockIdx.x * 32, e0 = (blockIdx.y * 4 + (threadIdx.x >> 6)) * 32;
  if (e0 >= E) return;  // uniform per wave
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (size_t)min(t0 + j, T - 1) * H) + hh;
  const u32x4* wrow = reinterpret_cast<const u32x4*>(wr + (size_t)min(e0 + j, E - 1) * H) + hh;
  const int steps = H / 16;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  int s = 0;
  for (; s + kRouterUnroll <= steps; s += kRouterUnroll) {
    u32x4 a[kRouterUnroll], b[kRouterUnroll];
#pragma unroll
    for (int u = 0; u < kRouterUnroll; ++u) {
      a[u] = wrow[2 * (s + u)];
      b[u] = xr[2 * (s + u)];
    }
#pragma unroll
    for (int u = 0; u < kRouterUnroll; ++u)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[u]), as_bf16x8(b[u]), acc, 0, 0, 0);
  }
  for (; s < steps; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(wrow[2 * s]), as_bf16x8(xr[2 * s]), acc, 0, 0, 0);
  if (t0 + j >= T) return;
  float* out = logits + (size_t)(t0 + j) * E;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int e = e0 + 8 * (v / 4) + 4 * hh + (v % 4);
    if (e < E) out[e] = acc[v];
  }
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E, float* logits,
                                hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (T >= 32 && H % 16 == 0) {
    const dim3 grid((unsigned)((T + 31) / 32), (unsigned)((E + 127) / 128)), block(256);
    hipLaunchKernelGGL(router_logits_mfma, grid, block, 0, st, x, wr, T, H, E, logits);
  } else {
    const dim3 grid((unsigned)T, (unsigned)((E + 4 * kRouterEPW - 1) / (4 * kRouterEPW))), block(256);
    hipLaunchKernelGGL(router_logits_kernel, grid, block, 0, st, x, wr, H, E, logits);
  }
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

// Top-k and permutation of a decode batch (T <= 8 tokens, T*k <= 64 pairs) in one
// small workgroup: wave t takes token t's top-k as above (the tokens in parallel),
// the ids meet in LDS behind one barrier, and wave 0 permutes the pairs in
// registers: lane p holds pair p = t*k + j, and one pass over the pairs (each
// broadcast with readlane) gives every lane the count and the number of smaller
// ids of its experts e = i*64 + lane (counts, offsets) and its own pair's place,
// the pairs of smaller experts plus those of the same expert with a smaller index
// (the stable order by r).  Ids lie in [0, E) here (they come from top-k).
constexpr int kRouteSmallMaxT = 8;
template <int EPL>
__global__ __launch_bounds__(64 * kRouteSmallMaxT) void route_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_rows,
    int32_t* __restrict__ inv_rows) {
  __shared__ int s_ids[64];
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
  if (t < T) {
    const TopkLane r = topk_row<EPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k);
    if (lane < k) s_ids[t * k + r.pos] = r.id;
  }
  __syncthreads();
  if (t != 0) return;
  const int n = T * k;
  const int my_e = lane < n ? s_ids[lane] : 0;
  int cnt[EPL], below[EPL], place = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) cnt[i] = below[i] = 0;
  for (int q = 0; q < n; ++q) {
    const int eq = __builtin_amdgcn_readlane(my_e, q);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = i * 64 + lane;
      cnt[i] += eq == e;
      below[i] += eq < e;
    }
    place += eq < my_e || (eq == my_e && q < lane);
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * 64 + lane;
    if (e < E) {
      counts[e] = cnt[i];
      offsets[e] = below[i];
    }
  }
  if (lane == 0) offsets[E] = n;
  if (lane < n) {
    sorted_rows[place] = lane;
    inv_rows[lane] = place;
  }
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_rows, int32_t* inv_rows, hipStream_t st) {
  if (T <= kRouteSmallMaxT && T * k <= 64) {
    const dim3 grid(1), block(64 * (T > 0 ? T : 1));
    if (E <= 64)
      hipLaunchKernelGGL(route_small_kernel<1>, grid, block, 0, st, logits, T, E, k, ids, w, counts, offsets, sorted_rows, inv_rows);
    else if (E <= 128)
      hipLaunchKernelGGL(route_small_kernel<2>, grid, block, 0, st, logits, T, E, k, ids, w, counts, offsets, sorted_rows, inv_rows);
    else if (E <= 256)
      hipLaunchKernelGGL(route_small_kernel<4>, grid, block, 0, st, logits, T, E, k, ids, w, counts, offsets, sorted_rows, inv_rows);
    else if (E <= 512)
      hipLaunchKernelGGL(route_small_kernel<8>, grid, block, 0, st, logits, T, E, k, ids, w, counts, offsets, sorted_rows, inv_rows);
    else
      hipLaunchKernelGGL(route_small_kernel<16>, grid, block, 0, st, logits, T, E, k, ids, w, counts, offsets, sorted_rows, inv_rows);
    return hipGetLastError();
  }
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
// thread owns 4 consecutive columns of one token.  The pairs go in groups of 8:
// every index, weight and row of a group is requested before the group's first
// multiply-add (one memory round trip per group instead of two per pair), then
// the group is added in increasing j, the same operations in the same order.
// ---------------------------------------------------------------------------
constexpr int kCombineGroup = 8;
template <bool BF16OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ rows, const float* __restrict__ w,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ shared, int k, int H,
                                                      void* __restrict__ y) {
  const int cb = (H / 4 + 255) / 256;
  const int t = blockIdx.x / cb;
  const int c4 = (blockIdx.x % cb) * 256 + threadIdx.x;
  if (c4 * 4 >= H) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (shared) s = reinterpret_cast<const float4*>(shared + (size_t)t * H)[c4];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += kCombineGroup) {
    int p[kCombineGroup];
    float wj[kCombineGroup];
    float4 o[kCombineGroup];
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u) {
      const int j = j0 + u;
      p[u] = j < k ? inv[(size_t)t * k + j] : -1;  // -1: no pair, or dropped by the permutation
      wj[u] = j < k ? w[(size_t)t * k + j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u)
      o[u] = p[u] >= 0 ? reinterpret_cast<const float4*>(rows + (size_t)p[u] * H)[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u) {
      if (p[u] < 0) continue;
      acc.x = fmaf(wj[u], o[u].x, acc.x);
      acc.y = fmaf(wj[u], o[u].y, acc.y);
      acc.z = fmaf(wj[u], o[u].z, acc.z);
      acc.w = fmaf(wj[u], o[u].w, acc.w);
    }
  }
  if (shared) {
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
