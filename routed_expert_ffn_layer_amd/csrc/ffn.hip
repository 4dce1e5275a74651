// ffn.hip -- grouped SwiGLU expert FFN for gfx950.
//
// Pages: "Meet FreeToken: An Edge-Native MoE Serving Engine that Runs 753B GLM-5.2
// on a Single Workstation GPU" (MarkTechPost).  The GPU computes the experts that
// are resident in its cache ("Three mechanisms": bandwidth-adaptive execution),
// with expert output bit-exact and no precision relaxation ("Key Takeaways"): MXFP4
// weights are expanded to bf16 exactly before the bf16 MFMA.  The FFN form
// (SwiGLU: down(SiLU(gate x) * up x)) is not on the pages; it is the standard
// MoE expert.
//
// Work decomposition.  A grid slot is (item, tile).  Items are the shared expert
// (if any) followed by up to min(E, T*k) routed experts; a block finds "its"
// routed expert as the a-th expert with pairs and a slot (a scan over offsets in
// L2), so the grid is sized from T alone and needs no host synchronisation.
// Weights are streamed from HBM exactly once per expert (per 16*NT tokens);
// the 4 waves of a block split the reduction dimension K and add their partial
// accumulators in a fixed order, so results are deterministic run to run.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16): weights are the A operand (16 rows),
// tokens the B operand (16 columns), so a single token costs one weight pass.
// Lane l supplies A[row l%16][8 values] and B[col l%16][8 values]; any fixed
// assignment of K indices to the 8-value groups is valid as long as A and B use
// the same one.  bf16 weights: lane group g = l/16 takes k = kb + 8g .. +7.
// MXFP4: lane group g loads one whole 32-element block (16 bytes of codes, one
// scale) at k = kb + 32g and feeds it to 4 MFMAs, the m-th taking elements
// 8m .. 8m+7.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

struct Item {
  const uint8_t* w;  // expert slot
  int I;             // intermediate size
  int n;             // tokens of the item
  int p0;            // first output row (routed: sorted position; shared: 0)
  int hrow0;         // first row of the item in the intermediate workspace
  int tile;          // tile index inside the item
  bool shared;
  bool valid;
};

__device__ __forceinline__ Item resolve_item(const FfnArgs& a, int shared_tiles, int routed_tiles) {
  Item it;
  int b = blockIdx.x;
  if (b < shared_tiles) {
    it.shared = true;
    it.valid = true;
    it.w = a.shared_w;
    it.I = a.I_shared;
    it.n = a.T;
    it.p0 = 0;
    it.hrow0 = a.T * a.k;
    it.tile = b;
    return it;
  }
  b -= shared_tiles;
  const int item = b / routed_tiles;
  it.tile = b - item * routed_tiles;
  it.shared = false;
  const int e = nth_active_expert(a.offsets, a.slot_of_expert, a.E, item);
  it.valid = e >= 0;
  if (!it.valid) return it;
  it.w = a.slot_pool + (uint64_t)a.slot_of_expert[e] * a.slot_stride;
  it.I = a.I;
  it.p0 = a.offsets[e];
  it.n = a.offsets[e + 1] - it.p0;
  it.hrow0 = it.p0;
  return it;
}

__device__ __forceinline__ int item_token(const FfnArgs& a, const Item& it, int i) {
  return it.shared ? i : a.sorted_rows[it.p0 + i] / a.k;
}

// ===========================================================================
// f32 weights: plain FMA, one wave per output element row, lanes split K,
// butterfly reduction.  Used by the small f32 layer.
// ===========================================================================
__global__ __launch_bounds__(256) void gate_up_f32(FfnArgs a, int shared_tiles, int routed_tiles) {
  const Item it = resolve_item(a, shared_tiles, routed_tiles);
  if (!it.valid) return;
  const int lane = threadIdx.x & 63;
  const int j = it.tile * 4 + (threadIdx.x >> 6);
  if (j >= it.I) return;
  const int H = a.H;
  const float* wg = reinterpret_cast<const float*>(it.w) + (size_t)j * H;
  const float* wu = reinterpret_cast<const float*>(it.w) + (size_t)(it.I + j) * H;
  float* h = reinterpret_cast<float*>(a.h);
  for (int i = 0; i < it.n; ++i) {
    const float* x = reinterpret_cast<const float*>(a.x) + (size_t)item_token(a, it, i) * H;
    float ga = 0.f, ua = 0.f;
    for (int c = lane; c < H; c += 64) {
      const float xv = x[c];
      ga = fmaf(wg[c], xv, ga);
      ua = fmaf(wu[c], xv, ua);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      ga += __shfl_xor(ga, d, 64);
      ua += __shfl_xor(ua, d, 64);
    }
    if (lane == 0) h[(size_t)(it.hrow0 + i) * a.h_ld + j] = silu_f32(ga) * ua;
  }
}

__global__ __launch_bounds__(256) void down_f32(FfnArgs a, int shared_tiles, int routed_tiles) {
  const Item it = resolve_item(a, shared_tiles, routed_tiles);
  if (!it.valid) return;
  const int lane = threadIdx.x & 63;
  const int r = it.tile * 4 + (threadIdx.x >> 6);
  const int H = a.H;
  if (r >= H) return;
  const float* wd = reinterpret_cast<const float*>(it.w) + (size_t)2 * it.I * H + (size_t)r * it.I;
  const float* h = reinterpret_cast<const float*>(a.h);
  for (int i = 0; i < it.n; ++i) {
    const float* hr = h + (size_t)(it.hrow0 + i) * a.h_ld;
    float acc = 0.f;
    for (int c = lane; c < it.I; c += 64) acc = fmaf(wd[c], hr[c], acc);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
    if (lane == 0) {
      if (it.shared)
        a.shared_out[(size_t)i * H + r] = acc;
      else
        a.out_rows[(size_t)(it.p0 + i) * H + r] = acc;
    }
  }
}

// ===========================================================================
// bf16 / MXFP4 weights on bf16 MFMA.
// ===========================================================================
template <int WT>
struct KStep {
  static constexpr int value = WT == W_MXFP4 ? 128 : 32;
};

// A fragments of one k step for weight row `wrow` of a K-wide matrix.
//   bf16:  a[0] = W[wrow][kb+8g .. +7]
//   mxfp4: a[m] = W[wrow][kb+32g+8m .. +7], m = 0..3 (zeros past K)
template <int WT>
__device__ __forceinline__ void load_a(const uint8_t* codes, const uint8_t* scales, int wrow, int K, int kb, int g,
                                       bf16x8 (&a)[WT == W_MXFP4 ? 4 : 1]) {
  if constexpr (WT == W_BF16) {
    a[0] = as_bf16x8(ldg16(codes + ((size_t)wrow * K + kb + 8 * g) * 2));
  } else {
    const int kk = kb + 32 * g;
    if (kk < K) {
      const u32x4 q = ldg16(codes + (size_t)wrow * (K / 2) + kk / 2);
      const float sc = e8m0_to_f32(scales[(size_t)wrow * (K / 32) + kk / 32]);
      a[0] = fp4x8_to_bf16x8(q[0], sc);
      a[1] = fp4x8_to_bf16x8(q[1], sc);
      a[2] = fp4x8_to_bf16x8(q[2], sc);
      a[3] = fp4x8_to_bf16x8(q[3], sc);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) a[m] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }
}

// B fragment m of one k step from a bf16 row `src` (nullptr = padding column).
template <int WT>
__device__ __forceinline__ bf16x8 load_b(const uint16_t* src, int K, int kb, int g, int m) {
  const int kk = WT == W_MXFP4 ? kb + 32 * g + 8 * m : kb + 8 * g;
  if (src == nullptr || kk >= K) return as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  return as_bf16x8(ldg16(src + kk));
}

// Byte offsets inside an expert slot.
template <int WT>
__device__ __forceinline__ void w13_ptrs(const uint8_t* slot, int H, int Ie, const uint8_t*& codes,
                                         const uint8_t*& scales) {
  codes = slot;
  scales = WT == W_MXFP4 ? slot + (size_t)3 * Ie * H / 2 : nullptr;
}
template <int WT>
__device__ __forceinline__ void w2_ptrs(const uint8_t* slot, int H, int Ie, const uint8_t*& codes,
                                        const uint8_t*& scales) {
  if constexpr (WT == W_MXFP4) {
    codes = slot + (size_t)Ie * H;
    scales = slot + (size_t)3 * Ie * H / 2 + (size_t)2 * Ie * (H / 32);
  } else {
    codes = slot + (size_t)4 * Ie * H;
    scales = nullptr;
  }
}

// gate_up: a block owns 8 intermediate indices j0..j0+7 of one item: one 16-row
// A tile = gate rows j0..j0+7 stacked on up rows j0..j0+7, so the epilogue pairs
// lane l (gate) with lane l+32 (up) and writes h = SiLU(gate) * up as bf16.
template <int WT, int NT>
__global__ __launch_bounds__(256) void gate_up_mfma(FfnArgs a, int shared_tiles, int routed_tiles) {
  const Item it = resolve_item(a, shared_tiles, routed_tiles);
  if (!it.valid) return;
  constexpr int KS = KStep<WT>::value;
  constexpr int NA = WT == W_MXFP4 ? 4 : 1;
  __shared__ f32x4 red[3][NT][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, Ie = it.I;
  const int j0 = it.tile * 8;
  const int wrow = r < 8 ? j0 + r : Ie + j0 + (r - 8);
  const int nsteps = (H + KS - 1) / KS;
  const int s0 = wv * nsteps / 4, s1 = (wv + 1) * nsteps / 4;
  const uint8_t *codes, *scales;
  w13_ptrs<WT>(it.w, H, Ie, codes, scales);
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(a.x);
  uint16_t* h = reinterpret_cast<uint16_t*>(a.h);
  for (int pass = 0; pass < it.n; pass += NT * 16) {
    const int ntl = min(NT, (it.n - pass + 15) / 16);
    const uint16_t* xrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int i = pass + nt * 16 + r;
      xrow[nt] = (nt < ntl && i < it.n) ? xb + (size_t)item_token(a, it, i) * H : nullptr;
    }
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s = s0; s < s1; ++s) {
      const int kb = s * KS;
      bf16x8 A[NA];
      load_a<WT>(codes, scales, wrow, H, kb, g, A);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (nt < ntl) {
#pragma unroll
          for (int m = 0; m < NA; ++m)
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[m], load_b<WT>(xrow[nt], H, kb, g, m), acc[nt], 0, 0, 0);
        }
      }
    }
    if (wv > 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) red[wv - 1][nt][lane] = acc[nt];
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (nt < ntl) {
          const f32x4 v = ((acc[nt] + red[0][nt][lane]) + red[1][nt][lane]) + red[2][nt][lane];
          f32x4 u;
#pragma unroll
          for (int q = 0; q < 4; ++q) u[q] = __shfl_xor(v[q], 32, 64);
          const int i = pass + nt * 16 + r;
          if (g < 2 && i < it.n) {
            uint2 packed;
            packed.x = (uint32_t)f32_to_bf16_rne(silu_f32(v[0]) * u[0]) |
                       ((uint32_t)f32_to_bf16_rne(silu_f32(v[1]) * u[1]) << 16);
            packed.y = (uint32_t)f32_to_bf16_rne(silu_f32(v[2]) * u[2]) |
                       ((uint32_t)f32_to_bf16_rne(silu_f32(v[3]) * u[3]) << 16);
            *reinterpret_cast<uint2*>(h + (size_t)(it.hrow0 + i) * a.h_ld + j0 + g * 4) = packed;
          }
        }
      }
    }
    __syncthreads();
  }
}

// down: a block owns 16 output columns (rows of W2) of one item.
template <int WT, int NT>
__global__ __launch_bounds__(256) void down_mfma(FfnArgs a, int shared_tiles, int routed_tiles) {
  const Item it = resolve_item(a, shared_tiles, routed_tiles);
  if (!it.valid) return;
  constexpr int KS = KStep<WT>::value;
  constexpr int NA = WT == W_MXFP4 ? 4 : 1;
  __shared__ f32x4 red[3][NT][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, Ie = it.I;
  const int row0 = it.tile * 16;
  const int nsteps = (Ie + KS - 1) / KS;
  const int s0 = wv * nsteps / 4, s1 = (wv + 1) * nsteps / 4;
  const uint8_t *codes, *scales;
  w2_ptrs<WT>(it.w, H, Ie, codes, scales);
  const uint16_t* hb = reinterpret_cast<const uint16_t*>(a.h);
  for (int pass = 0; pass < it.n; pass += NT * 16) {
    const int ntl = min(NT, (it.n - pass + 15) / 16);
    const uint16_t* hrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int i = pass + nt * 16 + r;
      hrow[nt] = (nt < ntl && i < it.n) ? hb + (size_t)(it.hrow0 + i) * a.h_ld : nullptr;
    }
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s = s0; s < s1; ++s) {
      const int kb = s * KS;
      bf16x8 A[NA];
      load_a<WT>(codes, scales, row0 + r, Ie, kb, g, A);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (nt < ntl) {
#pragma unroll
          for (int m = 0; m < NA; ++m)
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[m], load_b<WT>(hrow[nt], Ie, kb, g, m), acc[nt], 0, 0, 0);
        }
      }
    }
    if (wv > 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) red[wv - 1][nt][lane] = acc[nt];
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (nt < ntl) {
          const f32x4 v = ((acc[nt] + red[0][nt][lane]) + red[1][nt][lane]) + red[2][nt][lane];
          const int i = pass + nt * 16 + r;
          if (i < it.n) {
            float* dst = it.shared ? a.shared_out + (size_t)i * H : a.out_rows + (size_t)(it.p0 + i) * H;
            *reinterpret_cast<float4*>(dst + row0 + g * 4) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
    __syncthreads();
  }
}

// ===========================================================================
// Launchers
// ===========================================================================
size_t ffn_workspace_bytes(int wtype, int T, int k, int I, int I_shared) {
  const size_t rows = (size_t)T * k + (I_shared > 0 ? (size_t)T : 0);
  const size_t ld = (size_t)(I > I_shared ? I : I_shared);
  return rows * ld * (wtype == W_F32 ? 4 : 2);
}

template <int WT, int NT>
static void launch_gu(const FfnArgs& a, hipStream_t st, unsigned grid, int shared_tiles, int routed_tiles) {
  hipLaunchKernelGGL((gate_up_mfma<WT, NT>), dim3(grid), dim3(256), 0, st, a, shared_tiles, routed_tiles);
}
template <int WT, int NT>
static void launch_dn(const FfnArgs& a, hipStream_t st, unsigned grid, int shared_tiles, int routed_tiles) {
  hipLaunchKernelGGL((down_mfma<WT, NT>), dim3(grid), dim3(256), 0, st, a, shared_tiles, routed_tiles);
}

static int pick_nt(int T) {
  if (T <= 16) return 1;
  if (T <= 32) return 2;
  if (T <= 64) return 4;
  return 8;
}

template <int WT>
static void dispatch_gu(const FfnArgs& a, hipStream_t st, unsigned grid, int sh, int rt) {
  switch (pick_nt(a.T)) {
    case 1: launch_gu<WT, 1>(a, st, grid, sh, rt); break;
    case 2: launch_gu<WT, 2>(a, st, grid, sh, rt); break;
    case 4: launch_gu<WT, 4>(a, st, grid, sh, rt); break;
    default: launch_gu<WT, 8>(a, st, grid, sh, rt); break;
  }
}
template <int WT>
static void dispatch_dn(const FfnArgs& a, hipStream_t st, unsigned grid, int sh, int rt) {
  switch (pick_nt(a.T)) {
    case 1: launch_dn<WT, 1>(a, st, grid, sh, rt); break;
    case 2: launch_dn<WT, 2>(a, st, grid, sh, rt); break;
    case 4: launch_dn<WT, 4>(a, st, grid, sh, rt); break;
    default: launch_dn<WT, 8>(a, st, grid, sh, rt); break;
  }
}

hipError_t launch_ffn_gate_up(int wtype, const FfnArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const bool sh = a.shared_w != nullptr;
  if (wtype == W_F32) {
    const int shared_tiles = sh ? (a.I_shared + 3) / 4 : 0, routed_tiles = (a.I + 3) / 4;
    const unsigned grid = shared_tiles + a.routed_items * routed_tiles;
    if (grid) hipLaunchKernelGGL(gate_up_f32, dim3(grid), dim3(256), 0, st, a, shared_tiles, routed_tiles);
  } else {
    const int shared_tiles = sh ? a.I_shared / 8 : 0, routed_tiles = a.I / 8;
    const unsigned grid = shared_tiles + a.routed_items * routed_tiles;
    if (grid) {
      if (wtype == W_BF16) dispatch_gu<W_BF16>(a, st, grid, shared_tiles, routed_tiles);
      else dispatch_gu<W_MXFP4>(a, st, grid, shared_tiles, routed_tiles);
    }
  }
  return hipGetLastError();
}

hipError_t launch_ffn_down(int wtype, const FfnArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const bool sh = a.shared_w != nullptr;
  if (wtype == W_F32) {
    const int tiles = (a.H + 3) / 4;
    const int shared_tiles = sh ? tiles : 0;
    const unsigned grid = shared_tiles + a.routed_items * tiles;
    if (grid) hipLaunchKernelGGL(down_f32, dim3(grid), dim3(256), 0, st, a, shared_tiles, tiles);
  } else {
    const int tiles = a.H / 16;
    const int shared_tiles = sh ? tiles : 0;
    const unsigned grid = shared_tiles + a.routed_items * tiles;
    if (grid) {
      if (wtype == W_BF16) dispatch_dn<W_BF16>(a, st, grid, shared_tiles, tiles);
      else dispatch_dn<W_MXFP4>(a, st, grid, shared_tiles, tiles);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
