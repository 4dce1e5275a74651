// ffn_prefill.hip -- grouped SwiGLU expert FFN for prefill-sized batches on gfx950.
//
// Pages: "Meet FreeToken: An Edge-Native MoE Serving Engine that Runs 753B GLM-5.2
// on a Single Workstation GPU" (MarkTechPost): a prefill pass routes thousands of
// tokens per layer to nearly the whole expert set ("The gap it targets"), so every
// expert carries a batch of tokens and its weights are worth reading once for all
// of them.  Same arithmetic as the decode kernels (bf16 MFMA, MXFP4 expanded to
// bf16 exactly, SwiGLU intermediate rounded to bf16); only the data movement
// differs.
//
// Block = WAVES waves over 16*R*WAVES weight rows of one expert and up to 16*NT
// of its tokens.  Weights (A) stream from HBM in the tiled layout, one chunk of
// KC columns ahead of the MFMAs; the expert's token rows (B) are staged through
// LDS, KC columns at a time and double-buffered, and shared by all waves, so each
// weight fragment meets 16*NT tokens and each token fragment 16*R*WAVES weight
// rows.  One barrier per chunk.  Blocks are ordered so that all row blocks of an
// expert run on the same XCD in sequence (blockIdx b executes on XCD b % 8),
// keeping the expert's token rows in that XCD's L2.
#include "ffn_common.hpp"
#include "kernels.hpp"

namespace moe {

template <int WT, int R, int U>
struct AChunk {
  u32x4 qa[U][R];
  uint32_t qs[U][R];
};

// A fragments of U steps starting at step s (whole chunks only: s + U <= nK).
template <int WT, int R, int U>
__device__ __forceinline__ void load_a(AChunk<WT, R, U>& c, const Mat& w, const int (&atile)[R], int s) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int ts = atile[t] * w.nK + s;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      c.qa[u][t] = bld16(w.codes, lane * 16, (ts + u) * 1024);
      if constexpr (WT == W_MXFP4)
        c.qs[u][t] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(w.scales, lane, (ts + u) * 64, 0);
      else
        c.qs[u][t] = 0u;
    }
  }
}

// Token rows of one chunk: thread-owned 16-byte pieces, global -> registers -> LDS.
template <int NT, int KC, int WAVES>
struct BStage {
  static_assert((NT * 16 * (KC / 8)) % (WAVES * 64) == 0, "staging pieces must divide evenly over the block");
  static constexpr int kPieces = NT * 16 * (KC / 8) / (WAVES * 64);
  u32x4 v[kPieces];
};

template <int NT, int KC, int WAVES>
__device__ __forceinline__ void load_b(BStage<NT, KC, WAVES>& st, __amdgpu_buffer_rsrc_t src,
                                       const int (&row_off)[BStage<NT, KC, WAVES>::kPieces], int col0, int ntl) {
  constexpr int PR = KC / 8;  // pieces per row
#pragma unroll
  for (int i = 0; i < BStage<NT, KC, WAVES>::kPieces; ++i) {
    const int q = threadIdx.x + i * WAVES * 64;
    const int row = q / PR, c = q % PR;
    if (row < ntl * 16) st.v[i] = bld16(src, row_off[i] + (col0 + c * 8) * 2, 0);
  }
}

template <int NT, int KC, int WAVES>
__device__ __forceinline__ void store_b(const BStage<NT, KC, WAVES>& st, uint16_t (*buf)[KC + 8], int ntl) {
  constexpr int PR = KC / 8;
#pragma unroll
  for (int i = 0; i < BStage<NT, KC, WAVES>::kPieces; ++i) {
    const int q = threadIdx.x + i * WAVES * 64;
    const int row = q / PR, c = q % PR;
    if (row < ntl * 16) *reinterpret_cast<u32x4*>(&buf[row][c * 8]) = st.v[i];
  }
}

// acc[t][nt] += A_t . B_nt over one chunk: A from registers, B from LDS.  NTL
// (the token tiles of this pass) is a compile-time count, so the unrolled body
// has no branches.  The LDS reads of k-group m+1 are issued before the MFMAs of
// group m (scheduling barriers keep that order), so LDS latency hides behind
// R*NTL MFMAs; consecutive MFMAs update different accumulators.
template <int WT, int NTL, int R, int U, int KC>
__device__ __forceinline__ void compute_chunk_lds(const AChunk<WT, R, U>& c, const uint16_t (*buf)[KC + 8],
                                                  f32x4 (&acc)[R][NTL]) {
  constexpr int KS = KStep<WT>::value;
  constexpr int NA = WT == W_MXFP4 ? 4 : 1;
  constexpr int NG = U * NA;  // k-groups of 32 columns in the chunk
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  auto kcol = [&](int q) {
    const int u = q / NA, m = q % NA;
    return u * KS + (WT == W_MXFP4 ? 32 * g + 8 * m : 8 * g);
  };
  bf16x8 B[2][NTL];
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt) B[0][nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(&buf[nt * 16 + col][kcol(0)]));
#pragma unroll
  for (int u = 0; u < U; ++u) {
    bf16x8 A[R][NA];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      if constexpr (WT == W_BF16) {
        A[t][0] = as_bf16x8(c.qa[u][t]);
      } else {
        const float sc = e8m0_to_f32(c.qs[u][t]);
#pragma unroll
        for (int m = 0; m < 4; ++m) A[t][m] = fp4x8_to_bf16x8(c.qa[u][t][m], sc);
      }
    }
#pragma unroll
    for (int m = 0; m < NA; ++m) {
      const int q = u * NA + m;
      if (q + 1 < NG) {
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt)
          B[(q + 1) % 2][nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(&buf[nt * 16 + col][kcol(q + 1)]));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
        for (int t = 0; t < R; ++t)
          acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][m], B[q % 2][nt], acc[t][nt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

#ifndef MOE_PF_DA
#define MOE_PF_DA 4
#endif
constexpr int kPfDA = MOE_PF_DA;  // weight chunks in flight + 1

template <int WT, int NT, int NTL, int R, int KC, int WAVES>
__device__ __forceinline__ void prefill_rows(const Mat& w, const int (&atile)[R], __amdgpu_buffer_rsrc_t src,
                                             const int (&row_off)[BStage<NT, KC, WAVES>::kPieces],
                                             uint16_t (*sb)[NT * 16][KC + 8], f32x4 (&acc)[R][NTL]) {
  constexpr int U = KC / KStep<WT>::value;
  constexpr int DA = kPfDA;
  constexpr int UNROLL = DA % 2 == 0 ? DA : 2 * DA;  // both rotations static
  const int nchunks = w.K / KC;
  AChunk<WT, R, U> a[DA];
  BStage<NT, KC, WAVES> bs[2];
  load_b<NT, KC, WAVES>(bs[0], src, row_off, 0, NTL);
  load_b<NT, KC, WAVES>(bs[1], src, row_off, min(1, nchunks - 1) * KC, NTL);
#pragma unroll
  for (int d = 0; d < DA - 1; ++d) load_a<WT, R, U>(a[d], w, atile, min(d, nchunks - 1) * U);
  store_b<NT, KC, WAVES>(bs[0], sb[0], NTL);
  __syncthreads();
  // chunk ch: token rows of ch+2 and weights of ch+DA-1 are requested, ch is
  // computed from a[ch % DA] and sb[ch % 2], then the rows of ch+1 (requested a
  // chunk earlier) are written to sb[(ch+1) % 2].  The requests are not
  // conditional (past the last chunk they re-read it), so the compiler can count
  // exactly which loads a wait needs and leaves the later ones in flight.
  const int last = nchunks - 1;
  for (int ch0 = 0; ch0 < nchunks; ch0 += UNROLL) {
#pragma unroll
    for (int d = 0; d < UNROLL; ++d) {
      const int ch = ch0 + d;
      if (ch < nchunks) {
        load_b<NT, KC, WAVES>(bs[d % 2], src, row_off, min(ch + 2, last) * KC, NTL);
        load_a<WT, R, U>(a[(d + DA - 1) % DA], w, atile, min(ch + DA - 1, last) * U);
        compute_chunk_lds<WT, NTL, R, U, KC>(a[d % DA], sb[d % 2], acc);
        store_b<NT, KC, WAVES>(bs[(d + 1) % 2], sb[(d + 1) % 2], NTL);
        __syncthreads();
      }
    }
  }
}

// One pass of up to 16*NTL tokens, NTL fixed at compile time; returns the
// accumulators through the epilogue functor.
template <int WT, int NT, int NTL, int R, int KC, int WAVES, typename Epi>
__device__ __forceinline__ void prefill_pass(const Mat& w, const int (&atile)[R], __amdgpu_buffer_rsrc_t src,
                                             const int (&row_off)[BStage<NT, KC, WAVES>::kPieces],
                                             uint16_t (*sb)[NT * 16][KC + 8], const Epi& epi) {
  f32x4 acc[R][NTL];
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  prefill_rows<WT, NT, NTL, R, KC, WAVES>(w, atile, src, row_off, sb, acc);
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) epi(t, nt, acc[t][nt]);
}

template <int WT, int NT, int R, int KC, int WAVES, typename Epi>
__device__ __forceinline__ void prefill_dispatch(int ntl, const Mat& w, const int (&atile)[R],
                                                 __amdgpu_buffer_rsrc_t src,
                                                 const int (&row_off)[BStage<NT, KC, WAVES>::kPieces],
                                                 uint16_t (*sb)[NT * 16][KC + 8], const Epi& epi) {
  static_assert(NT == 8, "dispatch covers 1..8 token tiles");
  switch (ntl) {
    case 1: prefill_pass<WT, NT, 1, R, KC, WAVES>(w, atile, src, row_off, sb, epi); break;
    case 2: prefill_pass<WT, NT, 2, R, KC, WAVES>(w, atile, src, row_off, sb, epi); break;
    case 3: prefill_pass<WT, NT, 3, R, KC, WAVES>(w, atile, src, row_off, sb, epi); break;
    case 4: prefill_pass<WT, NT, 4, R, KC, WAVES>(w, atile, src, row_off, sb, epi); break;
    case 5: prefill_pass<WT, NT, 5, R, KC, WAVES>(w, atile, src, row_off, sb, epi); break;
    case 6: prefill_pass<WT, NT, 6, R, KC, WAVES>(w, atile, src, row_off, sb, epi); break;
    case 7: prefill_pass<WT, NT, 7, R, KC, WAVES>(w, atile, src, row_off, sb, epi); break;
    default: prefill_pass<WT, NT, 8, R, KC, WAVES>(w, atile, src, row_off, sb, epi); break;
  }
}

__device__ __forceinline__ int xcd_logical_block() {
  const int per = gridDim.x / 8;  // the grid is a multiple of 8
  return (blockIdx.x % 8) * per + blockIdx.x / 8;
}

template <int WT, int NT, int R, int KC, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void prefill_gate_up(FfnArgs a, int shared_tiles, int routed_tiles) {
  const Item it = resolve_item_at(a, xcd_logical_block(), shared_tiles, routed_tiles);
  if (!it.valid) return;
  constexpr int PIECES = BStage<NT, KC, WAVES>::kPieces;
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][NT * 16][KC + 8];
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, Ie = it.I;
  const int j0 = (it.tile * WAVES + wv) * 8 * R;  // this wave's first intermediate index
  const Mat w = w13_mat<WT>(it.w, H, Ie);
  const __amdgpu_buffer_rsrc_t src = make_rsrc(a.x, (size_t)a.T * H * 2);
  uint16_t* h = reinterpret_cast<uint16_t*>(a.h);
  int atile[R];
#pragma unroll
  for (int t = 0; t < R; ++t) atile[t] = min(j0 / 8 + t, Ie / 8 - 1);  // rows past I: loaded, never stored
  for (int pass = 0; pass < it.n; pass += NT * 16) {
    const int ntl = min(NT, (it.n - pass + 15) / 16);
    int row_off[PIECES];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int row = (threadIdx.x + i * WAVES * 64) / (KC / 8);
      row_off[i] = item_token(a, it, min(pass + row, it.n - 1)) * H * 2;
    }
    auto epi = [&](int t, int nt, const f32x4& v) {
      const int jt = j0 + 8 * t;
      f32x4 u;
#pragma unroll
      for (int q = 0; q < 4; ++q) u[q] = __shfl_xor(v[q], 32, 64);
      const int i = pass + nt * 16 + r;
      if (jt < Ie && g < 2 && i < it.n) {
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16_rne(silu_f32(v[0]) * u[0]) |
                   ((uint32_t)f32_to_bf16_rne(silu_f32(v[1]) * u[1]) << 16);
        packed.y = (uint32_t)f32_to_bf16_rne(silu_f32(v[2]) * u[2]) |
                   ((uint32_t)f32_to_bf16_rne(silu_f32(v[3]) * u[3]) << 16);
        *reinterpret_cast<uint2*>(h + (size_t)(it.hrow0 + i) * a.h_ld + jt + g * 4) = packed;
      }
    };
    prefill_dispatch<WT, NT, R, KC, WAVES>(ntl, w, atile, src, row_off, sb, epi);
  }
}

template <int WT, int NT, int R, int KC, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void prefill_down(FfnArgs a, int shared_tiles, int routed_tiles) {
  const Item it = resolve_item_at(a, xcd_logical_block(), shared_tiles, routed_tiles);
  if (!it.valid) return;
  constexpr int PIECES = BStage<NT, KC, WAVES>::kPieces;
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][NT * 16][KC + 8];
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, Ie = it.I;
  const int row0 = (it.tile * WAVES + wv) * 16 * R;  // this wave's first output column
  const Mat w = w2_mat<WT>(it.w, H, Ie);
  const __amdgpu_buffer_rsrc_t src =
      make_rsrc(a.h, ((size_t)a.T * a.k + (a.shared_w ? a.T : 0)) * a.h_ld * 2);
  int atile[R];
#pragma unroll
  for (int t = 0; t < R; ++t) atile[t] = min(row0 / 16 + t, H / 16 - 1);  // rows past H: loaded, never stored
  for (int pass = 0; pass < it.n; pass += NT * 16) {
    const int ntl = min(NT, (it.n - pass + 15) / 16);
    int row_off[PIECES];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int row = (threadIdx.x + i * WAVES * 64) / (KC / 8);
      row_off[i] = (it.hrow0 + min(pass + row, it.n - 1)) * a.h_ld * 2;
    }
    auto epi = [&](int t, int nt, const f32x4& v) {
      const int c0 = row0 + 16 * t;
      const int i = pass + nt * 16 + r;
      if (c0 < H && i < it.n) {
        float* dst = it.shared ? a.shared_out + (size_t)i * H : a.out_rows + (size_t)(it.p0 + i) * H;
        *reinterpret_cast<float4*>(dst + c0 + g * 4) = make_float4(v[0], v[1], v[2], v[3]);
      }
    };
    prefill_dispatch<WT, NT, R, KC, WAVES>(ntl, w, atile, src, row_off, sb, epi);
  }
}

// ---------------------------------------------------------------------------
// Launch: 8 waves, up to 128 tokens per pass, KC = 128 columns per chunk;
// R = 2 row tiles per wave (bf16 and MXFP4).
#ifndef MOE_PF_R
#define MOE_PF_R 2
#endif
#ifndef MOE_PF_KC_MX
#define MOE_PF_KC_MX 128
#endif
#ifndef MOE_PF_WAVES
#define MOE_PF_WAVES 8
#endif
constexpr int kPfNT = 8, kPfR = MOE_PF_R, kPfKC = 128, kPfKCmx = MOE_PF_KC_MX, kPfWaves = MOE_PF_WAVES;

bool prefill_supported(int wtype, int H, int I, int I_shared) {
  if (wtype != W_BF16 && wtype != W_MXFP4) return false;
  const int kc = wtype == W_MXFP4 ? kPfKCmx : kPfKC;
  return H % kc == 0 && I % kc == 0 && I_shared % kc == 0;
}

static unsigned pad8(unsigned g) { return (g + 7) / 8 * 8; }

hipError_t launch_prefill_gate_up(int wtype, const FfnArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const bool sh = a.shared_w != nullptr;
  constexpr int rb = 8 * kPfR * kPfWaves;  // intermediate indices per block
  const int shared_tiles = sh ? (a.I_shared + rb - 1) / rb : 0, routed_tiles = (a.I + rb - 1) / rb;
  const unsigned grid = pad8(shared_tiles + a.routed_items * routed_tiles);
  if (wtype == W_BF16)
    hipLaunchKernelGGL((prefill_gate_up<W_BF16, kPfNT, kPfR, kPfKC, kPfWaves>), dim3(grid), dim3(kPfWaves * 64), 0, st,
                       a, shared_tiles, routed_tiles);
  else
    hipLaunchKernelGGL((prefill_gate_up<W_MXFP4, kPfNT, kPfR, kPfKCmx, kPfWaves>), dim3(grid), dim3(kPfWaves * 64),
                       0, st, a, shared_tiles, routed_tiles);
  return hipGetLastError();
}

hipError_t launch_prefill_down(int wtype, const FfnArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const bool sh = a.shared_w != nullptr;
  constexpr int rb = 16 * kPfR * kPfWaves;  // output columns per block
  const int tiles = (a.H + rb - 1) / rb;
  const int shared_tiles = sh ? tiles : 0;
  const unsigned grid = pad8(shared_tiles + a.routed_items * tiles);
  if (wtype == W_BF16)
    hipLaunchKernelGGL((prefill_down<W_BF16, kPfNT, kPfR, kPfKC, kPfWaves>), dim3(grid), dim3(kPfWaves * 64), 0, st, a,
                       shared_tiles, tiles);
  else
    hipLaunchKernelGGL((prefill_down<W_MXFP4, kPfNT, kPfR, kPfKCmx, kPfWaves>), dim3(grid), dim3(kPfWaves * 64), 0,
                       st, a, shared_tiles, tiles);
  return hipGetLastError();
}

}  // namespace moe
