// ffn.hip -- grouped SwiGLU expert FFN for gfx950.
//
// Pages: "Meet FreeToken: An Edge-Native MoE Serving Engine that Runs 753B GLM-5.2
// on a Single Workstation GPU" (MarkTechPost).  The GPU computes the experts that
// are resident in its cache ("Three mechanisms": bandwidth-adaptive execution),
// with expert output exact and precision never lowered ("Key Takeaways"): MXFP4
// weights are expanded to bf16 exactly before the bf16 MFMA.  The FFN form
// (SwiGLU: down(SiLU(gate x) * up x)) is not on the pages; it is the standard
// MoE expert.
//
// Work decomposition.  A grid slot is (item, tile).  An item is one pass (up to
// 16*NT tokens) of one expert: the shared expert's passes (if any) come first, then
// the passes of the routed experts in ascending id; a block finds "its" item by a
// scan over the offsets (in L2), so the grid is sized from T alone (an upper bound
// on the items) and needs no host synchronisation.  Each pass streams its expert's
// weights once; the passes of one expert run side by side.
// The KW waves of a K split add their partial accumulators in a fixed order, so
// results are deterministic run to run.  Block shapes (waves, K split, row tiles
// per wave, token tiles per pass) are chosen per weight type and batch by the
// launchers below; MXFP4 passes of one token tile may first copy their token rows
// into LDS, and then stream weights through a ring of column steps.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16): weights are the A operand (16 rows),
// tokens the B operand (16 columns), so a single token costs one weight pass.
// Lane l supplies A[row l%16][8 values] and B[col l%16][8 values]; any fixed
// assignment of K indices to the 8-value groups is valid as long as A and B use
// the same one.  bf16 weights: lane group g = l/16 takes k = kb + 8g .. +7.
// MXFP4: lane group g takes one whole 32-element block (16 bytes of codes, one
// scale) at k = kb + 32g and feeds it to 4 MFMAs, the m-th taking elements
// 8m .. 8m+7.
//
// Weights are stored tiled to match (the slot layout of include/moe.h): every
// 16-row x 32-column (bf16) or 16-row x 128-column (MXFP4) tile is the 64 lanes'
// 16-byte A fragments in lane order, tiles row-tile major.  One wave load is
// therefore 1 KB of contiguous HBM, and a wave streams its row tile front to
// back.  W13 tiles hold 8 gate rows followed by the same 8 up rows.
#include "ffn_common.hpp"
#include "kernels.hpp"

namespace moe {

template <typename K, typename... Args>
static void launch_ffn_kernel(K kernel, unsigned grid, hipStream_t st, Args... args) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, st, args...);
}
// Waves per block of the MFMA decode kernels: bf16 splits K over up to 4 waves of a
// block; MXFP4 (no K split) uses 4 with one token tile (the block stages the
// tokens once for 4 waves) and 1 with more (smaller blocks even out the work per
// CU: one-wave blocks measured 14% faster at 64 tokens).
constexpr int kDecMx1Wpb = 4, kDecMxNWpb = 1;
template <int WT, int NT>
constexpr int dec_wpb() { return WT == W_MXFP4 ? (NT == 1 ? kDecMx1Wpb : kDecMxNWpb) : 4; }
static int dec_wpb_of(int wtype, int nt) {
  return wtype == W_MXFP4 ? (nt == 1 ? kDecMx1Wpb : kDecMxNWpb) : 4;
}

template <int WT, int NT, typename K, typename... Args>
static void launch_dec_kernel(K kernel, unsigned grid, size_t lds, hipStream_t st, Args... args) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(64 * dec_wpb<WT, NT>()), lds, st, args...);
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
// Register budget of the decode kernels.  A weight-streaming kernel needs many
// waves' loads in flight; MXFP4 kernels are compiled for at least 2 waves per
// SIMD (3 for the kernels that read their token rows from LDS), with their chunks
// of k steps halved to fit.
constexpr int kDecMxWaves = 2, kDecMxLdsWaves = 3, kDecMxDiv = 2;
constexpr int kDecRing = 4;  // weight steps in flight per wave (token rows in LDS)
template <int WT, int NT, bool LB = false>
struct DecTune {
  static constexpr bool mx = WT == W_MXFP4, mx1 = mx && NT == 1;
  static constexpr int waves = mx && LB ? kDecMxLdsWaves : mx ? kDecMxWaves : 1;
  static constexpr int div = mx ? kDecMxDiv : 1;
};
// k steps per chunk of loads (bounded by the registers two chunks take).
template <int WT, int NT, int R>
struct Unroll {
  static constexpr int raw = WT == W_MXFP4 ? (4 / (NT * R) > 0 ? 4 / (NT * R) : 1)
                                           : (8 / (NT * R) > 0 ? 8 / (NT * R) : 1);
  static constexpr int scaled = (raw > 4 ? 4 : raw) / DecTune<WT, NT>::div;
  static constexpr int value = scaled > 0 ? scaled : 1;
};

// Raw fragments of one chunk of U k steps: R weight rows (A) per step and the
// NT x NA token fragments (B) they share.
template <int WT, int NT, int R, int U>
struct Chunk {
  static constexpr int NA = WT == W_MXFP4 ? 4 : 1;
  u32x4 qa[U][R];
  uint32_t qs[U][R];
  u32x4 qb[U][NT][NA];
};

// Issue the loads of the chunk starting at step s.  Tile t of this wave is row
// tile atile[t] (wave-uniform); this lane's A fragment of step s is fragment
// `lane` of tile (atile[t], s).  B fragments come from row brow[nt] of `rows`.
// No load is predicated, so no lane diverges: padding token columns point at a
// real row (their MFMA columns are never stored) and token tiles nt >= ntl are
// skipped uniformly.  Without CLAMP the chunk must lie inside the wave's step
// range and (MXFP4) K must be a multiple of 128; with CLAMP, steps past s1
// re-read step s1-1 (never computed) and MXFP4 column groups past K (zero codes
// in the padded tile) re-read the row's last 8 values, so every access stays in
// its buffer.
template <int WT, int NT, int R, int U, bool CLAMP, bool SCALES = true, bool LB = false>
__device__ __forceinline__ void load_chunk(Chunk<WT, NT, R, U>& c, const Mat& w, const int (&atile)[R], int s,
                                           int s1, int g, const Rows& rows, const int (&brow)[NT], int ntl) {
  constexpr int KS = KStep<WT>::value;
  constexpr int NA = Chunk<WT, NT, R, U>::NA;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int tile_step = atile[t] * w.nK + s;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int du = CLAMP ? min(s + u, s1 - 1) - s : u;
      c.qa[u][t] = bld16(w.codes, lane * 16, (tile_step + du) * 1024);
      if constexpr (WT == W_MXFP4 && SCALES)
        c.qs[u][t] = load_scale_word(w, lane, atile[t], s + du);
      else
        c.qs[u][t] = 0u;
    }
  }
  if constexpr (LB) return;  // token fragments come from LDS at compute time
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (nt < ntl) {
      const int row_off = brow[nt] * rows.ld * 2;
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int m = 0; m < NA; ++m) {
          if constexpr (CLAMP) {
            const int su = min(s + u, s1 - 1);
            const int kk = WT == W_MXFP4 ? min(su * KS + 32 * g + 8 * m, w.K - 8) : su * KS + 8 * g;
            c.qb[u][nt][m] = bld16(rows.buf, row_off + kk * 2, 0);
          } else {
            const int goff = (WT == W_MXFP4 ? 32 * g : 8 * g) * 2;
            c.qb[u][nt][m] = bld16(rows.buf, row_off + goff, ((s + u) * KS + 8 * m) * 2);
          }
        }
      }
    }
  }
}

// MFMAs of one chunk.  MXFP4 scales come from the chunk's per-step words, or,
// with a scale block `sb` (16 steps per row tile, this lane's 16 bytes), from
// byte sofs + u of it (sofs = the chunk's first step inside the block).  Token
// fragments come from the chunk's registers, or with LB from the pass's rows in
// LDS (row brow[nt], the same column clamp as the global loads).
template <int WT, int NT, int R, int U, bool BLOCK = false, bool LB = false>
__device__ __forceinline__ void compute_chunk(const Chunk<WT, NT, R, U>& c, int s, int s1, int ntl,
                                              f32x4 (&acc)[R][NT], const u32x4* sb, int sofs, const Rows& rows,
                                              const int (&brow)[NT], int K) {
  constexpr int NA = Chunk<WT, NT, R, U>::NA;
  constexpr int KS = KStep<WT>::value;
  auto bfrag = [&](int u, int nt, int m) -> bf16x8 {
    if constexpr (LB) {
      const int g = (threadIdx.x & 63) >> 4;
      const int kk = WT == W_MXFP4 ? min((s + u) * KS + 32 * g + 8 * m, K - 8) : (s + u) * KS + 8 * g;
      return as_bf16x8(*reinterpret_cast<const u32x4*>(rows.lds + brow[nt] * rows.lds_ld + kk * 2));
    } else {
      return as_bf16x8(c.qb[u][nt][m]);
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (BLOCK || s + u < s1) {
#pragma unroll
      for (int t = 0; t < R; ++t) {
        bf16x8 A[NA];
        if constexpr (WT == W_BF16) {
          A[0] = as_bf16x8(c.qa[u][t]);
        } else {
          const float sc = BLOCK ? scale_of_word(sb[t][((sofs + u) % 16) / 4], sofs + u)
                                 : scale_of_word(c.qs[u][t], s + u);
#pragma unroll
          for (int m = 0; m < 4; ++m) A[m] = fp4x8_to_bf16x8(c.qa[u][t][m], sc);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (nt < ntl) {
#pragma unroll
            for (int m = 0; m < NA; ++m)
              acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[m], bfrag(u, nt, m), acc[t][nt], 0, 0, 0);
          }
        }
      }
    }
  }
}

// acc[t][nt] += A_t . B[nt] over the column steps [s0, s1) of matrix w, A_t
// being row tile atile[t] and B[nt] this lane's token row brow[nt] of `rows`.
// Two chunks of U steps alternate: the loads of chunk c+1 are in flight while
// chunk c is computed, so a wave keeps between U and 2U steps of weight loads
// outstanding; each token fragment is loaded once per step and reused by the R
// weight tiles.
template <int WT, int NT, int R, bool LB = false>
__device__ __forceinline__ void mfma_rows(const Mat& w, const int (&atile)[R], int s0, int s1, int g,
                                          const Rows& rows, const int (&brow)[NT], int ntl, f32x4 (&acc)[R][NT]) {
  constexpr int U = Unroll<WT, NT, R>::value;
  if (s0 >= s1) return;
  Chunk<WT, NT, R, U> c0, c1;
  if constexpr (WT == W_MXFP4 && LB) {
    // Token rows in LDS, so weight fragments are the only vector-memory loads:
    // a ring of kDecRing column steps per wave keeps that many steps of weights
    // in flight (step s requests step s + kDecRing - 1 into the slot step s - 1
    // has just used); scale blocks a block ahead as below.  The body is unrolled
    // over 16-step blocks, so ring slots and scale bytes are fixed positions.
    static_assert(16 % kDecRing == 0, "ring slots tile a scale block");
    if (s0 % 16 == 0 && (s1 - s0) % 16 == 0 && w.K % 128 == 0) {
      const int lane = threadIdx.x & 63, g = lane >> 4;
      const int nb = (s1 - s0) / 16;
      u32x4 ring[kDecRing][R];
      u32x4 sb[2][R];
      auto load_sb = [&](u32x4(&dst)[R], int step) {
#pragma unroll
        for (int t = 0; t < R; ++t) dst[t] = load_scale_block(w, lane, atile[t], step);
      };
      auto load_a = [&](u32x4(&dst)[R], int step) {
#pragma unroll
        for (int t = 0; t < R; ++t) dst[t] = bld16(w.codes, lane * 16, (atile[t] * w.nK + step) * 1024);
      };
      auto compute = [&](const u32x4(&a)[R], const u32x4(&sbk)[R], int sofs, int s) {
        bf16x8 B[NT][4];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int m = 0; m < 4; ++m)
            B[nt][m] = as_bf16x8(*reinterpret_cast<const u32x4*>(rows.lds + brow[nt] * rows.lds_ld +
                                                                 (s * 128 + 32 * g + 8 * m) * 2));
#pragma unroll
        for (int t = 0; t < R; ++t) {
          const float sc = scale_of_word(sbk[t][sofs / 4], sofs);
          bf16x8 A[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) A[m] = fp4x8_to_bf16x8(a[t][m], sc);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            if (nt < ntl)
#pragma unroll
              for (int m = 0; m < 4; ++m)
                acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[m], B[nt][m], acc[t][nt], 0, 0, 0);
        }
      };
      auto block = [&](u32x4(&cur)[R], u32x4(&next)[R], int sblk) {
        load_sb(next, min(sblk + 16, s1 - 16));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          load_a(ring[(i + kDecRing - 1) % kDecRing], min(sblk + i + kDecRing - 1, s1 - 1));
          __builtin_amdgcn_sched_barrier(0);  // keep the request ahead of this step's work
          compute(ring[i % kDecRing], cur, i, sblk + i);
        }
      };
      load_sb(sb[0], s0);
#pragma unroll
      for (int d = 0; d < kDecRing - 1; ++d) load_a(ring[d], min(s0 + d, s1 - 1));
      for (int b = 0; b < nb; b += 2) {
        block(sb[0], sb[1], s0 + 16 * b);
        if (b + 1 < nb) block(sb[1], sb[0], s0 + 16 * (b + 1));
      }
      return;
    }
  }
  if constexpr (WT == W_MXFP4) {
    // Whole 16-step scale blocks: one 16-byte scale load per lane and row tile
    // per block, issued a block ahead (two register sets, so the unrolled body
    // picks scale bytes at fixed positions); every load is unconditional (the
    // chunk past the end re-reads the last one, the block past the end the last
    // block).
    static_assert(16 % (2 * U) == 0, "chunk pairs tile a scale block");
    if (s0 % 16 == 0 && (s1 - s0) % 16 == 0 && w.K % 128 == 0) {
      const int lane = threadIdx.x & 63;
      const int nb = (s1 - s0) / 16;
      u32x4 sb[2][R];
      auto load_sb = [&](u32x4(&dst)[R], int step) {
#pragma unroll
        for (int t = 0; t < R; ++t) dst[t] = load_scale_block(w, lane, atile[t], step);
      };
      auto block = [&](u32x4(&cur)[R], u32x4(&next)[R], int sblk) {
        load_sb(next, min(sblk + 16, s1 - 16));
#pragma unroll
        for (int i = 0; i < 16 / (2 * U); ++i) {
          const int s = sblk + 2 * U * i;
          load_chunk<WT, NT, R, U, false, false, LB>(c1, w, atile, s + U, s1, g, rows, brow, ntl);
          compute_chunk<WT, NT, R, U, true, LB>(c0, s, s1, ntl, acc, cur, 2 * U * i, rows, brow, w.K);
          load_chunk<WT, NT, R, U, false, false, LB>(c0, w, atile, min(s + 2 * U, s1 - U), s1, g, rows, brow,
                                                     ntl);
          compute_chunk<WT, NT, R, U, true, LB>(c1, s + U, s1, ntl, acc, cur, 2 * U * i + U, rows, brow, w.K);
        }
      };
      load_sb(sb[0], s0);
      load_chunk<WT, NT, R, U, false, false, LB>(c0, w, atile, s0, s1, g, rows, brow, ntl);
      for (int b = 0; b < nb; b += 2) {
        block(sb[0], sb[1], s0 + 16 * b);
        if (b + 1 < nb) block(sb[1], sb[0], s0 + 16 * (b + 1));
      }
      return;
    }
  }
  if ((s1 - s0) % (2 * U) == 0 && (WT != W_MXFP4 || w.K % 128 == 0)) {
    load_chunk<WT, NT, R, U, false, true, LB>(c0, w, atile, s0, s1, g, rows, brow, ntl);
    for (int s = s0; s < s1; s += 2 * U) {
      load_chunk<WT, NT, R, U, false, true, LB>(c1, w, atile, s + U, s1, g, rows, brow, ntl);
      compute_chunk<WT, NT, R, U, false, LB>(c0, s, s1, ntl, acc, nullptr, 0, rows, brow, w.K);
      if (s + 2 * U < s1)
        load_chunk<WT, NT, R, U, false, true, LB>(c0, w, atile, s + 2 * U, s1, g, rows, brow, ntl);
      compute_chunk<WT, NT, R, U, false, LB>(c1, s + U, s1, ntl, acc, nullptr, 0, rows, brow, w.K);
    }
    return;
  }
  load_chunk<WT, NT, R, U, true, true, LB>(c0, w, atile, s0, s1, g, rows, brow, ntl);
  for (int s = s0; s < s1; s += 2 * U) {
    load_chunk<WT, NT, R, U, true, true, LB>(c1, w, atile, s + U, s1, g, rows, brow, ntl);
    compute_chunk<WT, NT, R, U, false, LB>(c0, s, s1, ntl, acc, nullptr, 0, rows, brow, w.K);
    load_chunk<WT, NT, R, U, true, true, LB>(c0, w, atile, s + 2 * U, s1, g, rows, brow, ntl);
    compute_chunk<WT, NT, R, U, false, LB>(c1, s + U, s1, ntl, acc, nullptr, 0, rows, brow, w.K);
  }
}

// Block shape (both phases): 4 waves.  Each wave owns R row tiles of 16 rows;
// KW waves split the K range of the same tiles and add their partial accumulators
// in a fixed order through LDS.  A block therefore covers 16 * R * (4/KW) rows of
// one item.

// Token rows of a pass in LDS (LB kernels): the block copies the pass's np real
// rows, K bf16 each, into rows of K*2 + 16 bytes (the 16 bytes of padding put the
// 16 rows of one 128-bit read on different banks); row_start(i) is the element
// offset of pass row i in `src`.  Lane rows past np re-read row np-1.
template <typename RowStart>
__device__ __forceinline__ void stage_rows(uint8_t* lds, const uint16_t* src, int np, int K,
                                           const RowStart& row_start) {
  const int pieces = K / 8, ld = K * 2 + 16;
  for (int q = threadIdx.x; q < np * pieces; q += blockDim.x) {
    const int row = q / pieces, pc = q - row * pieces;
    *reinterpret_cast<u32x4*>(lds + row * ld + pc * 16) =
        *reinterpret_cast<const u32x4*>(src + row_start(row) + (size_t)pc * 8);
  }
}

// gate_up: row tile t of a wave is 8 intermediate indices j..j+7 of one item: one
// 16-row A tile = gate rows j..j+7 stacked on up rows j..j+7, so the epilogue
// pairs lane l (gate) with lane l+32 (up) and writes h = SiLU(gate) * up as bf16.
template <int WT, int NT, int KW, int R, bool LB = false>
__global__ __launch_bounds__((64 * dec_wpb<WT, NT>())) __attribute__((amdgpu_waves_per_eu(DecTune<WT, NT, LB>::waves))) void gate_up_mfma(
    FfnArgs a, int shared_tiles, int routed_tiles) {
  constexpr int RT = dec_wpb<WT, NT>() / KW;
  static_assert(RT >= 1, "waves per block split by KW");
  const Item it = resolve_item<(NT > 1)>(a, shared_tiles, routed_tiles);  // one-tile passes never split
  if (!it.valid) return;
  __shared__ f32x4 red[KW > 1 ? dec_wpb<WT, NT>() : 1][R][NT][64];
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  const int rg = wv / KW, kp = wv % KW;
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, Ie = it.I;
  // tiles of this wave: j0 + 8 t, t < R (the last block of an item may hold fewer)
  const int j0 = (it.tile * RT + rg) * 8 * R;
  const int ntiles = max(0, min(R, (Ie - j0) / 8));
  // W13 row tile j0/8 + t holds gate and up rows of j0+8t .. j0+8t+7
  int atile[R];
#pragma unroll
  for (int t = 0; t < R; ++t) atile[t] = j0 / 8 + t;
  const int nsteps = ksteps<WT>(H);
  const int s0 = kp * nsteps / KW, s1 = (kp + 1) * nsteps / KW;
  const Mat w = w13_mat<WT>(it.w, H, Ie);
  Rows rows;
  rows.buf = make_rsrc(a.x, (size_t)a.T * H * 2);
  rows.ld = H;
  rows.lds = nullptr;
  rows.lds_ld = 0;
  uint16_t* h = reinterpret_cast<uint16_t*>(a.h);
  for (int pass = 0; pass < it.n; pass += NT * 16) {
    const int ntl = min(NT, (it.n - pass + 15) / 16);
    int xrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int i = min(pass + nt * 16 + r, it.n - 1);  // padding columns re-read a real row
      xrow[nt] = item_token<(NT > 1)>(a, it, i);
    }
    bool staged = false;  // uniform per block: this pass's token rows are in LDS
    if constexpr (LB) {
      extern __shared__ __attribute__((aligned(16))) uint8_t lds_rows[];
      const int np = min(NT * 16, it.n - pass);
      staged = np <= a.lds_rows;
      if (pass > 0) __syncthreads();  // the previous pass has finished reading
      if (staged)
        stage_rows(lds_rows, reinterpret_cast<const uint16_t*>(a.x), np, H,
                   [&](int i) { return (size_t)item_token<(NT > 1)>(a, it, pass + i) * H; });
      __syncthreads();
      if (staged) {
        rows.lds = lds_rows;
        rows.lds_ld = H * 2 + 16;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) xrow[nt] = min(nt * 16 + r, np - 1);
      }
    }
    f32x4 acc[R][NT];
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (ntiles == R) {
      if (staged)
        mfma_rows<WT, NT, R, LB>(w, atile, s0, s1, g, rows, xrow, ntl, acc);
      else
        mfma_rows<WT, NT, R, false>(w, atile, s0, s1, g, rows, xrow, ntl, acc);
    } else if (ntiles > 0) {
      // ragged last tiles of the item: one tile at a time
      for (int t = 0; t < ntiles; ++t) {
        f32x4 one[1][NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) one[0][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile1[1] = {j0 / 8 + t};
        if (staged)
          mfma_rows<WT, NT, 1, LB>(w, tile1, s0, s1, g, rows, xrow, ntl, one);
        else
          mfma_rows<WT, NT, 1, false>(w, tile1, s0, s1, g, rows, xrow, ntl, one);
#pragma unroll
        for (int tt = 0; tt < R; ++tt)
          if (tt == t)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[tt][nt] = one[0][nt];
      }
    }
    if (KW > 1) {
      if (kp > 0) {
#pragma unroll
        for (int t = 0; t < R; ++t)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) red[wv][t][nt][lane] = acc[t][nt];
      }
      __syncthreads();
    }
    if (kp == 0) {
#pragma unroll
      for (int t = 0; t < R; ++t) {
        if (t < ntiles) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if (nt < ntl) {
              f32x4 v = acc[t][nt];
#pragma unroll
              for (int q = 1; q < KW; ++q) v += red[wv + q][t][nt][lane];
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
                *reinterpret_cast<uint2*>(h + (size_t)(it.hrow0 + i) * a.h_ld + j0 + 8 * t + g * 4) = packed;
              }
            }
          }
        }
      }
    }
    if (KW > 1) __syncthreads();
  }
}

// down: row tile t of a wave is 16 output columns (rows of W2) of one item.
template <int WT, int NT, int KW, int R, bool LB = false>
__global__ __launch_bounds__((64 * dec_wpb<WT, NT>())) __attribute__((amdgpu_waves_per_eu(DecTune<WT, NT, LB>::waves))) void down_mfma(
    FfnArgs a, int shared_tiles, int routed_tiles) {
  constexpr int RT = dec_wpb<WT, NT>() / KW;
  static_assert(RT >= 1, "waves per block split by KW");
  const Item it = resolve_item<(NT > 1)>(a, shared_tiles, routed_tiles);  // one-tile passes never split
  if (!it.valid) return;
  __shared__ f32x4 red[KW > 1 ? dec_wpb<WT, NT>() : 1][R][NT][64];
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  const int rg = wv / KW, kp = wv % KW;
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, Ie = it.I;
  const int row0 = (it.tile * RT + rg) * 16 * R;
  const int ntiles = max(0, min(R, (H - row0) / 16));
  const int nsteps = ksteps<WT>(Ie);
  const int s0 = kp * nsteps / KW, s1 = (kp + 1) * nsteps / KW;
  const Mat w = w2_mat<WT>(it.w, H, Ie);
  Rows rows;
  rows.buf = make_rsrc(a.h, ((size_t)a.T * a.k + (a.shared_w ? a.T : 0)) * a.h_ld * 2);
  rows.ld = a.h_ld;
  rows.lds = nullptr;
  rows.lds_ld = 0;
  for (int pass = 0; pass < it.n; pass += NT * 16) {
    const int ntl = min(NT, (it.n - pass + 15) / 16);
    int hrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int i = min(pass + nt * 16 + r, it.n - 1);  // padding columns re-read a real row
      hrow[nt] = it.hrow0 + i;
    }
    bool staged = false;  // uniform per block: this pass's token rows are in LDS
    if constexpr (LB) {
      extern __shared__ __attribute__((aligned(16))) uint8_t lds_rows[];
      const int np = min(NT * 16, it.n - pass);
      staged = np <= a.lds_rows;
      if (pass > 0) __syncthreads();  // the previous pass has finished reading
      if (staged)
        stage_rows(lds_rows, reinterpret_cast<const uint16_t*>(a.h), np, Ie,
                   [&](int i) { return (size_t)(it.hrow0 + pass + i) * a.h_ld; });
      __syncthreads();
      if (staged) {
        rows.lds = lds_rows;
        rows.lds_ld = Ie * 2 + 16;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) hrow[nt] = min(nt * 16 + r, np - 1);
      }
    }
    f32x4 acc[R][NT];
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (ntiles == R) {
      int atile[R];
#pragma unroll
      for (int t = 0; t < R; ++t) atile[t] = row0 / 16 + t;
      if (staged)
        mfma_rows<WT, NT, R, LB>(w, atile, s0, s1, g, rows, hrow, ntl, acc);
      else
        mfma_rows<WT, NT, R, false>(w, atile, s0, s1, g, rows, hrow, ntl, acc);
    } else if (ntiles > 0) {
      for (int t = 0; t < ntiles; ++t) {
        f32x4 one[1][NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) one[0][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile1[1] = {row0 / 16 + t};
        if (staged)
          mfma_rows<WT, NT, 1, LB>(w, tile1, s0, s1, g, rows, hrow, ntl, one);
        else
          mfma_rows<WT, NT, 1, false>(w, tile1, s0, s1, g, rows, hrow, ntl, one);
#pragma unroll
        for (int tt = 0; tt < R; ++tt)
          if (tt == t)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[tt][nt] = one[0][nt];
      }
    }
    if (KW > 1) {
      if (kp > 0) {
#pragma unroll
        for (int t = 0; t < R; ++t)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) red[wv][t][nt][lane] = acc[t][nt];
      }
      __syncthreads();
    }
    if (kp == 0) {
#pragma unroll
      for (int t = 0; t < R; ++t) {
        if (t < ntiles) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if (nt < ntl) {
              f32x4 v = acc[t][nt];
#pragma unroll
              for (int q = 1; q < KW; ++q) v += red[wv + q][t][nt][lane];
              const int i = pass + nt * 16 + r;
              if (i < it.n) {
                float* dst = it.shared ? a.shared_out + (size_t)((NT > 1 ? it.p0 : 0) + i) * H : a.out_rows + (size_t)(it.p0 + i) * H;
                *reinterpret_cast<float4*>(dst + row0 + 16 * t + g * 4) = make_float4(v[0], v[1], v[2], v[3]);
              }
            }
          }
        }
      }
    }
    if (KW > 1) __syncthreads();
  }
}

// ===========================================================================
// Launchers
// ===========================================================================
size_t ffn_workspace_xq_offset(int T, int k, int I, int I_shared) {
  const size_t rows = (size_t)T * k + (I_shared > 0 ? (size_t)T : 0);
  const size_t ld = (size_t)(I > I_shared ? I : I_shared);
  return (rows * ld * 2 + 255) / 256 * 256;
}

size_t ffn_workspace_bytes(int wtype, int T, int k, int H, int I, int I_shared) {
  const size_t rows = (size_t)T * k + (I_shared > 0 ? (size_t)T : 0);
  const size_t ld = (size_t)(I > I_shared ? I : I_shared);
  if (wtype == W_MXFP4_A8)  // intermediate, then E4M3 codes [T][H] and E8M0 scales [T][H/32]
    return ffn_workspace_xq_offset(T, k, I, I_shared) + (size_t)T * H + ((size_t)T * H / 32 + 255) / 256 * 256;
  return rows * ld * (wtype == W_F32 ? 4 : 2);
}

// Block shapes by weight type, phase and batch, from a sweep on the MI355X
// (decode shapes: bf16 H=2048/I=512, MXFP4 H=4096/I=2048; T = 1 .. 64):
//   gate_up bf16   T <= 4: KW=4, R=1   else KW=2, R=1
//   gate_up MXFP4  T <= 16: KW=1, R=2  else KW=1, R=4
//   down    bf16   T = 1: KW=2, R=1   else KW=1, R=2
//   down    MXFP4  T <= 16: KW=1, R=2  else KW=1, R=4
struct Shape {
  int kw, r;
};
constexpr int kDecMx1R = 2, kDecMxNR = 4;  // MXFP4 row tiles per wave, T <= 16 / more
static Shape gate_up_shape(int wtype, int T) {
  if (wtype == W_BF16) return T <= 4 ? Shape{4, 1} : Shape{2, 1};
  return T <= 16 ? Shape{1, kDecMx1R} : Shape{1, kDecMxNR};
}
// bf16 down: one token's few experts fill the GPU only with K split over 2 waves of
// one row tile each (T = 1: 5% faster per layer); larger batches take 2 row tiles
// per wave over the whole K.
static Shape down_shape(int wtype, int T) {
  if (wtype == W_BF16) return T == 1 ? Shape{2, 1} : Shape{1, 2};
  return T <= 16 ? Shape{1, kDecMx1R} : Shape{1, kDecMxNR};
}

constexpr int kDecMxNtMax = 2;  // MXFP4: token tiles per pass
// The MXFP4 launchers build one kernel family per row-tile count of the shape
// table: kDecMx1R row tiles with one-tile passes (T <= 16), kDecMxNR with two.
static_assert(kDecMxNtMax == 2 && kDecMx1R != kDecMxNR, "MXFP4 decode shapes: (kDecMx1R, 1 tile), (kDecMxNR, 2 tiles)");
template <int WT, int R>
constexpr int mx_nt() { return R == kDecMx1R ? 1 : 2; }
static int pick_nt(int T, int wtype) {
  const int nt = T <= 16 ? 1 : T <= 32 ? 2 : T <= 64 ? 4 : 8;
  return wtype == W_MXFP4 && nt > kDecMxNtMax ? kDecMxNtMax : nt;
}

// Work items of the MFMA decode kernels are single passes: an expert with more pairs
// than one pass holds gives one item per pass, so its passes run on different waves
// at the same time (the waves of an item's passes stream the same weights, which the
// block order puts on one XCD, and each wave's work is at most one pass: a busy
// expert's second pass no longer decides when the launch ends).
static FfnArgs pass_split(const FfnArgs& a, int wtype) {
  FfnArgs b = a;
  const int P = 16 * pick_nt(a.T, wtype);  // a power of two
  // else no expert has more pairs than one pass holds (at most T); in particular the
  // one-tile kernels (T <= 16), compiled without the split, always get 0
  if (P < a.T) {
    b.pass_rows = P;
    b.routed_items = routed_item_bound(a.T, a.k, a.E, P);
  }
  return b;
}

// MXFP4 passes of one token tile take their token rows from LDS (staged once per
// pass and block): the launch's dynamic LDS holds as many rows of K columns as fit
// in the budget (more would cap the blocks per CU), at most min(T, 16); a block
// whose pass has more rows reads them from memory instead.  The budget is 48 KB, or
// up to 8 tokens 64 KB + 128 (8 rows at K = 4096): then every expert's rows are
// staged at the cost of one block fewer per CU, 2% faster per layer at 8 tokens
// (at 16 tokens the larger budget measured 1.5% slower).
constexpr size_t kDecLdsRowsMax = 49152, kDecLdsRowsMaxSmallT = 8 * (4096 * 2 + 16);
static int lds_rows_for(int T, int K) {
  if (T < 1) return 0;
  const size_t budget = T <= 8 ? kDecLdsRowsMaxSmallT : kDecLdsRowsMax;
  const int fit = (int)(budget / ((size_t)K * 2 + 16));
  const int want = T < 16 ? T : 16;
  return fit < want ? fit : want;
}

template <int WT, int KW, int R>
static void gu_nt(const FfnArgs& a0, hipStream_t st, unsigned grid, int sh, int rt) {
  FfnArgs a = a0;
  a.lds_rows = WT == W_MXFP4 && KW == 1 ? lds_rows_for(a.T, a.H) : 0;
  const size_t lb = (size_t)a.lds_rows * ((size_t)a.H * 2 + 16);
  if constexpr (WT == W_MXFP4) {  // the pass width the shape table pairs with R
    if constexpr (mx_nt<WT, R>() == 1) {
      if (a.lds_rows > 0)
        launch_dec_kernel<WT, 1>(gate_up_mfma<WT, 1, KW, R, KW == 1>, grid, lb, st, a, sh, rt);
      else
        launch_dec_kernel<WT, 1>(gate_up_mfma<WT, 1, KW, R>, grid, 0, st, a, sh, rt);
    } else {
      launch_dec_kernel<WT, 2>(gate_up_mfma<WT, 2, KW, R>, grid, 0, st, a, sh, rt);
    }
  } else {
    switch (pick_nt(a.T, WT)) {
      case 1: launch_dec_kernel<WT, 1>(gate_up_mfma<WT, 1, KW, R>, grid, 0, st, a, sh, rt); break;
      case 2: launch_dec_kernel<WT, 2>(gate_up_mfma<WT, 2, KW, R>, grid, 0, st, a, sh, rt); break;
      case 4: launch_dec_kernel<WT, 4>(gate_up_mfma<WT, 4, KW, R>, grid, 0, st, a, sh, rt); break;
      default: launch_dec_kernel<WT, 8>(gate_up_mfma<WT, 8, KW, R>, grid, 0, st, a, sh, rt); break;
    }
  }
}
template <int WT, int KW, int R>
static void dn_nt(const FfnArgs& a0, hipStream_t st, unsigned grid, int sh, int rt) {
  FfnArgs a = a0;
  const int kmax = a.I > a.I_shared ? a.I : a.I_shared;
  a.lds_rows = WT == W_MXFP4 && KW == 1 ? lds_rows_for(a.T, kmax) : 0;
  const size_t lb = (size_t)a.lds_rows * ((size_t)kmax * 2 + 16);
  if constexpr (WT == W_MXFP4) {  // the pass width the shape table pairs with R
    if constexpr (mx_nt<WT, R>() == 1) {
      if (a.lds_rows > 0)
        launch_dec_kernel<WT, 1>(down_mfma<WT, 1, KW, R, KW == 1>, grid, lb, st, a, sh, rt);
      else
        launch_dec_kernel<WT, 1>(down_mfma<WT, 1, KW, R>, grid, 0, st, a, sh, rt);
    } else {
      launch_dec_kernel<WT, 2>(down_mfma<WT, 2, KW, R>, grid, 0, st, a, sh, rt);
    }
  } else {
    switch (pick_nt(a.T, WT)) {
      case 1: launch_dec_kernel<WT, 1>(down_mfma<WT, 1, KW, R>, grid, 0, st, a, sh, rt); break;
      case 2: launch_dec_kernel<WT, 2>(down_mfma<WT, 2, KW, R>, grid, 0, st, a, sh, rt); break;
      case 4: launch_dec_kernel<WT, 4>(down_mfma<WT, 4, KW, R>, grid, 0, st, a, sh, rt); break;
      default: launch_dec_kernel<WT, 8>(down_mfma<WT, 8, KW, R>, grid, 0, st, a, sh, rt); break;
    }
  }
}

hipError_t launch_ffn_gate_up(int wtype, const FfnArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const bool sh = a.shared_w != nullptr;
  if (wtype == W_F32) {
    const int shared_tiles = sh ? (a.I_shared + 3) / 4 : 0, routed_tiles = (a.I + 3) / 4;
    const unsigned grid = shared_tiles + a.routed_items * routed_tiles;
    if (grid) launch_ffn_kernel(gate_up_f32, grid, st, a, shared_tiles, routed_tiles);
    return hipGetLastError();
  }
  const Shape sp = gate_up_shape(wtype, a.T);
  const FfnArgs b = pass_split(a, wtype);
  const int rb = 8 * sp.r * (dec_wpb_of(wtype, pick_nt(a.T, wtype)) / sp.kw);  // intermediate indices per block
  const int shared_tiles = sh ? (a.I_shared + rb - 1) / rb : 0, routed_tiles = (a.I + rb - 1) / rb;
  const unsigned grid = shared_tiles * shared_items(a.T, b.pass_rows) + b.routed_items * routed_tiles;
  if (!grid) return hipSuccess;
  if (wtype == W_BF16) {
    if (sp.kw == 4) gu_nt<W_BF16, 4, 1>(b, st, grid, shared_tiles, routed_tiles);
    else gu_nt<W_BF16, 2, 1>(b, st, grid, shared_tiles, routed_tiles);
  } else {
    if (sp.r == kDecMx1R) gu_nt<W_MXFP4, 1, kDecMx1R>(b, st, grid, shared_tiles, routed_tiles);
    else gu_nt<W_MXFP4, 1, kDecMxNR>(b, st, grid, shared_tiles, routed_tiles);
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
    if (grid) launch_ffn_kernel(down_f32, grid, st, a, shared_tiles, tiles);
    return hipGetLastError();
  }
  const Shape sp = down_shape(wtype, a.T);
  const FfnArgs b = pass_split(a, wtype);
  const int rb = 16 * sp.r * (dec_wpb_of(wtype, pick_nt(a.T, wtype)) / sp.kw);  // output columns per block
  const int tiles = (a.H + rb - 1) / rb;
  const int shared_tiles = sh ? tiles : 0;
  const unsigned grid = shared_tiles * shared_items(a.T, b.pass_rows) + b.routed_items * tiles;
  if (!grid) return hipSuccess;
  if (wtype == W_BF16) {
    if (sp.kw == 2) dn_nt<W_BF16, 2, 1>(b, st, grid, shared_tiles, tiles);
    else dn_nt<W_BF16, 1, 2>(b, st, grid, shared_tiles, tiles);
  }
  else if (sp.r == kDecMx1R) dn_nt<W_MXFP4, 1, kDecMx1R>(b, st, grid, shared_tiles, tiles);
  else dn_nt<W_MXFP4, 1, kDecMxNR>(b, st, grid, shared_tiles, tiles);
  return hipGetLastError();
}

}  // namespace moe
