// ffn_prefill.hip -- grouped SwiGLU expert FFN for prefill-sized batches on gfx950:
// one grouped GEMM per phase (gate_up with the SiLU * up epilogue, then down).
//
// Pages: "Meet FreeToken: An Edge-Native MoE Serving Engine that Runs 753B GLM-5.2
// on a Single Workstation GPU" (MarkTechPost): a prefill pass sends thousands of
// tokens to nearly every expert of a layer ("The gap it targets"), so each expert
// carries a batch of tokens and its weights are worth reading once for all of
// them.  Same arithmetic as the decode kernels (bf16 MFMA with f32 accumulation,
// MXFP4 expanded to bf16 exactly, SwiGLU intermediate rounded to bf16); only the
// data movement differs.
//
// MFMA: v_mfma_f32_32x32x16_bf16.  Weights are the A operand (32 rows: two stored
// 16-row tiles), tokens the B operand (32 columns).  Lane l supplies row / column
// l % 32; the lane half h = l / 32 supplies 8 of the 16 k of every step, and A and B
// use the same assignment, so the products pair up whatever the order inside the
// instruction.  MXFP4: a lane's 16 bytes of codes are one 32-element block (one
// E8M0 scale); over a 64-column chunk lane half h takes block h, and k-step m of
// the chunk uses elements 8m .. 8m+7 of it.  bf16: k-step m takes k = 16m + 8h.
// D: lane l, element v holds row 8 (v / 4) + 4 h + v % 4, column l % 32.
//
// Block (MXFP4) = 8 waves (two per SIMD, so one wave's conversions and address
// work overlap the other's MFMAs) over 16 32-row tiles of one expert (wave w:
// tiles 2w, 2w + 1; bf16 weights: 4 waves, one per SIMD) and up to 128 of its
// tokens per pass (NT tiles of 32, a compile-time
// count): 512 weight rows per block.  Each LDS B fragment feeds 2 MFMAs.  The K
// dimension is walked in chunks of 64 columns with a ring of 4:
//  * weights stream from HBM straight into registers (each wave its own rows);
//  * token rows go from global memory straight into LDS (buffer loads with the
//    LDS destination), shared by the block's waves; a 128-byte row of a chunk is 8 pieces
//    of 16 bytes, piece p of row r stored at position p ^ ((r + r / 8) % 8), so the
//    rows one 128-bit LDS read touches land in distinct bank groups whether the
//    read is served 8 or 16 lanes at a time;
//  * the loads of chunk c+3 are issued before chunk c is computed; every load is
//    unconditional (past the end they re-read the last chunk), so each wave issues
//    exactly NL loads per chunk and "chunk c+1 has landed" is the wait vmcnt(2 NL),
//    followed by a barrier that makes the LDS rows visible.
// Measured on the MI355X (same box, MXFP4 gate_up at the 4096-token shape): this
// shape 988-996 us, one wave per SIMD with 4 tiles per wave 1067 us, the earlier
// 16x16x32 design 1080-1091 us.
// Blocks are ordered so that the blocks of one expert run together on one XCD
// (blockIdx b executes on XCD b % 8), keeping its token rows in that XCD's L2.
#include "ffn_common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace moe {

constexpr int kGKC = 64;                            // K columns per chunk
constexpr int kGRowBytes = kGKC * 2;                // one token row of a chunk (bf16)
constexpr int kGMaxNT = 4;                          // token tiles of 32 per pass
constexpr int kGPassRows = 32 * kGMaxNT;            // 128 tokens per pass
constexpr int kGBufBytes = kGPassRows * kGRowBytes; // 16 KB per ring slot
constexpr int kGDepth = 4;                          // ring slots (LDS buffers, register sets)

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int WT>
struct GCfg {
  // waves per block: two per SIMD for MXFP4; bf16 weights need 4 code loads per
  // tile and chunk, whose ring fits only at one wave per SIMD
  static constexpr int W = WT == W_MXFP4 ? 8 : 4;
  static constexpr int R = 2;                        // 32-row weight tiles per wave
  static constexpr int LPT = WT == W_MXFP4 ? 1 : 4;  // 16-byte code loads per row tile and chunk
  static constexpr int SPT = WT == W_MXFP4 ? 1 : 0;  // scale words per row tile and chunk
};

// Token-row pieces of 1 KB (8 rows of a chunk) per wave per chunk: 4 NT pieces
// spread over the waves (a wave past the last piece re-loads it).
template <int WT, int NT>
struct GPieces {
  static constexpr int value = (4 * NT + GCfg<WT>::W - 1) / GCfg<WT>::W;
};
// Loads per wave per chunk: its token-row pieces plus the weights.
template <int WT, int NT>
struct GLoads {
  static constexpr int value = GPieces<WT, NT>::value + GCfg<WT>::R * (GCfg<WT>::LPT + GCfg<WT>::SPT);
};

// One ring slot of weight registers: the wave's R row tiles for one chunk.
template <int WT>
struct GA {
  u32x4 code[GCfg<WT>::R][GCfg<WT>::LPT];
  uint32_t sw[GCfg<WT>::R];
};

__device__ __forceinline__ int g_swz(int r) { return (r + (r >> 3)) & 7; }

// Wait until at most N vector loads of this wave are outstanding and its LDS
// accesses are done, then barrier.  The wait goes through the builtin so that the
// compiler's own wait placement knows the older loads have landed; the empty asm
// statements keep memory accesses from moving across.
template <int N>
__device__ __forceinline__ void g_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt fields: vmcnt[3:0] and [15:14], expcnt[6:4] (7: no wait), lgkmcnt[11:8].
  constexpr int imm = (N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane of token rows, global memory -> LDS at buf + 16 * lane.
__device__ __forceinline__ void g_dma16(__amdgpu_buffer_rsrc_t src, int voff, int soff, uint8_t* buf) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_ptr_t)buf, 16, voff, soff, 0, 0);
}

// Per-lane offsets of the wave's weight fragments inside a tiled matrix (the
// uniform part, tile and column step, goes into the scalar offset).
struct GLane {
  int code_voff;   // lane's fragment inside the (tile, step) pair it reads
  int scale_voff;  // MXFP4: lane's bytes inside the scale block pair
};

template <int WT>
__device__ __forceinline__ void g_issue_weights(GA<WT>& a, const Mat& w, const GLane& ln, const int (&st0)[GCfg<WT>::R],
                                                int c) {
  constexpr int R = GCfg<WT>::R;
#pragma unroll
  for (int t = 0; t < R; ++t) {
    if constexpr (WT == W_MXFP4) {
      const int s = c >> 1;  // 128-column step holding the chunk
      a.code[t][0] = bld16(w.codes, ln.code_voff, (st0[t] * w.nK + s) * 1024 + (c & 1) * 512);
      a.sw[t] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
          w.scales, ln.scale_voff, (st0[t] * w.nKs + (s >> 4)) * 1024 + (c & 1) * 512 + ((s & 15) >> 2) * 4, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)  // k-step j of the chunk: 32-column step 2c + j / 2, half j % 2
        a.code[t][j] = bld16(w.codes, ln.code_voff, (st0[t] * w.nK + 2 * c + (j >> 1)) * 1024 + (j & 1) * 512);
      a.sw[t] = 0u;
    }
  }
}

// acc[t][nt] += A_t . B_nt over one chunk (4 k-steps of 16): A from registers, B
// from the LDS ring slot `buf`.  The LDS reads and the conversions of k-step m+1
// are issued before the MFMAs of step m (two operand sets), and the steps are
// fenced, so that the reads have R * NT MFMAs to land behind and only two steps'
// operands are live at a time.
template <int WT, int NT>
__device__ __forceinline__ void g_compute(const GA<WT>& a, const uint8_t* buf, int c, const int (&brow)[NT],
                                          const int (&bswz)[NT], f32x16 (&acc)[GCfg<WT>::R][NT]) {
  constexpr int R = GCfg<WT>::R;
  const int h = (threadIdx.x & 63) >> 5;
  float sc[R];
  if constexpr (WT == W_MXFP4) {
    const int sh = 8 * ((c >> 1) & 3);
#pragma unroll
    for (int t = 0; t < R; ++t) sc[t] = e8m0_to_f32((a.sw[t] >> sh) & 0xffu);
  }
  bf16x8 B[2][NT], A[2][R];
  auto operands = [&](int m, bf16x8 (&b)[NT], bf16x8 (&aa)[R]) {
    const int p = WT == W_MXFP4 ? 4 * h + m : 2 * m + h;  // 16-byte piece of the token row
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      b[nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(buf + brow[nt] + ((p ^ bswz[nt]) << 4)));
#pragma unroll
    for (int t = 0; t < R; ++t) {
      if constexpr (WT == W_MXFP4)
        aa[t] = fp4x8_to_bf16x8(a.code[t][0][m], sc[t]);
      else
        aa[t] = as_bf16x8(a.code[t][m]);
    }
  };
  operands(0, B[0], A[0]);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m + 1 < 4) operands(m + 1, B[(m + 1) & 1], A[(m + 1) & 1]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int t = 0; t < R; ++t)
        acc[t][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[m & 1][t], B[m & 1][nt], acc[t][nt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One pass of up to 32 NT tokens over the wave's R row tiles, the whole K loop.
// row_start(i): byte offset of pass row i's first element in the B source (rows
// past the expert's tokens repeat its last token: loaded, never stored).
// tile_of(t): the wave's t-th 32-row tile (clamped to the matrix);
// epi(t, nt, acc) stores one 32 x 32 result tile.
template <int WT, int NT, typename RowStart, typename TileOf, typename Epi>
__device__ __forceinline__ void g_pass(const Mat& w, const TileOf& tile_of, __amdgpu_buffer_rsrc_t src,
                                       const RowStart& row_start, uint8_t* lds, const Epi& epi) {
  constexpr int R = GCfg<WT>::R;
  constexpr int NL = GLoads<WT, NT>::value;
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  const int rho = lane & 31, h = lane >> 5;
  GLane ln;
  ln.code_voff = (rho >> 4) * w.nK * 1024 + (rho & 15) * 16 + h * 256;
  ln.scale_voff = WT == W_MXFP4 ? (rho >> 4) * w.nKs * 1024 + (rho & 15) * 16 + h * 256 : 0;
  int st0[R];
#pragma unroll
  for (int t = 0; t < R; ++t) st0[t] = 2 * tile_of(t);
  // token-row pieces: this wave fills 1 KB pieces d = wv + W i (rows 8 d .. 8 d + 7);
  // lane l writes position l % 8 of row 8 d + l / 8, i.e. source piece pos ^ swz(row)
  constexpr int PW = GPieces<WT, NT>::value;
  constexpr int W = GCfg<WT>::W;
  int dvoff[PW], dpiece[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    dpiece[i] = min(wv + W * i, 4 * NT - 1);
    const int row = 8 * dpiece[i] + (lane >> 3);
    dvoff[i] = row_start(row) + (((lane & 7) ^ g_swz(row)) << 4);
  }
  // this lane's B rows: token tile nt, column lane % 32
  int brow[NT], bswz[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = 32 * nt + rho;
    brow[nt] = r * kGRowBytes;
    bswz[nt] = g_swz(r);
  }
  const int nch = w.K / kGKC;
  GA<WT> a[kGDepth];
  f32x16 acc[R][NT];
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][nt][v] = 0.0f;
  auto issue = [&](int slot, int c) {
#pragma unroll
    for (int i = 0; i < PW; ++i)
      g_dma16(src, dvoff[i], c * kGRowBytes, lds + slot * kGBufBytes + dpiece[i] * 1024);
    g_issue_weights<WT>(a[slot], w, ln, st0, c);
  };
  // The prologue's chunks are kept apart (and in order) like the loop's, so that
  // "two chunks back" counts the same loads.
#pragma unroll
  for (int d = 0; d < kGDepth - 1; ++d) {
    issue(d, min(d, nch - 1));
    asm volatile("" ::: "memory");
  }
  g_wait_barrier<2 * NL>();
  auto step = [&](int d, int c) {
    issue((d + kGDepth - 1) % kGDepth, min(c + kGDepth - 1, nch - 1));
    g_compute<WT, NT>(a[d], lds + d * kGBufBytes, c, brow, bswz, acc);
    g_wait_barrier<2 * NL>();
  };
  int c0 = 0;
  for (; c0 + kGDepth <= nch; c0 += kGDepth) {
#pragma unroll
    for (int d = 0; d < kGDepth; ++d) step(d, c0 + d);
  }
  // K a multiple of 128 but not of 256: two chunks left, ring slots 0 and 1
  if (c0 < nch) {
    step(0, c0);
    step(1, c0 + 1);
  }
  // one result tile at a time: the fence keeps the compiler from converting all
  // R * NT accumulator tiles at once (which would need them all in VGPRs)
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      epi(t, nt, acc[t][nt]);
      __builtin_amdgcn_sched_barrier(0);
    }
}

template <int WT, typename RowStart, typename TileOf, typename Epi>
__device__ __forceinline__ void g_dispatch(int nt, const Mat& w, const TileOf& tile_of, __amdgpu_buffer_rsrc_t src,
                                           const RowStart& row_start, uint8_t* lds, const Epi& epi) {
  switch (nt) {
    case 1: g_pass<WT, 1>(w, tile_of, src, row_start, lds, epi); break;
    case 2: g_pass<WT, 2>(w, tile_of, src, row_start, lds, epi); break;
    case 3: g_pass<WT, 3>(w, tile_of, src, row_start, lds, epi); break;
    default: g_pass<WT, 4>(w, tile_of, src, row_start, lds, epi); break;
  }
}

__device__ __forceinline__ int xcd_logical_block() {
  const int per = gridDim.x / 8;  // the grid is a multiple of 8
  return (blockIdx.x % 8) * per + blockIdx.x / 8;
}

// Blocks per item: 32-row tiles of a routed expert and of the shared expert.
struct GGrid {
  int tiles_per_block;                 // 32-row tiles per block (4 R)
  int shared_tiles, routed_tiles;      // 32-row tiles per item
  int shared_blocks, routed_blocks;    // blocks per item
};

template <int WT>
__global__ __launch_bounds__(GCfg<WT>::W * 64) __attribute__((amdgpu_waves_per_eu(GCfg<WT>::W / 4, GCfg<WT>::W / 4))) void prefill_gate_up(
    FfnArgs a, GGrid gr) {
  const Item it = resolve_item_at(a, xcd_logical_block(), gr.shared_blocks, gr.routed_blocks);
  if (!it.valid) return;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kGDepth * kGBufBytes];
  constexpr int R = GCfg<WT>::R;
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  const int j = lane & 31, h = lane >> 5;
  const int H = a.H, Ie = it.I;
  const int ntiles = Ie / 16;  // 32-row tiles of W13 (2 Ie rows)
  const int tile0 = it.tile * gr.tiles_per_block + wv * R;
  auto tile_of = [&](int t) { return min(tile0 + t, ntiles - 1); };
  const Mat w = w13_mat<WT>(it.w, H, Ie);
  const __amdgpu_buffer_rsrc_t src = make_rsrc(a.x, (size_t)a.T * H * 2);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(a.h);
  for (int pass = 0; pass < it.n; pass += kGPassRows) {
    const int nt = min(kGMaxNT, (it.n - pass + 31) / 32);
    auto row_start = [&](int row) { return item_token(a, it, min(pass + row, it.n - 1)) * H * 2; };
    // 32-row tile T holds gate and up of intermediate indices 16 T .. 16 T + 15:
    // elements 0-3 gate and 4-7 up of 16 T + 4 h + (0..3), 8-11 gate and 12-15 up
    // of 16 T + 8 + 4 h + (0..3)
    auto epi = [&](int t, int ntile, const f32x16& v) {
      const int T = tile0 + t, i = pass + 32 * ntile + j;
      if (T >= ntiles || i >= it.n) return;
      uint16_t* dst = hbuf + (size_t)(it.hrow0 + i) * a.h_ld + 16 * T + 4 * h;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int b = 8 * half;
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16_rne(silu_f32(v[b + 0]) * v[b + 4]) |
                   ((uint32_t)f32_to_bf16_rne(silu_f32(v[b + 1]) * v[b + 5]) << 16);
        packed.y = (uint32_t)f32_to_bf16_rne(silu_f32(v[b + 2]) * v[b + 6]) |
                   ((uint32_t)f32_to_bf16_rne(silu_f32(v[b + 3]) * v[b + 7]) << 16);
        *reinterpret_cast<uint2*>(dst + 8 * half) = packed;
      }
    };
    g_dispatch<WT>(nt, w, tile_of, src, row_start, lds, epi);
  }
}

template <int WT>
__global__ __launch_bounds__(GCfg<WT>::W * 64) __attribute__((amdgpu_waves_per_eu(GCfg<WT>::W / 4, GCfg<WT>::W / 4))) void prefill_down(
    FfnArgs a, GGrid gr) {
  const Item it = resolve_item_at(a, xcd_logical_block(), gr.shared_blocks, gr.routed_blocks);
  if (!it.valid) return;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kGDepth * kGBufBytes];
  constexpr int R = GCfg<WT>::R;
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  const int j = lane & 31, h = lane >> 5;
  const int H = a.H, Ie = it.I;
  const int ntiles = H / 32;  // 32-row tiles of W2 (H rows)
  const int tile0 = it.tile * gr.tiles_per_block + wv * R;
  auto tile_of = [&](int t) { return min(tile0 + t, ntiles - 1); };
  const Mat w = w2_mat<WT>(it.w, H, Ie);
  const __amdgpu_buffer_rsrc_t src =
      make_rsrc(a.h, ((size_t)a.T * a.k + (a.shared_w ? a.T : 0)) * a.h_ld * 2);
  for (int pass = 0; pass < it.n; pass += kGPassRows) {
    const int nt = min(kGMaxNT, (it.n - pass + 31) / 32);
    auto row_start = [&](int row) { return (it.hrow0 + min(pass + row, it.n - 1)) * a.h_ld * 2; };
    // 32-row tile T holds output columns 32 T .. 32 T + 31: elements 4 q .. 4 q + 3
    // are columns 32 T + 8 q + 4 h + (0..3)
    auto epi = [&](int t, int ntile, const f32x16& v) {
      const int T = tile0 + t, i = pass + 32 * ntile + j;
      if (T >= ntiles || i >= it.n) return;
      float* dst = (it.shared ? a.shared_out + (size_t)i * H : a.out_rows + (size_t)(it.p0 + i) * H) + 32 * T + 4 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(dst + 8 * q) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    };
    g_dispatch<WT>(nt, w, tile_of, src, row_start, lds, epi);
  }
}

// ---------------------------------------------------------------------------
bool prefill_supported(int wtype, int H, int I, int I_shared) {
  if (wtype != W_BF16 && wtype != W_MXFP4) return false;
  return H % 128 == 0 && I % 128 == 0 && I_shared % 128 == 0;
}

static unsigned pad8(unsigned g) { return (g + 7) / 8 * 8; }

static GGrid g_grid(int wtype, int routed_tiles, int shared_tiles) {
  GGrid g;
  g.tiles_per_block = wtype == W_MXFP4 ? GCfg<W_MXFP4>::W * GCfg<W_MXFP4>::R : GCfg<W_BF16>::W * GCfg<W_BF16>::R;
  g.routed_tiles = routed_tiles;
  g.shared_tiles = shared_tiles;
  g.routed_blocks = (routed_tiles + g.tiles_per_block - 1) / g.tiles_per_block;
  g.shared_blocks = (shared_tiles + g.tiles_per_block - 1) / g.tiles_per_block;
  return g;
}

hipError_t launch_prefill_gate_up(int wtype, const FfnArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const GGrid gr = g_grid(wtype, a.I / 16, a.shared_w ? a.I_shared / 16 : 0);
  const unsigned grid = pad8(gr.shared_blocks + a.routed_items * gr.routed_blocks);
  if (wtype == W_BF16)
    hipLaunchKernelGGL(prefill_gate_up<W_BF16>, dim3(grid), dim3(GCfg<W_BF16>::W * 64), 0, st, a, gr);
  else
    hipLaunchKernelGGL(prefill_gate_up<W_MXFP4>, dim3(grid), dim3(GCfg<W_MXFP4>::W * 64), 0, st, a, gr);
  return hipGetLastError();
}

hipError_t launch_prefill_down(int wtype, const FfnArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int tiles = a.H / 32;
  const GGrid gr = g_grid(wtype, tiles, a.shared_w ? tiles : 0);
  const unsigned grid = pad8(gr.shared_blocks + a.routed_items * gr.routed_blocks);
  if (wtype == W_BF16)
    hipLaunchKernelGGL(prefill_down<W_BF16>, dim3(grid), dim3(GCfg<W_BF16>::W * 64), 0, st, a, gr);
  else
    hipLaunchKernelGGL(prefill_down<W_MXFP4>, dim3(grid), dim3(GCfg<W_MXFP4>::W * 64), 0, st, a, gr);
  return hipGetLastError();
}

}  // namespace moe
