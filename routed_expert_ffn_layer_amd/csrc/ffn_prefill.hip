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
//    at least NL loads per chunk and "chunk c+1 has landed" is the wait vmcnt(2 NL),
//    followed by a barrier that makes the LDS rows visible;
//  * MXFP4 scales: each wave copies its tiles' E8M0 bytes for 32 chunks at a time
//    into LDS (one 1 KB load per 16-row tile) and reads one byte per tile and chunk
//    from there, instead of re-loading from memory, every chunk, a word that serves
//    8 chunks (a load as costly to the memory pipeline as the code load beside it).
// Measured on the MI355X (same box, MXFP4 gate_up at the 4096-token shape): this
// shape 988-996 us, one wave per SIMD with 4 tiles per wave 1067 us, the earlier
// 16x16x32 design 1080-1091 us; later, on another box, the scales in LDS 938-941 us
// against 959 us for the per-chunk scale loads (913 us with no scale loads at all).
// Blocks are ordered so that the blocks of one expert run together on one XCD
// (blockIdx b executes on XCD b % 8), keeping its token rows in that XCD's L2, and
// (without a shared expert) the experts go longest first, dealt round robin over
// the XCDs: each XCD gets an even share of the token tiles and ends on its shortest
// items, instead of a run of ascending ids whose last blocks leave CUs idle.
#include "ffn_common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace moe {

constexpr int kGKC = 64;                            // K columns per chunk
constexpr int kGRowBytes = kGKC * 2;                // one token row of a chunk (bf16)

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Kernel shape: weight type, waves per block W, 32-row weight tiles per wave R,
// ring depth D (chunks in flight: LDS slots and weight register sets), token
// tiles of 32 per pass MAXNT, and NATIVE: MXFP4 weights against MXFP8 activations
// on the scaled f8f6f4 MFMA (one 32x32x64 instruction per chunk, no conversion),
// instead of bf16 MFMAs on weights expanded to bf16.
template <int WT_, int W_, int R_, int D_, int MAXNT_, bool NATIVE_ = false>
struct GConf {
  static constexpr int WT = WT_, W = W_, R = R_, D = D_, MAXNT = MAXNT_;
  static constexpr bool NATIVE = NATIVE_;
  static constexpr int LPT = WT == W_MXFP4 ? 1 : 4;  // 16-byte code loads per row tile and chunk
  static constexpr int ROWB = NATIVE ? kGKC : 2 * kGKC;  // bytes of one token row of a chunk
  static constexpr int RPP = 1024 / ROWB;            // token rows per 1 KB piece
  static constexpr int PASS = 32 * MAXNT;            // tokens per pass
  // NATIVE: after the token rows, one 4-byte word of E8M0 scales per pass row
  // (the blocks of the chunk pair holding the chunk)
  static constexpr int ROWS_BYTES = PASS * ROWB;
  static constexpr int BUF = ROWS_BYTES + (NATIVE ? PASS * 4 : 0);  // bytes of one LDS ring slot
  // MXFP4: after the ring, each wave's E8M0 weight scales, two windows of 32
  // chunks (16 steps of 128 columns: one 1 KB scale block per 16-row tile)
  static constexpr int WIN = 2 * 1024;               // one window of one 32-row tile
  static constexpr int SCALE_LDS = WT == W_MXFP4 ? W * 2 * R * WIN : 0;
  static constexpr int LDS = D * BUF + SCALE_LDS;
  // token-row pieces of 1 KB per wave per chunk for NT tiles, spread over the
  // waves (a wave past the last piece re-loads it)
  template <int NT>
  static constexpr int pieces() { return (32 * NT / RPP + W - 1) / W; }
  // NATIVE: scale-word pieces of 256 bytes (64 rows) for NT tiles, likewise
  template <int NT>
  static constexpr int scale_pieces_total() { return NATIVE ? (NT + 1) / 2 : 0; }
  template <int NT>
  static constexpr int scale_pieces() { return (scale_pieces_total<NT>() + W - 1) / W; }
  // vector loads per wave per chunk (besides the weight-scale windows' loads,
  // which only some chunks issue)
  template <int NT>
  static constexpr int loads() { return pieces<NT>() + R * LPT + scale_pieces<NT>(); }
  // position of piece p of token row r inside the row: the rows one 128-bit LDS read
  // touches land in distinct bank groups whether it is served 8 or 16 lanes at a time
  static __device__ __forceinline__ int swz(int r) {
    return NATIVE ? ((r >> 1) ^ (r >> 3)) & 3 : (r + (r >> 3)) & 7;
  }
};

// Grouped GEMM for prefill batches.  MXFP4: two waves per SIMD, so one wave's
// conversions and address work overlap the other's MFMAs; bf16 weights need 4 code
// loads per tile and chunk, whose ring fits only at one wave per SIMD.
template <int WT>
using PrefillConf = GConf<WT, WT == W_MXFP4 ? 8 : 4, 2, 4, 4>;
// Native FP4 x FP8: no conversions, so one wave per SIMD, and 256 tokens per pass
// (the accumulators of 2 x 8 tiles fill the AGPRs): an expert with up to 256
// tokens streams its weights once.
using NativeConf = GConf<W_MXFP4, 4, 2, 5, 8, true>;

// One ring slot of weight registers: the wave's R row tiles for one chunk
// (MXFP4: sw[t] the E8M0 scale of the lane's 32-column block, read from LDS).
template <typename CF>
struct GA {
  u32x4 code[CF::R][CF::LPT];
  uint32_t sw[CF::R];
};

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
// 4 bytes per lane, global memory -> LDS at buf + 4 * lane.
__device__ __forceinline__ void g_dma4(__amdgpu_buffer_rsrc_t src, int voff, int soff, uint8_t* buf) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_ptr_t)buf, 4, voff, soff, 0, 0);
}

// Per-lane offsets of the wave's weight fragments inside a tiled matrix (the
// uniform part, tile and column step, goes into the scalar offset).
struct GLane {
  int code_voff;   // lane's fragment inside the (tile, step) pair it reads
  int scale_off;   // MXFP4: lane's scale bytes inside its tile's LDS window
};

template <typename CF>
__device__ __forceinline__ void g_issue_weights(GA<CF>& a, const Mat& w, const GLane& ln, const int (&st0)[CF::R],
                                                int c) {
  constexpr int R = CF::R, WT = CF::WT;
#pragma unroll
  for (int t = 0; t < R; ++t) {
    if constexpr (WT == W_MXFP4) {
      // 128-column step c / 2, its half c % 2
      a.code[t][0] = bld16(w.codes, ln.code_voff, (st0[t] * w.nK + (c >> 1)) * 1024 + (c & 1) * 512);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)  // k-step j of the chunk: 32-column step 2c + j / 2, half j % 2
        a.code[t][j] = bld16(w.codes, ln.code_voff, (st0[t] * w.nK + 2 * c + (j >> 1)) * 1024 + (j & 1) * 512);
    }
  }
}

// acc[t][nt] += A_t . B_nt over one chunk (4 k-steps of 16): A from registers, B
// from the LDS ring slot `buf`.  The LDS reads and the conversions of k-step m+1
// are issued before the MFMAs of step m (two operand sets), and the steps are
// fenced, so that the reads have R * NT MFMAs to land behind and only two steps'
// operands are live at a time.
template <typename CF, int NT>
__device__ __forceinline__ void g_compute(const GA<CF>& a, const uint8_t* buf, int c, const int (&brow)[NT],
                                          const int (&bswz)[NT], f32x16 (&acc)[CF::R][NT]) {
  constexpr int R = CF::R, WT = CF::WT;
  const int h = (threadIdx.x & 63) >> 5;
  float sc[R];
  if constexpr (WT == W_MXFP4) {
#pragma unroll
    for (int t = 0; t < R; ++t) sc[t] = e8m0_to_f32(a.sw[t]);
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

typedef int i32x8 __attribute__((ext_vector_type(8)));

// NATIVE: acc[t][nt] += A_t . B_nt over one 64-column chunk with one scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, A E2M1, B E4M3).  Operand layout of that
// instruction (established by in-bounds probes of single products and of the
// scales): an E2M1 lane of half h holds columns 32 h .. 32 h + 31 in nibble order
// (its 16 bytes of codes as loaded); an E4M3 lane of half h holds columns
// 16 h .. 16 h + 15 in bytes 0-15 and 32 + 16 h .. 32 + 16 h + 15 in bytes 16-31
// (pieces h and h + 2 of its token row); the scale operand of half h (low byte,
// E8M0) multiplies the products of columns 32 h .. 32 h + 31 on either side.  The
// token scales come from the slot's scale words (one per pass row, after the rows).
template <typename CF>
__device__ __forceinline__ void g_read_native(const uint8_t* buf, int nt, int brow, int bswz, i32x8& B, uint32_t& bsw) {
  const int rho = threadIdx.x & 31, h = (threadIdx.x & 63) >> 5;
  bsw = *reinterpret_cast<const uint32_t*>(buf + CF::ROWS_BYTES + 4 * (32 * nt + rho));
  const u32x4 lo = *reinterpret_cast<const u32x4*>(buf + brow + ((h ^ bswz) << 4));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(buf + brow + (((h + 2) ^ bswz) << 4));
  B = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// The MFMAs of chunk c (weights a, token operands B / bsw already in registers);
// once token tile nt+1's MFMAs are issued, tile nt's registers are refilled with
// chunk c+1's operands from the LDS slot `next`, so the LDS reads run under the
// MFMAs instead of ahead of them.  The refill waits one tile: an LDS read into the
// B registers of the two MFMAs just issued gave wrong sums on the MI355X (the
// instruction can still be reading its B operand then); two MFMAs later, the
// issue of the second one means the first pair has finished.  The fences keep the
// compiler from moving the reads down to their uses in the next step (which would
// put one LDS latency in front of every MFMA pair).
template <typename CF, int NT>
__device__ __forceinline__ void g_mma_native(const GA<CF>& a, int c, const uint8_t* next, const int (&brow)[NT],
                                             const int (&bswz)[NT], i32x8 (&B)[NT], uint32_t (&bsw)[NT],
                                             f32x16 (&acc)[CF::R][NT]) {
  constexpr int R = CF::R;
  const int h = (threadIdx.x & 63) >> 5;
  const int shb = 8 * (2 * (c & 1) + h);
  i32x8 A[R];
  int sa[R];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const u32x4 q = a.code[t][0];
    A[t] = i32x8{(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
    sa[t] = (int)a.sw[t];
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int t = 0; t < R; ++t)
      acc[t][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[t], B[nt], acc[t][nt], 4, 0, 0, sa[t], 0,
                                                                   (int)(bsw[nt] >> shb));
    if (nt > 0) g_read_native<CF>(next, nt - 1, brow[nt - 1], bswz[nt - 1], B[nt - 1], bsw[nt - 1]);
    __builtin_amdgcn_sched_barrier(0);
  }
  g_read_native<CF>(next, NT - 1, brow[NT - 1], bswz[NT - 1], B[NT - 1], bsw[NT - 1]);
}

// One pass of up to 32 NT tokens over the wave's R row tiles, the whole K loop.
// row_start(i): byte offset of pass row i's first element in the B source (rows
// past the expert's tokens repeat its last token: loaded, never stored).
// tile_of(t): the wave's t-th 32-row tile (clamped to the matrix);
// epi(t, nt, acc) stores one 32 x 32 result tile.
// NATIVE: src holds E4M3 codes (one byte per element) and bscale the E8M0 scale
// rows of the same tokens, scale_off(i) the byte offset of pass row i's scales
// (rows past the expert's tokens clamped like row_start's).
template <typename CF, int NT, typename RowStart, typename ScaleOff, typename TileOf, typename Epi>
__device__ __forceinline__ void g_pass(const Mat& w, const TileOf& tile_of, __amdgpu_buffer_rsrc_t src,
                                       const RowStart& row_start, __amdgpu_buffer_rsrc_t bscale,
                                       const ScaleOff& scale_off, uint8_t* lds, const Epi& epi) {
  constexpr int R = CF::R, WT = CF::WT, D = CF::D;
  constexpr int NL = CF::template loads<NT>();
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  const int rho = lane & 31, h = lane >> 5;
  GLane ln;
  ln.code_voff = (rho >> 4) * w.nK * 1024 + (rho & 15) * 16 + h * 256;
  ln.scale_off = (rho >> 4) * 1024 + h * 256 + (rho & 15) * 16;
  int st0[R];
#pragma unroll
  for (int t = 0; t < R; ++t) st0[t] = 2 * tile_of(t);
  // token-row pieces: this wave fills 1 KB pieces d = wv + W i (rows RPP d ..
  // RPP d + RPP - 1); lane l writes position l % PPR of row RPP d + l / PPR, i.e.
  // source piece pos ^ swz(row)
  constexpr int PW = CF::template pieces<NT>();
  constexpr int W = CF::W, PPR = CF::ROWB / 16;
  int dvoff[PW], dpiece[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    dpiece[i] = min(wv + W * i, 32 * NT / CF::RPP - 1);
    const int row = CF::RPP * dpiece[i] + lane / PPR;
    dvoff[i] = row_start(row) + (((lane % PPR) ^ CF::swz(row)) << 4);
  }
  // NATIVE: scale-word pieces d = wv + W i (rows 64 d .. 64 d + 63, lane l row
  // 64 d + l); 64 ceil(NT / 2) <= PASS rows, so they stay inside the slot
  constexpr int SPW = CF::template scale_pieces<NT>() > 0 ? CF::template scale_pieces<NT>() : 1;
  int svoff[SPW], spiece[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    spiece[i] = min(wv + W * i, CF::template scale_pieces_total<NT>() - 1);
    svoff[i] = CF::NATIVE ? scale_off(64 * spiece[i] + lane) : 0;
  }
  // this lane's B rows: token tile nt, column lane % 32
  int brow[NT], bswz[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = 32 * nt + rho;
    brow[nt] = r * CF::ROWB;
    bswz[nt] = CF::swz(r);
  }
  const int nch = w.K / kGKC;
  GA<CF> a[D];
  f32x16 acc[R][NT];
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][nt][v] = 0.0f;
  // MXFP4 weight scales: window v (chunks 32 v .. 32 v + 31) of the wave's row
  // tiles goes to LDS set v % 2 with one 1 KB load per 16-row tile.  Window v + 1
  // is loaded at the top of the first loop round that starts at chunk 32 v + 8 or
  // later (before that round's loads, at most D - 1 chunks later), so it replaces
  // window v - 1 after that window's last read (chunk 32 v - 1, read during step
  // 32 v - 2) and has landed with the round's first chunk, long before its own
  // first read (step 32 v + 31).  Only this wave reads its windows, so its own
  // vmcnt waits order them.  The loads sit outside the unrolled steps: a branch
  // inside them costs the native kernel a great many spills.
  uint8_t* const wsc = lds + D * CF::BUF + wv * 2 * R * CF::WIN;
  auto issue_scales = [&](int v) {
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        g_dma16(w.scales, 16 * lane, ((st0[t] + q) * w.nKs + v) * 1024, wsc + ((v & 1) * R + t) * CF::WIN + q * 1024);
  };
  // the scale bytes of chunk c into ring slot g (step c / 2 within its window)
  auto read_scales = [&](GA<CF>& g, int c) {
    if constexpr (WT == W_MXFP4) {
      const uint8_t* p = wsc + ((c >> 5) & 1) * R * CF::WIN + (c & 1) * 512 + ((c >> 1) & 15) + ln.scale_off;
#pragma unroll
      for (int t = 0; t < R; ++t) g.sw[t] = p[t * CF::WIN];
    }
  };
  int next_win = 1;
  auto round_scales = [&](int c0) {
    if constexpr (WT == W_MXFP4) {
      if (next_win < w.nKs && c0 + 24 >= 32 * next_win) {
        issue_scales(next_win);
        ++next_win;
      }
    }
  };
  // chunk c's loads into ring slot `slot` (past the end the last chunk is re-loaded)
  auto issue = [&](int slot, int c) {
#pragma unroll
    for (int i = 0; i < PW; ++i)
      g_dma16(src, dvoff[i], c * CF::ROWB, lds + slot * CF::BUF + dpiece[i] * 1024);
    g_issue_weights<CF>(a[slot], w, ln, st0, c);
    if constexpr (CF::NATIVE) {
      // the scale word of blocks 2 (c & ~1) .. + 3 of each pass row (both chunks of
      // a pair; the odd chunk re-loads it so that every chunk issues NL loads)
#pragma unroll
      for (int i = 0; i < CF::template scale_pieces<NT>(); ++i)
        g_dma4(bscale, svoff[i], 2 * (c & ~1), lds + slot * CF::BUF + CF::ROWS_BYTES + spiece[i] * 256);
    }
  };
  // The prologue's chunks are kept apart (and in order) like the loop's, so that
  // the waits below count the same loads.  Window 0 goes first: it has landed once
  // chunk 0 has.  The windows' loads come on top of some chunks' NL, which only
  // makes the waits below (at most so many loads outstanding) wait a little longer.
  if constexpr (WT == W_MXFP4) issue_scales(0);
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    issue(d, min(d, nch - 1));
    asm volatile("" ::: "memory");
  }
  // Step c (slot d = c % D) issues the loads of chunk c + D - 1 into the slot of
  // chunk c - 1 (read during step c - 2, before the barrier that ended step c - 1).
  int c0 = 0;
  if constexpr (CF::NATIVE) {
    // chunk c+1's token operands are read while chunk c's MFMAs run, so step c
    // ends with chunk c+2 in LDS: D - 3 chunks may stay in flight
    static_assert(D >= 4, "ring of at least 4 chunks");
    g_wait_barrier<(D - 3) * NL>();
    i32x8 B[NT];
    uint32_t bsw[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) g_read_native<CF>(lds, nt, brow[nt], bswz[nt], B[nt], bsw[nt]);
    read_scales(a[0], 0);
    // step c also reads chunk c+1's weight scales (its window landed long before)
    auto step = [&](int d, int c) {
      issue((d + D - 1) % D, min(c + D - 1, nch - 1));
      read_scales(a[(d + 1) % D], min(c + 1, nch - 1));
      __builtin_amdgcn_sched_barrier(0);
      g_mma_native<CF, NT>(a[d], c, lds + ((d + 1) % D) * CF::BUF, brow, bswz, B, bsw, acc);
      g_wait_barrier<(D - 3) * NL>();
    };
    for (; c0 + D <= nch; c0 += D) {
      round_scales(c0);
#pragma unroll
      for (int d = 0; d < D; ++d) step(d, c0 + d);
    }
    // the chunks left when K / 64 is not a multiple of D
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
      if (c0 + d < nch) step(d, c0 + d);
  } else {
    // step c ends with chunk c+1 in LDS: D - 2 chunks may stay in flight
    g_wait_barrier<(D - 2) * NL>();
    read_scales(a[0], 0);
    auto step = [&](int d, int c) {
      issue((d + D - 1) % D, min(c + D - 1, nch - 1));
      read_scales(a[(d + 1) % D], min(c + 1, nch - 1));
      g_compute<CF, NT>(a[d], lds + d * CF::BUF, c, brow, bswz, acc);
      g_wait_barrier<(D - 2) * NL>();
    };
    for (; c0 + D <= nch; c0 += D) {
      round_scales(c0);
#pragma unroll
      for (int d = 0; d < D; ++d) step(d, c0 + d);
    }
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
      if (c0 + d < nch) step(d, c0 + d);
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

template <typename CF, typename RowStart, typename ScaleOff, typename TileOf, typename Epi>
__device__ __forceinline__ void g_dispatch(int nt, const Mat& w, const TileOf& tile_of, __amdgpu_buffer_rsrc_t src,
                                           const RowStart& row_start, __amdgpu_buffer_rsrc_t bscale,
                                           const ScaleOff& scale_off, uint8_t* lds, const Epi& epi) {
#define MOE_G_PASS(N) g_pass<CF, N>(w, tile_of, src, row_start, bscale, scale_off, lds, epi)
  if constexpr (CF::MAXNT == 8) {
    switch (nt) {
      case 1: MOE_G_PASS(1); break;
      case 2: MOE_G_PASS(2); break;
      case 3: MOE_G_PASS(3); break;
      case 4: MOE_G_PASS(4); break;
      case 5: MOE_G_PASS(5); break;
      case 6: MOE_G_PASS(6); break;
      case 7: MOE_G_PASS(7); break;
      default: MOE_G_PASS(8); break;
    }
  } else {
    static_assert(CF::MAXNT == 4, "passes of 4 or 8 token tiles");
    switch (nt) {
      case 1: MOE_G_PASS(1); break;
      case 2: MOE_G_PASS(2); break;
      case 3: MOE_G_PASS(3); break;
      default: MOE_G_PASS(4); break;
    }
  }
#undef MOE_G_PASS
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
  int longest;                         // items longest first, round robin over the XCDs (no shared expert)
};

__device__ __forceinline__ Item g_item(const FfnArgs& a, const GGrid& gr) {
  return gr.longest ? resolve_item_longest(a, gr.routed_blocks)
                    : resolve_item_at(a, xcd_logical_block(), gr.shared_blocks, gr.routed_blocks);
}

template <typename CF>
__global__ __launch_bounds__(CF::W * 64) __attribute__((amdgpu_waves_per_eu(CF::W / 4, CF::W / 4))) void grouped_gate_up(
    FfnArgs a, GGrid gr) {
  const Item it = g_item(a, gr);
  if (!it.valid) return;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[CF::LDS];
  constexpr int R = CF::R, WT = CF::WT;
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  const int j = lane & 31, h = lane >> 5;
  const int H = a.H, Ie = it.I;
  const int ntiles = Ie / 16;  // 32-row tiles of W13 (2 Ie rows)
  const int tile0 = it.tile * gr.tiles_per_block + wv * R;
  auto tile_of = [&](int t) { return min(tile0 + t, ntiles - 1); };
  const Mat w = w13_mat<WT>(it.w, H, Ie);
  // token rows: bf16 x, or (NATIVE) its E4M3 codes with their E8M0 scale rows
  constexpr int xb = CF::NATIVE ? 1 : 2;
  const __amdgpu_buffer_rsrc_t src = make_rsrc(CF::NATIVE ? (const void*)a.xq : a.x, (size_t)a.T * H * xb);
  const __amdgpu_buffer_rsrc_t bscale = make_rsrc(CF::NATIVE ? (const void*)a.xs : a.x, (size_t)a.T * (H / 32));
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(a.h);
  for (int pass = 0; pass < it.n; pass += CF::PASS) {
    const int nt = min(CF::MAXNT, (it.n - pass + 31) / 32);
    auto row_start = [&](int row) { return item_token(a, it, min(pass + row, it.n - 1)) * H * xb; };
    auto scale_off = [&](int row) { return item_token(a, it, min(pass + row, it.n - 1)) * (H / 32); };
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
    g_dispatch<CF>(nt, w, tile_of, src, row_start, bscale, scale_off, lds, epi);
  }
}

template <typename CF>
__global__ __launch_bounds__(CF::W * 64) __attribute__((amdgpu_waves_per_eu(CF::W / 4, CF::W / 4))) void grouped_down(
    FfnArgs a, GGrid gr) {
  const Item it = g_item(a, gr);
  if (!it.valid) return;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[CF::LDS];
  constexpr int R = CF::R, WT = CF::WT;
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  const int j = lane & 31, h = lane >> 5;
  const int H = a.H, Ie = it.I;
  const int ntiles = H / 32;  // 32-row tiles of W2 (H rows)
  const int tile0 = it.tile * gr.tiles_per_block + wv * R;
  auto tile_of = [&](int t) { return min(tile0 + t, ntiles - 1); };
  const Mat w = w2_mat<WT>(it.w, H, Ie);
  const __amdgpu_buffer_rsrc_t src =
      make_rsrc(a.h, ((size_t)a.T * a.k + (a.shared_w ? a.T : 0)) * a.h_ld * 2);
  for (int pass = 0; pass < it.n; pass += CF::PASS) {
    const int nt = min(CF::MAXNT, (it.n - pass + 31) / 32);
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
    g_dispatch<CF>(nt, w, tile_of, src, row_start, src, [](int) { return 0; }, lds, epi);
  }
}

// ---------------------------------------------------------------------------
bool prefill_supported(int wtype, int H, int I, int I_shared) {
  if (wtype != W_BF16 && wtype != W_MXFP4) return false;
  return H % 128 == 0 && I % 128 == 0 && I_shared % 128 == 0;
}

static unsigned pad8(unsigned g) { return (g + 7) / 8 * 8; }

// Blocks of a launch: longest-first order, ceil(items / 8) items per XCD; else the
// shared expert's blocks and every item's, padded to a multiple of 8.
static unsigned g_blocks(const GGrid& gr, int routed_items) {
  if (gr.longest) return 8u * (unsigned)((routed_items + 7) / 8) * (unsigned)gr.routed_blocks;
  return pad8(gr.shared_blocks + routed_items * gr.routed_blocks);
}

template <typename CF>
static GGrid g_grid(int routed_tiles, int shared_tiles) {
  GGrid g;
  g.longest = shared_tiles == 0;
  g.tiles_per_block = CF::W * CF::R;
  g.routed_tiles = routed_tiles;
  g.shared_tiles = shared_tiles;
  g.routed_blocks = (routed_tiles + g.tiles_per_block - 1) / g.tiles_per_block;
  g.shared_blocks = (shared_tiles + g.tiles_per_block - 1) / g.tiles_per_block;
  return g;
}

template <typename CF>
static hipError_t launch_gu(const FfnArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const GGrid gr = g_grid<CF>(a.I / 16, a.shared_w ? a.I_shared / 16 : 0);
  const unsigned grid = g_blocks(gr, a.routed_items);
  hipLaunchKernelGGL(grouped_gate_up<CF>, dim3(grid), dim3(CF::W * 64), 0, st, a, gr);
  return hipGetLastError();
}

template <typename CF>
static hipError_t launch_dn(const FfnArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int tiles = a.H / 32;
  const GGrid gr = g_grid<CF>(tiles, a.shared_w ? tiles : 0);
  const unsigned grid = g_blocks(gr, a.routed_items);
  hipLaunchKernelGGL(grouped_down<CF>, dim3(grid), dim3(CF::W * 64), 0, st, a, gr);
  return hipGetLastError();
}

hipError_t launch_prefill_gate_up(int wtype, const FfnArgs& a, hipStream_t st) {
  return wtype == W_BF16 ? launch_gu<PrefillConf<W_BF16>>(a, st) : launch_gu<PrefillConf<W_MXFP4>>(a, st);
}

// ---------------------------------------------------------------------------
// MXFP8 activations for the native FP4 path (OCP Microscaling Formats v1.0): per
// block of 32 consecutive elements of a token row, X = floor(log2(max |x|)) - 8
// (8 = the largest E4M3 exponent; X = -127 for an all-zero block), scale byte
// X + 127, and each element x / 2^X rounded to the nearest E4M3 value, ties to
// even, clamped to +-448.  Scaling by 2^-X is exact, so the codes depend on x alone.

// E4M3 code of v (finite): below 2^-6 the subnormal steps of 2^-9, else three
// mantissa bits at v's own exponent; S.1111.111 is NaN, so 448 is the largest.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.0f);  // 0 .. 8 (8 is 2^-6, the smallest normal)
  } else {
    int e = ilogbf(a);
    float m = rintf(ldexpf(a, 3 - e));  // 8 .. 16
    if (m == 16.0f) {
      e += 1;
      m = 8.0f;
    }
    code = (e > 8 || (e == 8 && m > 14.0f)) ? 0x7Eu : ((uint32_t)(e + 7) << 3) | ((uint32_t)m - 8u);
  }
  return sign | code;
}

// One thread per 32-element block: 64 bytes in, 32 code bytes and 1 scale out.
__global__ __launch_bounds__(256) void mx8_quantize_kernel(const uint16_t* __restrict__ x, int nblocks,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)b * 32);
  u32x4 v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = src[q];
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax = fmaxf(amax, fabsf(__uint_as_float(v[q][i] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(v[q][i] & 0xffff0000u)));
    }
  const int X = amax == 0.0f ? -127 : max(-127, ilogbf(amax) - 8);
  const float inv = ldexpf(1.0f, -X);
  u32x4 out[2];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // elements 8q + 2i (low half) and 8q + 2i + 1 (high half) -> bytes of word 2q + i / 2
      const uint32_t c0 = e4m3_code(__uint_as_float(v[q][i] << 16) * inv);
      const uint32_t c1 = e4m3_code(__uint_as_float(v[q][i] & 0xffff0000u) * inv);
      const uint32_t pair = c0 | (c1 << 8);
      const int word = 2 * q + i / 2;
      if (i % 2 == 0)
        out[word / 4][word % 4] = pair;
      else
        out[word / 4][word % 4] |= pair << 16;
    }
  u32x4* dst = reinterpret_cast<u32x4*>(codes + (size_t)b * 32);
  dst[0] = out[0];
  dst[1] = out[1];
  scales[b] = (uint8_t)(X + 127);
}

hipError_t launch_mx8_quantize(const uint16_t* x, int T, int H, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int nblocks = (int)((int64_t)T * H / 32);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx8_quantize_kernel, dim3((nblocks + 255) / 256), dim3(256), 0, st, x, nblocks, codes, scales);
  return hipGetLastError();
}

hipError_t launch_native_gate_up(const FfnArgs& a, hipStream_t st) { return launch_gu<NativeConf>(a, st); }

hipError_t launch_prefill_down(int wtype, const FfnArgs& a, hipStream_t st) {
  return wtype == W_BF16 ? launch_dn<PrefillConf<W_BF16>>(a, st) : launch_dn<PrefillConf<W_MXFP4>>(a, st);
}

}  // namespace moe
