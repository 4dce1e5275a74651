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
// Block = WAVES waves over 16*R*WAVES weight rows of one expert and up to 128 of
// its tokens per pass.  The K dimension is walked in chunks of 128 columns.
//  * Weights (MFMA A operand) stream from HBM in the tiled layout straight into
//    registers, each wave its own rows.
//  * The expert's token rows (B operand) go from global memory straight into LDS
//    (buffer loads with the LDS destination, no registers on the way) and are
//    shared by all waves.  A row of a chunk is 256 bytes = 16 pieces of 16 bytes;
//    piece c of token row r is stored at position c ^ (r % 16), so the 16 rows that
//    one 128-bit LDS read touches hit 16 different bank groups.
//  * Four LDS buffers and four register sets: the loads of chunk ch+3 are issued
//    before chunk ch is computed.  Every load in the loop is unconditional (past the
//    last chunk they re-read it), so each wave issues exactly NL loads per chunk and
//    "everything issued two chunks back has landed" is the wait vmcnt(2*NL); the
//    barrier that follows makes the LDS rows visible to the other waves.
// Blocks are ordered so that all row blocks of an expert run on the same XCD in
// sequence (blockIdx b executes on XCD b % 8), keeping the expert's token rows in
// that XCD's L2.
#include "ffn_common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace moe {

constexpr int kPfKC = 128;                          // columns per chunk
constexpr int kPfRows = 128;                        // token rows per pass
constexpr int kPfRowBytes = kPfKC * 2;              // one token row of a chunk in LDS
constexpr int kPfBufBytes = kPfRows * kPfRowBytes;  // 32 KB per LDS buffer
constexpr int kPfDepth = 4;                         // buffers / register sets

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 1 KB pieces (4 token rows of a chunk) each wave writes per chunk: 4*NTL pieces
// spread over the WAVES waves.
template <int NTL, int WAVES>
struct PfPieces {
  static constexpr int value = (4 * NTL + WAVES - 1) / WAVES;
};

template <int WT, int R, int U>
struct AChunk {
  u32x4 qa[U][R];
  uint32_t qs[U][R];
};

// A fragments of the U column steps of chunk `s` (in steps) for the R row tiles.
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
        c.qs[u][t] = load_scale_word(w, lane, atile[t], s + u);
      else
        c.qs[u][t] = 0u;
    }
  }
}

// One 16-byte piece per lane of token rows, global memory -> LDS at
// buf + 16 * lane (the instruction writes 1 KB contiguously for the wave).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t src, int voff, int soff, uint8_t* buf) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_ptr_t)buf, 16, voff, soff, 0, 0);
}

// Wait until at most N vector loads of this wave are outstanding and its LDS
// accesses are done, then barrier.  The wait goes through the builtin so that
// the compiler's own wait placement knows the older loads have landed; the empty
// asm statements keep memory accesses from moving across.
template <int N>
__device__ __forceinline__ void vm_lds_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt fields: vmcnt[3:0] and [15:14], expcnt[6:4] (7: no wait), lgkmcnt[11:8].
  constexpr int imm = (N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS byte offset (inside a buffer, token tile 0) of this lane's B fragment for
// k-group q of a chunk: MXFP4 groups are 8-column slices of the lane's 32-column
// run (piece 4g + q), bf16 groups are the chunk's 32-column steps (piece 4q + g).
template <int WT>
__device__ __forceinline__ int b_frag_offset(int q) {
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  const int piece = WT == W_MXFP4 ? 4 * g + q : 4 * q + g;
  return col * kPfRowBytes + ((piece ^ col) << 4);
}

// acc[t][nt] += A_t . B_nt over one chunk: A from registers, B from LDS.  NTL
// (the token tiles of this pass) is a compile-time count, so the unrolled body
// has no branches.  The LDS reads of k-group q+1 are issued in program order
// before the MFMAs of group q, so LDS latency can hide behind R*NTL MFMAs; the
// compiler is left free to interleave the conversions, reads and MFMAs (fencing
// each group with scheduling barriers measured 5-9% slower); consecutive MFMAs
// update different accumulators.
template <int WT, int NTL, int R, int U>
__device__ __forceinline__ void compute_chunk_lds(const AChunk<WT, R, U>& c, const uint8_t* buf,
                                                  const int (&boff)[4], int step4, f32x4 (&acc)[R][NTL]) {
  constexpr int NA = WT == W_MXFP4 ? 4 : 1;
  constexpr int NG = U * NA;  // k-groups of 32 columns in the chunk
  static_assert(NG == 4, "a chunk is four k-groups");
  auto ldb = [&](int q, int nt) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(buf + boff[q] + nt * 16 * kPfRowBytes));
  };
  bf16x8 B[2][NTL];
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt) B[0][nt] = ldb(0, nt);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    bf16x8 A[R][NA];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      if constexpr (WT == W_BF16) {
        A[t][0] = as_bf16x8(c.qa[u][t]);
      } else {
        const float sc = scale_of_word(c.qs[u][t], step4 + u);
#pragma unroll
        for (int m = 0; m < 4; ++m) A[t][m] = fp4x8_to_bf16x8(c.qa[u][t][m], sc);
      }
    }
#pragma unroll
    for (int m = 0; m < NA; ++m) {
      const int q = u * NA + m;
      if (q + 1 < NG) {
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) B[(q + 1) % 2][nt] = ldb(q + 1, nt);
      }
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
        for (int t = 0; t < R; ++t)
          acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t][m], B[q % 2][nt], acc[t][nt], 0, 0, 0);
    }
  }
}

// The four LDS buffers of a block.
struct PfBufs {
  uint8_t* b[kPfDepth];
};

// K loops of one pass over up to 16*NTL tokens for the block's nu row tiles
// ("units") in sequence, on one flat chunk index f = unit * nchunks + ch.  Step f:
// the loads of chunk f+3 go to buffer / register set (f+3) % 4 (so the next
// unit's first chunks are requested while the current one finishes), chunk f is
// computed from set f % 4, then everything issued up to step f-2 (which includes
// the token rows of chunk f+1) is waited for and the block synchronises.  After a
// unit's last chunk its accumulators go to the epilogue.  atile_of(u, t) is row
// tile t of unit u for this wave; epi(u, t, nt, acc) stores a result tile.
template <int WT, int NTL, int R, int WAVES, typename ATileOf, typename Epi>
__device__ __forceinline__ void prefill_units(const Mat& w, int nu, const ATileOf& atile_of,
                                              __amdgpu_buffer_rsrc_t src, const int (&voff)[PfPieces<NTL, WAVES>::value],
                                              const PfBufs& bufs, const Epi& epi) {
  constexpr int U = kPfKC / KStep<WT>::value;
  constexpr int PW = PfPieces<NTL, WAVES>::value;            // B pieces per wave
  constexpr int NL = PW + R * U * (WT == W_MXFP4 ? 2 : 1);  // vector loads per chunk
  const int wv = uniform(threadIdx.x >> 6);
  const int nchunks = w.K / kPfKC, lastf = nu * nchunks - 1;
  AChunk<WT, R, U> a[kPfDepth];
  f32x4 acc[R][NTL];
  // Token rows of a chunk: wave wv writes the 1 KB pieces P = WAVES*i + wv (token rows
  // 4P..4P+3), i < PW; lane l fills position l % 16 of row 4P + l / 16.  voff[i]
  // holds the lane's row start plus its swizzled piece offset.  The weights come
  // from the unit's row tiles.
  auto issue = [&](int set, int f) {
    const int u = f / nchunks, ch = f - u * nchunks;
#pragma unroll
    for (int i = 0; i < PW; ++i) dma16(src, voff[i], ch * kPfRowBytes, bufs.b[set] + (WAVES * i + wv) * 1024);
    int at[R];
#pragma unroll
    for (int t = 0; t < R; ++t) at[t] = atile_of(u, t);
    load_a<WT, R, U>(a[set], w, at, ch * U);
  };
  auto zero = [&]() {
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto finish = [&](int u) {
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) epi(u, t, nt, acc[t][nt]);
  };
  int boff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) boff[q] = b_frag_offset<WT>(q);
  // The prologue's batches are kept apart (and in order) like the loop's chunks,
  // so that "two batches back" counts the same loads.
#pragma unroll
  for (int d = 0; d < kPfDepth - 1; ++d) {
    issue(d, min(d, lastf));
    asm volatile("" ::: "memory");
  }
  vm_lds_barrier<2 * NL>();
  auto step = [&](int d, int f) {
    issue((d + kPfDepth - 1) % kPfDepth, min(f + kPfDepth - 1, lastf));
    compute_chunk_lds<WT, NTL, R, U>(a[d], bufs.b[d], boff, d, acc);  // chunk index = d mod 4
    vm_lds_barrier<2 * NL>();
  };
  if (nchunks % kPfDepth == 0) {
    // Whole groups of four chunks carry no conditions, so every path back to a
    // loop head has issued the same loads (the compiler's own waits stay late),
    // and each unit starts on set 0.
    for (int u = 0; u < nu; ++u) {
      zero();
      for (int ch0 = 0; ch0 < nchunks; ch0 += kPfDepth) {
#pragma unroll
        for (int d = 0; d < kPfDepth; ++d) step(d, u * nchunks + ch0 + d);
      }
      finish(u);
    }
  } else {
    // One unit (the launch asks for no more), whole groups then the rest.
    zero();
    int ch0 = 0;
    for (; ch0 + kPfDepth <= nchunks; ch0 += kPfDepth) {
#pragma unroll
      for (int d = 0; d < kPfDepth; ++d) step(d, ch0 + d);
    }
#pragma unroll
    for (int d = 0; d < kPfDepth - 1; ++d)
      if (ch0 + d < nchunks) step(d, ch0 + d);
    finish(0);
  }
}

// One pass of up to 16*NTL tokens, NTL fixed at compile time.  row_start(i) is the
// byte offset of pass row i's first element in the B source; rows past the
// expert's tokens repeat its last token (loaded, never stored).
template <int WT, int NTL, int R, int WAVES, typename RowStart, typename ATileOf, typename Epi>
__device__ __forceinline__ void prefill_pass(const Mat& w, int nu, const ATileOf& atile_of,
                                             __amdgpu_buffer_rsrc_t src, const RowStart& row_start,
                                             const PfBufs& bufs, const Epi& epi) {
  constexpr int PW = PfPieces<NTL, WAVES>::value;
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  int voff[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int row = 4 * (WAVES * i + wv) + (lane >> 4);
    voff[i] = row_start(row) + (((lane & 15) ^ (row & 15)) << 4);
  }
  prefill_units<WT, NTL, R, WAVES>(w, nu, atile_of, src, voff, bufs, epi);
}

template <int WT, int R, int WAVES, typename RowStart, typename ATileOf, typename Epi>
__device__ __forceinline__ void prefill_dispatch(int ntl, const Mat& w, int nu, const ATileOf& atile_of,
                                                 __amdgpu_buffer_rsrc_t src, const RowStart& row_start,
                                                 const PfBufs& bufs, const Epi& epi) {
  switch (ntl) {
    case 1: prefill_pass<WT, 1, R, WAVES>(w, nu, atile_of, src, row_start, bufs, epi); break;
    case 2: prefill_pass<WT, 2, R, WAVES>(w, nu, atile_of, src, row_start, bufs, epi); break;
    case 3: prefill_pass<WT, 3, R, WAVES>(w, nu, atile_of, src, row_start, bufs, epi); break;
    case 4: prefill_pass<WT, 4, R, WAVES>(w, nu, atile_of, src, row_start, bufs, epi); break;
    case 5: prefill_pass<WT, 5, R, WAVES>(w, nu, atile_of, src, row_start, bufs, epi); break;
    case 6: prefill_pass<WT, 6, R, WAVES>(w, nu, atile_of, src, row_start, bufs, epi); break;
    case 7: prefill_pass<WT, 7, R, WAVES>(w, nu, atile_of, src, row_start, bufs, epi); break;
    default: prefill_pass<WT, 8, R, WAVES>(w, nu, atile_of, src, row_start, bufs, epi); break;
  }
}

__device__ __forceinline__ int xcd_logical_block() {
  const int per = gridDim.x / 8;  // the grid is a multiple of 8
  return (blockIdx.x % 8) * per + blockIdx.x / 8;
}

#define MOE_PF_LDS_BUFFERS                                            \
  __shared__ __attribute__((aligned(1024))) uint8_t sb0[kPfBufBytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t sb1[kPfBufBytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t sb2[kPfBufBytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t sb3[kPfBufBytes]; \
  const PfBufs bufs{{sb0, sb1, sb2, sb3}}

// Work of one block: `upb` consecutive row tiles ("units") of one expert.
// unit_tiles = row tiles of a routed expert, shared_units likewise for the
// shared expert; block counts per item follow from them.
struct PfGrid {
  int upb;
  int shared_units, routed_units;  // row tiles per item
  int shared_blocks, routed_blocks;  // blocks per item
};

template <int WT, int R, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void prefill_gate_up(FfnArgs a, PfGrid gr) {
  const Item it = resolve_item_at(a, xcd_logical_block(), gr.shared_blocks, gr.routed_blocks);
  if (!it.valid) return;
  MOE_PF_LDS_BUFFERS;
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, Ie = it.I;
  const int tile0 = it.tile * gr.upb;
  const int nu = min(gr.upb, (it.shared ? gr.shared_units : gr.routed_units) - tile0);
  // First intermediate index of unit u for this wave; rows past I are loaded
  // (clamped) and never stored.
  auto j0_of = [&](int u) { return ((tile0 + u) * WAVES + wv) * 8 * R; };
  auto atile_of = [&](int u, int t) { return min(j0_of(u) / 8 + t, Ie / 8 - 1); };
  const Mat w = w13_mat<WT>(it.w, H, Ie);
  const __amdgpu_buffer_rsrc_t src = make_rsrc(a.x, (size_t)a.T * H * 2);
  uint16_t* h = reinterpret_cast<uint16_t*>(a.h);
  for (int pass = 0; pass < it.n; pass += kPfRows) {
    const int ntl = min(kPfRows / 16, (it.n - pass + 15) / 16);
    auto row_start = [&](int row) { return item_token(a, it, min(pass + row, it.n - 1)) * H * 2; };
    auto epi = [&](int u, int t, int nt, const f32x4& v) {
      const int jt = j0_of(u) + 8 * t;
      f32x4 uu;
#pragma unroll
      for (int q = 0; q < 4; ++q) uu[q] = __shfl_xor(v[q], 32, 64);
      const int i = pass + nt * 16 + r;
      if (jt < Ie && g < 2 && i < it.n) {
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16_rne(silu_f32(v[0]) * uu[0]) |
                   ((uint32_t)f32_to_bf16_rne(silu_f32(v[1]) * uu[1]) << 16);
        packed.y = (uint32_t)f32_to_bf16_rne(silu_f32(v[2]) * uu[2]) |
                   ((uint32_t)f32_to_bf16_rne(silu_f32(v[3]) * uu[3]) << 16);
        *reinterpret_cast<uint2*>(h + (size_t)(it.hrow0 + i) * a.h_ld + jt + g * 4) = packed;
      }
    };
    prefill_dispatch<WT, R, WAVES>(ntl, w, nu, atile_of, src, row_start, bufs, epi);
  }
}

template <int WT, int R, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void prefill_down(FfnArgs a, PfGrid gr) {
  const Item it = resolve_item_at(a, xcd_logical_block(), gr.shared_blocks, gr.routed_blocks);
  if (!it.valid) return;
  MOE_PF_LDS_BUFFERS;
  const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int H = a.H, Ie = it.I;
  const int tile0 = it.tile * gr.upb;
  const int nu = min(gr.upb, (it.shared ? gr.shared_units : gr.routed_units) - tile0);
  // First output column of unit u for this wave; rows past H are loaded
  // (clamped) and never stored.
  auto row0_of = [&](int u) { return ((tile0 + u) * WAVES + wv) * 16 * R; };
  auto atile_of = [&](int u, int t) { return min(row0_of(u) / 16 + t, H / 16 - 1); };
  const Mat w = w2_mat<WT>(it.w, H, Ie);
  const __amdgpu_buffer_rsrc_t src =
      make_rsrc(a.h, ((size_t)a.T * a.k + (a.shared_w ? a.T : 0)) * a.h_ld * 2);
  for (int pass = 0; pass < it.n; pass += kPfRows) {
    const int ntl = min(kPfRows / 16, (it.n - pass + 15) / 16);
    auto row_start = [&](int row) { return (it.hrow0 + min(pass + row, it.n - 1)) * a.h_ld * 2; };
    auto epi = [&](int u, int t, int nt, const f32x4& v) {
      const int c0 = row0_of(u) + 16 * t;
      const int i = pass + nt * 16 + r;
      if (c0 < H && i < it.n) {
        float* dst = it.shared ? a.shared_out + (size_t)i * H : a.out_rows + (size_t)(it.p0 + i) * H;
        *reinterpret_cast<float4*>(dst + c0 + g * 4) = make_float4(v[0], v[1], v[2], v[3]);
      }
    };
    prefill_dispatch<WT, R, WAVES>(ntl, w, nu, atile_of, src, row_start, bufs, epi);
  }
}

// ---------------------------------------------------------------------------
// Launch: 8 waves and 128 KB of LDS; R row tiles per wave: 2 for MXFP4 (four
// register sets of 2 x 80 bytes per lane), 1 for bf16 (a bf16 chunk is four column
// steps, so one row tile already holds 4 x 16 bytes per set).
#ifndef MOE_PF_WAVES
#define MOE_PF_WAVES 8
#endif
#ifndef MOE_PF_R_MX
#define MOE_PF_R_MX 2
#endif
constexpr int kPfWaves = MOE_PF_WAVES;
template <int WT>
constexpr int pf_r() { return WT == W_MXFP4 ? MOE_PF_R_MX : 1; }

bool prefill_supported(int wtype, int H, int I, int I_shared) {
  if (wtype != W_BF16 && wtype != W_MXFP4) return false;
  return H % kPfKC == 0 && I % kPfKC == 0 && I_shared % kPfKC == 0;
}

static unsigned pad8(unsigned g) { return (g + 7) / 8 * 8; }

// Row tiles per block when the K loop is whole groups of four chunks.
#ifndef MOE_PF_UPB
#define MOE_PF_UPB 4
#endif
constexpr int kPfUpb = MOE_PF_UPB;

static PfGrid pf_grid(int routed_units, int shared_units, bool multi) {
  PfGrid g;
  g.upb = multi ? kPfUpb : 1;
  g.routed_units = routed_units;
  g.shared_units = shared_units;
  g.routed_blocks = (routed_units + g.upb - 1) / g.upb;
  g.shared_blocks = (shared_units + g.upb - 1) / g.upb;
  return g;
}

static bool whole_groups(int K) { return (K / kPfKC) % kPfDepth == 0; }

hipError_t launch_prefill_gate_up(int wtype, const FfnArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const bool sh = a.shared_w != nullptr;
  auto launch = [&](auto wt) {
    constexpr int WT = decltype(wt)::value, R = pf_r<WT>();
    constexpr int rb = 8 * R * kPfWaves;  // intermediate indices per row tile
    const PfGrid gr = pf_grid((a.I + rb - 1) / rb, sh ? (a.I_shared + rb - 1) / rb : 0, whole_groups(a.H));
    const unsigned grid = pad8(gr.shared_blocks + a.routed_items * gr.routed_blocks);
    hipLaunchKernelGGL((prefill_gate_up<WT, R, kPfWaves>), dim3(grid), dim3(kPfWaves * 64), 0, st, a, gr);
  };
  if (wtype == W_BF16)
    launch(std::integral_constant<int, W_BF16>{});
  else
    launch(std::integral_constant<int, W_MXFP4>{});
  return hipGetLastError();
}

hipError_t launch_prefill_down(int wtype, const FfnArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const bool sh = a.shared_w != nullptr;
  auto launch = [&](auto wt) {
    constexpr int WT = decltype(wt)::value, R = pf_r<WT>();
    constexpr int rb = 16 * R * kPfWaves;  // output columns per row tile
    const int tiles = (a.H + rb - 1) / rb;
    const PfGrid gr = pf_grid(tiles, sh ? tiles : 0, whole_groups(a.I) && (!sh || whole_groups(a.I_shared)));
    const unsigned grid = pad8(gr.shared_blocks + a.routed_items * gr.routed_blocks);
    hipLaunchKernelGGL((prefill_down<WT, R, kPfWaves>), dim3(grid), dim3(kPfWaves * 64), 0, st, a, gr);
  };
  if (wtype == W_BF16)
    launch(std::integral_constant<int, W_BF16>{});
  else
    launch(std::integral_constant<int, W_MXFP4>{});
  return hipGetLastError();
}

}  // namespace moe
