// cache_move.hip -- moving kept experts between slot pools on an elastic resize.
//
// Pages: "Meet FreeToken: An Edge-Native MoE Serving Engine that Runs 753B GLM-5.2
// on a Single Workstation GPU" (MarkTechPost), "Three mechanisms", elastic memory
// management: the expert pool grows and shrinks without reloading experts from the
// host.  One launch moves up to kMoveBatch experts (their old and new slots travel
// in the kernel arguments, so the move needs no device table): the grid is
// (piece of an expert, expert), each thread copying 16-byte words with
// non-temporal vector loads and stores (the moved bytes are not reused soon), so
// the copy runs as one stream at HBM speed instead of one copy call per expert.
// One word per thread measured fastest (3.2 TB/s moved, i.e. 6.3 TB/s of reads
// and writes, against 2.0 TB/s for 8 words without the non-temporal hint).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

struct MoveBatch {
  const uint8_t* src;
  uint8_t* dst;
  uint64_t src_stride, dst_stride, bytes;
  int n;
  int32_t from[kMoveBatch];  // old slot of each move
  int32_t to[kMoveBatch];    // new slot of each move
};

constexpr int kMoveThreads = 256, kMoveWordsPerThread = 1;  // per block: 4 KB x words
constexpr uint64_t kMoveBlockBytes = (uint64_t)kMoveThreads * kMoveWordsPerThread * 16;

__global__ __launch_bounds__(kMoveThreads) void move_slots_kernel(MoveBatch m) {
  const int i = blockIdx.y;
  if (i >= m.n) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(m.src + (uint64_t)m.from[i] * m.src_stride);
  u32x4* dst = reinterpret_cast<u32x4*>(m.dst + (uint64_t)m.to[i] * m.dst_stride);
  const uint64_t words = m.bytes / 16;
  const uint64_t w0 = (uint64_t)blockIdx.x * kMoveBlockBytes / 16 + threadIdx.x;
  u32x4 v[kMoveWordsPerThread];
#pragma unroll
  for (int j = 0; j < kMoveWordsPerThread; ++j) {
    const uint64_t w = w0 + (uint64_t)j * kMoveThreads;
    if (w < words) v[j] = __builtin_nontemporal_load(src + w);
  }
#pragma unroll
  for (int j = 0; j < kMoveWordsPerThread; ++j) {
    const uint64_t w = w0 + (uint64_t)j * kMoveThreads;
    if (w < words) __builtin_nontemporal_store(v[j], dst + w);
  }
}

hipError_t launch_move_slots(const uint8_t* src, uint64_t src_stride, uint8_t* dst, uint64_t dst_stride,
                             uint64_t bytes, const int32_t* from, const int32_t* to, int n, hipStream_t st) {
  for (int b = 0; b < n; b += kMoveBatch) {
    MoveBatch m;
    m.src = src;
    m.dst = dst;
    m.src_stride = src_stride;
    m.dst_stride = dst_stride;
    m.bytes = bytes;
    m.n = n - b < kMoveBatch ? n - b : kMoveBatch;
    for (int i = 0; i < m.n; ++i) {
      m.from[i] = from[b + i];
      m.to[i] = to[b + i];
    }
    const dim3 grid((unsigned)((bytes + kMoveBlockBytes - 1) / kMoveBlockBytes), (unsigned)m.n);
    hipLaunchKernelGGL(move_slots_kernel, grid, dim3(kMoveThreads), 0, st, m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Slot tables of one cache wave, written by a kernel whose arguments carry the
// wave's (expert, slot) pairs: no staging copy of the whole table from host memory
// (a small host-to-device copy runs as a runtime copy kernel that reads the host
// buffer over the link).  Every entry of the table(s) becomes -1, then each pair is
// written into table a or b; one block, so a barrier orders the two.
__global__ __launch_bounds__(256) void write_slot_tables_kernel(SlotPairs p) {
  for (int e = threadIdx.x; e < p.E; e += 256) {
    p.table_a[e] = -1;
    if (p.table_b) p.table_b[e] = -1;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < p.n; i += 256) {
    const int e = p.key[i] & 0xffff;
    int32_t* t = (p.key[i] >> 16) ? p.table_b : p.table_a;
    t[e] = p.slot[i];
  }
}

hipError_t launch_write_slot_tables(const SlotPairs& p, hipStream_t st) {
  hipLaunchKernelGGL(write_slot_tables_kernel, dim3(1), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace moe
