// Paged KV-cache block movement for gfx950: block copy, gather and scatter,
// and the block-table remap of a compaction (Loom Kernels home page, "Next
// boundaries": KV-cache movement, scheduler-facing block copy, gather,
// scatter and compact work for prefix reuse and preemption).
//
// A block (all block_size rows of all KV heads of one cache) is the unit of
// movement, moved as raw bytes, so one kernel serves any element type. Item i
// of a call moves one block of each cache from source slot s_i to
// destination slot d_i, where (s_i, d_i) is
//   copy:    pairs[i]       (pool -> pool)
//   gather:  (ids[i], i)    (pool -> contiguous buffer)
//   scatter: (i, ids[i])    (contiguous buffer -> pool)
// A workgroup of 256 threads moves one 4 KiB chunk of one item of one cache,
// one 16-byte load and store per thread, both streaming (nontemporal); the
// grid is (items x chunks, caches). Many small workgroups keep more of the
// moves in flight across the GPU than fewer large ones: against 16 KiB chunks
// (four loads per thread issued before any store) a 4,096-block gather took
// 87.5 instead of 91.2 us and a scatter 95.5 instead of 102.5 us; 32 KiB
// chunks took 133-139 us, and plain (cached) stores 3-7% longer. HBM-bound:
// the bytes read and written are the bytes moved. Pool ids are
// bounds-checked on the device (an item with an id outside the pool moves
// nothing).
//
// The remap kernel rewrites block tables in place after a compaction: each
// entry e with 0 <= e < num_blocks becomes remap[e]; other entries (padding)
// stay.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/paged_decode.h"
#include "pd_internal.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPerThread = 1;                          // 16-byte moves per thread
constexpr int64_t kChunk = kThreads * kPerThread * 16;  // 4 KiB per workgroup

enum Mode { kCopy = 0, kGather = 1, kScatter = 2 };

struct MoveArgs {
  const char* src[2];  // per cache: pool (copy, gather) or buffer (scatter)
  char* dst[2];        // per cache: pool (copy, scatter) or buffer (gather)
  const int32_t* ids;  // pairs [n, 2] (copy) or ids [n]
  int64_t block_bytes;
  int32_t n;           // items
  int32_t num_blocks;  // pool size
  int32_t chunks;      // chunks per block
};

template <int MODE>
__global__ __launch_bounds__(kThreads) void move_blocks_kernel(const MoveArgs a) {
  const int64_t x = blockIdx.x;
  const int64_t item = x / a.chunks;
  const int64_t chunk = x - item * a.chunks;
  if (item >= a.n) return;
  const int cache = blockIdx.y;
  int64_t s, d;
  if constexpr (MODE == kCopy) {
    s = a.ids[2 * item];
    d = a.ids[2 * item + 1];
    if ((uint64_t)s >= (uint64_t)a.num_blocks || (uint64_t)d >= (uint64_t)a.num_blocks) return;
  } else if constexpr (MODE == kGather) {
    s = a.ids[item];
    d = item;
    if ((uint64_t)s >= (uint64_t)a.num_blocks) return;
  } else {
    s = item;
    d = a.ids[item];
    if ((uint64_t)d >= (uint64_t)a.num_blocks) return;
  }
  const char* src = a.src[cache] + s * a.block_bytes;
  char* dst = a.dst[cache] + d * a.block_bytes;
  const int64_t base = chunk * kChunk + 16 * (int64_t)threadIdx.x;
  u32x4 v[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int64_t off = base + (int64_t)k * kThreads * 16;
    if (off < a.block_bytes) v[k] = __builtin_nontemporal_load((const u32x4*)(src + off));
  }
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int64_t off = base + (int64_t)k * kThreads * 16;
    if (off < a.block_bytes) __builtin_nontemporal_store(v[k], (u32x4*)(dst + off));
  }
}

__global__ __launch_bounds__(kThreads) void remap_table_kernel(int32_t* table, int64_t entries,
                                                               const int32_t* remap,
                                                               int32_t num_blocks) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= entries) return;
  const int32_t e = table[i];
  if ((uint32_t)e < (uint32_t)num_blocks) table[i] = remap[e];
}

}  // namespace

namespace pd {

int32_t launch_move_blocks(const MoveLaunch& l) {
  MoveArgs a;
  for (int c = 0; c < 2; ++c) {
    a.src[c] = (const char*)l.src[c];
    a.dst[c] = (char*)l.dst[c];
  }
  a.ids = l.ids;
  a.block_bytes = l.block_bytes;
  a.n = l.n;
  a.num_blocks = l.num_blocks;
  a.chunks = (int32_t)((l.block_bytes + kChunk - 1) / kChunk);
  const dim3 grid((unsigned)((int64_t)l.n * a.chunks), (unsigned)l.caches);
  const hipStream_t st = (hipStream_t)l.stream;
  switch (l.mode) {
    case kCopy: hipLaunchKernelGGL(move_blocks_kernel<kCopy>, grid, dim3(kThreads), 0, st, a); break;
    case kGather: hipLaunchKernelGGL(move_blocks_kernel<kGather>, grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL(move_blocks_kernel<kScatter>, grid, dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError() == hipSuccess ? PD_OK : PD_ERR_HIP;
}

int64_t move_chunk_bytes() { return kChunk; }

int32_t launch_remap_table(int32_t* table, int64_t entries, const int32_t* remap,
                           int32_t num_blocks, void* stream) {
  const unsigned blocks = (unsigned)((entries + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(remap_table_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     table, entries, remap, num_blocks);
  return hipGetLastError() == hipSuccess ? PD_OK : PD_ERR_HIP;
}

}  // namespace pd
