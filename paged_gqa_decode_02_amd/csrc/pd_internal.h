// Internal interfaces shared by the C ABI (pd_api.cpp), the host planner
// (pd_plan.cpp) and the HIP kernels (pd_kernels.hip). Not installed.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pd {

// Head dimension and query heads per KV head the kernels are built for.
constexpr int kHeadDim = 128;
constexpr int kGroup = 4;

struct Shape {
  int32_t B, Hq, Hkv, D, max_blocks_per_seq, block_size, dtype;
};

// How one call is laid out on the GPU.
struct Plan {
  int32_t splits;            // S: context partitions per (sequence, KV head)
  int32_t partition_tokens;  // P: tokens per partition, a multiple of block_size
  int32_t waves;             // NW: wavefronts per workgroup (1, 2, 4 or 8)
  int32_t wave_tokens;       // Pw: tokens per wave, a multiple of block_size,
                             //     at most 64 blocks; NW * Pw >= P
};

// Most blocks one wave's range may span (one block id per lane).
constexpr int kMaxWaveBlocks = 64;
constexpr int kMaxWaves = 8;

// Host-only checks of the scalar shape arguments; PD_* status code.
int32_t check_shape(const Shape& s);

// Split plan: requested_splits <= 0 runs the heuristic, else S is forced.
int32_t make_plan(const Shape& s, int32_t requested_splits, Plan* plan);

// Workspace layout for S > 1: fp32 partial outputs [B, Hq, S, D] first,
// then fp32 partial log2-sum-exps [B, Hq, S], each 256-byte aligned.
size_t partials_bytes(const Shape& s, const Plan& p);
size_t workspace_bytes(const Shape& s, const Plan& p);

// Everything a launch needs, all validated by the caller.
struct Launch {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* context_lens;
  void* out;
  void* workspace;
  Shape shape;
  Plan plan;
  float scale;
  void* stream;
};

// Queues the decode (and, for S > 1, the merge) kernel; PD_* status code.
int32_t launch(const Launch& l);

}  // namespace pd
