// Internal interfaces shared by the C ABI (pd_api.cpp), the host planner
// (pd_plan.cpp) and the HIP kernels (pd_kernels.hip). Not installed.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pd {

// Geometries the decode kernels are built for: head dim 64 or 128 (16-bit
// and FP8 caches alike), and up to kMaxGroup query heads per KV head.
constexpr int kMaxGroup = 128;

struct Shape {
  int32_t B, Hq, Hkv, D, max_blocks_per_seq, block_size, dtype;
};

// How one call is laid out on the GPU: a grid of (S, HS*Hkv/NH, B)
// workgroups of NH x NT waves; wave w serves virtual KV head w % NH of its
// group over token slice w / NH (Pw tokens) of its partition (P tokens). A
// KV head with more than 16 query heads is HS virtual KV heads of G/HS query
// heads each (consecutive virtual heads read the same physical KV head).
struct Plan {
  int32_t splits;            // S: context partitions per (sequence, KV head)
  int32_t partition_tokens;  // P: tokens per partition, a multiple of block_size
  int32_t heads_per_group;   // NH: KV heads per workgroup (1, 2, 4 or 8)
  int32_t slices;            // NT: token slices per workgroup, NH * NT <= 8
  int32_t wave_tokens;       // Pw: tokens per slice, a multiple of block_size,
                             //     at most 256 blocks; NT * Pw >= P
  int32_t head_split;        // HS: virtual KV heads per KV head, G / HS <= 16
};

// Most blocks one wave's slice may span (four block ids per lane).
constexpr int kMaxWaveBlocks = 256;
// Most waves in a workgroup: each wave holds two 16-token K/V tiles in LDS
// (17.5 KiB at D = 128 for a 16-bit cache, 8.1 KiB for FP8 codes, which are
// widened in registers), so 8 waves fill at most 140 KiB of a CU's 160 KiB.
constexpr int kMaxWaves = 8;

// Host-only checks of the scalar shape arguments; PD_* status code.
int32_t check_shape(const Shape& s);

// Split plan: requested_splits <= 0 runs the heuristic, else S is forced.
// kv_fp8 may change the slices per workgroup, never S or P (so the plan
// and workspace queries, which do not know the cache format, stay right).
int32_t make_plan(const Shape& s, int32_t requested_splits, Plan* plan, bool kv_fp8 = false);

// Workspace layout for S > 1: fp32 partial outputs [B, Hq, S, D], then fp32
// partial log2-sum-exps [B, Hq, S], each 256-byte aligned. Every call
// writes what it reads, so the workspace holds no state between calls.
size_t partials_bytes(const Shape& s, const Plan& p);
size_t lse_bytes(const Shape& s, const Plan& p);
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
  bool kv_fp8;    // K/V hold E4M3FN codes (1 byte per element)
  float k_scale;  // with kv_fp8: value = code * k_scale
  float v_scale;  // with kv_fp8: value = code * v_scale
};

// Queues the decode kernel, and for S > 1 the merge kernel after it on the
// same stream; PD_* status code.
int32_t launch(const Launch& l);

// paged_decode_attention with scratch the library owns (pd_api.cpp): every
// host check first, then PD_ERR_SCRATCH if the plan needs more than
// scratch_bytes, else get_scratch(stream, &ptr) supplies the scratch (only
// when the plan needs any) and the kernel is queued.
int32_t attention_with_scratch(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* context_lens,
                               int32_t max_blocks_per_seq, void* out, int32_t B, int32_t Hq,
                               int32_t Hkv, int32_t D, int32_t block_size, float scale,
                               int32_t dtype, void* stream, size_t scratch_bytes,
                               int32_t (*get_scratch)(void* stream, void** ptr));

// Queues a kernel that zeroes `bytes` (a multiple of 4) at `ws`.
int32_t zero_workspace(void* ws, size_t bytes, void* stream);

// RoPE + paged KV-cache write (pd_rope.hip); everything validated by the
// caller. Row strides are in elements; heads of a row are D apart.
struct RopeLaunch {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_row_stride, k_row_stride, v_row_stride;
  const int32_t* positions;
  const int32_t* slot_mapping;
  const float* cos_sin;
  int32_t max_position;
  void* q_out;
  void* k_cache;
  void* v_cache;
  int32_t num_blocks;
  int32_t T, Hq, Hkv, D, block_size, dtype;
  void* stream;
  bool kv_fp8 = false;  // caches hold E4M3FN codes (1 byte per element)
  float k_scale = 1.0f, v_scale = 1.0f;
};
int32_t launch_rope_kv_write(const RopeLaunch& l);
int32_t launch_rope_table(float* table, int32_t max_position, int32_t D, double base,
                          void* stream);

// Block movement (pd_blocks.hip); validated by the caller. mode: 0 copy
// (ids = pairs [n, 2]), 1 gather (ids [n], pool -> buffer), 2 scatter
// (ids [n], buffer -> pool); caches: 1 (K only) or 2 (K and V).
struct MoveLaunch {
  int32_t mode;
  const void* src[2];
  void* dst[2];
  int32_t caches;
  const int32_t* ids;
  int64_t block_bytes;
  int32_t n;
  int32_t num_blocks;
  void* stream;
};
int32_t launch_move_blocks(const MoveLaunch& l);
int64_t move_chunk_bytes();  // bytes one workgroup moves
int32_t launch_remap_table(int32_t* table, int64_t entries, const int32_t* remap,
                           int32_t num_blocks, void* stream);

}  // namespace pd
