// C ABI of the paged decode library: argument checks, planning and launch.
//
// Entry points are versioned and contain every failure (Loom Kernels home
// page, "Architecture": a versioned, panic-contained boundary over borrowed
// streams and memory with explicit layouts and aliasing rules). Nothing here
// touches device memory; every check uses host-visible values only.
#include <math.h>
#include <stdint.h>

#include <exception>

#include "../../include/paged_decode.h"
#include "pd_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool positive_finite(float x) { return x > 0.0f && isfinite(x); }

// Every host-side check of an attention call, then its plan, filled into
// *l ready to launch. With `own_workspace` the workspace arguments are not
// checked (the caller supplies scratch of its own afterwards) and
// *workspace_need tells how much the plan needs.
int32_t prepare(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_table, const int32_t* context_lens,
                int32_t max_blocks_per_seq, void* out, int32_t B, int32_t Hq, int32_t Hkv,
                int32_t D, int32_t block_size, float scale, int32_t dtype, void* workspace,
                size_t workspace_bytes, void* stream, int32_t requested_splits, bool kv_fp8,
                float k_scale, float v_scale, bool own_workspace, pd::Launch* l,
                size_t* workspace_need) {
  pd::Shape s{B, Hq, Hkv, D, max_blocks_per_seq, block_size, dtype};
  pd::Plan plan;
  int32_t st = pd::make_plan(s, requested_splits, &plan, kv_fp8);
  if (st != PD_OK) return st;
  if (!positive_finite(scale)) return PD_ERR_VALUE;
  if (kv_fp8 && (!positive_finite(k_scale) || !positive_finite(v_scale))) return PD_ERR_VALUE;
  const size_t need = pd::workspace_bytes(s, plan);
  *workspace_need = need;
  if (B == 0) return PD_OK;  // empty batch: nothing to compute
  if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out) return PD_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(context_lens, 4))
    return PD_ERR_ALIGN;
  if (need > 0 && !own_workspace) {
    if (!workspace || workspace_bytes < need) return PD_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return PD_ERR_ALIGN;
  }
  const size_t qo_bytes = (size_t)B * Hq * D * 2;
  if (overlap(out, qo_bytes, q, qo_bytes) ||
      overlap(out, qo_bytes, block_table, (size_t)B * max_blocks_per_seq * 4) ||
      overlap(out, qo_bytes, context_lens, (size_t)B * 4) ||
      (need > 0 && !own_workspace && overlap(out, qo_bytes, workspace, need)))
    return PD_ERR_ALIAS;
  *l = pd::Launch{q,     k_cache, v_cache, block_table, context_lens, out,     workspace,
                  s,     plan,    scale,   stream,      kv_fp8,       k_scale, v_scale};
  return PD_OK;
}

int32_t attention_impl(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* context_lens,
                       int32_t max_blocks_per_seq, void* out, int32_t B, int32_t Hq,
                       int32_t Hkv, int32_t D, int32_t block_size, float scale, int32_t dtype,
                       void* workspace, size_t workspace_bytes, void* stream,
                       int32_t requested_splits, bool kv_fp8 = false, float k_scale = 1.0f,
                       float v_scale = 1.0f) {
  pd::Launch l;
  size_t need = 0;
  const int32_t st = prepare(q, k_cache, v_cache, block_table, context_lens, max_blocks_per_seq,
                             out, B, Hq, Hkv, D, block_size, scale, dtype, workspace,
                             workspace_bytes, stream, requested_splits, kv_fp8, k_scale,
                             v_scale, false, &l, &need);
  if (st != PD_OK || B == 0) return st;
  return pd::launch(l);
}

int32_t plan_impl(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_blocks_per_seq,
                  int32_t block_size, int32_t dtype, int32_t requested_splits,
                  int32_t* num_splits, int32_t* partition_tokens) {
  pd::Shape s{B, Hq, Hkv, D, max_blocks_per_seq, block_size, dtype};
  pd::Plan plan;
  int32_t st = pd::make_plan(s, requested_splits, &plan);
  if (st != PD_OK) return st;
  if (!num_splits || !partition_tokens) return PD_ERR_NULL;
  *num_splits = plan.splits;
  *partition_tokens = plan.partition_tokens;
  return PD_OK;
}

size_t workspace_impl(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                      int32_t max_blocks_per_seq, int32_t block_size, int32_t dtype,
                      int32_t requested_splits) {
  pd::Shape s{B, Hq, Hkv, D, max_blocks_per_seq, block_size, dtype};
  pd::Plan plan;
  if (pd::make_plan(s, requested_splits, &plan) != PD_OK) return 0;
  return pd::workspace_bytes(s, plan);
}

}  // namespace

namespace pd {

int32_t attention_with_scratch(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* context_lens,
                               int32_t max_blocks_per_seq, void* out, int32_t B, int32_t Hq,
                               int32_t Hkv, int32_t D, int32_t block_size, float scale,
                               int32_t dtype, void* stream, size_t scratch_bytes,
                               int32_t (*get_scratch)(void* stream, void** ptr)) {
  Launch l;
  size_t need = 0;
  int32_t st = prepare(q, k_cache, v_cache, block_table, context_lens, max_blocks_per_seq, out,
                       B, Hq, Hkv, D, block_size, scale, dtype, nullptr, 0, stream, 0, false,
                       1.0f, 1.0f, true, &l, &need);
  if (st != PD_OK || B == 0) return st;
  if (need > scratch_bytes) return PD_ERR_SCRATCH;
  if (need > 0) {
    st = get_scratch(stream, &l.workspace);
    if (st != PD_OK) return st;
  }
  return launch(l);
}

}  // namespace pd

extern "C" {

int32_t paged_decode_abi_version(void) { return PAGED_DECODE_ABI_VERSION; }

const char* paged_decode_strerror(int32_t code) {
  switch (code) {
    case PD_OK: return "ok";
    case PD_ERR_NULL: return "a required pointer is NULL";
    case PD_ERR_SHAPE: return "a size argument is out of range or inconsistent";
    case PD_ERR_DTYPE: return "dtype must be PD_DTYPE_F16 or PD_DTYPE_BF16";
    case PD_ERR_ALIGN: return "pointer misaligned (q/k/v/out 16 B, tables 4 B, workspace 256 B)";
    case PD_ERR_ALIAS: return "out overlaps an input or the workspace";
    case PD_ERR_WORKSPACE: return "workspace missing or too small";
    case PD_ERR_UNSUPPORTED:
      return "shape not supported (needs D 64|128, Hq/Hkv <= 128, block_size 16|32)";
    case PD_ERR_HIP: return "HIP runtime rejected the launch";
    case PD_ERR_INTERNAL: return "internal error";
    case PD_ERR_VALUE: return "scale (and k_scale, v_scale) must be finite and positive";
    case PD_ERR_SCRATCH:
      return "the split plan needs more scratch than the no-allocation entry point holds "
             "(PAGED_DECODE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status code";
  }
}

int32_t paged_decode_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                          int32_t max_blocks_per_seq, int32_t block_size, int32_t dtype,
                          int32_t* num_splits, int32_t* partition_tokens) {
  try {
    return plan_impl(B, Hq, Hkv, D, max_blocks_per_seq, block_size, dtype, 0, num_splits,
                     partition_tokens);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

int32_t paged_decode_plan_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t max_blocks_per_seq, int32_t block_size, int32_t dtype,
                                 int32_t requested_splits, int32_t* num_splits,
                                 int32_t* partition_tokens) {
  try {
    if (requested_splits < 1) return PD_ERR_SHAPE;
    return plan_impl(B, Hq, Hkv, D, max_blocks_per_seq, block_size, dtype, requested_splits,
                     num_splits, partition_tokens);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

size_t paged_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t max_blocks_per_seq, int32_t block_size,
                                    int32_t dtype) {
  try {
    return workspace_impl(B, Hq, Hkv, D, max_blocks_per_seq, block_size, dtype, 0);
  } catch (...) {
    return 0;
  }
}

size_t paged_decode_workspace_bytes_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                           int32_t max_blocks_per_seq, int32_t block_size,
                                           int32_t dtype, int32_t requested_splits) {
  try {
    if (requested_splits < 1) return 0;
    return workspace_impl(B, Hq, Hkv, D, max_blocks_per_seq, block_size, dtype,
                          requested_splits);
  } catch (...) {
    return 0;
  }
}

int32_t paged_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (workspace_bytes < 4) return PD_OK;
    if (!workspace) return PD_ERR_NULL;
    if (!aligned(workspace, 256)) return PD_ERR_ALIGN;
    return pd::zero_workspace(workspace, workspace_bytes & ~size_t(3), stream);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

int32_t paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* context_lens,
                               int32_t max_blocks_per_seq, void* out, int32_t B, int32_t Hq,
                               int32_t Hkv, int32_t D, int32_t block_size, float scale,
                               int32_t dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  try {
    return attention_impl(q, k_cache, v_cache, block_table, context_lens, max_blocks_per_seq,
                          out, B, Hq, Hkv, D, block_size, scale, dtype, workspace,
                          workspace_bytes, stream, 0);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

int32_t paged_decode_attention_splits(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* context_lens,
                                      int32_t max_blocks_per_seq, void* out, int32_t B,
                                      int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                      float scale, int32_t dtype, void* workspace,
                                      size_t workspace_bytes, void* stream,
                                      int32_t num_splits) {
  try {
    if (num_splits < 1) return PD_ERR_SHAPE;
    return attention_impl(q, k_cache, v_cache, block_table, context_lens, max_blocks_per_seq,
                          out, B, Hq, Hkv, D, block_size, scale, dtype, workspace,
                          workspace_bytes, stream, num_splits);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

int32_t paged_decode_attention_fp8(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* context_lens,
                                   int32_t max_blocks_per_seq, void* out, int32_t B, int32_t Hq,
                                   int32_t Hkv, int32_t D, int32_t block_size, float scale,
                                   int32_t dtype, float k_scale, float v_scale, void* workspace,
                                   size_t workspace_bytes, void* stream, int32_t num_splits) {
  try {
    if (num_splits < 0) return PD_ERR_SHAPE;
    return attention_impl(q, k_cache, v_cache, block_table, context_lens, max_blocks_per_seq,
                          out, B, Hq, Hkv, D, block_size, scale, dtype, workspace,
                          workspace_bytes, stream, num_splits, true, k_scale, v_scale);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

}  // extern "C"
