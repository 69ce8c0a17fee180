// C ABI of the KV-cache operations (include/paged_kv.h): argument checks,
// the host compaction planner, and launch. As in pd_api.cpp, every check uses host-visible values only and
// every export contains all failures.
#include <math.h>
#include <stdint.h>

#include <exception>

#include "../../include/paged_kv.h"
#include "pd_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Byte ranges [a, a + na) and [b, b + nb) intersect.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

struct Range {
  const void* p;
  size_t n;
};

// Bytes spanned by T rows of `row_elems` 16-bit elements `stride` elements apart.
size_t rows_bytes(int64_t T, int64_t stride, int64_t row_elems) {
  return T > 0 ? (size_t)(((T - 1) * stride + row_elems) * 2) : 0;
}

bool positive_finite(float x) { return x > 0.0f && isfinite(x); }

int32_t rope_write_impl(const pd::RopeLaunch& l) {
  if (l.dtype != PD_DTYPE_F16 && l.dtype != PD_DTYPE_BF16) return PD_ERR_DTYPE;
  if (l.T < 0 || l.Hq < 1 || l.Hkv < 1 || l.Hq > 1024 || l.Hkv > 1024 || l.D < 1 ||
      l.block_size < 1 || l.num_blocks < 1 || l.max_position < 1)
    return PD_ERR_SHAPE;
  if (l.D != 64 && l.D != 128 && l.D != 256) return PD_ERR_UNSUPPORTED;
  if (l.block_size != 16 && l.block_size != 32) return PD_ERR_UNSUPPORTED;
  const int64_t qrow = (int64_t)l.Hq * l.D, kvrow = (int64_t)l.Hkv * l.D;
  if (l.q_row_stride < qrow || l.k_row_stride < kvrow || l.v_row_stride < kvrow)
    return PD_ERR_SHAPE;
  // one launch: T * (Hq + 2 Hkv) * D/16 threads in 256-thread workgroups
  const int64_t units = (int64_t)l.T * (l.Hq + 2 * l.Hkv) * (l.D / 16);
  if (units > ((int64_t)1 << 31) - 256) return PD_ERR_SHAPE;
  if ((int64_t)l.max_position * l.D > ((int64_t)1 << 31)) return PD_ERR_SHAPE;
  if (l.kv_fp8 && (!positive_finite(l.k_scale) || !positive_finite(l.v_scale)))
    return PD_ERR_VALUE;
  if (l.T == 0) return PD_OK;
  if (!l.q || !l.k || !l.v || !l.positions || !l.slot_mapping || !l.cos_sin || !l.q_out ||
      !l.k_cache || !l.v_cache)
    return PD_ERR_NULL;
  const uintptr_t cache_align = l.kv_fp8 ? 8 : 16;  // FP8 codes move 8 bytes at a time
  if (!aligned(l.q, 16) || !aligned(l.k, 16) || !aligned(l.v, 16) || !aligned(l.q_out, 16) ||
      !aligned(l.k_cache, cache_align) || !aligned(l.v_cache, cache_align) ||
      !aligned(l.cos_sin, 16) ||
      !aligned(l.positions, 4) || !aligned(l.slot_mapping, 4) || l.q_row_stride % 8 ||
      l.k_row_stride % 8 || l.v_row_stride % 8)
    return PD_ERR_ALIGN;

  const size_t cache_bytes = (size_t)l.num_blocks * l.block_size * kvrow * (l.kv_fp8 ? 1 : 2);
  const Range q{l.q, rows_bytes(l.T, l.q_row_stride, qrow)};
  const Range k{l.k, rows_bytes(l.T, l.k_row_stride, kvrow)};
  const Range v{l.v, rows_bytes(l.T, l.v_row_stride, kvrow)};
  const Range pos{l.positions, (size_t)l.T * 4};
  const Range slots{l.slot_mapping, (size_t)l.T * 4};
  const Range table{l.cos_sin, (size_t)l.max_position * l.D * 4};
  const Range qo{l.q_out, (size_t)l.T * qrow * 2};
  const Range kc{l.k_cache, cache_bytes};
  const Range vc{l.v_cache, cache_bytes};
  const bool in_place = l.q_out == l.q && l.q_row_stride == qrow;
  const Range outs[3] = {qo, kc, vc};
  const Range ins[6] = {q, k, v, pos, slots, table};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 6; ++i) {
      if (o == 0 && i == 0 && in_place) continue;  // q_out == q, element by element
      if (overlap(outs[o].p, outs[o].n, ins[i].p, ins[i].n)) return PD_ERR_ALIAS;
    }
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlap(outs[o].p, outs[o].n, outs[o2].p, outs[o2].n)) return PD_ERR_ALIAS;
  }
  return pd::launch_rope_kv_write(l);
}

// Checks shared by the three block moves; on success fills the launch.
int32_t move_impl(pd::MoveLaunch& l, const void* k_cache, const void* v_cache, const void* k_buf,
                  const void* v_buf, bool buf_is_output) {
  if (l.n < 0 || l.num_blocks < 1 || l.block_bytes < 16 || l.block_bytes % 16) return PD_ERR_SHAPE;
  const int64_t chunks = (l.block_bytes + pd::move_chunk_bytes() - 1) / pd::move_chunk_bytes();
  if ((int64_t)l.n * chunks >= ((int64_t)1 << 24)) return PD_ERR_SHAPE;
  if (l.n == 0) return PD_OK;
  const bool copy = l.mode == 0;
  if (!k_cache || !l.ids || (!copy && !k_buf) || (!copy && (v_cache != nullptr) != (v_buf != nullptr)))
    return PD_ERR_NULL;
  if (!aligned(k_cache, 16) || (v_cache && !aligned(v_cache, 16)) ||
      (k_buf && !aligned(k_buf, 16)) || (v_buf && !aligned(v_buf, 16)) || !aligned(l.ids, 4))
    return PD_ERR_ALIGN;
  const size_t pool = (size_t)l.num_blocks * (size_t)l.block_bytes;
  const size_t buf = (size_t)l.n * (size_t)l.block_bytes;
  const size_t ids = (size_t)l.n * (copy ? 8 : 4);
  if (overlap(k_cache, pool, v_cache, pool) || overlap(k_cache, pool, l.ids, ids) ||
      overlap(v_cache, pool, l.ids, ids))
    return PD_ERR_ALIAS;
  if (!copy) {
    const void* bufs[2] = {k_buf, v_buf};
    for (const void* b : bufs) {
      if (overlap(b, buf, k_cache, pool) || overlap(b, buf, v_cache, pool)) return PD_ERR_ALIAS;
      if (buf_is_output && overlap(b, buf, l.ids, ids)) return PD_ERR_ALIAS;
    }
    if (overlap(k_buf, buf, v_buf, buf)) return PD_ERR_ALIAS;
  }
  l.caches = v_cache ? 2 : 1;
  return pd::launch_move_blocks(l);
}

}  // namespace

extern "C" {

int32_t rope_cos_sin_table(float* table, int32_t max_position, int32_t rotary_dim, double base,
                           void* stream) {
  try {
    if (max_position < 1 || rotary_dim < 2 || rotary_dim > 4096 || rotary_dim % 2 ||
        (int64_t)max_position * rotary_dim > ((int64_t)1 << 31))
      return PD_ERR_SHAPE;
    if (!(base > 0.0) || !isfinite(base)) return PD_ERR_VALUE;
    if (!table) return PD_ERR_NULL;
    if (!aligned(table, 16)) return PD_ERR_ALIGN;
    return pd::launch_rope_table(table, max_position, rotary_dim, base, stream);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

int32_t rope_paged_kv_write(const void* q, const void* k, const void* v, int64_t q_row_stride,
                            int64_t k_row_stride, int64_t v_row_stride, const int32_t* positions,
                            const int32_t* slot_mapping, const float* cos_sin,
                            int32_t max_position, void* q_out, void* k_cache, void* v_cache,
                            int32_t num_blocks, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                            int32_t block_size, int32_t dtype, void* stream) {
  try {
    pd::RopeLaunch l{q,        k,         v,         q_row_stride, k_row_stride, v_row_stride,
                     positions, slot_mapping, cos_sin, max_position, q_out,     k_cache,
                     v_cache,  num_blocks, T,        Hq,           Hkv,          D,
                     block_size, dtype,   stream};
    return rope_write_impl(l);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

int32_t rope_paged_kv_write_fp8(const void* q, const void* k, const void* v,
                                int64_t q_row_stride, int64_t k_row_stride,
                                int64_t v_row_stride, const int32_t* positions,
                                const int32_t* slot_mapping, const float* cos_sin,
                                int32_t max_position, void* q_out, void* k_cache, void* v_cache,
                                int32_t num_blocks, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t block_size, int32_t dtype, float k_scale, float v_scale,
                                void* stream) {
  try {
    pd::RopeLaunch l{q,        k,         v,         q_row_stride, k_row_stride, v_row_stride,
                     positions, slot_mapping, cos_sin, max_position, q_out,     k_cache,
                     v_cache,  num_blocks, T,        Hq,           Hkv,          D,
                     block_size, dtype,   stream};
    l.kv_fp8 = true;
    l.k_scale = k_scale;
    l.v_scale = v_scale;
    return rope_write_impl(l);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

int32_t paged_kv_copy_blocks(void* k_cache, void* v_cache, int32_t num_blocks,
                             int64_t block_bytes, const int32_t* pairs, int32_t num_pairs,
                             void* stream) {
  try {
    pd::MoveLaunch l{0, {k_cache, v_cache}, {k_cache, v_cache}, 0, pairs, block_bytes,
                     num_pairs, num_blocks, stream};
    return move_impl(l, k_cache, v_cache, nullptr, nullptr, false);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

int32_t paged_kv_gather_blocks(const void* k_cache, const void* v_cache, int32_t num_blocks,
                               int64_t block_bytes, const int32_t* ids, int32_t n, void* k_out,
                               void* v_out, void* stream) {
  try {
    pd::MoveLaunch l{1, {k_cache, v_cache}, {k_out, v_out}, 0, ids, block_bytes, n, num_blocks,
                     stream};
    return move_impl(l, k_cache, v_cache, k_out, v_out, true);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

int32_t paged_kv_scatter_blocks(const void* k_in, const void* v_in, const int32_t* ids,
                                int32_t n, void* k_cache, void* v_cache, int32_t num_blocks,
                                int64_t block_bytes, void* stream) {
  try {
    pd::MoveLaunch l{2, {k_in, v_in}, {k_cache, v_cache}, 0, ids, block_bytes, n, num_blocks,
                     stream};
    return move_impl(l, k_cache, v_cache, k_in, v_in, false);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

int32_t paged_kv_compact_plan(const uint8_t* live, int32_t num_blocks, int32_t* pairs,
                              int32_t pairs_capacity, int32_t* num_pairs, int32_t* remap,
                              int32_t* n_live) {
  try {
    if (num_blocks < 1 || pairs_capacity < 0) return PD_ERR_SHAPE;
    if (!live || !num_pairs || !remap || !n_live || (pairs_capacity > 0 && !pairs))
      return PD_ERR_NULL;
    int32_t n = 0;
    for (int32_t b = 0; b < num_blocks; ++b) n += live[b] != 0;
    int32_t moves = 0;
    for (int32_t b = n; b < num_blocks; ++b) moves += live[b] != 0;
    if (moves > pairs_capacity) return PD_ERR_SHAPE;
    // two cursors: the next free id below n, the next live id at or above n
    int32_t hole = 0, k = 0;
    for (int32_t b = 0; b < num_blocks; ++b) remap[b] = b;
    for (int32_t src = n; src < num_blocks; ++src) {
      if (!live[src]) continue;
      while (live[hole]) ++hole;  // a free id below n exists for every mover
      pairs[2 * k] = src;
      pairs[2 * k + 1] = hole;
      remap[src] = hole;
      ++k;
      ++hole;
    }
    *num_pairs = moves;
    *n_live = n;
    return PD_OK;
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

int32_t paged_kv_remap_block_table(int32_t* block_table, int64_t entries, const int32_t* remap,
                                   int32_t num_blocks, void* stream) {
  try {
    if (entries < 0 || entries >= ((int64_t)1 << 31) || num_blocks < 1) return PD_ERR_SHAPE;
    if (entries == 0) return PD_OK;
    if (!block_table || !remap) return PD_ERR_NULL;
    if (!aligned(block_table, 4) || !aligned(remap, 4)) return PD_ERR_ALIGN;
    if (overlap(block_table, (size_t)entries * 4, remap, (size_t)num_blocks * 4))
      return PD_ERR_ALIAS;
    return pd::launch_remap_table(block_table, entries, remap, num_blocks, stream);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}

}  // extern "C"
