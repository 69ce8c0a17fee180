/*
 * paged_kv.h - C ABI of the operations around the paged KV cache that the
 * decode attention of paged_decode.h reads: the fused RoPE + cache write
 * that fills it, and the block movement (copy, gather, scatter, compaction)
 * a scheduler applies to it.
 *
 * Same library, status codes and dtype codes as paged_decode.h; the same
 * rules for every entry point: pointers are borrowed device memory the
 * caller keeps alive until the queued work has finished (host pointers
 * only where a function says so); nothing is allocated or synchronised and
 * no device memory is read on the host, so calls can be captured in a HIP
 * graph (positions, slot mappings, block ids and tables are read on the
 * device when the kernel runs); a call that fails its checks returns the
 * code and queues nothing; no C++ exception crosses the ABI.
 */
#ifndef PAGED_KV_H
#define PAGED_KV_H

#include <stddef.h>
#include <stdint.h>

#include "paged_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * cos/sin table of the rotary embedding (RoFormer, section 3.2): a float32
 * array [max_position, rotary_dim] whose row m holds cos(m * theta_i) in
 * column i and sin(m * theta_i) in column rotary_dim/2 + i, i < rotary_dim/2,
 * theta_i = base^(-2i / rotary_dim). Each entry is the float32 rounding
 * (nearest-even) of the value computed in fp64. Build it once per model;
 * rope_paged_kv_write reads it.
 *
 * table: device, 16-byte aligned, max_position * rotary_dim floats, written.
 * Errors: PD_ERR_SHAPE (max_position < 1, rotary_dim odd or outside
 * [2, 4096], or more than 2^31 entries), PD_ERR_VALUE (base not finite and
 * positive), PD_ERR_NULL, PD_ERR_ALIGN, PD_ERR_HIP.
 */
int32_t rope_cos_sin_table(float* table, int32_t max_position, int32_t rotary_dim, double base,
                           void* stream);

/*
 * RoPE + paged KV-cache write (Loom Kernels home page, "Supported now": "RoPE +
 * paged-KV write", a packed Q/K rotation and a write into the native cache;
 * benchmark page, "What the ratios mean": 1-512 tokens). For each token
 * t < T with m = positions[t] and s = slot_mapping[t]:
 *
 *   q_out[t][h]             = rot(q[t][h], m)        h < Hq
 *   k_cache[s / bs][s % bs][g] = rot(k[t][g], m)     g < Hkv, when s >= 0
 *   v_cache[s / bs][s % bs][g] = v[t][g]             g < Hkv, when s >= 0
 *
 * where rot turns pair i = (x[i], x[i + D/2]) by the angle of row m of the
 * table (x[i] c - x[i+D/2] s, x[i+D/2] c + x[i] s with c, s the table's
 * float32 cos and sin). Rotation in fp32, each output rounded once to dtype
 * (nearest-even); values are copied bit for bit.
 *
 * Layouts (element type dtype unless stated; heads of one token are D
 * elements apart, tokens q_row_stride / k_row_stride / v_row_stride elements
 * apart, so q, k and v may be views into one packed [T, Hq + 2 Hkv, D] QKV
 * array):
 *   q            [T, Hq, D] (row stride q_row_stride >= Hq * D)
 *   k, v         [T, Hkv, D] (row strides >= Hkv * D)
 *   positions    int32 [T]
 *   slot_mapping int32 [T]; a negative slot marks a padding token, whose
 *                K/V are not written (its q_out row still is)
 *   cos_sin      float32 [max_position, D] from rope_cos_sin_table (rotary
 *                dim = D)
 *   q_out        [T, Hq, D] contiguous; may be q itself (in place) when
 *                q_row_stride == Hq * D, else must not overlap any input
 *   k_cache, v_cache [num_blocks, block_size, Hkv, D], written at the slots
 *                named, every other byte left as it was
 *
 * Device-side contract (the caller's duty): 0 <= positions[t] <
 * max_position and slot_mapping[t] < num_blocks * block_size. The kernel
 * bounds-checks both and skips what falls outside (a token with a bad
 * position writes nothing at all; a bad slot writes no K/V), so memory
 * outside the arrays is never touched. Two tokens must not name one slot
 * (which of them lands is then unspecified).
 *
 * Supported: dtype f16 or bf16, D in {64, 128, 256}, block_size 16 or 32,
 * any Hq, Hkv >= 1 (at most 1024 each). T = 0 queues nothing.
 * Errors: PD_ERR_DTYPE, PD_ERR_SHAPE (negative sizes, strides too small, T
 * too large for one launch), PD_ERR_UNSUPPORTED (D, block_size), PD_ERR_NULL,
 * PD_ERR_ALIGN (q, k, v, q_out, caches, cos_sin not 16-byte aligned, row
 * strides not multiples of 8, positions/slots not 4-byte aligned),
 * PD_ERR_ALIAS (an output overlapping an input or another output other than
 * the in-place q_out), PD_ERR_HIP.
 */
int32_t rope_paged_kv_write(const void* q, const void* k, const void* v,
                            int64_t q_row_stride, int64_t k_row_stride, int64_t v_row_stride,
                            const int32_t* positions, const int32_t* slot_mapping,
                            const float* cos_sin, int32_t max_position,
                            void* q_out, void* k_cache, void* v_cache, int32_t num_blocks,
                            int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                            int32_t dtype, void* stream);

/*
 * The same step into an FP8 KV cache (Loom Kernels home page, "Next
 * boundaries": FP8 KV-cache compression; the cache paged_decode_attention_fp8
 * reads). k_cache and v_cache hold one OCP E4M3FN code per element in the
 * same [num_blocks, block_size, Hkv, D] layout; q, k, v and q_out stay
 * 16-bit of dtype, and q_out is written exactly as rope_paged_kv_write
 * writes it. At each named slot:
 *
 *   k code = E(fl(x' * fl(1 / k_scale))),  v code = E(fl(v * fl(1 / v_scale)))
 *
 * where x' is the key rotated in float32 in a fixed order, x'[i] =
 * fl(fl(x[i] c) - fl(x[i+D/2] s)) and x'[i+D/2] = fl(fl(x[i+D/2] c) +
 * fl(x[i] s)) (fl the float32 rounding, nearest-even, no fused
 * multiply-add), v is widened exactly, and E gives the E4M3FN code of the
 * nearest value (ties to the even code), holding magnitudes beyond the
 * largest finite 448 at 448 and NaN as 0x7F. The decode then reads the
 * value code * scale, so one scale per tensor serves the whole cache.
 *
 * Arguments, layouts, contract and errors as rope_paged_kv_write, except:
 * k_cache and v_cache are 8-byte aligned (PD_ERR_ALIGN otherwise) and span
 * num_blocks * block_size * Hkv * D bytes; k_scale and v_scale are finite
 * and positive (PD_ERR_VALUE otherwise).
 */
int32_t rope_paged_kv_write_fp8(const void* q, const void* k, const void* v,
                                int64_t q_row_stride, int64_t k_row_stride,
                                int64_t v_row_stride, const int32_t* positions,
                                const int32_t* slot_mapping, const float* cos_sin,
                                int32_t max_position, void* q_out, void* k_cache, void* v_cache,
                                int32_t num_blocks, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t block_size, int32_t dtype, float k_scale, float v_scale,
                                void* stream);

/*
 * KV-cache block movement (Loom Kernels home page, "Next boundaries":
 * KV-cache movement, block copy, gather, scatter and compact work for prefix
 * reuse and preemption). A block is one [block_size, Hkv, D] slab of a cache,
 * block_bytes bytes (block_size * Hkv * D * element size, any element type:
 * blocks move as raw bytes, unchanged). Each call moves blocks of k_cache
 * and, when v_cache is not NULL, the same blocks of v_cache; both caches
 * are [num_blocks, ...] arrays of block_bytes-sized blocks.
 *
 * Common rules: caches, buffers 16-byte aligned, block_bytes a positive
 * multiple of 16; id arrays int32 on the device, 4-byte aligned; k_cache and
 * v_cache overlap neither each other nor the ids; n = 0 queues nothing. Device-side contract: ids in [0, num_blocks) (an item
 * naming an id outside the pool is skipped, so nothing outside the arrays
 * is touched). Errors: PD_ERR_SHAPE (negative counts, num_blocks < 1,
 * block_bytes not a positive multiple of 16, too many items for one
 * launch: n * ceil(block_bytes / 4096) >= 2^24), PD_ERR_NULL, PD_ERR_ALIGN,
 * PD_ERR_ALIAS, PD_ERR_HIP.
 */

/*
 * Copy: for each i < num_pairs, block pairs[2i+1] (dst) of each cache
 * becomes a copy of block pairs[2i] (src) (copy-on-write of a shared
 * prefix). Sources may repeat; destinations must be distinct and no block
 * may be both a source and a destination (else the result is unspecified).
 * pairs must not overlap the caches.
 */
int32_t paged_kv_copy_blocks(void* k_cache, void* v_cache, int32_t num_blocks,
                             int64_t block_bytes, const int32_t* pairs, int32_t num_pairs,
                             void* stream);

/*
 * Gather: k_out[i] = k_cache[ids[i]] (and v_out[i] = v_cache[ids[i]]) for
 * i < n, into contiguous [n, ...] buffers (blocks leaving the pool on
 * preemption). v_out is needed exactly when v_cache is given. Outputs must
 * not overlap the caches, the ids or each other.
 */
int32_t paged_kv_gather_blocks(const void* k_cache, const void* v_cache, int32_t num_blocks,
                               int64_t block_bytes, const int32_t* ids, int32_t n, void* k_out,
                               void* v_out, void* stream);

/*
 * Scatter: k_cache[ids[i]] = k_in[i] (and v_cache[ids[i]] = v_in[i]) for
 * i < n (blocks coming back). ids must be distinct (else which lands is
 * unspecified). Inputs must not overlap the caches; the caches must not
 * overlap the ids or each other.
 */
int32_t paged_kv_scatter_blocks(const void* k_in, const void* v_in, const int32_t* ids,
                                int32_t n, void* k_cache, void* v_cache, int32_t num_blocks,
                                int64_t block_bytes, void* stream);

/*
 * Compaction plan, on the host (no device is touched): with live[b] != 0
 * for the n_live blocks in use, every live block whose id is >= n_live is
 * moved to a free id < n_live, the k-th such block (increasing ids) to the
 * k-th free id (increasing), so the live blocks fill [0, n_live) with the
 * fewest moves. Writes the moves as (src, dst) pairs, *num_pairs of them
 * (at most min(n_live, num_blocks - n_live)); remap[b] = the new id of
 * block b (b itself for a block that does not move); and *n_live. Sources
 * and destinations never meet, so the pairs are a valid
 * paged_kv_copy_blocks argument; paged_kv_remap_block_table with remap then
 * rewrites the block tables.
 *
 * live: host uint8 [num_blocks]; pairs: host int32 [pairs_capacity, 2];
 * remap: host int32 [num_blocks]. Errors: PD_ERR_SHAPE (num_blocks < 1, or
 * more moves than pairs_capacity: nothing is written then), PD_ERR_NULL.
 */
int32_t paged_kv_compact_plan(const uint8_t* live, int32_t num_blocks, int32_t* pairs,
                              int32_t pairs_capacity, int32_t* num_pairs, int32_t* remap,
                              int32_t* n_live);

/*
 * Rewrites a block table in place on the device: each of the `entries`
 * int32 values e with 0 <= e < num_blocks becomes remap[e] (remap: device
 * int32 [num_blocks]); any other value (padding such as -1) stays. The
 * table must not overlap remap. Errors: PD_ERR_SHAPE (entries < 0 or
 * >= 2^31, num_blocks < 1), PD_ERR_NULL, PD_ERR_ALIGN, PD_ERR_ALIAS,
 * PD_ERR_HIP.
 */
int32_t paged_kv_remap_block_table(int32_t* block_table, int64_t entries, const int32_t* remap,
                                   int32_t num_blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H */
