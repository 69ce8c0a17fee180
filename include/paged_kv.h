/*
 * paged_kv.h - C ABI of the operations around the paged KV cache that the
 * decode attention of paged_decode.h reads: the fused RoPE + cache write
 * that fills it.
 *
 * Same library, status codes and dtype codes as paged_decode.h; the same
 * rules for every entry point: pointers are borrowed device memory the
 * caller keeps alive until the queued work has finished; nothing is
 * allocated, synchronised or read on the host, so calls can be captured in a
 * HIP graph (positions and slot mappings are read on the device when the
 * kernel runs); a call that fails its checks returns the code and queues
 * nothing; no C++ exception crosses the ABI.
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
 * RoPE + paged KV-cache write (Loom Kernels home page, operator list: "RoPE +
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

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H */
