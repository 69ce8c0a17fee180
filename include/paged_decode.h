/*
 * paged_decode.h - C ABI of the MI355X (gfx950) paged GQA decode library.
 *
 * One query token per head attends over a KV cache scattered in fixed-size
 * blocks through a block table, with the query heads that share a KV head
 * packed into one pass over that head's K/V bytes, and long contexts split
 * into partitions whose partial results are merged by log-sum-exp (Loom
 * Kernels home page, "Supported now": paged MQA/GQA decode, GQA packing +
 * local split-K/LSE; benchmark page, "What the ratios mean": the
 * native-cache short-context route and the D128 long-context split-K/LSE
 * path at Hq/Hkv 32/8).
 *
 * What a call computes, for every sequence b < B and query head h < Hq, with
 * G = Hq / Hkv, g = h / G (consecutive grouping) and L = context_lens[b]:
 *
 *   s_t   = scale * sum_d q[b][h][d] * K[blk(t)][t % block_size][g][d],  t < L
 *   out[b][h][:] = sum_t softmax(s)_t * V[blk(t)][t % block_size][g][:]
 *
 * where blk(t) = block_table[b][t / block_size]. L = 0 gives a zero row.
 * Scores, softmax and accumulation run in fp32; the output is rounded once
 * to the input dtype, round-to-nearest-even.
 *
 * Layouts (row-major, contiguous, element type = dtype unless stated):
 *   q, out         [B, Hq, D]
 *   k_cache        [num_blocks, block_size, Hkv, D]
 *   v_cache        [num_blocks, block_size, Hkv, D]
 *   block_table    int32 [B, max_blocks_per_seq]
 *   context_lens   int32 [B]
 *   workspace      caller-owned device scratch for the split-K partials
 *
 * Ownership: every pointer is borrowed device memory that the caller keeps
 * alive until the work queued on `stream` has finished. The library never
 * allocates, frees, synchronises, or reads device memory on the host, so a
 * call can be captured in a HIP graph; block_table and context_lens are read
 * on the device when the kernels run. Inputs are never written; only `out`
 * and the workspace are.
 *
 * Device-side contract (not checkable on the host, the caller's duty):
 * 0 <= context_lens[b] <= max_blocks_per_seq * block_size, and every block
 * id the first ceil(L / block_size) entries of a row hold is in
 * [0, num_blocks). The decode does not check block ids against the pool (it
 * is not told num_blocks): an id outside it makes the kernel read outside
 * the caches, which can fault the GPU. Entries of a row past the first
 * ceil(L / block_size) may be loaded but are never used as addresses, and
 * cache slots at or after L in the last block are never read. Lengths
 * outside that range still keep the kernels inside the row: a length above
 * max_blocks_per_seq * block_size is taken as that, and a negative length
 * as 0 (zero output rows).
 *
 * Workspace contract (split plans, S > 1): the workspace holds the
 * partitions' fp32 partial outputs and log-sum-exps, which a second kernel,
 * queued right after the first on the same stream, merges into `out`. A
 * call writes every workspace byte it reads, so the workspace needs no
 * initialisation and keeps nothing from one call to the next; any
 * workspace at least as large as the shape needs serves it. Calls that
 * share a workspace must not overlap in time (issue them on one stream, or
 * order them with events).
 *
 * Errors: every entry point returns PD_OK or one of the codes below and
 * writes nothing when it fails before launching. No C++ exception crosses
 * the ABI. Supported now: D = 64 or 128; any G = Hq / Hkv from 1 to 128
 * (MHA, GQA with odd groups such as 14/2, MQA such as 32/1); block_size 16
 * or 32; dtype f16 or bf16. Other valid shapes return PD_ERR_UNSUPPORTED.
 */
#ifndef PAGED_DECODE_H
#define PAGED_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAGED_DECODE_ABI_VERSION 1

/* dtype codes */
#define PD_DTYPE_F16 0
#define PD_DTYPE_BF16 1

/* status codes */
#define PD_OK 0
#define PD_ERR_NULL 1          /* a required pointer is NULL */
#define PD_ERR_SHAPE 2         /* a size is out of range or inconsistent */
#define PD_ERR_DTYPE 3         /* dtype is not PD_DTYPE_F16 / PD_DTYPE_BF16 */
#define PD_ERR_ALIGN 4         /* q/k/v/out not 16-byte, tables not 4-byte, workspace not 256-byte aligned */
#define PD_ERR_ALIAS 5         /* out overlaps q, block_table, context_lens or the workspace */
#define PD_ERR_WORKSPACE 6     /* workspace missing or smaller than required */
#define PD_ERR_UNSUPPORTED 7   /* valid but not built (D, group size > 128, block size) */
#define PD_ERR_HIP 8           /* the HIP runtime rejected a launch */
#define PD_ERR_INTERNAL 9      /* unexpected internal failure */
#define PD_ERR_VALUE 10        /* scale is not a finite positive number */
#define PD_ERR_SCRATCH 11      /* the split plan needs more than the no-allocation scratch */

/* Version of this ABI (PAGED_DECODE_ABI_VERSION of the built library). */
int32_t paged_decode_abi_version(void);

/* Static, NUL-terminated description of a status code; never NULL. */
const char* paged_decode_strerror(int32_t code);

/*
 * Split plan for a shape: the number of context partitions S and the tokens
 * per partition P (a multiple of block_size) that paged_decode_attention
 * will use. Partition p covers tokens [p*P, min((p+1)*P, L)) of a sequence;
 * S = 1 means a single pass that writes `out` directly. A pure function of
 * its arguments: the heuristic is tuned for a whole MI355X (256 CUs) and
 * does not query the device, so a device with fewer CUs (a partition of
 * the GPU) gets the same plan, with the same results. It touches no device.
 * Returns PD_OK, or the error the attention call would give for the shape.
 */
int32_t paged_decode_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                          int32_t max_blocks_per_seq, int32_t block_size, int32_t dtype,
                          int32_t* num_splits, int32_t* partition_tokens);

/*
 * Workspace bytes paged_decode_attention needs for this shape: 0 when the
 * plan has S = 1, else room for fp32 partial outputs [B, Hq, S, D] and fp32
 * partial log-sum-exps [B, Hq, S], each rounded up to 256 bytes. Returns 0
 * for an invalid shape too (paged_decode_plan tells the two apart).
 */
size_t paged_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t max_blocks_per_seq, int32_t block_size,
                                    int32_t dtype);

/*
 * Zeroes `workspace_bytes` bytes (rounded down to a multiple of 4) of a
 * workspace on `stream` with a fill kernel (no memset node, so it is safe
 * to capture). `workspace` must be 256-byte aligned. PD_OK for 0 bytes.
 * The decode never needs it (see the workspace contract); it gives a
 * workspace defined contents for callers that want them.
 */
int32_t paged_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged decode attention (see the top of this file). Queues its kernel on
 * `stream` (a hipStream_t; NULL is the null stream), and for split plans
 * the merge kernel after it, and returns without waiting. `workspace` may be NULL when paged_decode_workspace_bytes(...)
 * is 0; otherwise it must follow the workspace contract above. `scale` is
 * usually 1/sqrt(D) rounded to float.
 */
int32_t paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* context_lens,
                               int32_t max_blocks_per_seq, void* out,
                               int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                               int32_t block_size, float scale, int32_t dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Same kernels with the split count forced to `num_splits` (>= 1) instead
 * of the heuristic's; P becomes the smallest multiple of block_size with
 * S*P >= max_blocks_per_seq * block_size, and S is then recomputed as
 * ceil(max_blocks_per_seq * block_size / P), so it can come out smaller than
 * asked. A partition never exceeds what one workgroup's token slices cover,
 * 256 blocks each: 4 slices (16,384 tokens at block size 16), or 2 when KV
 * heads are served in pairs, so a very long context can also get more splits
 * than asked. For tests and measurements of the split path; the result
 * equals the planned call's up to fp32 rounding order.
 */
int32_t paged_decode_attention_splits(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* context_lens,
                                      int32_t max_blocks_per_seq, void* out,
                                      int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                      int32_t block_size, float scale, int32_t dtype,
                                      void* workspace, size_t workspace_bytes, void* stream,
                                      int32_t num_splits);

/* Plan and workspace size for a forced split count, as used by
 * paged_decode_attention_splits. */
int32_t paged_decode_plan_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t max_blocks_per_seq, int32_t block_size, int32_t dtype,
                                 int32_t requested_splits,
                                 int32_t* num_splits, int32_t* partition_tokens);
size_t paged_decode_workspace_bytes_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                           int32_t max_blocks_per_seq, int32_t block_size,
                                           int32_t dtype, int32_t requested_splits);

/* Paged decode attention over an FP8 KV cache (Loom Kernels home page,
 * "Next boundaries": FP8 KV-cache compression, which halves the cache bytes
 * the bandwidth-bound path reads).
 *
 * k_cache and v_cache hold one byte per element in the same
 * [num_blocks, block_size, Hkv, D] layout: OCP FP8 E4M3FN codes (1 sign, 4
 * exponent bits with bias 7, 3 fraction bits; 0x7F and 0xFF are NaN; largest
 * finite 448). The element a code stands for is code * k_scale (K) or
 * code * v_scale (V), one float32 scale per tensor. q and out stay 16-bit of
 * `dtype` (PD_DTYPE_F16 or PD_DTYPE_BF16); every other argument, the layout,
 * ownership, workspace and error rules are those of paged_decode_attention,
 * and the plan and workspace size are paged_decode_plan's and
 * paged_decode_workspace_bytes' for the same shape and dtype (num_splits = 0)
 * or their _splits forms (num_splits > 0 forces S).
 *
 * The codes are widened exactly; the scales are applied in fp32 to the scores
 * (k_scale * scale) and to the normalised output (v_scale).
 *
 * Errors as paged_decode_attention, plus PD_ERR_VALUE when k_scale or
 * v_scale is not finite and positive and PD_ERR_SHAPE for num_splits < 0.
 * The FP8 kernels take every geometry the 16-bit path takes (D 64 or 128,
 * group sizes 1 to 128, block size 16 or 32).
 */
int32_t paged_decode_attention_fp8(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* context_lens,
                                   int32_t max_blocks_per_seq, void* out,
                                   int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                   int32_t block_size, float scale, int32_t dtype,
                                   float k_scale, float v_scale,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   int32_t num_splits);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * paged_decode_attention without a workspace argument. The split-K scratch
 * is one static device array per GPU of PAGED_DECODE_NOALLOC_SCRATCH_BYTES
 * (32 MiB of fp32 partials), held from the library's first call on that GPU
 * until the process ends; nothing is allocated or freed per call. Same
 * arguments (minus the workspace), plan, kernels and result as
 * paged_decode_attention, bit for bit.
 *
 * The first call on a GPU looks up that GPU's copy of the array. A call
 * writes every byte of it that it reads, so nothing needs clearing; but all
 * calls on one GPU share the array: calls that overlap in time on one GPU
 * (on different streams without ordering) race and give wrong results, so
 * order them (one stream, or events).
 *
 * Errors as paged_decode_attention, plus PD_ERR_SCRATCH (nothing queued)
 * when the shape's split plan needs more than the array holds, i.e. when
 * paged_decode_workspace_bytes(...) > PAGED_DECODE_NOALLOC_SCRATCH_BYTES.
 */
#define PAGED_DECODE_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
int32_t paged_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_table, const int32_t* context_lens,
                                       int32_t max_blocks_per_seq, void* out,
                                       int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                       int32_t block_size, float scale, int32_t dtype,
                                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_DECODE_H */
