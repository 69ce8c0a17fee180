// Paged GQA decode attention kernel for gfx950 (CDNA4, wave64).
//
// Method (Loom Kernels home page, "Supported now": paged MQA/GQA decode with
// GQA packing and local split-K/LSE): one query token per head attends over
// a paged K/V cache; the G = Hq / Hkv query heads that share a KV head are
// served by one pass over that head's K/V bytes, and a long context is cut
// into partitions whose normalised partial outputs and log-sum-exps are
// merged. Built for head dims D = 64 and 128 and any G up to 128 (MQA such
// as 32/1 or 64/1 included). The query heads of a wave fill the 16 columns of an MFMA
// block (spare columns repeat heads); a KV head with more than 16 query
// heads is served by HS "virtual" KV heads of G / HS <= 16 query heads each,
// whose waves sit in one workgroup and read the same K/V blocks together.
// An FP8 (E4M3FN) cache is read as codes and widened in registers.
//
// One kernel. Workgroup (partition p, KV-head group hg, sequence b) has
// NH x NT wave64s: wave w serves KV head hg*NH + w%NH over token slice w/NH
// of the partition (a block-aligned range of at most 256 blocks). Waves of
// the same slice read the same physical blocks, so a workgroup sweeps whole
// blocks (all heads of a token are one contiguous row group) rather than
// slivers of them.
//   * K/V move in tiles of 16 tokens from HBM straight into LDS with
//     bounds-checked buffer loads whose resource is the current physical
//     block (base = pool + id * block bytes, size = block bytes), so an
//     access cannot leave the block; lanes past the context get an offset
//     beyond the block and read nothing. Each 128-bit load instruction of a
//     wave reads 1 KiB: four whole 256-byte rows (D = 128) or eight 128-byte
//     rows (D = 64) of 16-bit values, or eight or sixteen rows of FP8 codes. One or two tiles stay in flight while the oldest is
//     computed; the loads use the streaming (nt) cache policy since every
//     K/V byte is read once.
//   * block ids: each lane loads up to four block-table entries of the
//     wave's range before the context length is known; a tile takes its
//     (wave-uniform) id with v_readlane, so addresses are scalar.
//   * scores: q . k for the 16 tokens of a tile and 16 query-head columns
//     are one 16x16 output of D/32 v_mfma_f32_16x16x32 (bf16 or f16 inputs,
//     exact products, fp32 sums), read from LDS in the operand order; one
//     multiply by scale*log2(e) puts the softmax in base 2 (v_exp_f32).
//   * softmax: per head column, a reference maximum that only moves when a
//     ballot finds a tile maximum more than 8 (f16: 6) above it in log2
//     units, i.e. a weight above 2^8 (2^6) (then the accumulators are
//     rescaled); each lane keeps its own partial sum of weights.
//   * PV: per 16-dim block and 16-bit weight term, a 16x16x16 MFMA of V^T
//     (read from LDS with the transposing ds_read_b64_tr_b16) and the
//     weights, accumulating in fp32.
//   * end of slice: each head's D sums sit in the 4 lanes of its column;
//     the NT slices of a head are merged through LDS, every wave of the
//     workgroup taking a share of the outputs.
//   * S == 1: the workgroup writes `out`, rounded to the dtype.
//   * S > 1: the workgroup writes its fp32 partial output and log2-sum-exp
//     (write-through stores), and a second kernel, queued right after on the
//     same stream, merges the non-empty partitions of every (sequence, query
//     head) in fixed order p = 0..n-1 and writes `out`. The kernel boundary
//     orders the partials' stores before the merge's loads; no state is kept
//     between calls.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/paged_decode.h"
#include "pd_internal.h"

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kIdRegs = pd::kMaxWaveBlocks / 64;  // block ids per lane
constexpr uint32_t kOutOfBlock = 0x80000000u;  // buffer offset that reads as zero
constexpr int kRsrcWord3 = 0x00020000;         // raw 32-bit buffer, gfx9 data format
constexpr int kStream = 2;                     // cache policy "nt": read once
constexpr int kCoherent = 16;                  // cache policy "sc1": device-coherent

struct KArgs {
  const uint16_t* q;
  const char* k;
  const char* v;
  const int32_t* bt;
  const int32_t* cl;
  void* out;
  float* o_part;      // [B, Hq, S, D]
  float* lse_part;    // [B, Hq, S], log2 domain
  // Hkv, HS, NH and groups serve the host: the kernel takes NH, HS and the
  // physical KV heads packed in its preloaded `geo` argument
  int32_t Hkv;  // virtual KV heads: physical KV heads x HS
  int32_t HS;   // virtual KV heads per physical KV head
  int32_t G;    // query heads per virtual KV head, <= 16
  int32_t MB;
  int32_t S;
  int32_t P;
  int32_t Pw;  // tokens per slice, a multiple of the block size, <= 256 blocks
  int32_t NH;  // KV heads per workgroup
  int32_t NT;  // token slices per workgroup
  int32_t groups;  // head groups (workgroups per partition) per sequence: Hkv / NH
  float scale_log2;    // scale * log2(e), times k_scale for an FP8 cache
  float out_scale;     // v_scale for an FP8 cache, else 1
  uint32_t blk_bytes;  // block_size * Hkv * D * element bytes
};

template <bool BF16>
__device__ __forceinline__ float lo_f(uint32_t u) {
  if constexpr (BF16) return __uint_as_float(u << 16);
  else return (float)__builtin_bit_cast(f16x2_t, u)[0];
}

template <bool BF16>
__device__ __forceinline__ float hi_f(uint32_t u) {
  if constexpr (BF16) return __uint_as_float(u & 0xffff0000u);
  else return (float)__builtin_bit_cast(f16x2_t, u)[1];
}

template <bool BF16>
__device__ __forceinline__ uint16_t to_bits(float x) {
  if constexpr (BF16) return __builtin_bit_cast(uint16_t, (__bf16)x);
  else return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)to_bits<BF16>(a) | ((uint32_t)to_bits<BF16>(b) << 16);
}

// DPP helpers (row = 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                        0xf, 0xf, false));
}

__device__ __forceinline__ float swap16_lo(float a, float b, float* b_out) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a),
                                            __builtin_bit_cast(uint32_t, b), false, false);
  *b_out = __builtin_bit_cast(float, (uint32_t)r[1]);
  return __builtin_bit_cast(float, (uint32_t)r[0]);
}

__device__ __forceinline__ float swap32_lo(float a, float b, float* b_out) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                            __builtin_bit_cast(uint32_t, b), false, false);
  *b_out = __builtin_bit_cast(float, (uint32_t)r[1]);
  return __builtin_bit_cast(float, (uint32_t)r[0]);
}

// Maximum / sum over the 4 token rows of the wave (lanes with equal lane%16).
__device__ __forceinline__ float max_rows(float x) {
  float y;
  float a = swap16_lo(x, x, &y);
  x = fmaxf(a, y);
  a = swap32_lo(x, x, &y);
  return fmaxf(a, y);
}

__device__ __forceinline__ float sum_rows(float x) {
  float y;
  float a = swap16_lo(x, x, &y);
  x = a + y;
  a = swap32_lo(x, x, &y);
  return a + y;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float uniform_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, kRsrcWord3);
}

// Tiles of 16 tokens of one KV head go from HBM straight into LDS (buffer
// loads with the LDS destination, no VGPRs held while in flight). A token row
// of one KV head is C = D/8 16-byte chunks; one load instruction moves R =
// 64 / C rows (4 at D = 128, 8 at D = 64), lane (r, sl) = (lane / C, lane %
// C) reading 16 bytes of row r, so every C lanes read one whole row, and
// lands them as one 1 KiB group in LDS. Which chunk a lane takes is rotated
// per row, and the 16/R groups of a tile are padded apart, so that the LDS
// reads below spread over the banks:
//   K: lane sl takes chunk (sl - r) mod C, groups 1088 bytes apart; read
//      back 16 bytes per lane in MFMA operand order (token lane%16, chunk
//      4s + lane/16);
//   V: lane sl takes chunk (sl - 2r) mod C, groups 1152 bytes apart; read
//      back with the transposing ds_read_b64_tr_b16, 8 bytes per lane
//      (token 4(lane/16) + (lane%16)/4, dims 4(lane%4) of a 16-dim block).
// At D = 128 any 16 lanes of the K read, and each 32 lanes of the V read,
// hit distinct 16-byte (8-byte) bank slots.
constexpr int kTileTok = 16;
template <int D>
struct Geo {
  static constexpr int kChunks = D / 8;                     // C
  static constexpr uint32_t kRowBytes = 2 * D;              // one 16-bit row of one KV head
  static constexpr int kRowsPerLoad = 64 / kChunks;         // R
  static constexpr int kGroups = kTileTok / kRowsPerLoad;   // load instructions per tile and tensor
  static constexpr uint32_t kKGroup = 1024 + 64;
  static constexpr uint32_t kVGroup = 1024 + 128;
  static constexpr uint32_t kKTile = kGroups * kKGroup;
  static constexpr uint32_t kLdsTile = kKTile + kGroups * kVGroup;  // K then V
  static constexpr int kSteps = D / 32;   // score MFMAs per column block
  static constexpr int kBlocks = D / 16;  // 16-dim output blocks (PV MFMAs)
};
static_assert(Geo<128>::kLdsTile == 8960 && Geo<64>::kLdsTile == 4480, "tile layout");
// An FP8 cache stays in its codes in LDS: a tile is 16 rows of D bytes for
// K, then for V, in 1 KiB groups of one load instruction each (64/(D/16)
// rows: 8 rows of 128 bytes at D = 128, groups 1040 bytes apart; all 16 rows
// of 64 bytes at D = 64, unpadded); the D/16 16-byte chunks of a row are
// rotated: chunk c of row r of a group sits at slot (c + rot(r)) mod D/16,
// rot(r) = r & ~1 at D = 128 and (0, 2, 1, 3)[r / 4] at D = 64. The tile
// path reads it in operand order and widens in registers:
//   K: ds_read_b64 of token lane%16, dims 32s + 8(lane/16) .. +8;
//   V: ds_read_b64_tr_b8, source lane 16g + a + 2k giving token 4g + k%4,
//      dims 16(m + k/4) + 8a .. +8, so that lane l receives dim 16m +
//      l%16 of tokens 4(l/16)..+4 (bytes 0..3) and dim 16(m+1) + l%16 of
//      the same tokens (bytes 4..7): two 16-dim blocks per read.
// Within each half-wave these reads touch 32 distinct 8-byte bank slots
// (no bank conflicts: measured with the LDS conflict counter at D = 128,
// enumerated lane by lane at D = 64).
template <int D>
struct Geo8 {
  static constexpr uint32_t kRowBytes = D;                  // one FP8 row of one KV head
  static constexpr int kChunks = D / 16;                    // 16-byte chunks per row
  static constexpr int kRowsPerLoad = 64 / kChunks;         // rows per 1 KiB load
  static constexpr int kGroups = kTileTok / kRowsPerLoad;   // loads per tile and tensor
  static constexpr uint32_t kGroup = D == 128 ? 1024 + 16 : 1024;
  static constexpr uint32_t kKTile = kGroups * kGroup;
  static constexpr uint32_t kStage = 2 * kKTile;
  // rotation of the chunks of row r (< kRowsPerLoad) of a group
  __host__ __device__ static constexpr int rot(int r) {
    return D == 128 ? (r & ~1) : (((r >> 2) & 1) << 1) | (r >> 3);
  }
};
static_assert(Geo8<128>::kStage == 4160 && Geo8<64>::kStage == 2048, "FP8 tile layout");
// the slice merge's per-wave scratch: G * (D + 2) floats for G <= 16
template <int D>
constexpr uint32_t merge_bytes() { return 16u * (D + 2) * 4u; }

// Two tile buffers per wave: one tile in flight while the other is
// computed. (Three and four buffers, all tiles of a short slice in flight at
// once, measured slower on every decode shape.)
template <int D, bool KV8>
constexpr uint32_t stage_bytes() { return KV8 ? Geo8<D>::kStage : Geo<D>::kLdsTile; }
template <int D, bool KV8>
constexpr int tile_buffers(int) { return 2; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef int v2i32_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t* lds_v4i16_ptr_t;

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8) that waits for vmcnt <= n and nothing else.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// ... and one that waits for every LDS access of the wave (lgkmcnt 0) only
constexpr int kWaitLds = 15 | (3 << 14) | (7 << 4);

template <bool BF16>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Softmax weights enter the PV products as a sum of 16-bit terms: hi =
// round(p), lo = round(p - hi), and for bf16 a third term lo2 = round(p - hi
// - lo) (each difference is exact in fp32), so p is carried to about 2^-27
// (bf16, three 8-bit terms) or 2^-22 (f16, two 11-bit terms) relative, the
// level of the fp32 arithmetic around it. For f16 the weights are scaled by
// 2^8 (the scale cancels in acc / l), which keeps lo of small weights out of
// the subnormal range.
template <bool BF16>
struct Weights {
  u32x4 hi_lo;   // words 0, 1: hi of the lane's 4 tokens; words 2, 3: lo
  uint32_t lo2[2];  // bf16 only: the third term of the 4 tokens
};
template <bool BF16>
__device__ __forceinline__ Weights<BF16> split_weights(const float (&p)[4]) {
  Weights<BF16> w;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t hi = pack2<BF16>(p[2 * i], p[2 * i + 1]);
    const float r0 = p[2 * i] - lo_f<BF16>(hi);
    const float r1 = p[2 * i + 1] - hi_f<BF16>(hi);
    const uint32_t lo = pack2<BF16>(r0, r1);
    w.hi_lo[i] = hi;
    w.hi_lo[2 + i] = lo;
    if constexpr (BF16) w.lo2[i] = pack2<BF16>(r0 - lo_f<BF16>(lo), r1 - hi_f<BF16>(lo));
  }
  return w;
}
template <bool BF16>
struct WeightBias {
  static constexpr float log2 = BF16 ? 0.f : 8.f;
  // the running maximum that serves as the weights' reference moves only
  // when a tile's maximum exceeds it by more than `lazy` (log2 units): the
  // result does not depend on the reference, and the accumulators are
  // rescaled far less often. Weights then stay below 2^(lazy + log2): 2^8
  // for bf16, 2^14 for f16 (whose largest finite value is 65504).
  static constexpr float lazy = BF16 ? 8.f : 6.f;
};

// v_mfma_f32_16x16x16: A lane l = row l%16, k 4(l/16) .. +4; B lane l =
// column l%16, the same k; two 32-bit words (four 16-bit values) each
template <bool BF16>
__device__ __forceinline__ f32x4 mfma_16x16x16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                               f32x4 c) {
  const u32x2_t a = {a0, a1}, b = {b0, b1};
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16_t, a),
                                                     __builtin_bit_cast(v4i16_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

// Per-lane state of one wave's online softmax over its token slice. Lane l
// follows head column l%16 (query head (l%16) % G of the virtual KV head);
// acc[m][i] is its unnormalised PV sum for dim 16m + 4(l/16) + i.
template <int D>
struct WaveState {
  f32x4 acc[Geo<D>::kBlocks];
  float lsum;  // sum of weights over the tokens of this lane's row
  float m;     // running maximum (log2 domain)
};

// One 16-token tile, already in LDS at kt (K) and kt + kKTile (V).
//   scores: the K tile is the A operand of D/32 16x16x32 MFMAs (row = token
//     lane%16, k = dims 32s + 8(lane/16) .. +8), q the B operand (column =
//     lane%16 -> its head): lane l gets the scores of tokens 4(l/16) + i,
//     i < 4, for its column;
//   softmax: the tile maximum per column (4 registers, then the 4 rows); the
//     reference maximum only moves when a ballot finds a tile maximum more
//     than WeightBias::lazy above it;
//   PV: per 16-dim block, 16x16x16 MFMAs with A = V^T (row = dim, k = the
//     lane's 4 tokens) and B = those tokens' weights, which is the layout
//     the scores came out in: one for the hi terms, one for lo, and for
//     bf16 a third for lo2.
// The math of one tile: ka[s] the K tile as score-MFMA A operands, v01/v23
// the V^T operand of each 16-dim block (16-bit values of tokens 4(lane/16)
// + 0,1 and + 2,3 for dim lane%16 of the block).
template <bool BF16, int D>
__device__ __forceinline__ void tile_math(WaveState<D>& st, const u32x4 (&ka)[Geo<D>::kSteps],
                                          uint32_t (&v01)[Geo<D>::kBlocks],
                                          uint32_t (&v23)[Geo<D>::kBlocks],
                                          const u32x4 (&qb)[Geo<D>::kSteps], int tok_row0,
                                          int tw1, bool partial, float c) {
  constexpr int kS = Geo<D>::kSteps, kM = Geo<D>::kBlocks;
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kS; ++s) sc = mfma_16x16x32<BF16>(ka[s], qb[s], sc);
  float s_[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s_[i] = sc[i] * c;
  if (partial) {
    // tokens past the slice get no weight, and their V values (whatever the
    // LDS holds there) are replaced by zeros
#pragma unroll
    for (int i = 0; i < 4; ++i) s_[i] = tok_row0 + i < tw1 ? s_[i] : -INFINITY;
    const uint32_t keep01 = (tok_row0 < tw1 ? 0xffffu : 0u) | (tok_row0 + 1 < tw1 ? 0xffff0000u : 0u);
    const uint32_t keep23 =
        (tok_row0 + 2 < tw1 ? 0xffffu : 0u) | (tok_row0 + 3 < tw1 ? 0xffff0000u : 0u);
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      v01[m] &= keep01;
      v23[m] &= keep23;
    }
  }
  const float tm = max_rows(fmaxf(fmaxf(s_[0], s_[1]), fmaxf(s_[2], s_[3])));
  if (__builtin_amdgcn_ballot_w64(tm > st.m + WeightBias<BF16>::lazy) != 0) {
    const float mn = fmaxf(st.m, tm);
    const float alpha = exp2_fast(st.m - mn);  // 1 where the maximum stays, 0 from -inf
    st.m = mn;
    st.lsum *= alpha;
#pragma unroll
    for (int m = 0; m < kM; ++m) st.acc[m] *= alpha;
  }
  float pr[4];
  const float mref = BF16 ? st.m : st.m - WeightBias<BF16>::log2;
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = exp2_fast(s_[i] - mref);
  st.lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  const Weights<BF16> wb = split_weights<BF16>(pr);
  // PV: one 16x16x16 MFMA per weight term and 16-dim block, A = V^T exactly
  // as the transposing read delivered it (dim lane%16, the lane's 4 tokens)
#pragma unroll
  for (int m = 0; m < kM; ++m)
    st.acc[m] = mfma_16x16x16<BF16>(v01[m], v23[m], wb.hi_lo[0], wb.hi_lo[1], st.acc[m]);
#pragma unroll
  for (int m = 0; m < kM; ++m)
    st.acc[m] = mfma_16x16x16<BF16>(v01[m], v23[m], wb.hi_lo[2], wb.hi_lo[3], st.acc[m]);
  if constexpr (BF16) {
#pragma unroll
    for (int m = 0; m < kM; ++m)
      st.acc[m] = mfma_16x16x16<BF16>(v01[m], v23[m], wb.lo2[0], wb.lo2[1], st.acc[m]);
  }
}

// One 16-bit tile, already in LDS at kt (K) and kt + kKTile (V): its LDS
// reads go out first (K in operand order, V^T through the transposing read),
// then the math.
template <bool BF16, int D>
__device__ __forceinline__ void tile_compute(WaveState<D>& st, const char* kt,
                                             const u32x4 (&qb)[Geo<D>::kSteps],
                                             const uint32_t (&koff)[Geo<D>::kSteps],
                                             const uint32_t (&voff)[Geo<D>::kBlocks],
                                             int tok_row0, int tw1, bool partial, float c) {
  constexpr int kS = Geo<D>::kSteps, kM = Geo<D>::kBlocks;
  u32x4 ka[kS];
#pragma unroll
  for (int s = 0; s < kS; ++s) ka[s] = *(const u32x4*)(kt + koff[s]);
  uint32_t v01[kM], v23[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const v4i16_t vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr_t)(kt + voff[m]));
    v01[m] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(vt, vt, 0, 1));
    v23[m] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(vt, vt, 2, 3));
  }
  tile_math<BF16, D>(st, ka, v01, v23, qb, tok_row0, tw1, partial, c);
}

// Two E4M3FN codes (bytes 2 HI, 2 HI + 1 of x) -> two 16-bit values, exact.
template <bool BF16, bool HI>
__device__ __forceinline__ uint32_t widen_pair(uint32_t x) {
  if constexpr (BF16)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, HI));
}

typedef __attribute__((address_space(3))) v2i32_t* lds_v2i32_ptr_t;

// One 16-token FP8 tile at kt: K codes widened into the score MFMA's A
// operand, V^T codes (two 16-dim blocks per transposing read) widened into
// the PV operand; then the same math as the 16-bit tile.
template <bool BF16, int D>
__device__ __forceinline__ void tile_compute_fp8(WaveState<D>& st, const char* kt,
                                                 const u32x4 (&qb)[D / 32],
                                                 const uint32_t (&koff)[D / 32],
                                                 const uint32_t (&voff)[D / 32], int tok_row0,
                                                 int tw1, bool partial, float c) {
  constexpr int kS = D / 32;
  u32x4 ka[kS];
#pragma unroll
  for (int s = 0; s < kS; ++s) {
    const u32x2_t x = *(const u32x2_t*)(kt + koff[s]);
    ka[s] = u32x4{widen_pair<BF16, false>(x[0]), widen_pair<BF16, true>(x[0]),
                  widen_pair<BF16, false>(x[1]), widen_pair<BF16, true>(x[1])};
  }
  uint32_t v01[2 * kS], v23[2 * kS];
#pragma unroll
  for (int mm = 0; mm < kS; ++mm) {
    const v2i32_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32_ptr_t)(kt + voff[mm]));
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      v01[2 * mm + u] = widen_pair<BF16, false>((uint32_t)x[u]);
      v23[2 * mm + u] = widen_pair<BF16, true>((uint32_t)x[u]);
    }
  }
  tile_math<BF16, D>(st, ka, v01, v23, qb, tok_row0, tw1, partial, c);
}

// Block id number idx (< 256, wave-uniform) of the wave's range.
__device__ __forceinline__ int pick_id(const int (&ids)[kIdRegs], int idx) {
  const int l = idx & 63;
  const int c = idx >> 6;
  int r = __builtin_amdgcn_readlane(ids[0], l);
#pragma unroll
  for (int i = 1; i < kIdRegs; ++i) {
    const int x = __builtin_amdgcn_readlane(ids[i], l);
    r = c == i ? x : r;
  }
  return r;
}

// Four consecutive output elements, rounded to the dtype (8 bytes).
template <bool BF16>
__device__ __forceinline__ void store4(uint16_t* o, f32x4 r, float inv) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  *(u32x2*)o = u32x2{pack2<BF16>(r[0] * inv, r[1] * inv), pack2<BF16>(r[2] * inv, r[3] * inv)};
}

// Lane ownership of the results: lane l (column u = l%16, rows 4(l/16)..+4
// of each 16-dim block) speaks for query head u % G. Every head has 16 / G
// column copies; the first `copies` of them (a power of
// two, at most D/16) split the head's D/16 dim blocks into runs of nown =
// (D/16) / copies, copy q taking blocks [q nown, (q+1) nown), so each (head,
// dim) is written by exactly one lane. Kernels built FAST (G <= 4) use four
// copies, so nown = D/64 is known when compiling and the epilogue is
// straight-line code.
struct Owner {
  int head;  // query head of the KV head, < G
  int copy;  // u / G
  int nown;  // dim blocks per owning lane
  bool active;
  __device__ int block(int k) const { return copy * nown + k; }
};

template <bool FAST>
__device__ __forceinline__ Owner make_owner(int u, int G, int kM) {
  int p2 = 4;
  if constexpr (!FAST) {
    const int copies = 16 / G;
    p2 = 1;
    while (2 * p2 <= copies && 2 * p2 <= kM) p2 *= 2;
  }
  Owner o;
  o.head = u % G;
  o.copy = u / G;
  o.nown = kM / p2;
  o.active = o.copy < p2;
  return o;
}

// The arguments the first loads depend on come first and on their own, so
// that they can arrive preloaded in scalar registers (the library is built
// with kernel-argument preloading); the rest are read from the argument
// segment.
template <bool BF16, int BS, bool SPLIT, int NW, bool KV8, int D, bool FAST>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
void pd_decode_kernel(const int32_t* __restrict__ bt_arg, const int32_t* __restrict__ cl_arg,
                      const uint16_t* __restrict__ q_arg, int32_t MB, int32_t P_arg,
                      int32_t Pw_arg, int32_t G_arg, int32_t geo, const KArgs a) {
  using Gm = Geo<D>;
  constexpr int kS = Gm::kSteps, kM = Gm::kBlocks;
  constexpr int kOwn = FAST ? kM / 4 : kM;  // most dim blocks a lane owns
  constexpr int kNBuf = tile_buffers<D, KV8>(NW);
  using G8 = Geo8<D>;
  constexpr int kLoads = KV8 ? 2 * G8::kGroups : 2 * Gm::kGroups;  // load instructions per tile
  constexpr int kWaitTile = waitcnt_vm((kNBuf - 1) * kLoads);
  constexpr uint32_t kStage = stage_bytes<D, KV8>();
  // one array per tile buffer, so the compiler can wait for exactly the
  // loads of the buffer about to be read
  // the first also holds the slice merge's scratch after the loop
  __shared__ __align__(16) char lds0[NW * (kStage > merge_bytes<D>() ? kStage : merge_bytes<D>())];
  __shared__ __align__(16) char lds1[NW * kStage];
  __shared__ __align__(16) char lds2[kNBuf > 2 ? NW * kStage : 16];
  // grid (head group, sequence, partition), x fastest: the partitions of a
  // head group are B * groups workgroups apart, so with the usual multiple
  // of 8 head groups per partition they share one XCD (workgroups are dealt
  // to the 8 XCDs in turn) and every XCD gets an even share of every
  // sequence's heads
  const int hg = blockIdx.x;
  const int b = blockIdx.y;
  const int p = blockIdx.z;
  const int G = G_arg;
  // the geometry the first loads' addresses need, from a preloaded argument:
  // NH (bits 0-3), HS (bits 4-11), physical KV heads (bits 12-31)
  const int NH = geo & 15, HS = (geo >> 4) & 255, Hkv_phys = geo >> 12;
  const int Hq = Hkv_phys * HS * G;
  const int nw = NH * a.NT;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = w % NH;  // KV head within the workgroup's group
  const int ts = w / NH;  // token slice
  const int g = hg * NH + hl;  // virtual KV head
  const int gk = g / HS;        // the physical KV head it reads
  const int row = lane >> 4;
  auto tile_buf = [&](int d) -> char* {
    char* base = d == 0 ? lds0 : d == 1 ? lds1 : lds2;
    return base + w * kStage;
  };

  const int t0 = p * P_arg;
  const int tw0 = t0 + ts * Pw_arg;
  const int bi0 = tw0 / BS;
  // q as the MFMA B operand: column lane%16 -> head (lane%16) % G, dims
  // 32s + 8(lane/16) .. +8. Loaded before the block ids, so that waiting for
  // the ids (which the first K/V addresses need) also covers q, and no later
  // wait has to drain the tile loads.
  u32x4 qb[kS];
  {
    const int hc = (lane & 15) % G;
    const uint16_t* qp = q_arg + ((size_t)b * Hq + (size_t)g * G + hc) * D + 8 * row;
#pragma unroll
    for (int s = 0; s < kS; ++s) qb[s] = *(const u32x4*)(qp + 32 * s);
  }
  // block ids of the wave's whole slice, fetched before the context length
  // is known (entries past the live ones are loaded but never used)
  const int nb_max = min(Pw_arg / BS, MB - bi0);
  const int32_t* btrow = bt_arg + (size_t)b * MB + bi0;
  int ids[kIdRegs];
#pragma unroll
  for (int i = 0; i < kIdRegs; ++i) ids[i] = 64 * i + lane < nb_max ? btrow[64 * i + lane] : 0;

  WaveState<D> st;
  st.lsum = 0.f;
  st.m = -INFINITY;
#pragma unroll
  for (int m = 0; m < kM; ++m) st.acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  // wave-uniform by construction; readfirstlane lets the compiler keep the
  // loop bounds and block addresses in scalar registers. A length past the
  // row's MB blocks counts as MB blocks (a negative one is an empty context).
  const int L = min(__builtin_amdgcn_readfirstlane(cl_arg[b]), MB * BS);
  if constexpr (!SPLIT) {
    if (L <= 0) {
      // empty context: zero rows for every query head of the group
      uint16_t* o = (uint16_t*)a.out + ((size_t)b * Hq + (size_t)hg * NH * G) * D;
      for (int i = threadIdx.x; i < NH * G * D / 8; i += nw * 64)
        *(u32x4*)(o + i * 8) = u32x4{0u, 0u, 0u, 0u};
      return;
    }
  } else {
    // an empty partition publishes nothing: the merge reads partitions
    // 0 .. ceil(L / P) - 1 only, and writes the zero rows of an empty context
    if (t0 >= L) return;
  }
  const int tw1 = min(min(tw0 + Pw_arg, t0 + P_arg), L);
  const int nst = __builtin_amdgcn_readfirstlane(
      tw0 < tw1 ? (tw1 - tw0 + kTileTok - 1) / kTileTok : 0);
  const float c = a.scale_log2;
  constexpr uint32_t kRow = KV8 ? G8::kRowBytes : Gm::kRowBytes;
  constexpr int kChunks = KV8 ? G8::kChunks : Gm::kChunks;  // 16-byte chunks per row as loaded
  const uint32_t tok_bytes = Hkv_phys * kRow;  // a token row: every physical KV head
  // global offsets of this lane's 16 bytes in load instruction 0 of a tile:
  // a row takes C lanes (64 / C rows per instruction), the chunks in the
  // rotated order of the tile layouts above
  const int lrow = lane / kChunks;
  const int lsl = lane % kChunks;
  const uint32_t head_off = (uint32_t)lrow * tok_bytes + (uint32_t)gk * kRow;
  const uint32_t koff_g =
      head_off + (uint32_t)(KV8 ? (lsl - G8::rot(lrow) + kChunks) % kChunks
                                : (lsl - lrow + kChunks) % kChunks) *
                     16u;
  const uint32_t voff_g =
      head_off + (uint32_t)(KV8 ? (lsl - G8::rot(lrow) + kChunks) % kChunks
                                : (lsl - 2 * lrow + 2 * kChunks) % kChunks) *
                     16u;
  // LDS offsets of the two read patterns (see the tile layouts above)
  uint32_t koff[kS], voff[kM];
  uint32_t koff8[kS], voff8[kS];  // FP8 tiles
  if constexpr (KV8) {
    constexpr int R8 = G8::kRowsPerLoad;
    auto at = [](int t, int chunk, int half) -> uint32_t {
      return (uint32_t)(t / R8) * G8::kGroup + (uint32_t)(t % R8) * G8::kRowBytes +
             16u * (uint32_t)((chunk + G8::rot(t % R8)) % G8::kChunks) + 8u * (uint32_t)half;
    };
#pragma unroll
    for (int s = 0; s < kS; ++s) koff8[s] = at(lane & 15, 2 * s + (row >> 1), row & 1);
    const int j = lane & 15, a8 = j & 1, k8 = j >> 1;
#pragma unroll
    for (int mm = 0; mm < kS; ++mm)
      voff8[mm] = G8::kKTile + at(4 * row + (k8 & 3), 2 * mm + (k8 >> 2), a8);
  }
  {
    constexpr int C = Gm::kChunks, R = Gm::kRowsPerLoad;
    const int t = lane & 15, r = t % R;
#pragma unroll
    for (int s = 0; s < kS; ++s)
      koff[s] = (uint32_t)(t / R) * Gm::kKGroup + (uint32_t)r * Gm::kRowBytes +
                16u * (uint32_t)((4 * s + row + r) % C);
    // source lane of the transposing read: token 4(lane/16) + (lane%16)/4,
    // dims 16m + 4(lane%4) .. +4, i.e. chunk 2m + (lane%4)/2, half lane%2
    const int tt = 4 * row + ((lane & 15) >> 2), a4 = lane & 3, rr = tt % R;
#pragma unroll
    for (int m = 0; m < kM; ++m)
      voff[m] = Gm::kKTile + (uint32_t)(tt / R) * Gm::kVGroup + (uint32_t)rr * Gm::kRowBytes +
                16u * (uint32_t)((2 * m + (a4 >> 1) + 2 * rr) % C) + 8u * (uint32_t)(a4 & 1);
  }

  // Queue the loads of tile j into buffer d. Straight-line, always kLoads
  // loads, so the wait counts stay exact: past the slice (j >= nst) every
  // lane's token is >= tw1 and its offset is out of the block, and the block
  // id is forced to 0, so those loads read nothing.
  auto issue = [&](int j, int d) {
    const int tok = kTileTok * j;  // offset in the slice
    const int idx = min(tok / BS, kIdRegs * 64 - 1);
    const int id = pick_id(ids, idx) * (int)(j < nst);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + (int64_t)id * a.blk_bytes, a.blk_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + (int64_t)id * a.blk_bytes, a.blk_bytes);
    const uint32_t tb = (uint32_t)(tok % BS) * tok_bytes;
    char* kt = tile_buf(d);
    constexpr int kRowsPerLoad = 64 / kChunks;
#pragma unroll
    for (int n = 0; n < kLoads / 2; ++n) {
      const bool ok = tw0 + tok + kRowsPerLoad * n + lrow < tw1;
      const uint32_t nb = tb + (uint32_t)(kRowsPerLoad * n) * tok_bytes;
      uint32_t ko = ok ? nb + koff_g : kOutOfBlock;
      uint32_t vo = ok ? nb + voff_g : kOutOfBlock;
      // the offsets are plain register values to the optimizer, so it cannot
      // turn the selects into a divergent branch around the loads (which
      // would issue a load twice and break the exact wait counts)
      asm("" : "+v"(ko), "+v"(vo));
      const uint32_t kd = KV8 ? n * G8::kGroup : n * Gm::kKGroup;
      const uint32_t vd = KV8 ? G8::kKTile + n * G8::kGroup : Gm::kKTile + n * Gm::kVGroup;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(kt + kd), 16, ko, 0, 0, kStream);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(kt + vd), 16, vo, 0, 0, kStream);
    }
  };

  // The loads leave in tile order, in the prologue as in the loop, so that
  // the wait for tile j never has to drain the later tiles.
#pragma unroll
  for (int d = 0; d < kNBuf; ++d) {
    issue(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int j0 = 0; j0 < nst; j0 += kNBuf) {
#pragma unroll
    for (int d = 0; d < kNBuf; ++d) {
      const int j = j0 + d;
      // tile j's loads are the oldest in flight: wait until only the later
      // tiles' (kNBuf - 1) * kLoads loads are outstanding. Explicit, because
      // the compiler does not always see that these LDS reads depend on them.
      __builtin_amdgcn_s_waitcnt(kWaitTile);
      __builtin_amdgcn_sched_barrier(0);
      // Before a buffer is refilled every LDS read of it has completed: the
      // refill's LDS writes are not ordered after reads still in flight, and
      // a refill past the slice reads no memory, so it lands at once.
      if (j < nst) {
        const int tile0 = tw0 + kTileTok * j;
        if constexpr (KV8)
          tile_compute_fp8<BF16, D>(st, tile_buf(d), qb, koff8, voff8, tile0 + 4 * row, tw1,
                                 tile0 + kTileTok > tw1, c);
        else
          tile_compute<BF16, D>(st, tile_buf(d), qb, koff, voff, tile0 + 4 * row, tw1,
                                tile0 + kTileTok > tw1, c);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitLds);
      __builtin_amdgcn_sched_barrier(0);
      issue(j + kNBuf, d);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // every tile load (the trailing ones read nothing) has landed before the
  // tile buffers are reused below
  __builtin_amdgcn_s_waitcnt(0);

  // ---- the lane's head, its owned dim blocks gathered into o[0..nown),
  // running maximum and weight sum
  const Owner own = make_owner<FAST>(lane & 15, G, kM);
  f32x4 o[kOwn];
#pragma unroll
  for (int k = 0; k < kOwn; ++k) {
    o[k] = st.acc[k];
    if constexpr (FAST) {
#pragma unroll
      for (int q = 1; q < 4; ++q)
        if (own.copy == q) o[k] = st.acc[q * kOwn + k];
    } else {
#pragma unroll
      for (int m = k + 1; m < kM; ++m)
        if (m == own.block(k)) o[k] = st.acc[m];
    }
  }
  float m_r = st.m;
  float l_r = sum_rows(st.lsum);
  const int h = own.head;
  const int nown = FAST ? kOwn : own.nown;
  const int d0 = 16 * own.block(0) + 4 * row;  // first owned dim; runs of 4 every 16

  // ---- merge the NT slices of each head through LDS (the first tile
  // buffer, sized to hold G * (D + 2) floats per wave as G <= 16): every
  // wave writes its slice's sums, then all the workgroup's waves share the
  // merge, one thread per (KV head of the group, query head, 4 dims), each
  // combining the NT slices in order i = 0..NT-1, and store the result
  if (a.NT > 1) {
    __syncthreads();  // every wave is done with its tile buffers
    float* s_acc = (float*)lds0;                 // [(w*G + h)*D + dim]
    float* s_m = s_acc + nw * G * D;             // [w*G + h]
    float* s_l = s_m + nw * G;
    if (own.active) {
#pragma unroll
      for (int k = 0; k < kOwn; ++k)
        if (k < nown) *(f32x4*)(s_acc + (w * G + h) * D + d0 + 16 * k) = o[k];
      if (row == 0 && own.copy == 0) {
        s_m[w * G + h] = m_r;
        s_l[w * G + h] = l_r;
      }
    }
    __syncthreads();
    constexpr int kD4 = D / 4;
    const int units = NH * G * kD4;
    // the head group's rows of the partial buffers (split calls only)
    const size_t gslot0 = ((size_t)b * Hq + (size_t)hg * NH * G) * a.S;
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(SPLIT ? a.o_part + gslot0 * D : nullptr,
                  SPLIT ? (uint32_t)(NH * G) * a.S * D * 4 : 0u);
    const __amdgpu_buffer_rsrc_t rl =
        make_rsrc(SPLIT ? a.lse_part + gslot0 : nullptr, SPLIT ? (uint32_t)(NH * G) * a.S * 4 : 0u);
    for (int u = threadIdx.x; u < units; u += nw * 64) {
      const int uh = u / kD4;  // hl * G + h: the group's query head
      const int d4 = u - uh * kD4;
      const int uhl = uh / G, uhh = uh - uhl * G;
      float M = -INFINITY;
      for (int i = 0; i < a.NT; ++i) M = fmaxf(M, s_m[(i * NH + uhl) * G + uhh]);
      float den = 0.f;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int i = 0; i < a.NT; ++i) {
        const int wi = (i * NH + uhl) * G + uhh;
        const float wt = exp2_fast(s_m[wi] - M);  // 0 for a slice with no tokens
        den = fmaf(wt, s_l[wi], den);
        const f32x4 x = *(const f32x4*)(s_acc + wi * D + 4 * d4);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(wt, x[e], acc[e]);
      }
      if constexpr (!SPLIT) {
        uint16_t* op = (uint16_t*)a.out + ((size_t)b * Hq + (size_t)hg * NH * G + uh) * D + 4 * d4;
        store4<BF16>(op, acc, a.out_scale / den);
      } else {
        // this partition's (o_p, lse_p), write-through; the raw buffer
        // builtins move 32-bit words, so floats go through bit casts
        const uint32_t row_off = (uint32_t)(uh * a.S + p);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc * (1.0f / den)), ro,
                                               (row_off * D + 4 * d4) * 4, 0, kCoherent);
        if (d4 == 0)
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(uint32_t, M + __builtin_amdgcn_logf(den) -
                                               WeightBias<BF16>::log2),
              rl, row_off * 4, 0, kCoherent);
      }
    }
    return;
  }

  // ---- one slice per head: the lanes that own the results store them
  if (!own.active) return;
  if constexpr (!SPLIT) {
    uint16_t* op = (uint16_t*)a.out + ((size_t)b * Hq + (size_t)g * G + h) * D + d0;
    const float inv = a.out_scale / l_r;
#pragma unroll
    for (int k = 0; k < kOwn; ++k)
      if (k < nown) store4<BF16>(op + 16 * k, o[k], inv);
  } else {
    // ---- publish this partition's (o_p, lse_p), write-through
    const size_t slot0 = ((size_t)b * Hq + (size_t)g * G) * a.S;  // (head 0, partition 0)
    const uint32_t rows_bytes = (uint32_t)G * a.S * D * 4;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o_part + slot0 * D, rows_bytes);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lse_part + slot0, (uint32_t)G * a.S * 4);
    // the raw buffer builtins move 32-bit words: floats go through bit casts
    const float inv = 1.0f / l_r;
    const uint32_t off = ((uint32_t)(h * a.S + p) * D + d0) * 4;
#pragma unroll
    for (int k = 0; k < kOwn; ++k)
      if (k < nown)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[k] * inv), ro,
                                               off + 64 * k, 0, kCoherent);
    if (row == 0 && own.copy == 0)
      __builtin_amdgcn_raw_buffer_store_b32(
          __builtin_bit_cast(uint32_t, m_r + __builtin_amdgcn_logf(l_r) -
                                           WeightBias<BF16>::log2),
          rl, (uint32_t)(h * a.S + p) * 4, 0, kCoherent);
  }
}

// Zero a workspace (paged_decode_workspace_init; the decode itself needs no
// zeroed memory).
__global__ void pd_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The LSE merge of a split call, queued after the decode kernel on the same
// stream: one wave per (query head, sequence) of a (Hq, B) grid, lane l holding dims
// [l * D/64, (l + 1) * D/64) of the head, the n = ceil(L / P) non-empty
// partitions merged in order p = 0 .. n-1 in batches of KB loads (an
// empty context writes a zero row); the first batch is loaded beside the
// context length rather than after it. A merge spread over B * Hq waves reads
// the partials at the whole GPU's rate; merging in the workgroup that
// finishes a head group last was slower on every split shape measured.
template <bool BF16, int D, int KB>
__global__ __launch_bounds__(64) void pd_merge_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      const int32_t* __restrict__ cl,
                                                      uint16_t* __restrict__ out, int32_t Hq,
                                                      int32_t S, int32_t P, int32_t cap,
                                                      float out_scale) {
  constexpr int kDl = D / 64;  // dims per lane
  constexpr int kBatch = KB;  // S <= KB (one batch) unless KB = 16
  const int b = blockIdx.y;
  const size_t bh = (size_t)b * Hq + blockIdx.x;  // (sequence, query head)
  const int lane = threadIdx.x;
  const int L_arg = __builtin_amdgcn_readfirstlane(cl[b]);
  const float* orow = o_part + bh * S * D + lane * kDl;
  const float* lrow = lse_part + bh * S;
  // Every load of a batch is issued before any is used. Row i of a batch
  // reads partition min(i, last) (inside the call's rows), so no load waits
  // alone inside a branch.
  float x[kBatch][kDl], lse[kBatch];
  auto load_batch = [&](int i0, int last) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = min(i0 + u, last);
      lse[u] = lrow[i];
      const float* r = orow + (size_t)i * D;
      if constexpr (kDl == 2) {
        const float2 v2 = *(const float2*)r;
        x[u][0] = v2.x;
        x[u][1] = v2.y;
      } else {
        x[u][0] = r[0];
      }
    }
  };
  // The first batch goes out together with the length, over all S rows:
  // rows of partitions past the live ones hold whatever an earlier call
  // left (or nothing written yet) and are excluded by selects below, never
  // multiplied in.
  // (An empty context runs the same code with n = 0 and stores a zero row
  // by a select at the end: a branch on the length here would let the
  // compiler sink these loads behind the length's arrival.)
  load_batch(0, S - 1);
  const int L = min(L_arg, cap);
  const int n = L > 0 ? (L + P - 1) / P : 0;
  float M = -INFINITY, den = 0.f, acc[kDl];
#pragma unroll
  for (int e = 0; e < kDl; ++e) acc[e] = 0.f;
  for (int i0 = 0;;) {
    float bm = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) bm = fmaxf(bm, i0 + u < n ? lse[u] : -INFINITY);
    const float alpha = exp2_fast(M - bm);  // 0 on the first batch
    den *= alpha;
#pragma unroll
    for (int e = 0; e < kDl; ++e) acc[e] *= alpha;
    M = bm;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool live = i0 + u < n;
      const float wt = live ? exp2_fast(lse[u] - M) : 0.f;
      den += wt;
#pragma unroll
      for (int e = 0; e < kDl; ++e) acc[e] = live ? fmaf(wt, x[u][e], acc[e]) : acc[e];
    }
    i0 += kBatch;
    if (i0 >= n) break;
    load_batch(i0, n - 1);
  }
  const float inv = out_scale / den;
  uint16_t* op = out + bh * D + lane * kDl;
#pragma unroll
  for (int e = 0; e < kDl; ++e) op[e] = n > 0 ? to_bits<BF16>(acc[e] * inv) : (uint16_t)0;
}

// The merge instance for a call: the batch is the smallest of 4, 8 and 16
// loads that holds S rows (16 for more), so no load repeats a row in vain.
template <bool BF16, int D>
const void* pick_merge_batch(int S) {
  return S <= 4   ? (const void*)&pd_merge_kernel<BF16, D, 4>
         : S <= 8 ? (const void*)&pd_merge_kernel<BF16, D, 8>
                  : (const void*)&pd_merge_kernel<BF16, D, 16>;
}

const void* pick_merge(bool bf16, int D, int S) {
  if (bf16) return D == 64 ? pick_merge_batch<true, 64>(S) : pick_merge_batch<true, 128>(S);
  return D == 64 ? pick_merge_batch<false, 64>(S) : pick_merge_batch<false, 128>(S);
}

template <bool BF16, int BS, bool SPLIT, bool KV8, int D, bool FAST>
hipError_t launch_decode(const KArgs& ka, dim3 grid, int nw, hipStream_t st) {
  const int32_t* bt = ka.bt;
  const int32_t* cl = ka.cl;
  const uint16_t* q = ka.q;
  int32_t mb = ka.MB, p = ka.P, pw = ka.Pw, g = ka.G;
  int32_t geo = ka.NH | (ka.HS << 4) | ((ka.Hkv / ka.HS) << 12);
  void* args[] = {(void*)&bt, (void*)&cl, (void*)&q, (void*)&mb, (void*)&p, (void*)&pw,
                  (void*)&g, (void*)&geo, (void*)&ka};
  // the LDS tile buffers are sized for the largest workgroup of the instance
  const void* f = nw <= 4
      ? (const void*)&pd_decode_kernel<BF16, BS, SPLIT, 4, KV8, D, FAST>
      : (const void*)&pd_decode_kernel<BF16, BS, SPLIT, 8, KV8, D, FAST>;
  return hipLaunchKernel(f, grid, dim3(nw * 64), args, 0, st);
}

template <bool BF16, bool SPLIT, bool KV8, int D, bool FAST>
hipError_t pick_block(const KArgs& ka, dim3 grid, int bs, int nw, hipStream_t st) {
  return bs == 32 ? launch_decode<BF16, 32, SPLIT, KV8, D, FAST>(ka, grid, nw, st)
                  : launch_decode<BF16, 16, SPLIT, KV8, D, FAST>(ka, grid, nw, st);
}

template <bool KV8, int D, bool FAST>
hipError_t pick_dtype(const KArgs& ka, dim3 grid, int bs, int nw, bool bf16, bool split,
                      hipStream_t st) {
  if (bf16)
    return split ? pick_block<true, true, KV8, D, FAST>(ka, grid, bs, nw, st)
                 : pick_block<true, false, KV8, D, FAST>(ka, grid, bs, nw, st);
  return split ? pick_block<false, true, KV8, D, FAST>(ka, grid, bs, nw, st)
               : pick_block<false, false, KV8, D, FAST>(ka, grid, bs, nw, st);
}

// Instances: D = 64 and 128 for 16-bit and for FP8 caches; each with a
// compile-time epilogue for G <= 4 query heads per virtual KV head (FAST)
// and a general one.
hipError_t pick_geometry(const KArgs& ka, dim3 grid, int bs, int nw, bool bf16, bool split,
                         bool kv8, int D, hipStream_t st) {
  const bool fast = ka.G <= 4;
  if (kv8 && D == 64)
    return fast ? pick_dtype<true, 64, true>(ka, grid, bs, nw, bf16, split, st)
                : pick_dtype<true, 64, false>(ka, grid, bs, nw, bf16, split, st);
  if (kv8)
    return fast ? pick_dtype<true, 128, true>(ka, grid, bs, nw, bf16, split, st)
                : pick_dtype<true, 128, false>(ka, grid, bs, nw, bf16, split, st);
  if (D == 64)
    return fast ? pick_dtype<false, 64, true>(ka, grid, bs, nw, bf16, split, st)
                : pick_dtype<false, 64, false>(ka, grid, bs, nw, bf16, split, st);
  return fast ? pick_dtype<false, 128, true>(ka, grid, bs, nw, bf16, split, st)
              : pick_dtype<false, 128, false>(ka, grid, bs, nw, bf16, split, st);
}

}  // namespace

namespace pd {

int32_t launch(const Launch& l) {
  KArgs ka;
  ka.q = (const uint16_t*)l.q;
  ka.k = (const char*)l.k_cache;
  ka.v = (const char*)l.v_cache;
  ka.bt = l.block_table;
  ka.cl = l.context_lens;
  ka.out = l.out;
  ka.o_part = nullptr;
  ka.lse_part = nullptr;
  if (l.plan.splits > 1) {
    char* ws = (char*)l.workspace;
    ka.o_part = (float*)ws;
    ka.lse_part = (float*)(ws + partials_bytes(l.shape, l.plan));
  }
  const int hs = l.plan.head_split;
  ka.Hkv = l.shape.Hkv * hs;
  ka.HS = hs;
  ka.G = l.shape.Hq / ka.Hkv;
  ka.MB = l.shape.max_blocks_per_seq;
  ka.S = l.plan.splits;
  ka.P = l.plan.partition_tokens;
  ka.Pw = l.plan.wave_tokens;
  ka.NH = l.plan.heads_per_group;
  ka.NT = l.plan.slices;
  ka.groups = ka.Hkv / l.plan.heads_per_group;
  ka.scale_log2 = l.scale * 1.4426950408889634f * (l.kv_fp8 ? l.k_scale : 1.0f);
  ka.out_scale = l.kv_fp8 ? l.v_scale : 1.0f;
  ka.blk_bytes = (uint32_t)l.shape.block_size * (uint32_t)l.shape.Hkv *
                 (l.kv_fp8 ? 1u : 2u) * (uint32_t)l.shape.D;
  const dim3 grid((unsigned)ka.groups, (unsigned)l.shape.B, (unsigned)l.plan.splits);
  const int nw = l.plan.heads_per_group * l.plan.slices;
  // each wave owns a tile's bytes of every tile buffer of its workgroup; the
  // slice merge needs G * (D + 2) floats of them per wave, so G <= 16
  // (NH, HS and the physical KV heads travel packed in one argument)
  if (nw < 1 || nw > kMaxWaves || hs < 1 || hs > 255 || l.plan.heads_per_group > 15 ||
      l.shape.Hkv >= (1 << 19) || ka.Hkv % l.plan.heads_per_group != 0 ||
      ka.G * ka.Hkv != l.shape.Hq || ka.G > 16 || (l.shape.D != 64 && l.shape.D != 128))
    return PD_ERR_INTERNAL;
  hipStream_t st = (hipStream_t)l.stream;
  const bool split = l.plan.splits > 1;
  const bool bf16 = l.shape.dtype == PD_DTYPE_BF16;
  hipError_t e = pick_geometry(ka, grid, l.shape.block_size, nw, bf16, split, l.kv_fp8,
                               l.shape.D, st);
  if (e == hipSuccess && split) {
    int32_t hq = l.shape.Hq, S = ka.S, P = ka.P, cap = ka.MB * l.shape.block_size;
    float osc = ka.out_scale;
    const float* op = ka.o_part;
    const float* lp = ka.lse_part;
    const int32_t* cl = ka.cl;
    uint16_t* out = (uint16_t*)ka.out;
    void* margs[] = {(void*)&op, (void*)&lp, (void*)&cl, (void*)&out, (void*)&hq,
                     (void*)&S,  (void*)&P,  (void*)&cap, (void*)&osc};
    const void* mf = pick_merge(bf16, l.shape.D, S);
    e = hipLaunchKernel(mf, dim3((unsigned)l.shape.Hq, (unsigned)l.shape.B), dim3(64), margs, 0,
                        st);
  }
  return e == hipSuccess ? PD_OK : PD_ERR_HIP;
}

int32_t zero_workspace(void* ws, size_t bytes, void* stream) {
  const size_t n = bytes / 4;
  if (n == 0) return PD_OK;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  uint32_t* p = (uint32_t*)ws;
  size_t nn = n;
  void* args[] = {(void*)&p, (void*)&nn};
  hipError_t e = hipLaunchKernel((const void*)&pd_zero_kernel, dim3((unsigned)blocks), dim3(256),
                                 args, 0, (hipStream_t)stream);
  return e == hipSuccess ? PD_OK : PD_ERR_HIP;
}

}  // namespace pd
