// Paged GQA decode attention kernel for gfx950 (CDNA4, wave64).
//
// Method (Loom Kernels home page, "Supported now": paged MQA/GQA decode with
// GQA packing and local split-K/LSE): one query token per head attends over
// a paged K/V cache; the 4 query heads that share a KV head are served by one
// pass over that head's K/V bytes, and a long context is cut into
// partitions whose normalised partial outputs and log-sum-exps are merged.
//
// One kernel. Workgroup (partition p, KV-head group hg, sequence b) has
// NH x NT wave64s: wave w serves KV head hg*NH + w%NH over token slice w/NH
// of the partition (a block-aligned range of at most 256 blocks). Waves of
// the same slice read the same physical blocks, so a workgroup sweeps whole
// blocks (all heads of a token are one contiguous 2 KiB row group) rather
// than 256-byte slivers of them.
//   * K/V move in tiles of 16 tokens from HBM straight into LDS with
//     bounds-checked buffer loads whose resource is the current physical
//     block (base = pool + id * block bytes, size = block bytes), so an
//     access cannot leave the block; lanes past the context get an offset
//     beyond the block and read nothing. Each 128-bit load instruction of a
//     wave reads four whole 256-byte rows. One or two tiles stay in flight
//     while the oldest is computed; the loads use the streaming (nt) cache
//     policy since every K/V byte is read once.
//   * block ids: each lane loads up to four block-table entries of the
//     wave's range before the context length is known; a tile takes its
//     (wave-uniform) id with v_readlane, so addresses are scalar.
//   * scores: q . k for the 16 tokens of a tile and the 4 query heads of the
//     KV head are one 16x16 output of four v_mfma_f32_16x16x32 (bf16 or
//     f16 inputs, exact products, fp32 sums), read from LDS in the operand
//     order; one multiply by scale*log2(e) puts the softmax in base 2
//     (v_exp_f32).
//   * softmax: per head, a running maximum that only moves when a ballot
//     finds a tile maximum above it (then the accumulators are rescaled);
//     each lane keeps its own partial sum of weights.
//   * PV: fp32 FMA of each weight with the 16-bit V values widened exactly,
//     acc[4 heads][8 dims] per lane.
//   * end of slice: a reduce-scatter over the 4 rows (permlane32_swap, then
//     permlane16_swap) leaves query head r's 128 sums in row r; the NT slices
//     of a head are merged through LDS.
//   * S == 1: the workgroup writes `out`, rounded to the dtype.
//   * S > 1: the workgroup writes its fp32 partial output and log2-sum-exp
//     with write-through (device-coherent) stores, then bumps a per
//     (sequence, head group) counter; the workgroup that brings it to the
//     number of non-empty partitions merges them in fixed order p = 0..n-1
//     with L2-bypassing loads, writes `out` and resets the counter to zero.
//     No device-wide cache flush is involved.
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

constexpr int D = pd::kHeadDim;  // 128
constexpr int G = pd::kGroup;    // 4
constexpr int kIdRegs = pd::kMaxWaveBlocks / 64;  // block ids per lane
constexpr uint32_t kRowBytes = D * 2;          // one token row of one KV head (16-bit)
constexpr uint32_t kRowBytes8 = D;             // the same row of an FP8 cache
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
  int32_t* counters;  // [B, Hkv / NH], at the start of the workspace
  int32_t Hkv;
  int32_t MB;
  int32_t S;
  int32_t P;
  int32_t Pw;  // tokens per slice, a multiple of the block size, <= 256 blocks
  int32_t NH;  // KV heads per workgroup
  int32_t NT;  // token slices per workgroup
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
// loads with the LDS destination, no VGPRs held while in flight). Within a
// tile, load instruction n moves tokens 4n..4n+3: lane (row, sl) reads 16
// bytes of token 4n + row, so every 16 lanes read one whole 256-byte row.
// Which 16-byte chunk a lane takes is rotated per row, and the four 1 KiB
// groups of a tile are padded apart, so that the LDS reads below touch
// distinct bank groups:
//   K: lane sl takes chunk (sl - row) mod 16, groups 1088 bytes apart; read
//      back 16 bytes per lane in MFMA operand order (token lane%16, chunk
//      4s + lane/16): any 16 (and any 8 consecutive) lanes hit distinct
//      16-byte bank groups;
//   V: lane sl takes chunk (sl - 2 row) mod 16, groups 1152 bytes apart;
//      read back with the transposing ds_read_b64_tr_b16, 8 bytes per lane
//      (token 4(lane/16) + (lane%16)/4, dims 4(lane%4) of a 16-dim block):
//      each 32 lanes hit distinct 8-byte bank slots.
constexpr int kTileTok = 16;
constexpr uint32_t kKGroup = 4 * kRowBytes + 64;
constexpr uint32_t kVGroup = 4 * kRowBytes + 128;
constexpr uint32_t kKTile = 4 * kKGroup;             // 4352
constexpr uint32_t kLdsTile = kKTile + 4 * kVGroup;  // K then V: 8960
// An FP8 cache lands in a plain staging tile (16 rows of 128 bytes for K,
// then for V) and is converted into the 16-bit layout above before use.
constexpr uint32_t kStage8 = 2 * kTileTok * kRowBytes8;  // 4096

// Tile buffers per wave (tiles in flight while one is computed: buffers - 1),
// as many as fit the 160 KiB of LDS for the workgroup size, up to PD_NBUF.
#ifndef PD_NBUF
#define PD_NBUF 2
#endif
constexpr uint32_t kLdsBytes = 160 * 1024;
template <bool KV8>
constexpr uint32_t stage_bytes() { return KV8 ? kStage8 : kLdsTile; }
template <bool KV8>
constexpr int tile_buffers(int nw) {
  return PD_NBUF >= 3 && 3 * nw * stage_bytes<KV8>() + (KV8 ? nw * kLdsTile : 0) <= kLdsBytes
             ? 3 : 2;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
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
  u32x4 hi_lo;   // k 0..3: hi of the lane's 4 tokens, k 4..7: lo
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
};

// Per-lane state of one wave's online softmax over its token slice. Lane l
// follows query head l%4 of the KV head; acc[m][i] is its unnormalised PV
// sum for dim 16m + 4(l/16) + i (the four lane quads of a row hold copies).
struct WaveState {
  f32x4 acc[8];
  float lsum;  // sum of weights over the tokens of this lane's row
  float m;     // running maximum (log2 domain)
};

// One 16-token tile, already in LDS at kt (K) and kt + kKTile (V).
//   scores: the K tile is the A operand of four 16x16x32 MFMAs (row = token
//     lane%16, k = dims 32s + 8(lane/16) .. +8), q the B operand (column =
//     lane%16 -> query head (lane%16)%4, the 4 heads repeated 4 times): lane
//     l gets the scores of tokens 4(l/16) + i, i < 4, for head l%4;
//   softmax: the tile maximum per head (4 registers, then the 4 rows); the
//     running maximum only moves when a ballot finds a tile maximum above it;
//   PV: per 16-dim block, one 16x16x32 MFMA with A = V^T (row = dim, k = the
//     lane's 4 tokens, twice) and B = those tokens' weights (hi in k 0..3,
//     lo in k 4..7), which is the layout the scores came out in; for bf16 a
//     second one adds the third weight term.
template <bool BF16>
__device__ __forceinline__ void tile_compute(WaveState& st, const char* kt,
                                             const u32x4 (&qb)[4], const uint32_t (&koff)[4],
                                             const uint32_t (&voff)[8], int tok_row0, int tw1,
                                             bool partial, float c) {
  u32x4 ka[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) ka[s] = *(const u32x4*)(kt + koff[s]);
  v4i16_t vt[8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
    vt[m] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr_t)(kt + voff[m]));
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) sc = mfma_16x16x32<BF16>(ka[s], qb[s], sc);
  float s_[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s_[i] = sc[i] * c;
  if (partial) {
    // tokens past the slice get no weight, and their V rows (whatever the
    // LDS holds there) are replaced by zeros
#pragma unroll
    for (int i = 0; i < 4; ++i) s_[i] = tok_row0 + i < tw1 ? s_[i] : -INFINITY;
    // V^T element i of every block is token 4(lane/16) + i as well
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) vt[m][i] = tok_row0 + i < tw1 ? vt[m][i] : (short)0;
  }
  const float tm = max_rows(fmaxf(fmaxf(s_[0], s_[1]), fmaxf(s_[2], s_[3])));
  if (__builtin_amdgcn_ballot_w64(tm > st.m) != 0) {
    const float mn = fmaxf(st.m, tm);
    const float alpha = exp2_fast(st.m - mn);  // 1 where the maximum stays, 0 from -inf
    st.m = mn;
    st.lsum *= alpha;
#pragma unroll
    for (int m = 0; m < 8; ++m) st.acc[m] *= alpha;
  }
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = exp2_fast(s_[i] - st.m + WeightBias<BF16>::log2);
  st.lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  const Weights<BF16> wb = split_weights<BF16>(pr);
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const uint32_t v01 = __builtin_bit_cast(uint32_t, __builtin_shufflevector(vt[m], vt[m], 0, 1));
    const uint32_t v23 = __builtin_bit_cast(uint32_t, __builtin_shufflevector(vt[m], vt[m], 2, 3));
    st.acc[m] = mfma_16x16x32<BF16>(u32x4{v01, v23, v01, v23}, wb.hi_lo, st.acc[m]);
    if constexpr (BF16)  // k 4..7 of this one are zero on both sides
      st.acc[m] = mfma_16x16x32<BF16>(u32x4{v01, v23, 0u, 0u},
                                      u32x4{wb.lo2[0], wb.lo2[1], 0u, 0u}, st.acc[m]);
  }
}

// FP8 staging tile -> 16-bit tile layout. Lane l takes 16-byte chunks
// 64i + l (i < 2) of the K and of the V staging tile: token c/8, dims
// 16(c%8) .. +16; their 16 codes become two 16-byte chunks of 8 values each,
// written where the 16-bit layout keeps them. E4M3FN values are exact in
// both bf16 and f16, so the conversion (scale 1) loses nothing.
template <bool BF16>
__device__ __forceinline__ void convert_fp8_tile(const char* st, char* kt, int lane) {
#pragma unroll
  for (int tv = 0; tv < 2; ++tv) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = 64 * i + lane;
      const int t = c >> 3, c8 = c & 7, n = t >> 2, r = t & 3;
      const u32x4 x = *(const u32x4*)(st + tv * (kStage8 / 2) + 16 * c);
      u32x4 y[2];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t lo, hi;
        if constexpr (BF16) {
          lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, false));
          hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, true));
        } else {
          lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[w], 1.0f, false));
          hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[w], 1.0f, true));
        }
        y[w >> 1][2 * (w & 1)] = lo;
        y[w >> 1][2 * (w & 1) + 1] = hi;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int chunk = 2 * c8 + h;  // 16-bit chunk (8 dims) of the row
        const uint32_t off = tv == 0
            ? (uint32_t)n * kKGroup + (uint32_t)r * kRowBytes + 16u * (uint32_t)((chunk + r) & 15)
            : kKTile + (uint32_t)n * kVGroup + (uint32_t)r * kRowBytes +
                  16u * (uint32_t)((chunk + 2 * r) & 15);
        *(u32x4*)(kt + off) = y[h];
      }
    }
  }
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

template <bool BF16, int BS, bool SPLIT, int NW, bool KV8>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
void pd_decode_kernel(const KArgs a) {
  constexpr int kNBuf = tile_buffers<KV8>(NW);
  constexpr int kLoads = KV8 ? 4 : 8;  // load instructions per tile
  constexpr int kWaitTile = waitcnt_vm((kNBuf - 1) * kLoads);
  constexpr uint32_t kStage = stage_bytes<KV8>();
  // one array per tile buffer, so the compiler can wait for exactly the
  // loads of the buffer about to be read
  __shared__ __align__(16) char lds0[NW * kStage];
  __shared__ __align__(16) char lds1[NW * kStage];
  __shared__ __align__(16) char lds2[kNBuf > 2 ? NW * kStage : 16];
  __shared__ __align__(16) char ldsc[KV8 ? NW * kLdsTile : 16];  // converted FP8 tile
  const int p = blockIdx.x;
  const int hg = blockIdx.y;
  const int b = blockIdx.z;
  const int Hq = a.Hkv * G;
  const int nw = a.NH * a.NT;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = w % a.NH;  // KV head within the workgroup's group
  const int ts = w / a.NH;  // token slice
  const int g = hg * a.NH + hl;
  const int row = lane >> 4;
  const int sl = lane & 15;
  auto tile_buf = [&](int d) -> char* {
    char* base = d == 0 ? lds0 : d == 1 ? lds1 : lds2;
    return base + w * kStage;
  };

  const int t0 = p * a.P;
  const int tw0 = t0 + ts * a.Pw;
  const int bi0 = tw0 / BS;
  // q as the MFMA B operand: head lane%4, dims 32s + 8(lane/16) .. +8.
  // Loaded before the block ids, so that waiting for the ids (which the
  // first K/V addresses need) also covers q, and no later wait has to drain
  // the tile loads.
  u32x4 qb[4];
  const uint16_t* qp = a.q + ((size_t)b * Hq + (size_t)g * G + (lane & 3)) * D + 8 * row;
#pragma unroll
  for (int s = 0; s < 4; ++s) qb[s] = *(const u32x4*)(qp + 32 * s);
  // block ids of the wave's whole slice, fetched before the context length
  // is known (entries past the live ones are loaded but never used)
  const int nb_max = min(a.Pw / BS, a.MB - bi0);
  const int32_t* btrow = a.bt + (size_t)b * a.MB + bi0;
  int ids[kIdRegs];
#pragma unroll
  for (int i = 0; i < kIdRegs; ++i) ids[i] = 64 * i + lane < nb_max ? btrow[64 * i + lane] : 0;

  WaveState st;
  st.lsum = 0.f;
  st.m = -INFINITY;
#pragma unroll
  for (int m = 0; m < 8; ++m) st.acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  // wave-uniform by construction; readfirstlane lets the compiler keep the
  // loop bounds and block addresses in scalar registers
  const int L = __builtin_amdgcn_readfirstlane(a.cl[b]);
  if constexpr (!SPLIT) {
    if (L <= 0) {
      // empty context: zero rows for every query head of the group
      uint16_t* o = (uint16_t*)a.out + ((size_t)b * Hq + (size_t)hg * a.NH * G) * D;
      for (int i = threadIdx.x; i < a.NH * G * D / 8; i += nw * 64)
        *(u32x4*)(o + i * 8) = u32x4{0u, 0u, 0u, 0u};
      return;
    }
  } else {
    if (t0 >= L) {  // empty partition: neither counted nor merged
      if (L <= 0 && p == 0) {
        // empty context: partition 0 writes the zero rows, no merge runs
        uint16_t* o = (uint16_t*)a.out + ((size_t)b * Hq + (size_t)hg * a.NH * G) * D;
        for (int i = threadIdx.x; i < a.NH * G * D / 8; i += nw * 64)
          *(u32x4*)(o + i * 8) = u32x4{0u, 0u, 0u, 0u};
      }
      return;
    }
  }
  const int tw1 = min(min(tw0 + a.Pw, t0 + a.P), L);
  const int nst = __builtin_amdgcn_readfirstlane(
      tw0 < tw1 ? (tw1 - tw0 + kTileTok - 1) / kTileTok : 0);
  const float c = a.scale_log2;
  const uint32_t tok_bytes = a.Hkv * (KV8 ? kRowBytes8 : kRowBytes);
  // global offsets of this lane's 16 bytes in load instruction 0 of a tile:
  // 16-bit rows take 16 lanes each (4 rows per instruction), chunks rotated;
  // FP8 rows take 8 lanes each (8 rows per instruction), in order
  const int lrow = KV8 ? lane >> 3 : row;
  const uint32_t head_off =
      (uint32_t)lrow * tok_bytes + (uint32_t)g * (KV8 ? kRowBytes8 : kRowBytes);
  const uint32_t koff_g =
      head_off + (uint32_t)(KV8 ? (lane & 7) : ((sl - row) & 15)) * 16u;
  const uint32_t voff_g =
      head_off + (uint32_t)(KV8 ? (lane & 7) : ((sl - 2 * row) & 15)) * 16u;
  // LDS offsets of the two read patterns (see the tile layout above)
  uint32_t koff[4], voff[8];
  {
    const int t = lane & 15, r = t & 3;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      koff[s] = (uint32_t)(t >> 2) * kKGroup + (uint32_t)r * kRowBytes +
                16u * (uint32_t)((4 * s + row + r) & 15);
    // source lane of the transposing read: token 4(lane/16) + (lane%16)/4,
    // dims 16m + 4(lane%4) .. +4, i.e. chunk 2m + (lane%4)/2, half lane%2
    const int k = (lane & 15) >> 2, a4 = lane & 3;
#pragma unroll
    for (int m = 0; m < 8; ++m)
      voff[m] = kKTile + (uint32_t)row * kVGroup + (uint32_t)k * kRowBytes +
                16u * (uint32_t)((2 * m + (a4 >> 1) + 2 * k) & 15) + 8u * (uint32_t)(a4 & 1);
  }

  // Queue the 8 loads of tile j into buffer d. Straight-line, always eight
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
    constexpr int kRowsPerLoad = KV8 ? 8 : 4;
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
      const uint32_t kd = KV8 ? n * 1024u : n * kKGroup;
      const uint32_t vd = KV8 ? kStage8 / 2 + n * 1024u : kKTile + n * kVGroup;
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
      // tiles' (kNBuf - 1) * 8 loads are outstanding. Explicit, because the
      // compiler does not always see that these LDS reads depend on them.
      __builtin_amdgcn_s_waitcnt(kWaitTile);
      __builtin_amdgcn_sched_barrier(0);
      // Before a buffer is refilled every LDS read of it has completed: the
      // refill's LDS writes are not ordered after reads still in flight, and
      // a refill past the slice reads no memory, so it lands at once.
      if constexpr (KV8) {
        // convert, then refill the staging buffer before computing
        char* ct = ldsc + w * kLdsTile;
        if (j < nst) convert_fp8_tile<BF16>(tile_buf(d), ct, lane);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitLds);
        __builtin_amdgcn_sched_barrier(0);
        issue(j + kNBuf, d);
        __builtin_amdgcn_sched_barrier(0);
        if (j < nst) {
          const int tile0 = tw0 + kTileTok * j;
          tile_compute<BF16>(st, ct, qb, koff, voff, tile0 + 4 * row, tw1,
                             tile0 + kTileTok > tw1, c);
        }
      } else {
        if (j < nst) {
          const int tile0 = tw0 + kTileTok * j;
          tile_compute<BF16>(st, tile_buf(d), qb, koff, voff, tile0 + 4 * row, tw1,
                             tile0 + kTileTok > tw1, c);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitLds);
        __builtin_amdgcn_sched_barrier(0);
        issue(j + kNBuf, d);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // every tile load (the trailing ones read nothing) has landed before the
  // tile buffers are reused below
  __builtin_amdgcn_s_waitcnt(0);

  // ---- this lane's share of the result: query head h of the KV head, the
  // 8 dims [d0, d0+4) and [d0+16, d0+20) (one of the 4 copies of each)
  const int h = lane & 3;
  const int qd = (lane >> 2) & 3;
  const int d0 = 32 * qd + 4 * row;
  f32x4 o0 = qd == 0 ? st.acc[0] : qd == 1 ? st.acc[2] : qd == 2 ? st.acc[4] : st.acc[6];
  f32x4 o1 = qd == 0 ? st.acc[1] : qd == 1 ? st.acc[3] : qd == 2 ? st.acc[5] : st.acc[7];
  float m_r = st.m;
  float l_r = sum_rows(st.lsum);

  // ---- merge the NT slices of each head through LDS (the first tile
  // buffer); slice 0 keeps the result
  if (a.NT > 1) {
    __syncthreads();  // every wave is done with its tile buffers
    float* s_acc = (float*)lds0;            // [(w*G + h)*D + dim]
    float* s_m = (float*)lds0 + nw * G * D;  // [w*G + h]
    float* s_l = s_m + nw * G;
    *(f32x4*)(s_acc + (w * G + h) * D + d0) = o0;
    *(f32x4*)(s_acc + (w * G + h) * D + d0 + 16) = o1;
    if ((lane >> 2) == 0) {
      s_m[w * G + h] = m_r;
      s_l[w * G + h] = l_r;
    }
    __syncthreads();
    if (ts == 0) {
      float M = m_r;
      for (int i = 1; i < a.NT; ++i) M = fmaxf(M, s_m[(i * a.NH + hl) * G + h]);
      float den = 0.f;
      o0 = f32x4{0.f, 0.f, 0.f, 0.f};
      o1 = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int i = 0; i < a.NT; ++i) {
        const int wi = (i * a.NH + hl) * G + h;
        const float wt = exp2_fast(s_m[wi] - M);  // 0 for a slice with no tokens
        den = fmaf(wt, s_l[wi], den);
        const f32x4 x0 = *(const f32x4*)(s_acc + wi * D + d0);
        const f32x4 x1 = *(const f32x4*)(s_acc + wi * D + d0 + 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o0[e] = fmaf(wt, x0[e], o0[e]);
          o1[e] = fmaf(wt, x1[e], o1[e]);
        }
      }
      m_r = M;
      l_r = den;
    }
  }
  const bool owner = ts == 0;
  const int hq = g * G + h;  // query head of this lane

  if constexpr (!SPLIT) {
    if (owner) {
      uint16_t* o = (uint16_t*)a.out + ((size_t)b * Hq + hq) * D + d0;
      const float inv = a.out_scale / l_r;
      store4<BF16>(o, o0, inv);
      store4<BF16>(o + 16, o1, inv);
    }
    return;
  } else {
    // ---- publish this partition's (o_p, lse_p), write-through
    const size_t slot0 = ((size_t)b * Hq + (size_t)g * G) * a.S;  // (head 0, partition 0)
    const uint32_t rows_bytes = (uint32_t)G * a.S * D * 4;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o_part + slot0 * D, rows_bytes);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lse_part + slot0, (uint32_t)G * a.S * 4);
    if (owner) {
      // the raw buffer builtins move 32-bit words: floats go through bit casts
      const float inv = 1.0f / l_r;
      const uint32_t off = ((uint32_t)(h * a.S + p) * D + d0) * 4;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o0 * inv), ro, off, 0,
                                             kCoherent);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o1 * inv), ro, off + 64,
                                             0, kCoherent);
      if ((lane >> 2) == 0)
        __builtin_amdgcn_raw_buffer_store_b32(
            __builtin_bit_cast(uint32_t, m_r + __builtin_amdgcn_logf(l_r) -
                                             WeightBias<BF16>::log2),
            rl, (uint32_t)(h * a.S + p) * 4, 0, kCoherent);
    }
    // the stores are complete (and past every non-coherent cache) before the
    // counter moves
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ int s_last;
    const int n_live = (L + a.P - 1) / a.P;
    if (threadIdx.x == 0) {
      int32_t* cnt = a.counters + (size_t)b * (a.Hkv / a.NH) + hg;
      const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = old == n_live - 1;
      if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last || !owner) return;

    // ---- last workgroup: LSE merge over the n_live partitions, in order
    constexpr int kBatch = 8;
    float M = -INFINITY, den = 0.f;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < n_live; i0 += kBatch) {
      float lse[kBatch];
      f32x4 x0[kBatch], x1[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        // partitions past n_live read zeros and are skipped below
        const bool ok = i0 + u < n_live;
        const uint32_t slot = (uint32_t)(h * a.S + i0 + u);
        const uint32_t off = ok ? (slot * D + d0) * 4 : kOutOfBlock;
        x0[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0,
                                                                                kCoherent));
        x1[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              ro, ok ? off + 64 : kOutOfBlock, 0, kCoherent));
        lse[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               rl, ok ? slot * 4 : kOutOfBlock, 0, kCoherent));
      }
      float bm = M;
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (i0 + u < n_live) bm = fmaxf(bm, lse[u]);
      const float alpha = exp2_fast(M - bm);  // 0 on the first batch
      den *= alpha;
      acc0 *= alpha;
      acc1 *= alpha;
      M = bm;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (i0 + u < n_live) {
          const float wt = exp2_fast(lse[u] - M);
          den += wt;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc0[e] = fmaf(wt, x0[u][e], acc0[e]);
            acc1[e] = fmaf(wt, x1[u][e], acc1[e]);
          }
        }
      }
    }
    uint16_t* o = (uint16_t*)a.out + ((size_t)b * Hq + hq) * D + d0;
    const float inv = a.out_scale / den;
    store4<BF16>(o, acc0, inv);
    store4<BF16>(o + 16, acc1, inv);
  }
}

// Zero the workspace (the split path's counters must start at zero).
__global__ void pd_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

template <bool BF16, int BS, bool SPLIT, bool KV8>
hipError_t launch_decode(const KArgs& ka, dim3 grid, int nw, hipStream_t st) {
  void* args[] = {(void*)&ka};
  // the LDS tile buffers are sized for the largest workgroup of the instance
  const void* f = nw <= 4 ? (const void*)&pd_decode_kernel<BF16, BS, SPLIT, 4, KV8>
                          : (const void*)&pd_decode_kernel<BF16, BS, SPLIT, 8, KV8>;
  return hipLaunchKernel(f, grid, dim3(nw * 64), args, 0, st);
}

template <bool BF16, bool SPLIT, bool KV8>
hipError_t pick_block(const KArgs& ka, dim3 grid, int bs, int nw, hipStream_t st) {
  return bs == 32 ? launch_decode<BF16, 32, SPLIT, KV8>(ka, grid, nw, st)
                  : launch_decode<BF16, 16, SPLIT, KV8>(ka, grid, nw, st);
}

template <bool KV8>
hipError_t pick_dtype(const KArgs& ka, dim3 grid, int bs, int nw, bool bf16, bool split,
                      hipStream_t st) {
  if (bf16)
    return split ? pick_block<true, true, KV8>(ka, grid, bs, nw, st)
                 : pick_block<true, false, KV8>(ka, grid, bs, nw, st);
  return split ? pick_block<false, true, KV8>(ka, grid, bs, nw, st)
               : pick_block<false, false, KV8>(ka, grid, bs, nw, st);
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
  ka.counters = nullptr;
  if (l.plan.splits > 1) {
    char* ws = (char*)l.workspace;
    ka.counters = (int32_t*)ws;
    ka.o_part = (float*)(ws + kCounterBytes);
    ka.lse_part = (float*)(ws + kCounterBytes + partials_bytes(l.shape, l.plan));
  }
  ka.Hkv = l.shape.Hkv;
  ka.MB = l.shape.max_blocks_per_seq;
  ka.S = l.plan.splits;
  ka.P = l.plan.partition_tokens;
  ka.Pw = l.plan.wave_tokens;
  ka.NH = l.plan.heads_per_group;
  ka.NT = l.plan.slices;
  ka.scale_log2 = l.scale * 1.4426950408889634f * (l.kv_fp8 ? l.k_scale : 1.0f);
  ka.out_scale = l.kv_fp8 ? l.v_scale : 1.0f;
  ka.blk_bytes = (uint32_t)l.shape.block_size * (uint32_t)l.shape.Hkv *
                 (l.kv_fp8 ? kRowBytes8 : kRowBytes);
  const dim3 grid(l.plan.splits, l.shape.Hkv / l.plan.heads_per_group, l.shape.B);
  const int nw = l.plan.heads_per_group * l.plan.slices;
  // each wave owns kLdsTile bytes of every tile buffer of its workgroup
  if (nw < 1 || nw > kMaxWaves || l.shape.Hkv % l.plan.heads_per_group != 0)
    return PD_ERR_INTERNAL;
  hipStream_t st = (hipStream_t)l.stream;
  const bool split = l.plan.splits > 1;
  const bool bf16 = l.shape.dtype == PD_DTYPE_BF16;
  const hipError_t e = l.kv_fp8
      ? pick_dtype<true>(ka, grid, l.shape.block_size, nw, bf16, split, st)
      : pick_dtype<false>(ka, grid, l.shape.block_size, nw, bf16, split, st);
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
