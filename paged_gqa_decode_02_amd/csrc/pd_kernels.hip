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
//   * lanes: 16 lanes per token row. A 4-token step gives lane
//     (row = lane/16, sl = lane%16) token `row` of the step and head-dim
//     elements [8sl, 8sl+8): each 128-bit load instruction of the wave reads
//     four whole 256-byte rows.
//   * K/V come straight from HBM into registers with bounds-checked buffer
//     loads whose resource is the current physical block (base = pool +
//     id * block bytes, size = block bytes), so an access cannot leave the
//     block; lanes past the context get an offset beyond the block and read
//     zeros with no memory access. Three 8-token stages of loads stay in
//     flight while the oldest is computed; the loads use the streaming (nt)
//     cache policy since every K/V byte is read once.
//   * block ids: each lane loads up to four block-table entries of the
//     wave's range before the context length is known; a stage takes its
//     (wave-uniform) id with v_readlane, so addresses are scalar.
//   * scores: q stays as packed 16-bit pairs; v_dot2_f32_{bf16,f16} gives
//     fp32 sums of products with no conversion of K, a 4-step DPP butterfly
//     sums the 16 lanes of a row, and one multiply by scale*log2(e) puts the
//     softmax in base 2 (v_exp_f32).
//   * softmax: a wave-uniform running maximum per head that only moves when
//     a ballot finds a score above it (then permlane16/32 swaps reduce over
//     the 4 rows and the accumulators are rescaled); each lane keeps its own
//     partial sum l and accumulator acc[4][8].
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int D = pd::kHeadDim;  // 128
constexpr int G = pd::kGroup;    // 4
constexpr int kMaxWaves = pd::kMaxWaves;
constexpr int kIdRegs = pd::kMaxWaveBlocks / 64;  // block ids per lane
constexpr uint32_t kRowBytes = D * 2;          // one token row of one KV head
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
  float scale_log2;    // scale * log2(e)
  uint32_t blk_bytes;  // block_size * Hkv * D * 2
};

template <bool BF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                  __builtin_bit_cast(f16x2_t, b), c, false);
}

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
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kRowMirror = 0x140;   // lane i <-> 15-i within the row

// Sum over the 16 lanes of a token row; every lane gets the total.
__device__ __forceinline__ float sum16(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  return x;
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

// Per-lane state of one wave's online softmax over its token slice.
template <bool BF16>
struct WaveState {
  u32x4 q[G];       // this lane's 8 q elements of each head, packed pairs
  float acc[G][8];  // unnormalised PV sums of the lane's token row
  float l[G];       // sum of weights of the lane's token row
  float m[G];       // wave-uniform running maximum (log2 domain)
};

// One stage = two 4-token steps = 8 consecutive tokens of one block.
// kb[i], vb[i]: this lane's 16 bytes of the K / V row of step i's token.
template <bool BF16>
__device__ __forceinline__ void stage_compute(WaveState<BF16>& st, const u32x4 (&kb)[2],
                                              const u32x4 (&vb)[2], bool valid0, bool valid1,
                                              float c) {
  float s[2][G];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const bool ok = i == 0 ? valid0 : valid1;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) d = dot2<BF16>(st.q[h][e], kb[i][e], d);
      d = sum16(d);
      s[i][h] = ok ? d * c : -INFINITY;
    }
  }
  // the running maximum only moves when some score exceeds it (wave vote)
  uint64_t above = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h = 0; h < G; ++h) above |= __builtin_amdgcn_ballot_w64(s[i][h] > st.m[h]);
  if (above != 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(st.m[h], max_rows(fmaxf(s[0][h], s[1][h])));
      const float alpha = exp2_fast(st.m[h] - mn);  // 0 when m was -inf
      st.l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[h][e] *= alpha;
      st.m[h] = uniform_f(mn);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    // a token past the range reads zeros (out-of-block offset), and its
    // weight is exp2(-inf) = 0, so it adds nothing
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pr = exp2_fast(s[i][h] - st.m[h]);
      st.l[h] += pr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st.acc[h][2 * e] = fmaf(pr, lo_f<BF16>(vb[i][e]), st.acc[h][2 * e]);
        st.acc[h][2 * e + 1] = fmaf(pr, hi_f<BF16>(vb[i][e]), st.acc[h][2 * e + 1]);
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

template <bool BF16>
__device__ __forceinline__ void store_row(uint16_t* o, const float (&r)[8], float inv) {
  u32x4 wv;
#pragma unroll
  for (int i = 0; i < 4; ++i) wv[i] = pack2<BF16>(r[2 * i] * inv, r[2 * i + 1] * inv);
  *(u32x4*)o = wv;
}

// Stages of K/V loads in flight per wave (the waves per SIMD the register
// budget is sized for, and with it the largest workgroup, is in pd_internal.h).
#ifndef PD_DEPTH
#define PD_DEPTH 3
#endif

template <bool BF16, int BS, bool SPLIT>
__global__ __launch_bounds__(kMaxWaves * 64)
__attribute__((amdgpu_waves_per_eu(PD_WAVES_PER_SIMD, 8)))
void pd_decode_kernel(const KArgs a) {
  constexpr int DEPTH = PD_DEPTH;
  constexpr int kStageTok = 8;
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

  const int t0 = p * a.P;
  const int tw0 = t0 + ts * a.Pw;
  const int bi0 = tw0 / BS;
  // block ids of the wave's whole slice, fetched before the context length
  // is known (entries past the live ones are loaded but never used)
  const int nb_max = min(a.Pw / BS, a.MB - bi0);
  const int32_t* btrow = a.bt + (size_t)b * a.MB + bi0;
  int ids[kIdRegs];
#pragma unroll
  for (int i = 0; i < kIdRegs; ++i) ids[i] = 64 * i + lane < nb_max ? btrow[64 * i + lane] : 0;

  WaveState<BF16> st;
  const uint16_t* qp = a.q + ((size_t)b * Hq + (size_t)g * G) * D + sl * 8;
#pragma unroll
  for (int h = 0; h < G; ++h) st.q[h] = *(const u32x4*)(qp + h * D);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.l[h] = 0.f;
    st.m[h] = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[h][e] = 0.f;
  }

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
      tw0 < tw1 ? (tw1 - tw0 + kStageTok - 1) / kStageTok : 0);
  const float c = a.scale_log2;
  const uint32_t lane_off = ((uint32_t)row * a.Hkv + g) * kRowBytes + sl * 16u;
  const uint32_t tok_bytes = a.Hkv * kRowBytes;

  u32x4 kb[DEPTH][2], vb[DEPTH][2];
  // Queue the loads of stage j. Straight-line code, always four loads, so
  // the wait counts stay exact: past the slice (j >= nst) every lane's token
  // is >= tw1 and its offset is out of the block, and the block id is forced
  // to 0, so those loads read nothing.
  auto issue = [&](int j, u32x4(&kr)[2], u32x4(&vr)[2]) {
    const int tok = kStageTok * j;  // offset in the slice
    const int idx = min(tok / BS, kIdRegs * 64 - 1);
    const int id = pick_id(ids, idx) * (int)(j < nst);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + (int64_t)id * a.blk_bytes, a.blk_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + (int64_t)id * a.blk_bytes, a.blk_bytes);
    const uint32_t base = (uint32_t)(tok % BS) * tok_bytes + lane_off;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bool ok = tw0 + tok + 4 * i + row < tw1;
      // the whole offset goes in the vector operand, which the range check covers
      const uint32_t vo = ok ? base + 4u * i * tok_bytes : kOutOfBlock;
      kr[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, vo, 0, kStream);
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo, 0, kStream);
    }
  };

  // The loads must leave in stage order, in the prologue as in the loop, so
  // that the wait for stage j never has to drain the later stages.
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    issue(d, kb[d], vb[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int j0 = 0; j0 < nst; j0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int j = j0 + d;
      if (j < nst) {
        const int tok = tw0 + kStageTok * j + row;
        stage_compute<BF16>(st, kb[d], vb[d], tok < tw1, tok + 4 < tw1, c);
      }
      issue(j + DEPTH, kb[d], vb[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- reduce over the 4 token rows of the wave
#pragma unroll
  for (int h = 0; h < G; ++h) st.l[h] = sum_rows(st.l[h]);
  // reduce-scatter: rows 0-1 keep heads {0,1}, rows 2-3 keep heads {2,3} ...
  float r1[2][8];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float y;
      const float x = swap32_lo(st.acc[hh][e], st.acc[hh + 2][e], &y);
      r1[hh][e] = x + y;
    }
  // ... then row r keeps head r.
  float r2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float y;
    const float x = swap16_lo(r1[0][e], r1[1][e], &y);
    r2[e] = x + y;
  }
  float m_r = row == 0 ? st.m[0] : row == 1 ? st.m[1] : row == 2 ? st.m[2] : st.m[3];
  float l_r = row == 0 ? st.l[0] : row == 1 ? st.l[1] : row == 2 ? st.l[2] : st.l[3];

  // ---- merge the NT slices of each head through LDS; slice 0 keeps the result
  if (a.NT > 1) {
    // dynamic LDS, sized by the host to the workgroup's waves:
    // acc [nw][G][D] floats, then m [nw][G], then l [nw][G]
    extern __shared__ __align__(16) float pd_lds[];
    f32x4* s_acc = (f32x4*)pd_lds;                  // [(w*G + row)*(D/4) + i]
    float* s_m = pd_lds + nw * G * D;               // [w*G + row]
    float* s_l = s_m + nw * G;
    s_acc[(w * G + row) * (D / 4) + 2 * sl] = f32x4{r2[0], r2[1], r2[2], r2[3]};
    s_acc[(w * G + row) * (D / 4) + 2 * sl + 1] = f32x4{r2[4], r2[5], r2[6], r2[7]};
    if (sl == 0) {
      s_m[w * G + row] = m_r;
      s_l[w * G + row] = l_r;
    }
    __syncthreads();
    if (ts == 0) {
      float M = m_r;
      for (int i = 1; i < a.NT; ++i) M = fmaxf(M, s_m[(i * a.NH + hl) * G + row]);
      float den = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) r2[e] = 0.f;
      for (int i = 0; i < a.NT; ++i) {
        const int wi = (i * a.NH + hl) * G + row;
        const float wt = exp2_fast(s_m[wi] - M);  // 0 for a slice with no tokens
        den = fmaf(wt, s_l[wi], den);
        const f32x4 x0 = s_acc[wi * (D / 4) + 2 * sl];
        const f32x4 x1 = s_acc[wi * (D / 4) + 2 * sl + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r2[e] = fmaf(wt, x0[e], r2[e]);
          r2[4 + e] = fmaf(wt, x1[e], r2[4 + e]);
        }
      }
      m_r = M;
      l_r = den;
    }
  }
  const bool owner = ts == 0;
  const int hq = g * G + row;  // query head of this lane's row

  if constexpr (!SPLIT) {
    if (owner)
      store_row<BF16>((uint16_t*)a.out + ((size_t)b * Hq + hq) * D + sl * 8, r2, 1.0f / l_r);
    return;
  } else {
    // ---- publish this partition's (o_p, lse_p), write-through
    const size_t slot0 = ((size_t)b * Hq + (size_t)g * G) * a.S;  // (row 0, partition 0)
    const uint32_t rows_bytes = (uint32_t)G * a.S * D * 4;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o_part + slot0 * D, rows_bytes);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lse_part + slot0, (uint32_t)G * a.S * 4);
    if (owner) {
      // the raw buffer builtins move 32-bit words: floats go through bit casts
      const float inv = 1.0f / l_r;
      const uint32_t off = ((uint32_t)(row * a.S + p) * D + sl * 8) * 4;
      const f32x4 o0 = {r2[0] * inv, r2[1] * inv, r2[2] * inv, r2[3] * inv};
      const f32x4 o1 = {r2[4] * inv, r2[5] * inv, r2[6] * inv, r2[7] * inv};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o0), ro, off, 0, kCoherent);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o1), ro, off + 16, 0,
                                             kCoherent);
      if (sl == 0)
        __builtin_amdgcn_raw_buffer_store_b32(
            __builtin_bit_cast(uint32_t, m_r + __builtin_amdgcn_logf(l_r)), rl,
            (uint32_t)(row * a.S + p) * 4, 0, kCoherent);
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
    float M = -INFINITY, den = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int i0 = 0; i0 < n_live; i0 += kBatch) {
      float lse[kBatch];
      f32x4 o0[kBatch], o1[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        // partitions past n_live read zeros and are skipped below
        const bool ok = i0 + u < n_live;
        const uint32_t slot = (uint32_t)(row * a.S + i0 + u);
        const uint32_t off = ok ? (slot * D + sl * 8) * 4 : kOutOfBlock;
        o0[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0,
                                                                                kCoherent));
        o1[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off + 16, 0,
                                                                                kCoherent));
        lse[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               rl, ok ? slot * 4 : kOutOfBlock, 0, kCoherent));
      }
      float bm = M;
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (i0 + u < n_live) bm = fmaxf(bm, lse[u]);
      const float alpha = exp2_fast(M - bm);  // 0 on the first batch
      den *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= alpha;
      M = bm;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (i0 + u < n_live) {
          const float wt = exp2_fast(lse[u] - M);
          den += wt;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[e] = fmaf(wt, o0[u][e], acc[e]);
            acc[4 + e] = fmaf(wt, o1[u][e], acc[4 + e]);
          }
        }
      }
    }
    store_row<BF16>((uint16_t*)a.out + ((size_t)b * Hq + hq) * D + sl * 8, acc, 1.0f / den);
  }
}

// Zero the workspace (the split path's counters must start at zero).
__global__ void pd_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

template <bool BF16, int BS, bool SPLIT>
hipError_t launch_decode(const KArgs& ka, dim3 grid, int nw, hipStream_t st) {
  void* args[] = {(void*)&ka};
  const size_t lds = ka.NT > 1 ? (size_t)nw * G * (D + 2) * sizeof(float) : 0;
  return hipLaunchKernel((const void*)&pd_decode_kernel<BF16, BS, SPLIT>, grid, dim3(nw * 64),
                         args, lds, st);
}

template <bool BF16, bool SPLIT>
hipError_t pick_block(const KArgs& ka, dim3 grid, int bs, int nw, hipStream_t st) {
  return bs == 32 ? launch_decode<BF16, 32, SPLIT>(ka, grid, nw, st)
                  : launch_decode<BF16, 16, SPLIT>(ka, grid, nw, st);
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
  ka.scale_log2 = l.scale * 1.4426950408889634f;
  ka.blk_bytes = (uint32_t)l.shape.block_size * (uint32_t)l.shape.Hkv * kRowBytes;
  const dim3 grid(l.plan.splits, l.shape.Hkv / l.plan.heads_per_group, l.shape.B);
  const int nw = l.plan.heads_per_group * l.plan.slices;
  hipStream_t st = (hipStream_t)l.stream;
  const bool split = l.plan.splits > 1;
  hipError_t e;
  if (l.shape.dtype == PD_DTYPE_BF16)
    e = split ? pick_block<true, true>(ka, grid, l.shape.block_size, nw, st)
              : pick_block<true, false>(ka, grid, l.shape.block_size, nw, st);
  else
    e = split ? pick_block<false, true>(ka, grid, l.shape.block_size, nw, st)
              : pick_block<false, false>(ka, grid, l.shape.block_size, nw, st);
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
