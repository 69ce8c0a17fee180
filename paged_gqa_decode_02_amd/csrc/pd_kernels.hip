// Paged GQA decode attention kernels for gfx950 (CDNA4, wave64).
//
// Method (Loom Kernels home page, "Supported now": paged MQA/GQA decode with
// GQA packing and local split-K/LSE): one query token per head attends over
// a paged K/V cache; the 4 query heads that share a KV head are served by one
// pass over that head's K/V bytes, and a long context is cut into
// partitions whose normalised partial outputs and log-sum-exps are merged.
//
// Decode kernel, one workgroup of NW wave64s per (partition p, KV head g,
// sequence b); wave w owns a block-aligned range of at most 64 blocks:
//   * lanes: 16 lanes per token row. A 4-token step gives lane
//     (row = lane/16, sl = lane%16) token `row` of the step and head-dim
//     elements [8sl, 8sl+8): each 128-bit load instruction of the wave reads
//     four whole 256-byte rows (eight 128-byte lines).
//   * K/V come straight from HBM into registers with bounds-checked buffer
//     loads whose resource is the current physical block (base = pool +
//     id * block bytes, size = block bytes), so an access cannot leave the
//     block; lanes past the context get an offset beyond the block and read
//     zeros with no memory access. Three 8-token stages of loads are kept in
//     flight while the oldest is computed.
//   * block ids: each lane loads one block-table entry of the wave's range
//     before the context length is known; a stage takes its (wave-uniform)
//     id with v_readlane, so addresses are scalar.
//   * scores: q stays as packed 16-bit pairs; v_dot2_f32_{bf16,f16} gives
//     fp32 sums of products with no conversion of K, a 4-step DPP butterfly
//     sums the 16 lanes of a row, and one multiply by scale*log2(e) puts the
//     softmax in base 2 (v_exp_f32).
//   * softmax: a wave-uniform running maximum per head that only moves when
//     a ballot finds a score above it (then permlane16/32 swaps reduce over
//     the 4 rows and the accumulators are rescaled); each lane keeps its own
//     partial sum l and accumulator acc[4][8].
//   * end of range: a reduce-scatter over the 4 rows (permlane32_swap, then
//     permlane16_swap) leaves head r's 128 sums in row r; the waves of a
//     workgroup are merged through LDS.
//   * S == 1 writes `out` rounded to the dtype; S > 1 writes fp32 o_p and
//     the partition's log2-sum-exp.
// Merge kernel, one workgroup per (query head, sequence): the LSE merge over
// the ceil(L/P) non-empty partitions in fixed order p = 0..n-1.
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
constexpr int kMaxWaveBlocks = pd::kMaxWaveBlocks;
constexpr int G = pd::kGroup;    // 4
constexpr uint32_t kRowBytes = D * 2;        // one token row of one KV head
constexpr uint32_t kOutOfBlock = 0x80000000u;  // buffer offset that reads as zero
constexpr int kRsrcWord3 = 0x00020000;        // raw 32-bit buffer, gfx9 data format
constexpr int kStream = 2;                    // cache policy "nt": K/V bytes are read once

struct KArgs {
  const uint16_t* q;
  const char* k;
  const char* v;
  const int32_t* bt;
  const int32_t* cl;
  void* out;
  float* o_part;    // [B, Hq, S, D]
  float* lse_part;  // [B, Hq, S], log2 domain
  int32_t Hkv;
  int32_t MB;
  int32_t S;
  int32_t P;
  int32_t Pw;          // tokens per wave, a multiple of the block size, <= 64 blocks
  float scale_log2;   // scale * log2(e)
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
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;   // lane i <-> 7-i within each 8 lanes
constexpr int kRowMirror = 0x140;    // lane i <-> 15-i within the row

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

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const char* base, int32_t id,
                                                             uint32_t blk_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      (void*)(base + (int64_t)id * (int64_t)blk_bytes), (short)0, (int)blk_bytes, kRsrcWord3);
}

// Sum over the 16 lanes of a token row; every lane gets the total.
__device__ __forceinline__ float sum16(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  return x;
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

// Per-lane state of one wave's online softmax over its token range.
// Lane (row r = lane/16, sub-lane sl = lane%16) owns token r of each 4-token
// step and head-dim elements [8sl, 8sl+8) of the group's 4 query heads.
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
      st.m[h] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                              __builtin_bit_cast(int, mn)));  // uniform
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

// Decode kernel: one workgroup of NW waves per (partition p, KV head g,
// sequence b); wave w owns tokens [p*P + w*Pw, +Pw) of the partition, at most
// 64 blocks. BS: block size. DEPTH: stages of loads kept in flight.
template <bool BF16, int BS, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 8)))
void pd_decode_kernel(const KArgs a) {
  constexpr int DEPTH = 3;
  constexpr int kStageTok = 8;
  const int p = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int Hq = a.Hkv * G;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane >> 4;
  const int sl = lane & 15;

  const int t0 = p * a.P;
  const int tw0 = t0 + w * a.Pw;
  const int bi0 = tw0 / BS;
  // block ids of the wave's whole range, fetched before the context length
  // is known (entries past the live ones are loaded but never used)
  const int nb_max = min(a.Pw / BS, a.MB - bi0);
  const int myid = lane < nb_max ? a.bt[(size_t)b * a.MB + bi0 + lane] : 0;

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
      // empty context: a zero row for each of the group's heads
      uint16_t* o = (uint16_t*)a.out + ((size_t)b * Hq + (size_t)g * G) * D;
      for (int i = threadIdx.x; i < G * D / 8; i += NW * 64)
        *(u32x4*)(o + i * 8) = u32x4{0u, 0u, 0u, 0u};
      return;
    }
  } else {
    if (t0 >= L) return;  // the merge reads only the ceil(L/P) non-empty partitions
  }
  const int tw1 = min(min(tw0 + a.Pw, t0 + a.P), L);
  const int nst = __builtin_amdgcn_readfirstlane(
      tw0 < tw1 ? (tw1 - tw0 + kStageTok - 1) / kStageTok : 0);
  const float c = a.scale_log2;
  const uint32_t lane_off = ((uint32_t)row * a.Hkv + g) * kRowBytes + sl * 16u;
  const uint32_t tok_bytes = a.Hkv * kRowBytes;

  u32x4 kb[DEPTH][2], vb[DEPTH][2];
  // Queue the loads of stage j. Straight-line code, always four loads, so
  // the wait counts stay exact: past the range (j >= nst) every lane's token
  // is >= tw1 and its offset is out of the block, and the block id is forced
  // to 0, so those loads read nothing.
  auto issue = [&](int j, u32x4(&kr)[2], u32x4(&vr)[2]) {
    const int tok = kStageTok * j;                        // offset in the wave range
    const int idx = min(tok / BS, kMaxWaveBlocks - 1);
    const int id = __builtin_amdgcn_readlane(myid, idx) * (int)(j < nst);
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(a.k, id, a.blk_bytes);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(a.v, id, a.blk_bytes);
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

  if constexpr (NW > 1) {
    // ---- merge the NW waves through LDS; wave 0 finishes
    __shared__ f32x4 s_acc[NW][G][D / 4];
    __shared__ float s_m[NW][G];
    __shared__ float s_l[NW][G];
    s_acc[w][row][2 * sl] = f32x4{r2[0], r2[1], r2[2], r2[3]};
    s_acc[w][row][2 * sl + 1] = f32x4{r2[4], r2[5], r2[6], r2[7]};
    if (sl == 0) {
      s_m[w][row] = m_r;
      s_l[w][row] = l_r;
    }
    __syncthreads();
    if (w != 0) return;
    float M = s_m[0][row];
#pragma unroll
    for (int i = 1; i < NW; ++i) M = fmaxf(M, s_m[i][row]);
    float den = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) r2[e] = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const float wt = exp2_fast(s_m[i][row] - M);  // 0 for a wave with no tokens
      den = fmaf(wt, s_l[i][row], den);
      const f32x4 x0 = s_acc[i][row][2 * sl];
      const f32x4 x1 = s_acc[i][row][2 * sl + 1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r2[e] = fmaf(wt, x0[e], r2[e]);
        r2[4 + e] = fmaf(wt, x1[e], r2[4 + e]);
      }
    }
    m_r = M;
    l_r = den;
  }

  // ---- epilogue: row r of wave 0 holds head g*G + r, elements [8sl, 8sl+8)
  const int hq = g * G + row;
  const float inv = 1.0f / l_r;
  if constexpr (!SPLIT) {
    uint16_t* o = (uint16_t*)a.out + ((size_t)b * Hq + hq) * D + sl * 8;
    u32x4 wv;
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[i] = pack2<BF16>(r2[2 * i] * inv, r2[2 * i + 1] * inv);
    *(u32x4*)o = wv;
  } else {
    const size_t slot = ((size_t)b * Hq + hq) * a.S + p;
    float* o = a.o_part + slot * D + sl * 8;
    *(f32x4*)o = f32x4{r2[0] * inv, r2[1] * inv, r2[2] * inv, r2[3] * inv};
    *(f32x4*)(o + 4) = f32x4{r2[4] * inv, r2[5] * inv, r2[6] * inv, r2[7] * inv};
    if (sl == 0) a.lse_part[slot] = m_r + __builtin_amdgcn_logf(l_r);
  }
}

// LSE merge: one workgroup of D threads per (query head, sequence).
template <bool BF16>
__global__ __launch_bounds__(D) void pd_merge_kernel(const float* __restrict__ o_part,
                                                     const float* __restrict__ lse_part,
                                                     const int32_t* __restrict__ cl,
                                                     void* __restrict__ out, int32_t S,
                                                     int32_t P) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int Hq = gridDim.x;
  const int d = threadIdx.x;
  const int L = cl[b];
  const int n = L > 0 ? (L + P - 1) / P : 0;
  const size_t rowi = (size_t)b * Hq + h;
  const float* lp = lse_part + rowi * S;
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, lp[i]);
  float num = 0.f, den = 0.f;
  for (int i = 0; i < n; ++i) {
    const float wt = exp2_fast(lp[i] - M);
    den += wt;
    num = fmaf(wt, o_part[(rowi * S + i) * D + d], num);
  }
  const float r = n > 0 ? num / den : 0.f;
  ((uint16_t*)out)[rowi * D + d] = to_bits<BF16>(r);
}

template <bool BF16, int BS, int NW, bool SPLIT>
hipError_t launch_decode(const KArgs& ka, dim3 grid, hipStream_t st) {
  void* args[] = {(void*)&ka};
  return hipLaunchKernel((const void*)&pd_decode_kernel<BF16, BS, NW, SPLIT>, grid,
                         dim3(NW * 64), args, 0, st);
}

template <bool BF16, int BS, bool SPLIT>
hipError_t pick_waves(const KArgs& ka, dim3 grid, int nw, hipStream_t st) {
  switch (nw) {
    case 8: return launch_decode<BF16, BS, 8, SPLIT>(ka, grid, st);
    case 4: return launch_decode<BF16, BS, 4, SPLIT>(ka, grid, st);
    case 2: return launch_decode<BF16, BS, 2, SPLIT>(ka, grid, st);
    default: return launch_decode<BF16, BS, 1, SPLIT>(ka, grid, st);
  }
}

template <bool BF16, bool SPLIT>
hipError_t pick_block(const KArgs& ka, dim3 grid, int bs, int nw, hipStream_t st) {
  return bs == 32 ? pick_waves<BF16, 32, SPLIT>(ka, grid, nw, st)
                  : pick_waves<BF16, 16, SPLIT>(ka, grid, nw, st);
}

template <bool BF16>
hipError_t launch_all(const KArgs& ka, const pd::Launch& l, hipStream_t st) {
  const dim3 grid(l.plan.splits, l.shape.Hkv, l.shape.B);
  if (l.plan.splits == 1)
    return pick_block<BF16, false>(ka, grid, l.shape.block_size, l.plan.waves, st);
  hipError_t e = pick_block<BF16, true>(ka, grid, l.shape.block_size, l.plan.waves, st);
  if (e != hipSuccess) return e;
  const float* op = ka.o_part;
  const float* lp = ka.lse_part;
  const int32_t* cl = ka.cl;
  void* out = ka.out;
  int32_t S = l.plan.splits, P = l.plan.partition_tokens;
  void* args[] = {(void*)&op, (void*)&lp, (void*)&cl, (void*)&out, (void*)&S, (void*)&P};
  return hipLaunchKernel((const void*)&pd_merge_kernel<BF16>, dim3(l.shape.Hq, l.shape.B),
                         dim3(D), args, 0, st);
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
    ka.o_part = (float*)l.workspace;
    ka.lse_part = (float*)((char*)l.workspace + partials_bytes(l.shape, l.plan));
  }
  ka.Hkv = l.shape.Hkv;
  ka.MB = l.shape.max_blocks_per_seq;
  ka.S = l.plan.splits;
  ka.P = l.plan.partition_tokens;
  ka.Pw = l.plan.wave_tokens;
  ka.scale_log2 = l.scale * 1.4426950408889634f;
  ka.blk_bytes = (uint32_t)l.shape.block_size * (uint32_t)l.shape.Hkv * kRowBytes;
  hipStream_t st = (hipStream_t)l.stream;
  hipError_t e = l.shape.dtype == PD_DTYPE_BF16 ? launch_all<true>(ka, l, st)
                                                : launch_all<false>(ka, l, st);
  return e == hipSuccess ? PD_OK : PD_ERR_HIP;
}

}  // namespace pd
