// Paged GQA decode attention kernels for gfx950 (CDNA4, wave64).
//
// Method (Loom Kernels home page, "Supported now": paged MQA/GQA decode with
// GQA packing and local split-K/LSE): one query token per head attends over
// a paged K/V cache; the 4 query heads that share a KV head are served by one
// pass over that head's K/V bytes, and a long context is cut into
// partitions whose normalised partial outputs and log-sum-exps are merged.
//
// Decode kernel, one workgroup per (partition p, KV head g, sequence b):
//   * lanes: 8 lanes per token row. A wave step covers 8 consecutive tokens;
//     lane (tg = lane/8, sl = lane%8) owns token tg of the step and the
//     16 head-dim elements [8sl, 8sl+8) and [64+8sl, 64+8sl+8). Each row is
//     256 contiguous bytes, so one 128-bit load instruction of the wave reads
//     eight whole 128-byte lines.
//   * K/V come straight from HBM into registers with bounds-checked buffer
//     loads whose resource is the current physical block (base = pool +
//     id * block bytes, size = block bytes). Lanes whose token lies past the
//     context get an offset beyond the block: the hardware returns zeros and
//     issues no memory access.
//   * block ids: each lane of a wave loads one block-table entry of the
//     wave's range up front; a step takes its (wave-uniform) id with
//     v_readlane, so the address is scalar and known before the K/V loads.
//   * scores: q stays as packed 16-bit pairs; v_dot2_f32_{bf16,f16} gives
//     fp32 products-and-sums with no conversion of K, then a 3-step DPP
//     butterfly over the 8 lanes of a row, then one multiply by
//     scale*log2(e) so the softmax runs in base 2 (v_exp_f32).
//   * softmax: per head, a wave-uniform running maximum updated once per
//     batch of steps (DPP + permlane16/32 swaps across the 8 token groups),
//     each lane keeping its own partial sum l and accumulator acc[4][16].
//   * end of range: a reduce-scatter over token groups (permlane32_swap,
//     permlane16_swap, then DPP row_ror:8) leaves head r's 128 sums in row r
//     of the wave; waves of a workgroup are merged through LDS.
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
constexpr int G = pd::kGroup;    // 4
constexpr uint32_t kRowBytes = D * 2;        // one token row of one KV head
constexpr uint32_t kOutOfBlock = 0x80000000u;  // buffer offset that reads as zero
constexpr int kRsrcWord3 = 0x00020000;        // raw 32-bit buffer, gfx9 data format

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
constexpr int kRowRor8 = 0x128;      // lane i <- (i+8) mod 16 within the row

// Sum over the 8 lanes of a token row; every lane gets the total.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kHalfMirror>(x);
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

// Maximum over the 8 token groups of the wave (lanes with equal lane%8).
__device__ __forceinline__ float max_groups(float x) {
  x = fmaxf(x, dpp<kRowRor8>(x));
  float y;
  float a = swap16_lo(x, x, &y);
  x = fmaxf(a, y);
  a = swap32_lo(x, x, &y);
  return fmaxf(a, y);
}

// Sum over the 8 token groups of the wave.
__device__ __forceinline__ float sum_groups(float x) {
  x += dpp<kRowRor8>(x);
  float y;
  float a = swap16_lo(x, x, &y);
  x = a + y;
  a = swap32_lo(x, x, &y);
  return a + y;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const char* base, int32_t id,
                                                             uint32_t blk_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      (void*)(base + (int64_t)id * (int64_t)blk_bytes), (short)0, (int)blk_bytes, kRsrcWord3);
}

// One workgroup of NW waves per (partition, KV head, sequence).
// BS: block size (16 or 32). U: wave steps (8 tokens each) per batch.
template <bool BF16, int BS, int NW, int U, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void pd_decode_kernel(const KArgs a) {
  static_assert(BS % (8 * U) == 0, "a batch must stay inside one block");
  constexpr int SPB = BS / 8;  // wave steps per block
  const int p = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int Hq = a.Hkv * G;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tg = lane >> 3;
  const int sl = lane & 7;
  const int row = lane >> 4;  // head this lane holds after the final reduction

  const int L = a.cl[b];
  const int t0 = p * a.P;

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
  const int t1 = min(t0 + a.P, L);

  // wave sub-range, block aligned
  const int Pw = ((a.P + NW - 1) / NW + BS - 1) / BS * BS;
  const int tw0 = t0 + w * Pw;
  const int tw1 = min(tw0 + Pw, t1);

  // q of the group's 4 heads: this lane's 16 elements of each, as packed pairs
  const uint16_t* qp = a.q + ((size_t)b * Hq + (size_t)g * G) * D;
  u32x4 qa[G], qb[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    qa[h] = *(const u32x4*)(qp + h * D + sl * 8);
    qb[h] = *(const u32x4*)(qp + h * D + 64 + sl * 8);
  }

  float acc[G][16];
  float l[G], m[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = 0.f;
    m[h] = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
  }
  const float c = a.scale_log2;

  if (tw0 < tw1) {
    const int bi0 = tw0 / BS;
    const int nblk = (tw1 - 1) / BS - bi0 + 1;
    const int32_t* btrow = a.bt + (size_t)b * a.MB + bi0;
    const uint32_t lane_off = ((uint32_t)tg * a.Hkv + g) * kRowBytes + sl * 16u;
    const uint32_t step_bytes = 8u * a.Hkv * kRowBytes;

    for (int cb = 0; cb < nblk; cb += 64) {
      const int nb_here = min(64, nblk - cb);
      const int myid = lane < nb_here ? btrow[cb + lane] : 0;
      for (int jb = 0; jb < nb_here; ++jb) {
        const int id = __builtin_amdgcn_readlane(myid, jb);
        const int blk_tok0 = (bi0 + cb + jb) * BS;
        const __amdgpu_buffer_rsrc_t rk = block_rsrc(a.k, id, a.blk_bytes);
        const __amdgpu_buffer_rsrc_t rv = block_rsrc(a.v, id, a.blk_bytes);
#pragma unroll
        for (int ub = 0; ub < SPB; ub += U) {
          if (blk_tok0 + ub * 8 >= tw1) break;  // rest of the block is past the range
          u32x4 kr[U][2], vr[U][2];
          bool valid[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int tok = blk_tok0 + (ub + u) * 8 + tg;
            valid[u] = tok < tw1;
            // the whole offset goes in the vector operand, which the range check covers
            const uint32_t vo = (valid[u] ? lane_off : kOutOfBlock) + (ub + u) * step_bytes;
            kr[u][0] = __builtin_amdgcn_raw_buffer_load_b128(rk, vo, 0, 0);
            kr[u][1] = __builtin_amdgcn_raw_buffer_load_b128(rk, vo + 128u, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const uint32_t vo = (valid[u] ? lane_off : kOutOfBlock) + (ub + u) * step_bytes;
            vr[u][0] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo, 0, 0);
            vr[u][1] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + 128u, 0, 0);
          }
          // scores (log2 domain)
          float s[U][G];
#pragma unroll
          for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
              float d = 0.f;
#pragma unroll
              for (int i = 0; i < 4; ++i) d = dot2<BF16>(qa[h][i], kr[u][0][i], d);
#pragma unroll
              for (int i = 0; i < 4; ++i) d = dot2<BF16>(qb[h][i], kr[u][1][i], d);
              d = sum8(d);
              s[u][h] = valid[u] ? d * c : -INFINITY;
            }
          }
          // running maximum, wave-uniform per head
          bool grow = false;
          float mn[G];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float bm = s[0][h];
#pragma unroll
            for (int u = 1; u < U; ++u) bm = fmaxf(bm, s[u][h]);
            bm = max_groups(bm);
            mn[h] = fmaxf(m[h], bm);
            grow |= mn[h] > m[h];
          }
          if (grow) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const float alpha = exp2_fast(m[h] - mn[h]);
              l[h] *= alpha;
#pragma unroll
              for (int e = 0; e < 16; ++e) acc[h][e] *= alpha;
              m[h] = mn[h];
            }
          }
          // weights and PV
#pragma unroll
          for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const float pr = exp2_fast(s[u][h] - m[h]);
              l[h] += pr;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                acc[h][2 * i] = fmaf(pr, lo_f<BF16>(vr[u][0][i]), acc[h][2 * i]);
                acc[h][2 * i + 1] = fmaf(pr, hi_f<BF16>(vr[u][0][i]), acc[h][2 * i + 1]);
                acc[h][8 + 2 * i] = fmaf(pr, lo_f<BF16>(vr[u][1][i]), acc[h][8 + 2 * i]);
                acc[h][9 + 2 * i] = fmaf(pr, hi_f<BF16>(vr[u][1][i]), acc[h][9 + 2 * i]);
              }
            }
          }
        }
      }
    }
  }

  // ---- reduce over the 8 token groups of the wave
#pragma unroll
  for (int h = 0; h < G; ++h) l[h] = sum_groups(l[h]);
  // reduce-scatter: rows 0-1 keep heads {0,1}, rows 2-3 keep heads {2,3} ...
  float r1[2][16];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float y;
      const float x = swap32_lo(acc[hh][e], acc[hh + 2][e], &y);
      r1[hh][e] = x + y;
    }
  // ... then row r keeps head r ...
  float r2[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float y;
    const float x = swap16_lo(r1[0][e], r1[1][e], &y);
    r2[e] = x + y;
  }
  // ... and the two 8-lane halves of each row are summed.
#pragma unroll
  for (int e = 0; e < 16; ++e) r2[e] += dpp<kRowRor8>(r2[e]);

  const float m_r = row == 0 ? m[0] : row == 1 ? m[1] : row == 2 ? m[2] : m[3];
  const float l_r = row == 0 ? l[0] : row == 1 ? l[1] : row == 2 ? l[2] : l[3];
  const bool writer = (lane & 8) == 0;  // first 8 lanes of each row
  const int h_out = g * G + row;

  if constexpr (NW == 1) {
    if (writer) {
      if constexpr (!SPLIT) {
        const float inv = 1.0f / l_r;
        uint16_t* o = (uint16_t*)a.out + ((size_t)b * Hq + h_out) * D;
        u32x4 w0, w1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w0[i] = pack2<BF16>(r2[2 * i] * inv, r2[2 * i + 1] * inv);
          w1[i] = pack2<BF16>(r2[8 + 2 * i] * inv, r2[9 + 2 * i] * inv);
        }
        *(u32x4*)(o + sl * 8) = w0;
        *(u32x4*)(o + 64 + sl * 8) = w1;
      } else {
        const float inv = 1.0f / l_r;
        const size_t slot = ((size_t)b * Hq + h_out) * a.S + p;
        float* o = a.o_part + slot * D;
        *(f32x4*)(o + sl * 8) = f32x4{r2[0] * inv, r2[1] * inv, r2[2] * inv, r2[3] * inv};
        *(f32x4*)(o + sl * 8 + 4) = f32x4{r2[4] * inv, r2[5] * inv, r2[6] * inv, r2[7] * inv};
        *(f32x4*)(o + 64 + sl * 8) =
            f32x4{r2[8] * inv, r2[9] * inv, r2[10] * inv, r2[11] * inv};
        *(f32x4*)(o + 64 + sl * 8 + 4) =
            f32x4{r2[12] * inv, r2[13] * inv, r2[14] * inv, r2[15] * inv};
        if (sl == 0) a.lse_part[slot] = m_r + __builtin_amdgcn_logf(l_r);
      }
    }
  } else {
    // ---- merge the NW waves through LDS
    __shared__ float s_acc[NW][G][D];
    __shared__ float s_m[NW][G];
    __shared__ float s_l[NW][G];
    if (writer) {
      float* dst = &s_acc[w][row][0];
      *(f32x4*)(dst + sl * 8) = f32x4{r2[0], r2[1], r2[2], r2[3]};
      *(f32x4*)(dst + sl * 8 + 4) = f32x4{r2[4], r2[5], r2[6], r2[7]};
      *(f32x4*)(dst + 64 + sl * 8) = f32x4{r2[8], r2[9], r2[10], r2[11]};
      *(f32x4*)(dst + 64 + sl * 8 + 4) = f32x4{r2[12], r2[13], r2[14], r2[15]};
      if (sl == 0) {
        s_m[w][row] = m_r;
        s_l[w][row] = l_r;
      }
    }
    __syncthreads();
    for (int o = threadIdx.x; o < G * D; o += NW * 64) {
      const int h = o / D;
      const int d = o % D;
      float M = s_m[0][h];
#pragma unroll
      for (int i = 1; i < NW; ++i) M = fmaxf(M, s_m[i][h]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const float wt = exp2_fast(s_m[i][h] - M);
        num = fmaf(wt, s_acc[i][h][d], num);
        den = fmaf(wt, s_l[i][h], den);
      }
      const int hq = g * G + h;
      if constexpr (!SPLIT) {
        uint16_t* out = (uint16_t*)a.out + ((size_t)b * Hq + hq) * D;
        out[d] = to_bits<BF16>(num / den);
      } else {
        const size_t slot = ((size_t)b * Hq + hq) * a.S + p;
        a.o_part[slot * D + d] = num / den;
        if (d == 0) a.lse_part[slot] = M + __builtin_amdgcn_logf(den);
      }
    }
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
  constexpr int U = 2;
  void* args[] = {(void*)&ka};
  return hipLaunchKernel((const void*)&pd_decode_kernel<BF16, BS, NW, U, SPLIT>, grid,
                         dim3(NW * 64), args, 0, st);
}

template <bool BF16, int BS, bool SPLIT>
hipError_t pick_waves(const KArgs& ka, dim3 grid, int nw, hipStream_t st) {
  switch (nw) {
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
  ka.scale_log2 = l.scale * 1.4426950408889634f;
  ka.blk_bytes = (uint32_t)l.shape.block_size * (uint32_t)l.shape.Hkv * kRowBytes;
  hipStream_t st = (hipStream_t)l.stream;
  hipError_t e = l.shape.dtype == PD_DTYPE_BF16 ? launch_all<true>(ka, l, st)
                                                : launch_all<false>(ka, l, st);
  return e == hipSuccess ? PD_OK : PD_ERR_HIP;
}

}  // namespace pd
