// RoPE + paged KV-cache write, and the cos/sin table it reads, for gfx950.
//
// Operation (Loom Kernels home page, "Supported now": "RoPE + paged-KV write",
// a packed Q/K rotation with a write into the native cache; it is the step
// that fills the cache the paged decode reads): for token t at position
// m = positions[t], every query and key head vector is rotated pair by pair,
// pair i = (x[i], x[i + D/2]) by the angle m * theta_i, theta_i =
// base^(-2i/D) (RoFormer, section 3.2, with rotate-half pairing); the rotated
// query goes to q_out, and the rotated key and the unchanged value go to
// cache slot slot_mapping[t] (block slot / block_size, row slot %
// block_size), which in the [num_blocks, block_size, Hkv, D] layout is simply
// row slot of a [num_blocks * block_size, Hkv, D] array.
//
// The write kernel is a pure stream: one thread per "unit", 8 elements of
// the first half of a head vector and their 8 partners in the second half
// (two 16-byte loads and two 16-byte stores), so a head of dimension D is
// D/16 units and a token (Hq + 2 Hkv) * D/16. Eight consecutive lanes cover
// one half-head (128 contiguous bytes at D = 128) and the two halves are
// issued back to back, so every 128-byte line of the token's rows is fully
// used. The rotation widens the 16-bit inputs exactly, reads the token's
// float32 cos/sin row (32 bytes of each per unit), computes in fp32 and
// rounds each output once to the dtype, round-to-nearest-even; value units
// are a bit-for-bit copy.
//
// Into an FP8 cache (home page, "Next boundaries": FP8 KV-cache
// compression) the K/V units store OCP E4M3FN codes, one byte per element,
// with one float32 scale per tensor: the code of x is the E4M3FN value
// nearest to x times the float32 reciprocal of the scale, ties to even,
// magnitudes past 448 held at 448. Keys are rotated in float32 in a fixed
// order, x' = fl(fl(x c) - fl(y s)) and y' = fl(fl(y c) + fl(x s)) (no fused
// multiply-add), then multiplied by fl(1 / k_scale); values are widened
// exactly and multiplied by fl(1 / v_scale). The query output stays 16-bit.
//
// The table kernel evaluates theta_i, the angle and its cosine and sine in
// fp64 and rounds each entry once to float32, so the table is the float32
// rounding of the exact one whatever the position (a float32 angle would be
// off by up to ~2e-3 rad at position 32768).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/paged_decode.h"
#include "pd_internal.h"

// e4m3_code: float32 -> OCP E4M3FN code (nearest value, ties to even,
// magnitudes from 464 up held at 448, NaN to 0x7F), built for the device
#define PD_FP8_FN __device__ __forceinline__
#include "pd_fp8_code.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

struct RopeArgs {
  const char* q;
  const char* k;
  const char* v;
  int64_t q_stride, k_stride, v_stride;  // bytes from one token's row to the next
  const int32_t* positions;
  const int32_t* slots;
  const float* table;  // [max_position, D]: cos of pair i at i, sin at D/2 + i
  char* q_out;         // [T, Hq, D]
  char* k_cache;       // [num_slots, Hkv, D]
  char* v_cache;
  int64_t num_slots;   // num_blocks * block_size
  int32_t max_position;
  int32_t T, Hq, Hkv, D;
  int32_t units_head;   // D / 16
  int32_t units_token;  // (Hq + 2 Hkv) * D / 16
  float k_inv, v_inv;  // FP8 caches: code = E4M3FN(x * inv), inv = fl(1 / scale)
};

// 8 16-bit values (one 16-byte chunk) <-> fp32, exact widening and
// round-to-nearest-even narrowing.
template <bool BF16>
__device__ __forceinline__ void widen8(const u32x4 x, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BF16) {
      f[2 * i] = __builtin_bit_cast(float, x[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, x[i] & 0xffff0000u);
    } else {
      f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(x[i] & 0xffffu));
      f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(x[i] >> 16));
    }
  }
}

template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  uint16_t lo, hi;
  if constexpr (BF16) {
    lo = __builtin_bit_cast(uint16_t, (__bf16)a);
    hi = __builtin_bit_cast(uint16_t, (__bf16)b);
  } else {
    lo = __builtin_bit_cast(uint16_t, (_Float16)a);
    hi = __builtin_bit_cast(uint16_t, (_Float16)b);
  }
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Rotation of the pairs (x[i], y[i]) in the order the FP8 write fixes.
__device__ __forceinline__ void rotate_exact(const float (&x)[8], const float (&y)[8],
                                             const float (&c)[8], const float (&s)[8],
                                             float (&rx)[8], float (&ry)[8]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float xc = x[i] * c[i], ys = y[i] * s[i], yc = y[i] * c[i], xs = x[i] * s[i];
    rx[i] = xc - ys;
    ry[i] = yc + xs;
  }
}

// 8 values -> 8 codes of x * inv (inv the float32 reciprocal of the scale),
// byte i = value i.
__device__ __forceinline__ u32x2 codes8(const float (&x)[8], float inv) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i / 4] |= e4m3_code(x[i] * inv) << (8 * (i % 4));
  return u32x2{w[0], w[1]};
}

template <bool BF16, bool FP8>
__global__ __launch_bounds__(kThreads) void rope_kv_write_kernel(const RopeArgs a) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t t = g / a.units_token;
  if (t >= a.T) return;
  const int u = (int)(g - t * a.units_token);
  const int h = u / a.units_head;
  const int j = u - h * a.units_head;
  const int64_t head_bytes = 2 * (int64_t)a.D;
  const int64_t half = head_bytes / 2;
  const int64_t o = 16 * (int64_t)j;
  const bool is_q = h < a.Hq, is_k = !is_q && h < a.Hq + a.Hkv, is_v = !is_q && !is_k;
  const int hk = is_q ? 0 : is_k ? h - a.Hq : h - a.Hq - a.Hkv;
  const char* src = is_q ? a.q + t * a.q_stride + h * head_bytes
                         : (is_k ? a.k + t * a.k_stride : a.v + t * a.v_stride) + hk * head_bytes;
  // the data loads do not wait for the position and slot checks
  const int32_t pos = a.positions[t];
  const int32_t slot = is_q ? 0 : a.slots[t];
  u32x4 x1 = *(const u32x4*)(src + o);
  u32x4 x2 = *(const u32x4*)(src + half + o);
  // a token whose position is outside the table is skipped entirely;
  // padding (negative slot) and slots outside the pool write no K/V
  if ((uint32_t)pos >= (uint32_t)a.max_position) return;
  if (!is_q && (slot < 0 || (int64_t)slot >= a.num_slots)) return;
  if constexpr (FP8) {
    if (!is_q) {
      // one byte per cached element: codes of 8 elements at 8 j and their
      // partners at D/2 + 8 j
      char* dst = (is_k ? a.k_cache : a.v_cache) + ((int64_t)slot * a.Hkv + hk) * a.D;
      float e1[8], e2[8];
      widen8<BF16>(x1, e1);
      widen8<BF16>(x2, e2);
      u32x2 w1, w2;
      if (is_k) {
        const float* row = a.table + (int64_t)pos * a.D + 8 * j;
        const f32x4 c0 = *(const f32x4*)row, c1 = *(const f32x4*)(row + 4);
        const f32x4 s0 = *(const f32x4*)(row + a.D / 2), s1 = *(const f32x4*)(row + a.D / 2 + 4);
        const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        float r1[8], r2[8];
        rotate_exact(e1, e2, c, s, r1, r2);
        w1 = codes8(r1, a.k_inv);
        w2 = codes8(r2, a.k_inv);
      } else {
        w1 = codes8(e1, a.v_inv);
        w2 = codes8(e2, a.v_inv);
      }
      *(u32x2*)(dst + 8 * j) = w1;
      *(u32x2*)(dst + a.D / 2 + 8 * j) = w2;
      return;
    }
  }
  char* dst = is_q ? a.q_out + (t * a.Hq + h) * head_bytes
                   : (is_k ? a.k_cache : a.v_cache) + ((int64_t)slot * a.Hkv + hk) * head_bytes;
  if (!is_v) {
    const float* row = a.table + (int64_t)pos * a.D + 8 * j;
    const f32x4 c0 = *(const f32x4*)row, c1 = *(const f32x4*)(row + 4);
    const f32x4 s0 = *(const f32x4*)(row + a.D / 2), s1 = *(const f32x4*)(row + a.D / 2 + 4);
    const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    float e1[8], e2[8], r1[8], r2[8];
    widen8<BF16>(x1, e1);
    widen8<BF16>(x2, e2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      r1[i] = e1[i] * c[i] - e2[i] * s[i];
      r2[i] = e2[i] * c[i] + e1[i] * s[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x1[i] = pack2<BF16>(r1[2 * i], r1[2 * i + 1]);
      x2[i] = pack2<BF16>(r2[2 * i], r2[2 * i + 1]);
    }
  }
  *(u32x4*)(dst + o) = x1;
  *(u32x4*)(dst + half + o) = x2;
}

__global__ __launch_bounds__(kThreads) void rope_table_kernel(float* table, int32_t max_position,
                                                              int32_t D, double base) {
  const int half = D / 2;
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g >= (int64_t)max_position * half) return;
  const int64_t p = g / half;
  const int i = (int)(g - p * half);
  const double theta = pow(base, (-2.0 * i) / D);
  const double ang = (double)p * theta;
  table[p * D + i] = (float)cos(ang);
  table[p * D + half + i] = (float)sin(ang);
}

}  // namespace

namespace pd {

int32_t launch_rope_table(float* table, int32_t max_position, int32_t D, double base,
                          void* stream) {
  const int64_t n = (int64_t)max_position * (D / 2);
  const unsigned blocks = (unsigned)((n + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     table, max_position, D, base);
  return hipGetLastError() == hipSuccess ? PD_OK : PD_ERR_HIP;
}

int32_t launch_rope_kv_write(const RopeLaunch& l) {
  RopeArgs a;
  a.q = (const char*)l.q;
  a.k = (const char*)l.k;
  a.v = (const char*)l.v;
  a.q_stride = 2 * l.q_row_stride;
  a.k_stride = 2 * l.k_row_stride;
  a.v_stride = 2 * l.v_row_stride;
  a.positions = l.positions;
  a.slots = l.slot_mapping;
  a.table = l.cos_sin;
  a.q_out = (char*)l.q_out;
  a.k_cache = (char*)l.k_cache;
  a.v_cache = (char*)l.v_cache;
  a.num_slots = (int64_t)l.num_blocks * l.block_size;
  a.max_position = l.max_position;
  a.T = l.T;
  a.Hq = l.Hq;
  a.Hkv = l.Hkv;
  a.D = l.D;
  a.units_head = l.D / 16;
  a.units_token = (l.Hq + 2 * l.Hkv) * a.units_head;
  // correctly rounded float32 reciprocals, once on the host
  a.k_inv = 1.0f / l.k_scale;
  a.v_inv = 1.0f / l.v_scale;
  const int64_t n = (int64_t)l.T * a.units_token;
  const unsigned blocks = (unsigned)((n + kThreads - 1) / kThreads);
  const hipStream_t st = (hipStream_t)l.stream;
  const bool bf16 = l.dtype == PD_DTYPE_BF16;
  if (l.kv_fp8) {
    if (bf16)
      hipLaunchKernelGGL((rope_kv_write_kernel<true, true>), dim3(blocks), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((rope_kv_write_kernel<false, true>), dim3(blocks), dim3(kThreads), 0, st, a);
  } else if (bf16) {
    hipLaunchKernelGGL((rope_kv_write_kernel<true, false>), dim3(blocks), dim3(kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((rope_kv_write_kernel<false, false>), dim3(blocks), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? PD_OK : PD_ERR_HIP;
}

}  // namespace pd
