// Host-side shape checks and the split-count heuristic.
//
// The split count is chosen per (batch, context) shape: the Loom Kernels
// benchmark page ("What the ratios mean") describes the decode route as
// shape-gated, with short contexts and a long-context split-K/LSE path. Here
// that becomes one kernel family whose partition count S is a pure function
// of the host-visible shape, so results are reproducible call to call and
// the same plan is baked into a captured graph.
#include <limits.h>

#include "../../include/paged_decode.h"
#include "pd_internal.h"

namespace pd {

namespace {

#ifndef PD_WAVES_PER_CU
#define PD_WAVES_PER_CU 16  // resident decode waves per CU (4 per SIMD at 128 VGPRs)
#endif
constexpr int64_t kCUs = 256;  // MI355X compute units
constexpr int64_t kTargetWaves = kCUs * PD_WAVES_PER_CU;
constexpr int64_t kMaxSplits = 1 << 16;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
int64_t pow2_ceil(int64_t x) {
  int64_t r = 1;
  while (r < x) r <<= 1;
  return r;
}
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

int32_t check_shape(const Shape& s) {
  if (s.dtype != PD_DTYPE_F16 && s.dtype != PD_DTYPE_BF16) return PD_ERR_DTYPE;
  if (s.B < 0 || s.Hq < 1 || s.Hkv < 1 || s.D < 1 || s.block_size < 1 ||
      s.max_blocks_per_seq < 1)
    return PD_ERR_SHAPE;
  if (s.Hq % s.Hkv != 0) return PD_ERR_SHAPE;
  if ((int64_t)s.max_blocks_per_seq * s.block_size > INT_MAX / 2) return PD_ERR_SHAPE;
  if (s.D != kHeadDim || s.Hq / s.Hkv != kGroup) return PD_ERR_UNSUPPORTED;
  if (s.block_size != 16 && s.block_size != 32) return PD_ERR_UNSUPPORTED;
  // grid limits: (S, Hkv, B) with y and z below 65536
  if (s.B > 65535 || s.Hkv > 65535) return PD_ERR_SHAPE;
  return PD_OK;
}

// The plan cuts each sequence's context (up to cap = max_blocks_per_seq *
// block_size tokens) into S partitions of P tokens, each served by
// workgroups of NH KV heads x NT token slices of Pw tokens. Pw is sized so
// that the whole grid is about one full round of resident waves
// (kTargetWaves): long work keeps every wave streaming, short work keeps
// every wave's loads in flight at once. Slices of one head merge in LDS,
// partitions merge across workgroups, so the plan first gives a head all the
// slices it needs inside one workgroup (NT up to 16, S = 1 when they fit),
// then fills the rest of the 16-wave workgroup with more KV heads (NH, a
// power of two dividing Hkv, at most 8) so that its waves read whole blocks.
// A forced S fixes P instead and sizes NT and Pw to it.
int32_t make_plan(const Shape& s, int32_t requested_splits, Plan* plan) {
  int32_t st = check_shape(s);
  if (st != PD_OK) return st;
  const int64_t bs = s.block_size;
  const int64_t cap = (int64_t)s.max_blocks_per_seq * bs;  // longest possible context
  const int64_t units = (int64_t)(s.B > 0 ? s.B : 1) * s.Hkv;
  int64_t nh_max = 8;
  while (s.Hkv % nh_max != 0) nh_max >>= 1;
  const int64_t pw_max = kMaxWaveBlocks * bs;
  int64_t pw_target = round_up(ceil_div(units * cap, kTargetWaves), bs);
  if (pw_target > pw_max) pw_target = pw_max;
  int64_t P, nt, pw;
  if (requested_splits > 0) {
    const int64_t want = requested_splits > kMaxSplits ? kMaxSplits : requested_splits;
    P = round_up(ceil_div(cap, want), bs);
    nt = pow2_ceil(ceil_div(P, pw_target));
  } else {
    nt = pow2_ceil(ceil_div(cap, pw_target));
    if (nt > kMaxWaves) nt = kMaxWaves;
    const int64_t s0 = ceil_div(cap, nt * pw_target);
    P = round_up(ceil_div(cap, s0), bs);
  }
  if (nt > kMaxWaves) nt = kMaxWaves;
  pw = round_up(ceil_div(P, nt), bs);
  if (pw > pw_max) {  // a slice cannot exceed 256 blocks: split more
    pw = pw_max;
    P = nt * pw;
  }
  nt = ceil_div(P, pw);  // drop slices that would start past the partition
  int64_t nh = nh_max;
  while (nh > 1 && nh * nt > kMaxWaves) nh >>= 1;
#ifdef PD_FORCE_NH
  if (PD_FORCE_NH > 0 && s.Hkv % PD_FORCE_NH == 0 && PD_FORCE_NH * nt <= kMaxWaves) nh = PD_FORCE_NH;
#endif
  const int64_t S = ceil_div(cap, P);
  if (S > kMaxSplits) return PD_ERR_SHAPE;
  // the split path keeps one arrival counter per (sequence, head group)
  if (S > 1 && (int64_t)s.B * (s.Hkv / nh) > kMaxCounters) return PD_ERR_UNSUPPORTED;
  plan->splits = (int32_t)S;
  plan->partition_tokens = (int32_t)P;
  plan->heads_per_group = (int32_t)nh;
  plan->slices = (int32_t)nt;
  plan->wave_tokens = (int32_t)pw;
  return PD_OK;
}

size_t partials_bytes(const Shape& s, const Plan& p) {
  return align256((size_t)s.B * s.Hq * p.splits * s.D * sizeof(float));
}

size_t lse_bytes(const Shape& s, const Plan& p) {
  return align256((size_t)s.B * s.Hq * p.splits * sizeof(float));
}

size_t workspace_bytes(const Shape& s, const Plan& p) {
  if (p.splits <= 1) return 0;
  return kCounterBytes + partials_bytes(s, p) + lse_bytes(s, p);
}

}  // namespace pd
