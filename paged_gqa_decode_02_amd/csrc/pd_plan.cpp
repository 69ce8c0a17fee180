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

constexpr int64_t kWavesSmall = 1024;       // waves for latency-bound calls
constexpr int64_t kWavesLarge = 2048;       // waves for streaming calls
constexpr int64_t kSmallWork = 128 * 1024;  // token-heads up to which a call is latency-bound
constexpr int64_t kPairWork = 256 * 1024;   // token-heads from which KV heads go in pairs
constexpr int64_t kSlices = 4;              // token slices per head in a workgroup
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
// block_size tokens) into S partitions of P tokens, each served by one
// workgroup per group of NH KV heads, made of NH x NT waves; a wave covers
// one slice of Pw tokens (block aligned, at most 256 blocks) of one head.
// Slices of a head merge in LDS, partitions merge across workgroups.
//
// The rule was fitted to sweeps of every (NH, NT, S) on an MI355X over the
// decode workloads (batch 1..64, contexts 16..4,096, block sizes 16/32):
//   * work = B * Hkv * cap token-heads sets the number of waves: about
//     kWavesSmall for work up to kSmallWork (latency-bound calls: all of a
//     wave's loads go out at once), kWavesLarge beyond (streaming calls:
//     two resident waves per SIMD, each with a long slice, beat four with
//     short ones), so Pw = work / waves, at least one block;
//   * NT = 4 slices per head (NT = 8 or 16 only added waiting for the
//     slowest wave; NT = 1 or 2 added cross-workgroup merges);
//   * NH = 2 heads per workgroup once work reaches kPairWork (the pair reads
//     512 contiguous bytes per token), else 1.
// S and P follow from NT * Pw. A forced S fixes P instead and cuts it into
// up to NT slices.
int32_t make_plan(const Shape& s, int32_t requested_splits, Plan* plan) {
  int32_t st = check_shape(s);
  if (st != PD_OK) return st;
  const int64_t bs = s.block_size;
  const int64_t cap = (int64_t)s.max_blocks_per_seq * bs;  // longest possible context
  const int64_t units = (int64_t)(s.B > 0 ? s.B : 1) * s.Hkv;
  const int64_t work = units * cap;
  const int64_t pw_max = kMaxWaveBlocks * bs;
  const int64_t waves = work <= kSmallWork ? kWavesSmall : kWavesLarge;
  int64_t nh = work >= kPairWork && s.Hkv % 2 == 0 ? 2 : 1;
  int64_t nt = kSlices;
  int64_t pw, P;
  if (requested_splits > 0) {
    const int64_t want = requested_splits > kMaxSplits ? kMaxSplits : requested_splits;
    P = round_up(ceil_div(cap, want), bs);
  } else {
    pw = round_up(ceil_div(work, waves), bs);
    if (pw > pw_max) pw = pw_max;
    P = nt * pw;
    if (P > cap) P = cap;  // one partition
  }
#ifdef PD_FORCE_NT  // tuning builds only: fix the slices per workgroup
  if (PD_FORCE_NT > 0) nt = PD_FORCE_NT;
#endif
  if (nt > P / bs) nt = P / bs;  // every slice at least one block
  pw = round_up(ceil_div(P, nt), bs);
  if (pw > pw_max) {  // a slice cannot exceed 256 blocks: split more
    pw = pw_max;
    P = nt * pw;
  }
  nt = ceil_div(P, pw);  // drop slices that would start past the partition
#ifdef PD_FORCE_NH  // tuning builds only: fix the KV heads per workgroup
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
