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

// The heuristic is tuned for a whole MI355X: 256 CUs of 4 SIMDs. It does not
// query the device (plan and workspace queries are pure functions of the
// shape); on a device with fewer CUs the same plan runs, equally correct.
constexpr int64_t kCUs = 256;
constexpr int64_t kFillWaves = 4 * kCUs;  // one wave per SIMD
constexpr int64_t kWaves = 4;         // waves per workgroup
constexpr int64_t kTileTok = 16;      // tokens per K/V tile of a wave
constexpr int64_t kMinSplitTiles = 2;  // tiles per wave a split must leave
constexpr int64_t kNoSplitTiles = 4;   // tiles per wave below which a split never pays
constexpr int64_t kPairTiles = 16;     // tiles per wave from which split KV heads go in pairs
constexpr int64_t kMergeBatch = 16;    // partitions the merge kernel loads in one batch
constexpr int64_t kMaxSplits = 65535;  // grid z

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

int32_t check_shape(const Shape& s) {
  if (s.dtype != PD_DTYPE_F16 && s.dtype != PD_DTYPE_BF16) return PD_ERR_DTYPE;
  if (s.B < 0 || s.Hq < 1 || s.Hkv < 1 || s.D < 1 || s.block_size < 1 ||
      s.max_blocks_per_seq < 1)
    return PD_ERR_SHAPE;
  if (s.Hq % s.Hkv != 0) return PD_ERR_SHAPE;
  if ((int64_t)s.max_blocks_per_seq * s.block_size > INT_MAX / 2) return PD_ERR_SHAPE;
  if ((s.D != 64 && s.D != 128) || s.Hq / s.Hkv > kMaxGroup) return PD_ERR_UNSUPPORTED;
  if (s.block_size != 16 && s.block_size != 32) return PD_ERR_UNSUPPORTED;
  // grid limits: (Hkv / NH, B, S) with y and z below 65536
  if (s.B > 65535 || s.Hkv > 65535) return PD_ERR_SHAPE;
  return PD_OK;
}

// The plan cuts each sequence's context (up to cap = max_blocks_per_seq *
// block_size tokens) into S partitions of P tokens, each served by one
// workgroup of 4 waves per group of NH KV heads; a wave covers one slice of
// Pw tokens (block aligned, at most 256 blocks) of one head, in tiles of 16.
// Slices of a head merge in LDS, partitions merge across workgroups. A KV
// head with more than 16 query heads (MQA) counts as HS virtual KV heads,
// paired in a workgroup when HS is even.
//
// The rule was fitted to sweeps of every (NH, NT, S) on an MI355X over the
// decode workloads (batch 1..64, contexts 16..4,096, block sizes 16/32):
//   * a call runs best with about one wave per SIMD (kFillWaves) in
//     workgroups of 4 waves: NH = 1, NT = 4 while B * Hkv < 512, else KV
//     heads in pairs (NH = 2, NT = 2, the pair reads 512 contiguous bytes
//     per token);
//   * when B * Hkv * NT / NH waves would leave SIMDs idle, the context is
//     split until they are filled, keeping at least kMinSplitTiles tiles per
//     wave; a split costs the partials' round trip through memory and a
//     second kernel that merges them, so it is not used when a wave would
//     have at most kNoSplitTiles tiles without it;
//   * a split call whose waves still have kPairTiles or more tiles each
//     does better with KV heads in pairs and twice the partitions;
//   * a split call that still has fewer workgroups than CUs (a small batch
//     whose split the kMinSplitTiles floor capped) takes workgroups of two
//     waves and up to twice the partitions, kept within one merge batch
//     (kMergeBatch): the same waves then spread over twice the CUs, and one
//     CU reads at most some 44 GB/s;
//   * tiles with more work per byte (an FP8 cache; 16 query heads per wave
//     at D 64) take four slices per KV-head pair instead of two, which puts
//     two waves on each SIMD (S and P are unchanged); an unsplit FP8 call
//     with one KV head per workgroup likewise takes eight slices instead
//     of four.
// A forced S fixes P instead and cuts it into up to NT slices.
int32_t make_plan(const Shape& s, int32_t requested_splits, Plan* plan, bool kv_fp8) {
  int32_t st = check_shape(s);
  if (st != PD_OK) return st;
  const int64_t bs = s.block_size;
  const int64_t cap = (int64_t)s.max_blocks_per_seq * bs;  // longest possible context
  // a wave serves at most 16 query heads: split each KV head into the fewest
  // virtual heads of equal size that respects that
  const int64_t G = s.Hq / s.Hkv;
  int64_t hs = 1;
  while (G % hs != 0 || G / hs > 16) ++hs;
  const int64_t hkv = s.Hkv * hs;  // virtual KV heads
  const int64_t units = (int64_t)(s.B > 0 ? s.B : 1) * hkv;
  const int64_t pw_max = kMaxWaveBlocks * bs;
  // virtual heads of one KV head pair up, so both waves of a pair read the
  // same blocks
  const bool pairs = hkv % 2 == 0;
  int64_t nh = pairs && (hs % 2 == 0 || units >= 2 * kFillWaves / kWaves) ? 2 : 1;
  int64_t nt = kWaves / nh;
  int64_t P;
  if (requested_splits > 0) {
    const int64_t want = requested_splits > kMaxSplits ? kMaxSplits : requested_splits;
    P = round_up(ceil_div(cap, want), bs);
  } else {
    int64_t S = 1;
    if (units * nt < kFillWaves && ceil_div(cap, nt * kTileTok) > kNoSplitTiles) {
      S = ceil_div(kFillWaves, units * nt);
      const int64_t s_max = cap / (nt * kMinSplitTiles * kTileTok);
      if (S > s_max) S = s_max;
      if (S < 1) S = 1;
      if (S > 1 && pairs && nh == 1 && cap / (S * nt) >= kPairTiles * kTileTok) {
        nh = 2;
        nt = kWaves / nh;
        S *= 2;
      }
      if (nh == 1 && nt == 4 && S > 1 && units * S < kCUs) {
        int64_t s2 = ceil_div(kFillWaves, units * 2);
        const int64_t s2_max = cap / (2 * kMinSplitTiles * kTileTok);
        if (s2 > s2_max) s2 = s2_max;
        if (s2 > kMergeBatch) s2 = kMergeBatch;
        if (s2 > S) {
          nt = 2;
          S = s2;
        }
      }
    }
    P = round_up(ceil_div(cap, S), bs);
  }
  if (nh * nt > kMaxWaves) nt = kMaxWaves / nh;
  if (nt > P / bs) nt = P / bs;  // every slice at least one block
  int64_t pw = round_up(ceil_div(P, nt), bs);
  if (pw > pw_max) {  // a slice cannot exceed 256 blocks: split more
    pw = pw_max;
    P = nt * pw;
  }
  // tiles with more work per byte (FP8 codes widened in registers; 16 query
  // heads per wave at D 64) run better with two waves per SIMD: paired KV
  // heads then cut the partition, now fixed, into four slices instead of two
  if (nh == 2 && nt == 2 && (kv_fp8 || (s.D == 64 && G / hs > 8)) && P / bs > 2) {
    nt = P / bs < 4 ? P / bs : 4;
    pw = round_up(ceil_div(P, nt), bs);
  }
  // likewise an unsplit FP8 call with one KV head per workgroup: eight
  // slices instead of four (a split one keeps four: its merge then reads
  // twice the slices and costs more than the second wave per SIMD gains)
  if (nh == 1 && nt == 4 && kv_fp8 && ceil_div(cap, P) == 1 && P / bs >= 8) {
    nt = 8;
    pw = round_up(ceil_div(P, nt), bs);
  }
  nt = ceil_div(P, pw);  // drop slices that would start past the partition
  const int64_t S = ceil_div(cap, P);
  if (S > kMaxSplits) return PD_ERR_SHAPE;
  if (hkv > 65535) return PD_ERR_SHAPE;
  // the merge kernel runs one workgroup per (sequence, query head): keep
  // their count within int32
  if (S > 1 && (int64_t)s.B * s.Hq > INT_MAX) return PD_ERR_SHAPE;
  plan->splits = (int32_t)S;
  plan->partition_tokens = (int32_t)P;
  plan->heads_per_group = (int32_t)nh;
  plan->slices = (int32_t)nt;
  plan->wave_tokens = (int32_t)pw;
  plan->head_split = (int32_t)hs;
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
  return partials_bytes(s, p) + lse_bytes(s, p);
}

}  // namespace pd
