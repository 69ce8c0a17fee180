// Host-side driver of the C ABI's argument handling, built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by the CPU tests: the ABI
// sources (pd_api.cpp, pd_kv_api.cpp, pd_plan.cpp) are linked against stub
// launchers that only record what would be queued, so no GPU is needed.
// Random argument sets, valid and extreme (zero, negative, INT32_MAX sizes,
// NULL and misaligned pointers that are never dereferenced), go through
// every entry point; each must return a documented status code, and a
// launch may only be recorded for a call that returned PD_OK. The host
// compaction planner runs on real host arrays and its output is checked.
// Exit status 0 when every check holds.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../include/paged_decode.h"
#include "../include/paged_kv.h"
#include "../paged_gqa_decode_02_amd/csrc/pd_internal.h"

namespace {
int g_launches = 0;
int g_fail = 0;
#define CHECK(c)                                                             \
  do {                                                                       \
    if (!(c)) {                                                              \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);        \
      if (++g_fail > 20) exit(1);                                            \
    }                                                                        \
  } while (0)
}  // namespace

// stub launchers: record, check what the ABI promised them, queue nothing
namespace pd {
int32_t launch(const Launch& l) {
  ++g_launches;
  CHECK(l.shape.B > 0 && l.plan.splits >= 1 && l.plan.partition_tokens > 0);
  CHECK((int64_t)l.plan.splits * l.plan.partition_tokens >=
        (int64_t)l.shape.max_blocks_per_seq * l.shape.block_size);
  CHECK(l.plan.splits == 1 || l.workspace != nullptr);
  return PD_OK;
}
int32_t zero_workspace(void*, size_t, void*) {
  ++g_launches;
  return PD_OK;
}
int32_t launch_rope_kv_write(const RopeLaunch& l) {
  ++g_launches;
  CHECK(l.T > 0);
  return PD_OK;
}
int32_t launch_rope_table(float*, int32_t, int32_t, double, void*) {
  ++g_launches;
  return PD_OK;
}
int32_t launch_move_blocks(const MoveLaunch& l) {
  ++g_launches;
  CHECK(l.n > 0);
  return PD_OK;
}
int64_t move_chunk_bytes() { return 16384; }
int32_t launch_remap_table(int32_t*, int64_t entries, const int32_t*, int32_t, void*) {
  ++g_launches;
  CHECK(entries > 0);
  return PD_OK;
}
}  // namespace pd

namespace {

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t rnd() {
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return g_rng;
}

int32_t pick_int(const int32_t* vals, int n) { return vals[rnd() % n]; }

int32_t an_int() {
  static const int32_t v[] = {0, 1, 2, 3, 4, 7, 8, 13, 14, 16, 17, 31, 32, 33, 40, 64, 96, 100,
                              127, 128, 129, 255, 256, 1000, 1024, 4096, 65535, 65536, 1 << 20,
                              INT_MAX, -1, -2, INT_MIN};
  return pick_int(v, sizeof v / sizeof v[0]);
}

// a fake device pointer: NULL, 256-aligned, or off by a few bytes; distinct
// regions 1 GiB apart so only deliberate choices alias
const void* a_ptr(int region) {
  const uint64_t r = rnd() % 8;
  if (r == 0) return nullptr;
  uintptr_t base = ((uintptr_t)(region + 1)) << 30;
  if (r == 1) base += 2;
  if (r == 2) base += 8;
  if (r == 3) base += 4;
  return (const void*)base;
}

bool known_status(int32_t st) { return st >= PD_OK && st <= PD_ERR_SCRATCH; }

void fuzz_decode(int iters) {
  for (int i = 0; i < iters; ++i) {
    const int before = g_launches;
    const int32_t B = an_int(), Hq = an_int(), Hkv = an_int(), D = an_int(), MB = an_int(),
                  bs = an_int(), dtype = (int32_t)(rnd() % 4) - 1, splits = an_int();
    const float scale = (rnd() % 5 == 0) ? -1.0f : 0.088f;
    const size_t wsb = (rnd() % 2) ? (size_t)an_int() * 4096u : (size_t)1 << 34;
    void* out = (void*)a_ptr(5);
    int32_t st;
    switch (rnd() % 3) {
      case 0:
        st = paged_decode_attention(a_ptr(0), a_ptr(1), a_ptr(2), (const int32_t*)a_ptr(3),
                                    (const int32_t*)a_ptr(4), MB, out, B, Hq, Hkv, D, bs, scale,
                                    dtype, (void*)a_ptr(6), wsb, nullptr);
        break;
      case 1:
        st = paged_decode_attention_splits(a_ptr(0), a_ptr(1), a_ptr(2),
                                           (const int32_t*)a_ptr(3), (const int32_t*)a_ptr(4),
                                           MB, out, B, Hq, Hkv, D, bs, scale, dtype,
                                           (void*)a_ptr(6), wsb, nullptr, splits);
        break;
      default:
        st = paged_decode_attention_fp8(a_ptr(0), a_ptr(1), a_ptr(2), (const int32_t*)a_ptr(3),
                                        (const int32_t*)a_ptr(4), MB, out, B, Hq, Hkv, D, bs,
                                        scale, dtype, (rnd() % 7) ? 0.5f : 0.0f, 0.25f,
                                        (void*)a_ptr(6), wsb, nullptr, (int32_t)(rnd() % 70) - 1);
    }
    CHECK(known_status(st));
    CHECK(g_launches == before || st == PD_OK);
    int32_t S = 0, P = 0;
    const int32_t sp = paged_decode_plan(B, Hq, Hkv, D, MB, bs, dtype, &S, &P);
    CHECK(known_status(sp));
    if (sp == PD_OK) {
      CHECK(S >= 1 && P >= 1 && (int64_t)S * P >= (int64_t)MB * bs);
      const size_t w = paged_decode_workspace_bytes(B, Hq, Hkv, D, MB, bs, dtype);
      CHECK((S == 1 || B == 0) == (w == 0));
    }
    const int32_t sps = paged_decode_plan_splits(B, Hq, Hkv, D, MB, bs, dtype, splits, &S, &P);
    CHECK(known_status(sps));
    (void)paged_decode_workspace_bytes_splits(B, Hq, Hkv, D, MB, bs, dtype, splits);
  }
  CHECK(paged_decode_plan(8, 32, 8, 128, 64, 16, 1, nullptr, nullptr) == PD_ERR_NULL);
  CHECK(paged_decode_workspace_init(nullptr, 4096, nullptr) == PD_ERR_NULL);
  CHECK(paged_decode_workspace_init((void*)(uintptr_t)(1 << 30), 0, nullptr) == PD_OK);
}

void fuzz_kv(int iters) {
  for (int i = 0; i < iters; ++i) {
    const int before = g_launches;
    const int32_t T = an_int(), Hq = an_int(), Hkv = an_int(), D = an_int(), bs = an_int(),
                  NB = an_int(), maxpos = an_int(), dtype = (int32_t)(rnd() % 3);
    const int64_t qs = (int64_t)an_int() * (rnd() % 3), ks = an_int(), vs = an_int();
    int32_t st;
    if (rnd() % 2)
      st = rope_paged_kv_write(a_ptr(0), a_ptr(1), a_ptr(2), qs, ks, vs,
                               (const int32_t*)a_ptr(3), (const int32_t*)a_ptr(4),
                               (const float*)a_ptr(5), maxpos, (void*)a_ptr(6), (void*)a_ptr(7),
                               (void*)a_ptr(8), NB, T, Hq, Hkv, D, bs, dtype, nullptr);
    else
      st = rope_paged_kv_write_fp8(a_ptr(0), a_ptr(1), a_ptr(2), qs, ks, vs,
                                   (const int32_t*)a_ptr(3), (const int32_t*)a_ptr(4),
                                   (const float*)a_ptr(5), maxpos, (void*)a_ptr(6),
                                   (void*)a_ptr(7), (void*)a_ptr(8), NB, T, Hq, Hkv, D, bs, dtype,
                                   (rnd() % 5) ? 0.01f : -1.0f, 0.02f, nullptr);
    CHECK(known_status(st));
    CHECK(g_launches == before || st == PD_OK);
    const int b2 = g_launches;
    st = rope_cos_sin_table((float*)a_ptr(0), maxpos, D, (rnd() % 4) ? 1e6 : -1.0, nullptr);
    CHECK(known_status(st) && (g_launches == b2 || st == PD_OK));
    const int b3 = g_launches;
    const int64_t bb = (int64_t)an_int() * (int64_t)(rnd() % 4);
    switch (rnd() % 4) {
      case 0:
        st = paged_kv_copy_blocks((void*)a_ptr(0), (void*)a_ptr(1), NB, bb,
                                  (const int32_t*)a_ptr(2), T, nullptr);
        break;
      case 1:
        st = paged_kv_gather_blocks(a_ptr(0), a_ptr(1), NB, bb, (const int32_t*)a_ptr(2), T,
                                    (void*)a_ptr(3), (void*)a_ptr(4), nullptr);
        break;
      case 2:
        st = paged_kv_scatter_blocks(a_ptr(0), a_ptr(1), (const int32_t*)a_ptr(2), T,
                                     (void*)a_ptr(3), (void*)a_ptr(4), NB, bb, nullptr);
        break;
      default:
        st = paged_kv_remap_block_table((int32_t*)a_ptr(0), (int64_t)an_int() * 3,
                                        (const int32_t*)a_ptr(1), NB, nullptr);
    }
    CHECK(known_status(st) && (g_launches == b3 || st == PD_OK));
  }
}

// the host compaction planner on real arrays: every live block at or above
// n_live moves to a hole below it, the remap is a bijection of live ids
// onto [0, n_live) and leaves the rest alone
void check_compaction(int iters) {
  for (int it = 0; it < iters; ++it) {
    const int32_t nb = (int32_t)(rnd() % 3000);
    std::vector<uint8_t> live(nb > 0 ? nb : 1);
    const int density = (int)(rnd() % 101);
    int32_t n_live_want = 0;
    for (int32_t i = 0; i < nb; ++i) {
      live[i] = (int)(rnd() % 100) < density;
      n_live_want += live[i];
    }
    const int32_t cap = (int32_t)(rnd() % 3 == 0 ? rnd() % (nb / 2 + 2) : nb / 2 + 1);
    std::vector<int32_t> pairs(2 * (cap > 0 ? cap : 1)), remap(nb > 0 ? nb : 1);
    int32_t n_pairs = -1, n_live = -1;
    const int32_t st = paged_kv_compact_plan(live.data(), nb, pairs.data(), cap, &n_pairs,
                                             remap.data(), &n_live);
    CHECK(known_status(st));
    if (st != PD_OK) continue;
    CHECK(n_live == n_live_want);
    int32_t movers = 0;
    for (int32_t i = n_live; i < nb; ++i) movers += live[i];
    CHECK(n_pairs == movers && n_pairs <= cap);
    std::vector<int> seen(nb > 0 ? nb : 1, 0);
    for (int32_t i = 0; i < nb; ++i) {
      if (!live[i]) continue;
      CHECK(remap[i] >= 0 && remap[i] < n_live);
      if (remap[i] >= 0 && remap[i] < nb) seen[remap[i]]++;
      if (i < n_live) CHECK(remap[i] == i);
    }
    for (int32_t i = 0; i < n_live; ++i) CHECK(seen[i] == 1);
    for (int32_t k = 0; k < n_pairs; ++k) {
      const int32_t s = pairs[2 * k], d = pairs[2 * k + 1];
      CHECK(s >= n_live && s < nb && live[s] && d >= 0 && d < n_live && !live[d]);
      CHECK(remap[s] == d);
    }
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 200000;
  fuzz_decode(iters);
  fuzz_kv(iters);
  check_compaction(iters / 100 + 1);
  printf("abi_sanitize: %d launches recorded, %d failures\n", g_launches, g_fail);
  return g_fail ? 1 : 0;
}
