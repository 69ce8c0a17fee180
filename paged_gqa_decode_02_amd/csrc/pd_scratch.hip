// The decode entry point for callers that cannot allocate: its split-K
// scratch (fp32 partial outputs and log-sum-exps) lives in one static device
// array per GPU instead of a caller-owned workspace.
//
// The array's name is a host-side stand-in in host code; the device address
// of each GPU's copy is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address ever reaches a kernel. Every
// GPU keeps its copy until the process ends. A call writes every byte of it
// that it reads, so no call depends on what an earlier one left; but all
// calls on one GPU share it, and calls that overlap in time on one GPU
// (different streams, unordered) race on it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/paged_decode.h"
#include "pd_internal.h"

namespace {

static_assert(PAGED_DECODE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __align__(256) char scratch[PAGED_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of each GPU's copy of `scratch`

// The device `stream` belongs to (the current device for the null stream).
int32_t stream_device(hipStream_t stream, int* dev) {
  if (hipStreamGetDevice(stream, dev) != hipSuccess) return PD_ERR_HIP;
  return *dev >= 0 && *dev < kMaxDevices ? PD_OK : PD_ERR_UNSUPPORTED;
}

// This GPU's copy of the scratch array, looked up on the first call on the
// device (with that device current).
int32_t device_scratch(void* stream_arg, void** out) {
  const hipStream_t stream = (hipStream_t)stream_arg;
  int dev = 0;
  int32_t st = stream_device(stream, &dev);
  if (st != PD_OK) return st;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return PD_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return PD_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return PD_ERR_HIP;
    if (e != hipSuccess || !p) return PD_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return PD_OK;
}

}  // namespace

extern "C" int32_t paged_decode_attention_noalloc(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
    const int32_t* context_lens, int32_t max_blocks_per_seq, void* out, int32_t B, int32_t Hq,
    int32_t Hkv, int32_t D, int32_t block_size, float scale, int32_t dtype, void* stream) {
  try {
    return pd::attention_with_scratch(q, k_cache, v_cache, block_table, context_lens,
                                      max_blocks_per_seq, out, B, Hq, Hkv, D, block_size, scale,
                                      dtype, stream, PAGED_DECODE_NOALLOC_SCRATCH_BYTES,
                                      device_scratch);
  } catch (...) {
    return PD_ERR_INTERNAL;
  }
}
