// Python binding of the per-step entry points of the C ABI (the decode
// attention of paged_decode.h, its FP8 and allocation-free forms, the RoPE +
// paged KV write of paged_kv.h and the workspace fill): it checks the torch
// tensors a call hands over (device, dtype, shape, layout), supplies `out`
// and the split-K workspace when the caller gives none, takes the stream
// (the given one, else the device's current one) and forwards pointers and
// sizes. Nothing here computes: every step of the decode and the write runs
// in the library's kernels. A check that fails raises ValueError before any
// HIP call; a status the library returns is handed back to Python, which
// raises it as PagedDecodeError.
//
// Compiled by build.py with g++ against the torch headers; linked to
// libpaged_decode.so, which the package loads first.
#include <ATen/core/Tensor.h>
#include <ATen/hip/impl/HIPGuardImplMasqueradingAsCUDA.h>
#include <ATen/hip/impl/HIPStreamMasqueradingAsCUDA.h>
#include <ATen/ops/empty.h>
#include <c10/hip/HIPGraphsC10Utils.h>
#include <torch/csrc/utils/pybind.h>

#include <climits>
#include <cmath>
#include <initializer_list>
#include <map>
#include <mutex>
#include <optional>
#include <stdexcept>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include "paged_decode.h"
#include "paged_kv.h"

namespace {

using at::Tensor;
using OptTensor = std::optional<Tensor>;
using OptInt = std::optional<int64_t>;
using Stream = c10::hip::HIPStreamMasqueradingAsCUDA;

[[noreturn]] void refuse(const std::string& msg) { throw std::invalid_argument(msg); }

std::string where(const Tensor& t) { return t.device().str(); }

// Index of the GPU holding `t`; a host tensor is refused (the library takes
// device pointers only, and a host pointer reaching a kernel faults the GPU).
int gpu_index(const Tensor& t, const char* name) {
  if (!t.is_cuda()) refuse(std::string(name) + " must be a GPU tensor, not on " + where(t));
  return t.get_device();
}

void same_gpu(int dev, const Tensor& t, const char* name) {
  if (!t.is_cuda() || t.get_device() != dev)
    refuse(std::string(name) + " must be a GPU tensor on cuda:" + std::to_string(dev) +
           " (got " + where(t) + ")");
}

int32_t dtype_code(at::ScalarType t) {
  return t == at::kHalf ? PD_DTYPE_F16 : t == at::kBFloat16 ? PD_DTYPE_BF16 : -1;
}

bool fp8_codes(at::ScalarType t) { return t == at::kFloat8_e4m3fn || t == at::kByte; }

// The stream a call runs on: the given raw handle, else the device's current one.
Stream stream_for(const OptInt& stream, int dev) {
  if (stream)
    return c10::hip::getStreamFromExternalMasqueradingAsCUDA(
        reinterpret_cast<hipStream_t>(static_cast<uintptr_t>(*stream)), (c10::DeviceIndex)dev);
  return c10::hip::getCurrentHIPStreamMasqueradingAsCUDA((c10::DeviceIndex)dev);
}

void* handle(const Stream& s) { return static_cast<void*>(static_cast<hipStream_t>(s)); }

// A tensor allocated by torch's allocator on `stream` (its blocks are then
// reused only in that stream's order).
Tensor empty_on(at::IntArrayRef shape, at::ScalarType dt, int dev, const OptInt& stream,
                const Stream& s) {
  const auto opts = at::TensorOptions().dtype(dt).device(at::kCUDA, (c10::DeviceIndex)dev);
  if (!stream) return at::empty(shape, opts);
  c10::hip::HIPStreamGuardMasqueradingAsCUDA guard(s);
  return at::empty(shape, opts);
}

bool fits_int32(std::initializer_list<int64_t> sizes) {
  for (int64_t x : sizes)
    if (x > INT32_MAX) return false;
  return true;
}

size_t nbytes(const Tensor& t) { return (size_t)t.numel() * t.element_size(); }

// Zeroed workspace of at least `need` bytes (at least 256), allocated and
// filled on `stream`; `rc` receives the fill's status.
Tensor fresh_workspace(size_t need, int dev, const OptInt& stream, const Stream& s, int32_t* rc) {
  Tensor ws = empty_on({(int64_t)std::max<size_t>(need, 256)}, at::kByte, dev, stream, s);
  *rc = paged_decode_workspace_init(ws.data_ptr(), nbytes(ws), handle(s));
  return ws;
}

// Workspaces supplied to eager calls on the current stream when the caller
// gives none: one per (GPU, stream), replaced by a larger one when a call
// needs more (the outgrown ones are kept, not freed, while calls queued
// earlier may still read them). The decode needs no particular contents (a
// call writes every workspace byte it reads), and calls on one stream run in
// order, so they can share one; calls on different streams use different
// workspaces, and captured calls get their own from the graph's pool.
// (Held in objects that are never destroyed: their tensors must not be freed
// by static destructors at exit, after torch's allocator may be gone.)
std::mutex g_ws_mu;
auto& g_ws = *new std::map<std::pair<int, uintptr_t>, Tensor>();
auto& g_ws_retired = *new std::vector<Tensor>();

// (pointer, bytes, keep-alive) of a workspace of at least `need` bytes for
// a call on `s`, or nulls when none is needed. An explicit stream or a call
// under graph capture gets one of its own, allocated on the stream the call
// runs on.
std::tuple<void*, size_t, Tensor> auto_workspace(size_t need, int dev, const OptInt& stream,
                                                 const Stream& s) {
  if (need == 0) return {nullptr, 0, Tensor()};
  const int64_t n = (int64_t)std::max<size_t>(need, 256);
  if (stream || c10::hip::currentStreamCaptureStatusMayInitCtx() != c10::hip::CaptureStatus::None) {
    Tensor ws = empty_on({n}, at::kByte, dev, stream, s);
    return {ws.data_ptr(), nbytes(ws), ws};
  }
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Tensor& ws = g_ws[{dev, reinterpret_cast<uintptr_t>(handle(s))}];
  if (!ws.defined() || nbytes(ws) < need) {
    Tensor fresh = empty_on({n}, at::kByte, dev, stream, s);
    if (ws.defined()) g_ws_retired.push_back(ws);
    ws = fresh;
  }
  return {ws.data_ptr(), nbytes(ws), ws};
}

enum Mode { kPlain = 0, kFp8 = 1, kNoalloc = 2 };

// paged_decode_attention and its forms. Returns (out, status).
std::tuple<Tensor, int64_t> decode(const Tensor& q, const Tensor& k, const Tensor& v,
                                   const Tensor& bt, const Tensor& cl, OptTensor out,
                                   const OptTensor& workspace, std::optional<double> scale,
                                   OptInt num_splits, OptInt stream, int64_t mode,
                                   double k_scale, double v_scale) {
  const int dev = gpu_index(q, "q");
  const Tensor* ts[] = {&q, &k, &v, &bt, &cl};
  const char* names[] = {"q", "k_cache", "v_cache", "block_table", "context_lens"};
  for (int i = 0; i < 5; ++i) {
    same_gpu(dev, *ts[i], names[i]);
    if (!ts[i]->is_contiguous()) refuse(std::string(names[i]) + " must be contiguous");
  }
  const auto qs = q.sizes(), ks = k.sizes();
  if (qs.size() != 3 || ks.size() != 4 || v.sizes() != ks || ks[3] != qs[2])
    refuse("q must be [B,Hq,D] and k_cache/v_cache [num_blocks,block_size,Hkv,D]");
  const at::ScalarType dt = q.scalar_type();
  const int32_t code = dtype_code(dt);
  if (mode == kFp8) {
    if (!fp8_codes(k.scalar_type()) || v.scalar_type() != k.scalar_type() || code < 0)
      refuse("k_cache/v_cache must be float8_e4m3fn (or uint8 codes), q f16 or bf16");
  } else if (k.scalar_type() != dt || v.scalar_type() != dt || code < 0) {
    refuse("q, k_cache and v_cache must share one dtype, float16 or bfloat16");
  }
  if (bt.scalar_type() != at::kInt || cl.scalar_type() != at::kInt)
    refuse("block_table and context_lens must be int32");
  const auto bts = bt.sizes();
  const int64_t B = qs[0];
  if (bts.size() != 2 || bts[0] != B || cl.dim() != 1 || cl.size(0) != B)
    refuse("block_table must be [B, max_blocks_per_seq] and context_lens [B]");
  if (!fits_int32({B, qs[1], ks[2], qs[2], bts[1], ks[1]}))
    refuse("a size of q, the caches or block_table exceeds the int32 range of the C ABI");
  if (num_splits && (*num_splits < INT32_MIN || *num_splits > INT32_MAX))
    refuse("num_splits exceeds the int32 range of the C ABI");
  const int32_t Hq = (int32_t)qs[1], Hkv = (int32_t)ks[2], D = (int32_t)qs[2];
  const int32_t MB = (int32_t)bts[1], bs = (int32_t)ks[1];
  if (out) {
    same_gpu(dev, *out, "out");
    if (out->sizes() != qs || out->scalar_type() != dt || !out->is_contiguous())
      refuse("out must be a contiguous tensor of q's shape and dtype");
  } else if (mode == kNoalloc) {
    refuse("out is required: this entry point allocates nothing");
  }
  if (workspace) {
    same_gpu(dev, *workspace, "workspace");
    if (!workspace->is_contiguous()) refuse("workspace must be contiguous");
  }
  const Stream s = stream_for(stream, dev);
  if (!out) out = empty_on(qs, dt, dev, stream, s);
  const float sc = (float)(scale ? *scale : std::pow((double)D, -0.5));
  int32_t rc;
  if (mode == kNoalloc) {
    rc = paged_decode_attention_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        bt.data_ptr<int32_t>(), cl.data_ptr<int32_t>(), MB,
                                        out->data_ptr(), (int32_t)B, Hq, Hkv, D, bs, sc, code,
                                        handle(s));
    return {*out, rc};
  }
  void* wp = nullptr;
  size_t wn = 0;
  Tensor keep;
  if (workspace) {
    wp = workspace->data_ptr();
    wn = nbytes(*workspace);
  } else {
    const size_t need =
        num_splits ? paged_decode_workspace_bytes_splits((int32_t)B, Hq, Hkv, D, MB, bs, code,
                                                         (int32_t)*num_splits)
                   : paged_decode_workspace_bytes((int32_t)B, Hq, Hkv, D, MB, bs, code);
    std::tie(wp, wn, keep) = auto_workspace(need, dev, stream, s);
  }
  if (mode == kFp8) {
    rc = paged_decode_attention_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    bt.data_ptr<int32_t>(), cl.data_ptr<int32_t>(), MB,
                                    out->data_ptr(), (int32_t)B, Hq, Hkv, D, bs, sc, code,
                                    (float)k_scale, (float)v_scale, wp, wn, handle(s),
                                    num_splits ? (int32_t)*num_splits : 0);
  } else if (num_splits) {
    rc = paged_decode_attention_splits(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       bt.data_ptr<int32_t>(), cl.data_ptr<int32_t>(), MB,
                                       out->data_ptr(), (int32_t)B, Hq, Hkv, D, bs, sc, code, wp,
                                       wn, handle(s), (int32_t)*num_splits);
  } else {
    rc = paged_decode_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                bt.data_ptr<int32_t>(), cl.data_ptr<int32_t>(), MB,
                                out->data_ptr(), (int32_t)B, Hq, Hkv, D, bs, sc, code, wp, wn,
                                handle(s));
  }
  return {*out, rc};
}

// Row stride (elements) of a [T, H, D] view whose heads are contiguous.
int64_t rows(const char* name, const Tensor& t, int64_t H, int64_t D) {
  const auto sh = t.sizes();
  if (sh.size() != 3 || sh[1] != H || sh[2] != D)
    refuse(std::string(name) + " must be [T, " + std::to_string(H) + ", " + std::to_string(D) +
           "]");
  const auto st = t.strides();
  if (sh[0] > 0 && (st[2] != 1 || st[1] != D))
    refuse(std::string(name) + ": heads of a token must be contiguous (strides [*, D, 1])");
  return sh[0] > 1 ? st[0] : H * D;
}

// rope_paged_kv_write and its FP8 form. Returns (q_out, status).
std::tuple<Tensor, int64_t> rope(const Tensor& q, const Tensor& k, const Tensor& v,
                                 const Tensor& positions, const Tensor& slots,
                                 const Tensor& cos_sin, const Tensor& k_cache,
                                 const Tensor& v_cache, OptTensor q_out, bool fp8, double k_scale,
                                 double v_scale, OptInt stream) {
  const int dev = gpu_index(q, "q");
  same_gpu(dev, k, "k");
  same_gpu(dev, v, "v");
  same_gpu(dev, positions, "positions");
  same_gpu(dev, slots, "slot_mapping");
  same_gpu(dev, cos_sin, "cos_sin");
  same_gpu(dev, k_cache, "k_cache");
  same_gpu(dev, v_cache, "v_cache");
  if (q_out) same_gpu(dev, *q_out, "q_out");
  const at::ScalarType dt = q.scalar_type();
  const int32_t code = dtype_code(dt);
  if (code < 0 || k.scalar_type() != dt || v.scalar_type() != dt)
    refuse("q, k and v must share one dtype, float16 or bfloat16");
  if (fp8) {
    if (!fp8_codes(k_cache.scalar_type()) || v_cache.scalar_type() != k_cache.scalar_type())
      refuse("FP8 caches must be float8_e4m3fn (or uint8 codes), both alike");
  } else if (k_cache.scalar_type() != dt || v_cache.scalar_type() != dt) {
    refuse("the caches must have q's dtype");
  }
  const auto cs = k_cache.sizes();
  if (cs.size() != 4 || v_cache.sizes() != cs || !k_cache.is_contiguous() ||
      !v_cache.is_contiguous())
    refuse("k_cache/v_cache must be contiguous [num_blocks,block_size,Hkv,D]");
  const int64_t NB = cs[0], bs = cs[1], Hkv = cs[2], D = cs[3];
  if (q.dim() != 3) refuse("q must be [T, Hq, D]");
  const int64_t T = q.size(0), Hq = q.size(1);
  const int64_t qs = rows("q", q, Hq, D), ks = rows("k", k, Hkv, D), vs = rows("v", v, Hkv, D);
  if (k.size(0) != T || v.size(0) != T) refuse("q, k and v must have the same number of tokens");
  const Tensor* idx[] = {&positions, &slots};
  const char* idx_names[] = {"positions", "slot_mapping"};
  for (int i = 0; i < 2; ++i) {
    const Tensor& t = *idx[i];
    if (t.scalar_type() != at::kInt || t.dim() != 1 || t.size(0) != T || !t.is_contiguous())
      refuse(std::string(idx_names[i]) + " must be a contiguous int32 [T] tensor");
  }
  if (cos_sin.scalar_type() != at::kFloat || cos_sin.dim() != 2 || cos_sin.size(1) != D ||
      !cos_sin.is_contiguous())
    refuse("cos_sin must be a contiguous float32 [max_position, D] tensor");
  if (q_out && (q_out->dim() != 3 || q_out->size(0) != T || q_out->size(1) != Hq ||
                q_out->size(2) != D || q_out->scalar_type() != dt || !q_out->is_contiguous()))
    refuse("q_out must be a contiguous [T, Hq, D] tensor of q's dtype");
  if (!fits_int32({NB, bs, Hkv, D, T, Hq, cos_sin.size(0)}))
    refuse("a size of q, the caches or cos_sin exceeds the int32 range of the C ABI");
  const Stream s = stream_for(stream, dev);
  if (!q_out) q_out = empty_on({T, Hq, D}, dt, dev, stream, s);
  const int32_t rc =
      fp8 ? rope_paged_kv_write_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), qs, ks, vs,
                                    positions.data_ptr<int32_t>(), slots.data_ptr<int32_t>(),
                                    cos_sin.data_ptr<float>(), (int32_t)cos_sin.size(0),
                                    q_out->data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                    (int32_t)NB, (int32_t)T, (int32_t)Hq, (int32_t)Hkv,
                                    (int32_t)D, (int32_t)bs, code, (float)k_scale,
                                    (float)v_scale, handle(s))
          : rope_paged_kv_write(q.data_ptr(), k.data_ptr(), v.data_ptr(), qs, ks, vs,
                                positions.data_ptr<int32_t>(), slots.data_ptr<int32_t>(),
                                cos_sin.data_ptr<float>(), (int32_t)cos_sin.size(0),
                                q_out->data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                (int32_t)NB, (int32_t)T, (int32_t)Hq, (int32_t)Hkv, (int32_t)D,
                                (int32_t)bs, code, handle(s));
  return {*q_out, rc};
}

// paged_decode_workspace_init on `workspace`. Returns the status.
int64_t workspace_init(const Tensor& workspace, OptInt stream) {
  const int dev = gpu_index(workspace, "workspace");
  if (!workspace.is_contiguous()) refuse("workspace must be contiguous");
  return paged_decode_workspace_init(workspace.data_ptr(), nbytes(workspace),
                                     handle(stream_for(stream, dev)));
}

// A zeroed uint8 workspace of `n` bytes (at least 256) on GPU `dev`,
// allocated and zeroed on the given stream (else the current one). Returns
// (workspace, status of the fill).
std::tuple<Tensor, int64_t> alloc_workspace_bytes(int64_t n, int64_t dev, OptInt stream) {
  if (n < 0) refuse("workspace bytes must be >= 0");
  const Stream s = stream_for(stream, (int)dev);
  int32_t rc;
  Tensor ws = fresh_workspace((size_t)n, (int)dev, stream, s, &rc);
  return {ws, rc};
}

}  // namespace

PYBIND11_MODULE(_pd_binding, m) {
  m.doc() = "Argument marshalling for the per-step entry points of libpaged_decode.so";
  m.def("decode", &decode);
  m.def("rope", &rope);
  m.def("workspace_init", &workspace_init);
  m.def("alloc_workspace_bytes", &alloc_workspace_bytes);
}
