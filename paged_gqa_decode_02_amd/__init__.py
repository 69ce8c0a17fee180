"""MI355X-native paged GQA decode attention.

A thin binding over the C ABI in ``include/paged_decode.h`` and
``include/paged_kv.h`` (built as ``_lib/libpaged_decode.so`` by ``python
paged_gqa_decode_02_amd/build.py``). The functions keep the C names; they only
marshal torch tensors into pointers, sizes and the HIP stream. The per-step
entry points (the decode attention in its forms, the RoPE + KV write, the
workspace fill) go through a compiled binding (``_lib/_pd_binding*.so``,
``csrc/pd_binding.cpp``) that checks the tensors and calls the library in
well under a microsecond; the rest use ctypes. Every step of the computation
runs in the library's HIP kernels. Importing this package fails if the
library or the binding has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libpaged_decode.so")

PD_DTYPE_F16 = 0
PD_DTYPE_BF16 = 1
_DTYPE_CODE = {torch.float16: PD_DTYPE_F16, torch.bfloat16: PD_DTYPE_BF16}

PD_OK = 0
STATUS_NAMES = {
    0: "PD_OK", 1: "PD_ERR_NULL", 2: "PD_ERR_SHAPE", 3: "PD_ERR_DTYPE", 4: "PD_ERR_ALIGN",
    5: "PD_ERR_ALIAS", 6: "PD_ERR_WORKSPACE", 7: "PD_ERR_UNSUPPORTED", 8: "PD_ERR_HIP",
    9: "PD_ERR_INTERNAL", 10: "PD_ERR_VALUE", 11: "PD_ERR_SCRATCH",
}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"paged_gqa_decode_02_amd: HIP library not built ({LIB_PATH} missing); "
        "run `python paged_gqa_decode_02_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)


def _load_binding():
    import importlib.util
    import sysconfig
    path = os.path.join(_HERE, "_lib", "_pd_binding" + sysconfig.get_config_var("EXT_SUFFIX"))
    if not os.path.exists(path):
        raise ImportError(f"paged_gqa_decode_02_amd: compiled binding not built ({path} "
                          "missing); run `python paged_gqa_decode_02_amd/build.py`")
    spec = importlib.util.spec_from_file_location("_pd_binding", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


# loaded after the library: it links to the copy loaded above
_b = _load_binding()
_P, _I, _Z, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
_PI = ctypes.POINTER(ctypes.c_int32)

lib.paged_decode_abi_version.argtypes = []
lib.paged_decode_abi_version.restype = _I
lib.paged_decode_strerror.argtypes = [_I]
lib.paged_decode_strerror.restype = ctypes.c_char_p
lib.paged_decode_plan.argtypes = [_I, _I, _I, _I, _I, _I, _I, _PI, _PI]
lib.paged_decode_plan.restype = _I
lib.paged_decode_plan_splits.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _PI, _PI]
lib.paged_decode_plan_splits.restype = _I
lib.paged_decode_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I, _I]
lib.paged_decode_workspace_bytes.restype = _Z
lib.paged_decode_workspace_bytes_splits.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I]
lib.paged_decode_workspace_bytes_splits.restype = _Z
lib.paged_decode_workspace_init.argtypes = [_P, _Z, _P]
lib.paged_decode_workspace_init.restype = _I
# The per-step entry points below are called through the compiled binding;
# their ctypes declarations serve direct calls of the C ABI (the host-side
# ABI tests make them).
_ATTN = [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]
lib.paged_decode_attention.argtypes = _ATTN
lib.paged_decode_attention.restype = _I
lib.paged_decode_attention_splits.argtypes = _ATTN + [_I]
lib.paged_decode_attention_splits.restype = _I
lib.paged_decode_attention_fp8.argtypes = _ATTN[:14] + [_F, _F] + _ATTN[14:] + [_I]
lib.paged_decode_attention_fp8.restype = _I
lib.paged_decode_attention_noalloc.argtypes = _ATTN[:14] + [_P]
lib.paged_decode_attention_noalloc.restype = _I
NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024  # PAGED_DECODE_NOALLOC_SCRATCH_BYTES


class PagedDecodeError(RuntimeError):
    def __init__(self, code: int):
        self.code = int(code)
        super().__init__(f"{STATUS_NAMES.get(self.code, self.code)}: {paged_decode_strerror(self.code)}")


# The raw HIP stream handle of a device's current stream, without building a
# torch Stream object per call.
_raw_stream = torch._C._cuda_getCurrentRawStream


def _gpu_index(t, name) -> int:
    """Index of the GPU holding `t`; a host tensor is refused (the library
    takes device pointers only, and a host pointer reaching a kernel faults
    the GPU)."""
    d = t.get_device()
    if d < 0:
        raise ValueError(f"{name} must be a GPU tensor, not on {t.device}")
    return d


def _same_gpu(dev, **tensors):
    """Every given tensor (None skipped) lives on GPU `dev`."""
    for name, t in tensors.items():
        if t is not None and t.get_device() != dev:
            raise ValueError(f"{name} must be a GPU tensor on cuda:{dev} (got {t.device})")


def _on_gpu(dev, **tensors):
    """As _same_gpu, for a torch.device `dev`."""
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, not {dev}")
    _same_gpu(dev.index if dev.index is not None else torch.cuda.current_device(), **tensors)


def _stream_handle(stream, dev: int) -> int:
    """HIP stream handle: the given stream (a torch stream or a raw handle) or
    the device's current stream."""
    if stream is None:
        return _raw_stream(dev)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def paged_decode_abi_version() -> int:
    return int(lib.paged_decode_abi_version())


def paged_decode_strerror(code: int) -> str:
    return lib.paged_decode_strerror(int(code)).decode()


def paged_decode_plan(B, Hq, Hkv, D, max_blocks_per_seq, block_size, dtype, num_splits=None):
    """(S, P) the library uses for this shape; ``num_splits`` forces S."""
    s, p = ctypes.c_int32(0), ctypes.c_int32(0)
    dt = _DTYPE_CODE.get(dtype, dtype)
    if num_splits is None:
        rc = lib.paged_decode_plan(B, Hq, Hkv, D, max_blocks_per_seq, block_size, dt,
                                   ctypes.byref(s), ctypes.byref(p))
    else:
        rc = lib.paged_decode_plan_splits(B, Hq, Hkv, D, max_blocks_per_seq, block_size, dt,
                                          int(num_splits), ctypes.byref(s), ctypes.byref(p))
    if rc != PD_OK:
        raise PagedDecodeError(rc)
    return s.value, p.value


def paged_decode_workspace_bytes(B, Hq, Hkv, D, max_blocks_per_seq, block_size, dtype,
                                 num_splits=None) -> int:
    dt = _DTYPE_CODE.get(dtype, dtype)
    if num_splits is None:
        return int(lib.paged_decode_workspace_bytes(B, Hq, Hkv, D, max_blocks_per_seq,
                                                    block_size, dt))
    return int(lib.paged_decode_workspace_bytes_splits(B, Hq, Hkv, D, max_blocks_per_seq,
                                                       block_size, dt, int(num_splits)))


_NEED = {}  # (shape, dtype, num_splits) -> workspace bytes (a pure function of them)


def _workspace_need(B, Hq, Hkv, D, MB, bs, dt, num_splits) -> int:
    key = (B, Hq, Hkv, D, MB, bs, dt, num_splits)
    n = _NEED.get(key)
    if n is None:
        n = paged_decode_workspace_bytes(B, Hq, Hkv, D, MB, bs, dt, num_splits)
        if len(_NEED) > 4096:
            _NEED.clear()
        _NEED[key] = n
    return n


def _shape(q, k_cache, block_table):
    B, Hq, D = q.shape
    _, bs, Hkv, _ = k_cache.shape
    return int(B), int(Hq), int(Hkv), int(D), int(block_table.shape[1]), int(bs)


def _stream_arg(stream):
    """None (the device's current stream) or the raw HIP handle of `stream`
    (a torch stream or a raw handle), for the compiled binding."""
    if stream is None:
        return None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(rc: int) -> None:
    if rc != PD_OK:
        raise PagedDecodeError(rc)


def paged_decode_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    """Zero a workspace on the current (or given) stream with the library's
    fill kernel (the decode does not need it: a call writes every workspace
    byte it reads)."""
    _check(_b.workspace_init(workspace, _stream_arg(stream)))


def alloc_workspace(q, k_cache, block_table, num_splits=None, stream=None) -> torch.Tensor:
    """A zeroed device workspace of the size the call needs (at least 256
    bytes), allocated and zeroed on the current (or given) stream."""
    B, Hq, Hkv, D, MB, bs = _shape(q, k_cache, block_table)
    _gpu_index(q, "q")
    n = _workspace_need(B, Hq, Hkv, D, MB, bs, _DTYPE_CODE.get(q.dtype, q.dtype), num_splits)
    return alloc_workspace_bytes(n, q.device, stream)


def alloc_workspace_bytes(nbytes, device, stream=None) -> torch.Tensor:
    """A zeroed uint8 device workspace of `nbytes` (at least 256), allocated
    and zeroed on the current (or given) stream."""
    device = torch.device(device)
    if device.type != "cuda":
        raise ValueError(f"a workspace must be on a GPU, not {device}")
    dev = device.index if device.index is not None else torch.cuda.current_device()
    ws, rc = _b.alloc_workspace_bytes(int(nbytes), dev, _stream_arg(stream))
    _check(rc)
    return ws


_PLAIN, _FP8_MODE, _NOALLOC = 0, 1, 2


def paged_decode_attention(q, k_cache, v_cache, block_table, context_lens, out=None, *,
                           scale=None, workspace=None, num_splits=None, stream=None):
    """Paged decode attention on the current (or given) stream.

    q [B,Hq,D], k_cache/v_cache [num_blocks,block_size,Hkv,D] (f16 or bf16,
    contiguous, on the GPU); block_table int32 [B,max_blocks_per_seq];
    context_lens int32 [B]. ``out`` (same shape/dtype as q) is allocated when
    not given. Without a ``workspace`` the binding supplies one: a buffer
    kept per (GPU, stream) for calls on the current stream, or one of
    the call's own, allocated on ``stream``, for calls given a stream or made
    under graph capture. ``scale`` defaults to D ** -0.5. ``num_splits``
    forces the split count (``paged_decode_attention_splits``). Returns
    ``out``.
    """
    out, rc = _b.decode(q, k_cache, v_cache, block_table, context_lens, out, workspace, scale,
                        num_splits, _stream_arg(stream), _PLAIN, 1.0, 1.0)
    _check(rc)
    return out


def paged_decode_attention_splits(q, k_cache, v_cache, block_table, context_lens, num_splits,
                                  out=None, **kw):
    """``paged_decode_attention`` with the split count forced to ``num_splits``."""
    return paged_decode_attention(q, k_cache, v_cache, block_table, context_lens, out,
                                  num_splits=num_splits, **kw)


def paged_decode_attention_noalloc(q, k_cache, v_cache, block_table, context_lens, out, *,
                                   scale=None, stream=None):
    """``paged_decode_attention`` for callers that cannot allocate: the
    library's static per-GPU scratch takes the workspace's place, and this
    binding allocates nothing either, so ``out`` is required. Calls that
    overlap in time on one GPU share that scratch and race. Returns ``out``.
    """
    if out is None:
        raise ValueError("out is required: this entry point allocates nothing")
    out, rc = _b.decode(q, k_cache, v_cache, block_table, context_lens, out, None, scale, None,
                        _stream_arg(stream), _NOALLOC, 1.0, 1.0)
    _check(rc)
    return out


def paged_decode_attention_fp8(q, k_cache, v_cache, block_table, context_lens, out=None, *,
                               k_scale, v_scale, scale=None, workspace=None, num_splits=None,
                               stream=None):
    """Paged decode attention over an FP8 (E4M3FN) cache.

    k_cache/v_cache: [num_blocks,block_size,Hkv,D] of torch.float8_e4m3fn (or
    uint8 holding the codes), standing for code * k_scale and code * v_scale;
    q (and out) f16 or bf16 [B,Hq,D]. Otherwise as ``paged_decode_attention``.
    """
    out, rc = _b.decode(q, k_cache, v_cache, block_table, context_lens, out, workspace, scale,
                        num_splits, _stream_arg(stream), _FP8_MODE, float(k_scale),
                        float(v_scale))
    _check(rc)
    return out


# --- KV-cache operations (include/paged_kv.h) --------------------------------

_L, _D = ctypes.c_int64, ctypes.c_double
lib.rope_cos_sin_table.argtypes = [_P, _I, _I, _D, _P]
lib.rope_cos_sin_table.restype = _I
lib.rope_paged_kv_write.argtypes = [_P, _P, _P, _L, _L, _L, _P, _P, _P, _I, _P, _P, _P, _I,
                                    _I, _I, _I, _I, _I, _I, _P]
lib.rope_paged_kv_write.restype = _I
lib.rope_paged_kv_write_fp8.argtypes = lib.rope_paged_kv_write.argtypes[:-1] + [_F, _F, _P]
lib.rope_paged_kv_write_fp8.restype = _I


def _handle(stream, device):
    """HIP stream handle for a call on `device` (a torch.device)."""
    return _stream_handle(stream, device.index if device.index is not None
                          else torch.cuda.current_device())


def rope_cos_sin_table(max_position, rotary_dim, base, *, device="cuda", out=None, stream=None):
    """float32 [max_position, rotary_dim] cos/sin table of the rotary
    embedding (``rope_cos_sin_table``), built on the GPU."""
    if out is None:
        out = torch.empty((max_position, rotary_dim), dtype=torch.float32, device=device)
    dev = _gpu_index(out, "out")
    if out.dtype != torch.float32 or not out.is_contiguous() or \
            tuple(out.shape) != (max_position, rotary_dim):
        raise ValueError("out must be a contiguous float32 [max_position, rotary_dim] tensor")
    rc = lib.rope_cos_sin_table(out.data_ptr(), int(max_position), int(rotary_dim), float(base),
                                _stream_handle(stream, dev))
    if rc != PD_OK:
        raise PagedDecodeError(rc)
    return out


def rope_paged_kv_write(q, k, v, positions, slot_mapping, cos_sin, k_cache, v_cache, q_out=None,
                        *, stream=None):
    """RoPE + paged KV-cache write (``rope_paged_kv_write``) on the current
    (or given) stream.

    q [T,Hq,D], k/v [T,Hkv,D] (f16 or bf16; views into one packed QKV array
    are fine as long as each head is contiguous); positions, slot_mapping
    int32 [T]; cos_sin float32 [max_position, D] (``rope_cos_sin_table``);
    k_cache/v_cache [num_blocks,block_size,Hkv,D] (written in place). Returns
    q_out [T,Hq,D] (allocated when not given; may be q itself).
    """
    q_out, rc = _b.rope(q, k, v, positions, slot_mapping, cos_sin, k_cache, v_cache, q_out,
                        False, 1.0, 1.0, _stream_arg(stream))
    _check(rc)
    return q_out


def rope_paged_kv_write_fp8(q, k, v, positions, slot_mapping, cos_sin, k_cache, v_cache,
                            q_out=None, *, k_scale, v_scale, stream=None):
    """The RoPE + KV write into an FP8 cache (``rope_paged_kv_write_fp8``):
    as ``rope_paged_kv_write`` with k_cache/v_cache float8_e4m3fn (or uint8)
    [num_blocks,block_size,Hkv,D] receiving the E4M3FN codes of the rotated
    key times the float32 reciprocal of k_scale and of the value times that
    of v_scale. Returns q_out (16-bit)."""
    q_out, rc = _b.rope(q, k, v, positions, slot_mapping, cos_sin, k_cache, v_cache, q_out,
                        True, float(k_scale), float(v_scale), _stream_arg(stream))
    _check(rc)
    return q_out


lib.paged_kv_copy_blocks.argtypes = [_P, _P, _I, _L, _P, _I, _P]
lib.paged_kv_copy_blocks.restype = _I
lib.paged_kv_gather_blocks.argtypes = [_P, _P, _I, _L, _P, _I, _P, _P, _P]
lib.paged_kv_gather_blocks.restype = _I
lib.paged_kv_scatter_blocks.argtypes = [_P, _P, _P, _I, _P, _P, _I, _L, _P]
lib.paged_kv_scatter_blocks.restype = _I
lib.paged_kv_compact_plan.argtypes = [_P, _I, _P, _I, _PI, _P, _PI]
lib.paged_kv_compact_plan.restype = _I
lib.paged_kv_remap_block_table.argtypes = [_P, _L, _P, _I, _P]
lib.paged_kv_remap_block_table.restype = _I


def _pool(k_cache, v_cache):
    """(num_blocks, block_bytes, v pointer) of a cache pair; v_cache may be None."""
    _on_gpu(k_cache.device, v_cache=v_cache)
    if not k_cache.is_contiguous() or k_cache.dim() < 1:
        raise ValueError("k_cache must be a contiguous [num_blocks, ...] tensor")
    if v_cache is not None and (v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype
                                or not v_cache.is_contiguous()):
        raise ValueError("v_cache must match k_cache (shape, dtype, contiguous)")
    nb = int(k_cache.shape[0])
    bb = (k_cache.numel() // max(nb, 1)) * k_cache.element_size()
    return nb, bb, (v_cache.data_ptr() if v_cache is not None else None)


def _ids(t, name):
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor")
    return t


def paged_kv_copy_blocks(k_cache, v_cache, pairs, *, stream=None):
    """Block pairs[i, 1] of each cache becomes a copy of block pairs[i, 0]
    (``paged_kv_copy_blocks``); pairs: device int32 [n, 2]. In place."""
    nb, bb, vp = _pool(k_cache, v_cache)
    _on_gpu(k_cache.device, pairs=pairs)
    _ids(pairs, "pairs")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n, 2]")
    rc = lib.paged_kv_copy_blocks(k_cache.data_ptr(), vp, nb, bb, pairs.data_ptr(),
                                  int(pairs.shape[0]), _handle(stream, k_cache.device))
    if rc != PD_OK:
        raise PagedDecodeError(rc)


def paged_kv_gather_blocks(k_cache, v_cache, ids, k_out=None, v_out=None, *, stream=None):
    """k_out[i] = k_cache[ids[i]] (and the same for V) into [n, ...] buffers
    (``paged_kv_gather_blocks``); returns (k_out, v_out)."""
    nb, bb, vp = _pool(k_cache, v_cache)
    _ids(ids, "ids")
    n = int(ids.numel())
    shape = (n,) + tuple(k_cache.shape[1:])
    if k_out is None:
        k_out = torch.empty(shape, dtype=k_cache.dtype, device=k_cache.device)
    if v_cache is not None and v_out is None:
        v_out = torch.empty(shape, dtype=k_cache.dtype, device=k_cache.device)
    _on_gpu(k_cache.device, ids=ids, k_out=k_out, v_out=v_out)
    for t in (k_out, v_out):
        if t is not None and (tuple(t.shape) != shape or t.dtype != k_cache.dtype
                              or not t.is_contiguous()):
            raise ValueError("outputs must be contiguous [n, ...] tensors of the cache dtype")
    rc = lib.paged_kv_gather_blocks(k_cache.data_ptr(), vp, nb, bb, ids.data_ptr(), n,
                                    k_out.data_ptr(),
                                    v_out.data_ptr() if v_out is not None else None,
                                    _handle(stream, k_cache.device))
    if rc != PD_OK:
        raise PagedDecodeError(rc)
    return k_out, v_out


def paged_kv_scatter_blocks(k_in, v_in, ids, k_cache, v_cache, *, stream=None):
    """k_cache[ids[i]] = k_in[i] (and the same for V)
    (``paged_kv_scatter_blocks``). In place on the caches."""
    nb, bb, vp = _pool(k_cache, v_cache)
    _ids(ids, "ids")
    n = int(ids.numel())
    shape = (n,) + tuple(k_cache.shape[1:])
    _on_gpu(k_cache.device, ids=ids, k_in=k_in, v_in=v_in)
    for t in (k_in, v_in):
        if t is not None and (tuple(t.shape) != shape or t.dtype != k_cache.dtype
                              or not t.is_contiguous()):
            raise ValueError("inputs must be contiguous [n, ...] tensors of the cache dtype")
    rc = lib.paged_kv_scatter_blocks(k_in.data_ptr(), v_in.data_ptr() if v_in is not None else None,
                                     ids.data_ptr(), n, k_cache.data_ptr(), vp, nb, bb,
                                     _handle(stream, k_cache.device))
    if rc != PD_OK:
        raise PagedDecodeError(rc)


def paged_kv_compact_plan(live):
    """Host compaction plan (``paged_kv_compact_plan``) of a live mask (any
    CPU array-like of num_blocks truthy values): returns (pairs int32 [m, 2],
    remap int32 [num_blocks], n_live) as CPU tensors / int."""
    live_t = torch.as_tensor(live).to(torch.uint8).contiguous().cpu()
    nb = int(live_t.numel())
    cap = nb // 2 + 1
    pairs = torch.empty((cap, 2), dtype=torch.int32)
    remap = torch.empty(nb, dtype=torch.int32)
    m, n = ctypes.c_int32(0), ctypes.c_int32(0)
    rc = lib.paged_kv_compact_plan(live_t.data_ptr(), nb, pairs.data_ptr(), cap, ctypes.byref(m),
                                   remap.data_ptr(), ctypes.byref(n))
    if rc != PD_OK:
        raise PagedDecodeError(rc)
    return pairs[: m.value].clone(), remap, n.value


def paged_kv_remap_block_table(block_table, remap, *, stream=None):
    """In place: every entry e of the device int32 block table with
    0 <= e < len(remap) becomes remap[e] (``paged_kv_remap_block_table``)."""
    _on_gpu(block_table.device, remap=remap)
    _ids(block_table, "block_table")
    _ids(remap, "remap")
    rc = lib.paged_kv_remap_block_table(block_table.data_ptr(), int(block_table.numel()),
                                        remap.data_ptr(), int(remap.numel()),
                                        _handle(stream, block_table.device))
    if rc != PD_OK:
        raise PagedDecodeError(rc)


def paged_kv_compact(k_cache, v_cache, live, block_tables, *, stream=None):
    """Compaction in one call: plan on the host from the live mask, copy the
    moved blocks and remap every given device block table in place. Returns
    (n_live, number of moved blocks, remap on the device)."""
    pairs, remap, n = paged_kv_compact_plan(live)
    dev = k_cache.device
    remap_d = remap.to(dev)
    if pairs.shape[0] > 0:
        paged_kv_copy_blocks(k_cache, v_cache, pairs.to(dev), stream=stream)
    for bt in block_tables:
        paged_kv_remap_block_table(bt, remap_d, stream=stream)
    return n, int(pairs.shape[0]), remap_d
