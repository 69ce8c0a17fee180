"""fp64 CPU oracle for paged GQA decode attention.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the HIP library
never does, and this package imports nothing from it.

The arithmetic lives in ``pd_oracle.c`` (plain C, fp64, threaded over
(sequence, query-head) pairs); this module only marshals numpy arrays into it.
What it computes follows the Loom Kernels home page ("Supported now": paged
MQA/GQA decode with GQA packing and local split-K/LSE): the exact softmax
attention of one query token per head over the paged cache, plus the
per-partition results and their log-sum-exp merge; and, for an FP8 cache
(same page, "Next boundaries": FP8 KV-cache compression), the same over
E4M3FN codes times a float32 scale per tensor.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, invariants and brute-force identities; see that file).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pd_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libpd_oracle.so")

F16, BF16 = 0, 1
_DT = {"f16": F16, "bf16": BF16, F16: F16, BF16: BF16}

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile pd_oracle.c with gcc into oracle/_build/libpd_oracle.so."""
    if not force and os.path.exists(_LIB):
        return _LIB
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-pthread", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        # PD_ORACLE_LIB: another build of the same source (the sanitizer
        # tests load an instrumented one)
        path = os.environ.get("PD_ORACLE_LIB")
        if not path:
            if not os.path.exists(_LIB):
                build()
            path = _LIB
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.pdo_attention.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i64,
                                      f64, i32, P, P, i32]
        lib.pdo_attention.restype = i32
        lib.pdo_partials.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i64,
                                     f64, i32, i32, i32, P, P, i32]
        lib.pdo_partials.restype = i32
        lib.pdo_merge.argtypes = [P, P, P, i32, i32, i32, i32, i32, P]
        lib.pdo_merge.restype = i32
        lib.pdo_round.argtypes = [P, i64, i32, P]
        lib.pdo_round.restype = None
        lib.pdo_widen.argtypes = [P, i64, i32, P]
        lib.pdo_widen.restype = None
        lib.pdo_widen_fp8.argtypes = [P, i64, P]
        lib.pdo_widen_fp8.restype = None
        lib.pdo_attention_fp8kv.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i64,
                                            f64, i32, f64, f64, P, P, i32]
        lib.pdo_attention_fp8kv.restype = i32
        lib.pdo_partials_fp8kv.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i64,
                                           f64, i32, f64, f64, i32, i32, P, P, i32]
        lib.pdo_partials_fp8kv.restype = i32
        _lib = lib
        return lib


class OracleError(RuntimeError):
    pass


_MSG = {-1: "bad shape", -2: "live block id outside the pool",
        -3: "context length outside [0, max_blocks_per_seq*block_size]",
        -4: "out of memory", -5: "bad dtype"}


def _c(a, dt):
    a = np.ascontiguousarray(a, dtype=dt)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc < 0:
        raise OracleError(_MSG.get(rc, f"status {rc}"))
    return rc


def _inputs(q, k_cache, v_cache, block_table, context_lens, kv=np.uint16):
    q, qp = _c(q, np.uint16)
    k, kp = _c(k_cache, kv)
    v, vp = _c(v_cache, kv)
    bt, btp = _c(block_table, np.int32)
    cl, clp = _c(context_lens, np.int32)
    if k.shape != v.shape or k.ndim != 4 or q.ndim != 3 or bt.ndim != 2:
        raise OracleError("bad shape")
    return (q, k, v, bt, cl), (qp, kp, vp, btp, clp)


def attention(q, k_cache, v_cache, block_table, context_lens, *, scale, dtype,
              nthreads: int = 0, return_threads: bool = False):
    """Exact single-pass attention in fp64.

    q: uint16 [B,Hq,D]; k_cache/v_cache: uint16 [NB,bs,Hkv,D];
    block_table: int32 [B,MB]; context_lens: int32 [B]; scale: the float32
    scale (widened exactly); dtype: 'bf16' | 'f16'.
    Returns (out fp64 [B,Hq,D], lse fp64 [B,Hq]) (and the thread count).
    """
    lib = _load()
    keep, (qp, kp, vp, btp, clp) = _inputs(q, k_cache, v_cache, block_table, context_lens)
    qa, k, _, bt, _ = keep
    B, Hq, D = qa.shape
    NB, bs, Hkv, Dk = k.shape
    if Dk != D or bt.shape[0] != B:
        raise OracleError("bad shape")
    out = np.empty((B, Hq, D), np.float64)
    lse = np.empty((B, Hq), np.float64)
    rc = lib.pdo_attention(qp, kp, vp, btp, clp, B, Hq, Hkv, D, bs, bt.shape[1], NB,
                           float(np.float32(scale)), _DT[dtype],
                           out.ctypes.data_as(ctypes.c_void_p),
                           lse.ctypes.data_as(ctypes.c_void_p), int(nthreads))
    nt = _check(rc)
    return (out, lse, nt) if return_threads else (out, lse)


def partials(q, k_cache, v_cache, block_table, context_lens, *, scale, dtype,
             partition_tokens: int, num_splits: int, nthreads: int = 0):
    """Per-partition (o_part [B,Hq,S,D], lse_part [B,Hq,S]) in fp64."""
    lib = _load()
    keep, (qp, kp, vp, btp, clp) = _inputs(q, k_cache, v_cache, block_table, context_lens)
    qa, k, _, bt, _ = keep
    B, Hq, D = qa.shape
    NB, bs, Hkv, _ = k.shape
    S = int(num_splits)
    o = np.empty((B, Hq, S, D), np.float64)
    lse = np.empty((B, Hq, S), np.float64)
    rc = lib.pdo_partials(qp, kp, vp, btp, clp, B, Hq, Hkv, D, bs, bt.shape[1], NB,
                          float(np.float32(scale)), _DT[dtype], int(partition_tokens), S,
                          o.ctypes.data_as(ctypes.c_void_p),
                          lse.ctypes.data_as(ctypes.c_void_p), int(nthreads))
    _check(rc)
    return o, lse


def merge(o_part, lse_part, context_lens, *, partition_tokens: int):
    """LSE merge of the non-empty partitions, in order, in fp64."""
    lib = _load()
    o, op = _c(o_part, np.float64)
    l, lp = _c(lse_part, np.float64)
    cl, clp = _c(context_lens, np.int32)
    B, Hq, S, D = o.shape
    out = np.empty((B, Hq, D), np.float64)
    _check(lib.pdo_merge(op, lp, clp, B, Hq, S, D, int(partition_tokens),
                         out.ctypes.data_as(ctypes.c_void_p)))
    return out


def round_to_dtype(x, dtype) -> np.ndarray:
    """fp64 -> 16-bit pattern, round-to-nearest-even in one step."""
    lib = _load()
    a, ap = _c(x, np.float64)
    out = np.empty(a.shape, np.uint16)
    lib.pdo_round(ap, a.size, _DT[dtype], out.ctypes.data_as(ctypes.c_void_p))
    return out


def widen(bits, dtype) -> np.ndarray:
    """16-bit pattern -> exact fp64 value."""
    lib = _load()
    a, ap = _c(bits, np.uint16)
    out = np.empty(a.shape, np.float64)
    lib.pdo_widen(ap, a.size, _DT[dtype], out.ctypes.data_as(ctypes.c_void_p))
    return out


def widen_fp8(codes) -> np.ndarray:
    """E4M3FN byte code -> exact fp64 value (NaN for the two NaN codes)."""
    lib = _load()
    a, ap = _c(codes, np.uint8)
    out = np.empty(a.shape, np.float64)
    lib.pdo_widen_fp8(ap, a.size, out.ctypes.data_as(ctypes.c_void_p))
    return out


def attention_fp8(q, k_cache, v_cache, block_table, context_lens, *, scale, dtype, k_scale,
                  v_scale, nthreads: int = 0, return_threads: bool = False):
    """``attention`` over an FP8 cache: k_cache/v_cache are uint8 E4M3FN codes
    [NB,bs,Hkv,D] standing for code * k_scale and code * v_scale (float32
    scales, widened exactly); q stays 16-bit."""
    lib = _load()
    keep, (qp, kp, vp, btp, clp) = _inputs(q, k_cache, v_cache, block_table, context_lens,
                                           kv=np.uint8)
    qa, k, _, bt, _ = keep
    B, Hq, D = qa.shape
    NB, bs, Hkv, Dk = k.shape
    if Dk != D or bt.shape[0] != B:
        raise OracleError("bad shape")
    out = np.empty((B, Hq, D), np.float64)
    lse = np.empty((B, Hq), np.float64)
    rc = lib.pdo_attention_fp8kv(qp, kp, vp, btp, clp, B, Hq, Hkv, D, bs, bt.shape[1], NB,
                                 float(np.float32(scale)), _DT[dtype],
                                 float(np.float32(k_scale)), float(np.float32(v_scale)),
                                 out.ctypes.data_as(ctypes.c_void_p),
                                 lse.ctypes.data_as(ctypes.c_void_p), int(nthreads))
    nt = _check(rc)
    return (out, lse, nt) if return_threads else (out, lse)


def partials_fp8(q, k_cache, v_cache, block_table, context_lens, *, scale, dtype, k_scale,
                 v_scale, partition_tokens: int, num_splits: int, nthreads: int = 0):
    """``partials`` over an FP8 cache."""
    lib = _load()
    keep, (qp, kp, vp, btp, clp) = _inputs(q, k_cache, v_cache, block_table, context_lens,
                                           kv=np.uint8)
    qa, k, _, bt, _ = keep
    B, Hq, D = qa.shape
    NB, bs, Hkv, _ = k.shape
    S = int(num_splits)
    o = np.empty((B, Hq, S, D), np.float64)
    lse = np.empty((B, Hq, S), np.float64)
    rc = lib.pdo_partials_fp8kv(qp, kp, vp, btp, clp, B, Hq, Hkv, D, bs, bt.shape[1], NB,
                                float(np.float32(scale)), _DT[dtype],
                                float(np.float32(k_scale)), float(np.float32(v_scale)),
                                int(partition_tokens), S, o.ctypes.data_as(ctypes.c_void_p),
                                lse.ctypes.data_as(ctypes.c_void_p), int(nthreads))
    _check(rc)
    return o, lse


def attention_case(case, **kw):
    """``attention`` (or ``attention_fp8`` for an FP8 cache) over a ``workloads.Case``."""
    if getattr(case, "kv_dtype", "") == "fp8":
        return attention_fp8(case.q, case.k_cache, case.v_cache, case.block_table,
                             case.context_lens, scale=case.scale, dtype=case.dtype,
                             k_scale=case.k_scale, v_scale=case.v_scale, **kw)
    return attention(case.q, case.k_cache, case.v_cache, case.block_table,
                     case.context_lens, scale=case.scale, dtype=case.dtype, **kw)
