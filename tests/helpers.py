"""Shared helpers of the GPU tests: upload a generated case, run the library,
and compare its 16-bit output with the fp64 oracle.

Tolerance (north-star bar "max abs 1e-2 and max rel 1e-2", read element-wise
as an allclose): |g - r| <= 1e-2 + 1e-2 * |r| for every element, where g is
the GPU value and r the unrounded fp64 oracle value. A second, tighter gate
catches indexing slips that 1e-2 would let through (a token dropped out of a
thousand moves the output by ~1e-3): g must be within one unit in the last
place of the dtype of RNE(r), the oracle rounded once to the dtype, unless
|g - r| <= FP32_FLOOR. The floor is the absolute error of fp32 accumulation
(output = sum_t p_t v_t / sum_t p_t in fp32, "fp32 accumulation, output
rounded to dtype"): its rounding error scales with the size of the summands
(|v| of order 1), not with the output, so an output that nearly cancels to
~1e-6 carries an absolute error of a few 1e-8 that is several bf16 ulps of
that tiny value. 1e-6 is 20x the largest such error seen and 1000x below the
shift a single dropped token causes at 1,024 tokens.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

ABS_TOL = 1e-2
REL_TOL = 1e-2
ULP_TOL = 1
FP32_FLOOR = 1e-6


def device_case(case, device="cuda"):
    """The case's tensors on the GPU: q, k_cache, v_cache, block_table, context_lens."""
    q, k, v = case.torch_views()
    return (q.to(device), k.to(device), v.to(device),
            torch.from_numpy(case.block_table).to(device),
            torch.from_numpy(case.context_lens).to(device))


def out_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def ordered(bits: np.ndarray) -> np.ndarray:
    """Map 16-bit float patterns onto integers in value order (for ulp distance)."""
    b = bits.astype(np.int32)
    neg = (b & 0x8000) != 0
    return np.where(neg, -(b & 0x7FFF), b)


def compare(gpu_bits: np.ndarray, ref: np.ndarray, dtype: str, *, what: str = ""):
    """Assert both gates; return a small report dict."""
    assert gpu_bits.shape == ref.shape, (gpu_bits.shape, ref.shape)
    g = oracle.widen(gpu_bits, dtype)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - ref)
    bound = ABS_TOL + REL_TOL * np.abs(ref)
    bad = err > bound
    rne = oracle.round_to_dtype(ref, dtype)
    ulp = np.abs(ordered(gpu_bits) - ordered(rne))
    big = np.abs(ref) >= 1e-2
    rep = {
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_rel": float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
        "max_ulp": int(ulp.max()) if ulp.size else 0,
        "frac_exact": float((ulp == 0).mean()) if ulp.size else 1.0,
    }
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: tolerance exceeded at {i}: gpu={g[i]!r} oracle={ref[i]!r} {rep}")
    far = (ulp > ULP_TOL) & (err > FP32_FLOOR)
    if far.any():
        i = np.unravel_index(np.argmax(np.where(far, ulp, -1)), ulp.shape)
        raise AssertionError(f"{what}: {int(ulp[i])} ulp from RNE(oracle) at {i}: "
                             f"gpu={g[i]!r} oracle={ref[i]!r} {rep}")
    return rep


def run_library(case, num_splits=None, dev=None):
    import paged_gqa_decode_02_amd as pd
    dev = dev if dev is not None else device_case(case)
    q, k, v, bt, cl = dev
    if getattr(case, "fp8", False):
        out = pd.paged_decode_attention_fp8(q, k, v, bt, cl, k_scale=case.k_scale,
                                            v_scale=case.v_scale, scale=case.scale,
                                            num_splits=num_splits)
    else:
        out = pd.paged_decode_attention(q, k, v, bt, cl, scale=case.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out


def check_case(case, num_splits=None, what=None):
    out = run_library(case, num_splits)
    ref, _ = oracle.attention_case(case)
    return compare(out_bits(out), ref, case.dtype, what=what or case.name)


__all__ = ["device_case", "out_bits", "compare", "run_library", "check_case", "workloads"]
