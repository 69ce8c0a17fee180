#!/usr/bin/env python3
"""Benchmark of paged GQA decode attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload large|splitk_B8_L1024|...]

Prints ONE JSON line. A step is one call of the library's entry point
(host plan + decode kernel [+ LSE merge kernel]) over one batch of synthetic
input that is already resident in HBM. `value` is the achieved algorithmic
bandwidth in GB/s: (K+V bytes of the valid tokens + Q + O bytes) / time per
call; `ms_per_step` is the time per call. The default workload is the
bandwidth-bound large decode: batch 64, context 4,096, Hq/Hkv 32/8, D 128,
bf16, block size 16, whose 1 GiB of K+V per call does not fit the 256 MB
Infinity Cache, so every call streams from HBM.

The output of the first call is kept; after the GPU timing (so that the
GPU does not sit idle during the CPU work right before its warmup), one call
of the fp64 CPU oracle checks it on its sampled sequences, and a case that
fails prints an error line instead of a result. Further oracle calls on the
same sequences give `cpu_baseline` (the median call). The secondary workloads get checks
that need no oracle (finite, bit-for-bit repeatable); their parity is what
the GPU tests cover.

Other modes:
  --calibrate-copy   only run device-to-device copies of a known size
                     (reference kernel for the HBM traffic counters)
  --extras-only      only the RoPE + KV write and block-movement tables
  --ingest-pmc F W CF CW
                     turn four rocprofv3 --pmc counter CSVs (FETCH_SIZE and
                     WRITE_SIZE of the bench run, then of the copy run) into
                     profiles/traffic_<workload>.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call + achieved HBM GB/s (% of peak), paged GQA decode Hq/Hkv 32/8 D128"
PEAK_GBPS = 8000.0          # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "paged_gqa_decode_02_amd", "csrc", "pd_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")
DECODE_KERNEL = "pd_decode_kernel"
COPY_BYTES = 1 << 30


def kernel_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def make_workload(name: str, seed: int = 0):
    """Workload by name; a trailing "_fp8" stores the K/V cache as E4M3FN codes."""
    import workloads
    kv = ""
    if name.endswith("_fp8"):
        name, kv = name[:-4], "fp8"
    if name == "large":
        return workloads.large(seed, kv_dtype=kv)
    if name == "ragged":
        return workloads.ragged(seed, kv_dtype=kv)
    if name == "tiny":
        return workloads.tiny(seed, kv_dtype=kv)
    if name.startswith("splitk_"):
        _, b, l = name.split("_")
        return workloads.splitk(int(b[1:]), int(l[1:]), seed, kv_dtype=kv)
    if name.startswith("geom_"):
        # geom_14x2_D64_B32_L1024
        _, hh, d, b, l = name.split("_")
        hq, hkv = hh.split("x")
        return workloads.geometry(int(hq), int(hkv), int(d[1:]), int(b[1:]), int(l[1:]), seed,
                                  kv_dtype=kv)
    if name.startswith("short_"):
        # short_B32_L64_bf16_bs16
        _, b, l, dt, bs = name.split("_")
        return workloads.short(int(b[1:]), int(l[1:]), dt, int(bs[2:]), seed, kv_dtype=kv)
    raise SystemExit(f"unknown workload {name!r}")


def attend(pd, case, q, k, v, bt, cl, out, ws, num_splits=None):
    """One library call on the workload's inputs (the FP8 entry point for an FP8 cache)."""
    if case.fp8:
        return pd.paged_decode_attention_fp8(q, k, v, bt, cl, out, k_scale=case.k_scale,
                                             v_scale=case.v_scale, scale=case.scale,
                                             workspace=ws, num_splits=num_splits)
    return pd.paged_decode_attention(q, k, v, bt, cl, out, scale=case.scale, workspace=ws,
                                     num_splits=num_splits)


def upload(case, torch):
    q, k, v = (t.to("cuda") for t in case.torch_views())
    bt = torch.from_numpy(case.block_table).to("cuda")
    cl = torch.from_numpy(case.context_lens).to("cuda")
    return q, k, v, bt, cl


def self_check(out, again, torch):
    """Checks of a GPU output that need no oracle: every element finite, and
    a second call over the same inputs gives the same bits."""
    finite = bool(torch.isfinite(out.float()).all())
    stable = bool(torch.equal(out.view(torch.int16), again.view(torch.int16)))
    return finite and stable, {"finite": finite, "bitwise_repeatable": stable}


def time_calls(fn, iters: int, warmup: int, torch) -> float:
    """Average ms per call over `iters` calls, HIP events on the current stream."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def time_samples(fn, iters: int, samples: int, torch, check=None) -> list:
    """ms per call of each of `samples` back-to-back blocks of `iters` calls,
    every block between its own pair of HIP events; `check()` (if given) runs
    after each block, outside the timed span."""
    out = []
    for _ in range(samples):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / iters)
        if check is not None:
            check()
    return out


def sample_stats(ms_list) -> dict:
    """Median, min and max µs per call over timing samples."""
    us = sorted(m * 1e3 for m in ms_list)
    n = len(us)
    med = us[n // 2] if n % 2 else 0.5 * (us[n // 2 - 1] + us[n // 2])
    return {"n": n, "median_us": round(med, 3), "min_us": round(us[0], 3),
            "max_us": round(us[-1], 3)}


def graph_of(fn, iters: int, torch):
    """`iters` calls captured in one HIP graph, after three eager calls on the
    capture stream; the graph has been replayed once."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    return g


def time_graph(fn, iters: int, torch) -> float:
    """Average ms per call when `iters` calls are captured in one HIP graph."""
    return time_graph_samples(fn, iters, 1, torch)[0]


def time_graph_samples(fn, iters: int, samples: int, torch, check=None) -> list:
    """ms per call of each of `samples` replays of one graph of `iters` calls."""
    g = graph_of(fn, iters, torch)
    out = []
    for _ in range(samples):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / iters)
        if check is not None:
            check()
    return out


def replicas_for(case, torch, pd, min_bytes=1 << 30):
    """Device replicas of the whole input set, enough to cover min_bytes, so
    that a rotating loop cannot be served from the 256 MB Infinity Cache."""
    base = upload(case, torch)
    foot = sum(t.numel() * t.element_size() for t in base)
    R = max(1, math.ceil(min_bytes / foot))
    reps = [base] + [tuple(t.clone() for t in base) for _ in range(R - 1)]
    outs = [torch.empty_like(base[0]) for _ in range(R)]
    wss = [pd.alloc_workspace(r[0], r[1], r[3]) for r in reps]
    return reps, outs, wss, foot


def overhead_bytes(case, S: int) -> dict:
    """Bytes a call moves beyond the algorithmic ones (not counted in GB/s):
    the block table and context lengths it reads, and at S > 1 the fp32
    partial outputs and log-sum-exps, written once and read back once."""
    return {"block_table": 4 * case.B * case.max_blocks_per_seq, "context_lens": 4 * case.B,
            "split_workspace_each_way": 4 * case.B * case.Hq * S * (case.D + 1) if S > 1 else 0}


def bench_other(name, torch, pd, iters=200, warmup=20, samples=7):
    case = make_workload(name)
    reps, outs, wss, foot = replicas_for(case, torch, pd)
    R = len(reps)

    def call(i):
        q, k, v, bt, cl = reps[i % R]
        attend(pd, case, q, k, v, bt, cl, outs[i % R], wss[i % R])

    call(0)
    torch.cuda.synchronize()
    first = outs[0].clone()
    call(0)
    torch.cuda.synchronize()
    ok, chk = self_check(outs[0], first, torch)
    if not ok:
        return {"check": "FAIL", **chk}
    time_calls(call, iters, warmup, torch)
    st = sample_stats(time_samples(call, iters, samples, torch))
    iters_g = max(R, (iters // R) * R)
    gt = sample_stats(time_graph_samples(call, iters_g, samples, torch))
    ms, ms_g = st["median_us"] * 1e-3, gt["median_us"] * 1e-3
    S, P = pd.paged_decode_plan(case.B, case.Hq, case.Hkv, case.D, case.max_blocks_per_seq,
                                case.block_size, torch.bfloat16 if case.dtype == "bf16"
                                else torch.float16)
    nbytes = case.algorithmic_bytes()
    res = {"us_per_call": round(ms * 1e3, 3), "us_per_call_graph": round(ms_g * 1e3, 3),
           "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "GBps_graph": round(nbytes / (ms_g * 1e-3) / 1e9, 1),
           "frac_of_peak_graph": round(nbytes / (ms_g * 1e-3) / 1e9 / PEAK_GBPS, 4),
           "algorithmic_bytes": nbytes, "overhead_bytes": overhead_bytes(case, S),
           "splits": S, "partition_tokens": P, "replicas": R, "rotated_bytes": R * foot, "check": chk,
           "samples": {"calls_per_sample": iters, "stream": st, "graph": gt}}
    if case.fp8:
        res["kv_dtype"] = "fp8_e4m3fn"
    del reps, outs, wss
    torch.cuda.empty_cache()
    return res


ROPE_CASES = ("scatter_T1", "scatter_T8", "scatter_T32", "scatter_T64", "scatter_T128",
              "scatter_T512", "prefill_4x4096", "scatter_T64_fp8", "prefill_4x4096_fp8")


def rope_fp8_scales(case, torch):
    """Per-tensor scales of an FP8 cache write, from the inputs' largest
    magnitudes (keys: times sqrt 2, the most a rotation can grow a
    coordinate): amax / 448, so no code saturates."""
    import workloads
    x = torch.from_numpy(case.qkv.view(np.int16)).view(workloads.DTYPES[case.dtype]).float()
    H, G = case.Hq, case.Hkv
    k_amax = float(x[:, H:H + G].abs().max()) * math.sqrt(2.0)
    v_amax = float(x[:, H + G:].abs().max())
    return max(k_amax, 1e-30) / 448.0, max(v_amax, 1e-30) / 448.0


def rope_check(case, qkv, qo, vc, torch):
    """Oracle-free checks of one RoPE + KV write: q_out finite, each rotated
    pair as long as before up to the output rounding, and the value rows at
    the written slots equal to the inputs bit for bit."""
    H, D = case.Hq, case.D
    q = qkv[:, :H].float()
    r = qo.float()
    h = D // 2
    n0 = torch.hypot(q[..., :h], q[..., h:])
    n1 = torch.hypot(r[..., :h], r[..., h:])
    ulp = 2.0 ** -7 if case.dtype == "bf16" else 2.0 ** -10
    norm_ok = bool((n1 - n0).abs().le(ulp * n0 + 1e-6).all())
    finite = bool(torch.isfinite(r).all())
    chk = {"finite": finite, "pair_norms_kept": norm_ok}
    if vc is None:  # the caller checks the cache itself
        return finite and norm_ok, chk
    live = torch.from_numpy(case.slot_mapping).cuda().long()
    live = live[live >= 0]
    vrows = vc.view(-1, case.Hkv, D)[live]
    v_in = qkv[:, H + case.Hkv:][torch.from_numpy(case.slot_mapping >= 0).cuda()]
    v_ok = bool(torch.equal(vrows.view(torch.int16), v_in.reshape(vrows.shape).view(torch.int16)))
    chk["values_copied_exactly"] = v_ok
    return finite and norm_ok and v_ok, chk


def rope_check_fp8(case, qkv, qo, vc, torch, vs):
    """Oracle-free checks of one RoPE write into an FP8 cache: q_out as in
    rope_check, and each value code within half an E4M3FN step of value /
    v_scale, held at 448 (torch's own float8 widening)."""
    H, G, D = case.Hq, case.Hkv, case.D
    ok16, chk = rope_check(case, qkv, qo, None, torch)
    live = torch.from_numpy(case.slot_mapping).cuda().long()
    live = live[live >= 0]
    got = vc.view(-1, G, D)[live].view(torch.float8_e4m3fn).float()
    v_in = qkv[:, H + G:][torch.from_numpy(case.slot_mapping >= 0).cuda()].float() / vs
    v_in = v_in.reshape(got.shape).clamp(-448.0, 448.0)
    close = bool(((got - v_in).abs() <= 2.0 ** -4 * v_in.abs() + 2.0 ** -10).all())
    chk["value_codes_nearest"] = close
    return ok16 and close, chk


def bench_rope(name, torch, pd, table, iters=200, warmup=20):
    """RoPE + paged KV write at the decode geometry (Hq/Hkv 32/8, D 128,
    bf16, block size 16): T tokens at random positions into distinct random
    slots, or a 4 x 4,096-token prefill through block tables; a "_fp8"
    suffix writes E4M3FN codes into an FP8 cache instead."""
    from workloads import rope as wrope
    fp8 = name.endswith("_fp8")
    if fp8:
        name = name[:-4]
    if name.startswith("scatter_T"):
        case = wrope.scatter(int(name[len("scatter_T"):]), seed=1)
    else:
        n, t = name[len("prefill_"):].split("x")
        case = wrope.prefill(int(n), int(t), seed=1)
    dt = torch.bfloat16

    def up():
        qkv = case.torch_qkv().cuda()
        if fp8:
            kc, vc = (torch.zeros(case.k_cache.shape, dtype=torch.uint8, device="cuda")
                      for _ in range(2))
        else:
            kc, vc = (t.cuda() for t in case.torch_caches())
        return (qkv, kc, vc, torch.from_numpy(case.positions).cuda(),
                torch.from_numpy(case.slot_mapping).cuda(),
                torch.empty((case.T, case.Hq, case.D), dtype=dt, device="cuda"))

    base = up()
    foot = sum(t.numel() * t.element_size() for t in base)
    # big cases rotate over replicas that overflow the 256 MB Infinity Cache;
    # small ones stay cache-resident, as they are when a projection has just
    # written q, k and v
    R = max(1, math.ceil((1 << 30) / foot)) if foot > (64 << 20) else 1
    reps = [base] + [up() for _ in range(R - 1)]
    H, G = case.Hq, case.Hkv
    # the q, k and v views of each packed QKV array, made once (as a serving
    # loop holds them): slicing a tensor costs microseconds of host time
    views = [(r[0][:, :H], r[0][:, H:H + G], r[0][:, H + G:]) + r[1:] for r in reps]

    ks, vs = rope_fp8_scales(case, torch) if fp8 else (1.0, 1.0)

    def call(i):
        q, k, v, kc, vc, pos, slots, qo = views[i % R]
        if fp8:
            pd.rope_paged_kv_write_fp8(q, k, v, pos, slots, table, kc, vc, q_out=qo, k_scale=ks,
                                       v_scale=vs)
        else:
            pd.rope_paged_kv_write(q, k, v, pos, slots, table, kc, vc, q_out=qo)

    call(0)
    torch.cuda.synchronize()
    if fp8:
        ok, chk = rope_check_fp8(case, base[0], base[5], base[2], torch, vs)
    else:
        ok, chk = rope_check(case, base[0], base[5], base[2], torch)
    if not ok:
        return {"check": "FAIL", **chk}
    time_calls(call, iters, warmup, torch)
    st = sample_stats(time_samples(call, iters, 7, torch))
    gt = sample_stats(time_graph_samples(call, max(R, (iters // R) * R), 7, torch))
    ms, ms_g = st["median_us"] * 1e-3, gt["median_us"] * 1e-3
    nbytes = case.algorithmic_bytes(1 if fp8 else 2)
    res = {"tokens": case.T, "us_per_call": round(ms * 1e3, 3),
           "us_per_call_graph": round(ms_g * 1e3, 3),
           "GBps_graph": round(nbytes / (ms_g * 1e-3) / 1e9, 1),
           "frac_of_peak_graph": round(nbytes / (ms_g * 1e-3) / 1e9 / PEAK_GBPS, 4),
           "algorithmic_bytes": nbytes, "replicas": R, "check": chk,
           "samples": {"calls_per_sample": iters, "stream": st, "graph": gt}}
    del reps, base, views
    torch.cuda.empty_cache()
    return res


BLOCK_CASES = ("copy_4096", "gather_4096", "scatter_4096", "compact_16384")


def bench_blocks(name, torch, pd, iters=100, warmup=10):
    """KV-cache block movement at the decode geometry (32 KiB blocks: block
    size 16, Hkv 8, D 128, bf16; K and V): 4,096 blocks copied, gathered or
    scattered in a 16,384-block pool, or the compaction of such a pool with
    half its blocks live, dealt to 64 sequences (device part: the moves and
    the remap of their block table; the host plan is timed on its own). Two pools
    alternate so the moved bytes do not stay in the 256 MB Infinity Cache."""
    from workloads import blocks as wb
    nb, n = 16384, 4096
    pools = []
    for r in range(2):
        case = wb.pool(nb, seed=r) if r == 0 else None
        kc = torch.empty((nb, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
        vc = torch.empty_like(kc)
        if case is not None:
            k0, v0 = case.torch_caches()
            kc.copy_(k0)
            vc.copy_(v0)
        else:
            kc.copy_(pools[0][0])
            vc.copy_(pools[0][1])
        pools.append((kc, vc))
    bb = 16 * 8 * 128 * 2
    res = {"block_bytes": bb, "pool_blocks": nb}
    kind = name.split("_")[0]
    if kind == "copy":
        pairs = torch.from_numpy(wb.copy_pairs(nb, n, seed=1)).cuda()

        def call(i):
            kc, vc = pools[i % 2]
            pd.paged_kv_copy_blocks(kc, vc, pairs)
        nbytes = 2 * 2 * n * bb + 8 * n
    elif kind in ("gather", "scatter"):
        ids = torch.from_numpy(wb.block_ids(nb, n, seed=1)).cuda()
        bufs = [(torch.empty((n, 16, 8, 128), dtype=torch.bfloat16, device="cuda"),
                 torch.empty((n, 16, 8, 128), dtype=torch.bfloat16, device="cuda"))
                for _ in range(2)]

        def call(i):
            kc, vc = pools[i % 2]
            ko, vo = bufs[i % 2]
            if kind == "gather":
                pd.paged_kv_gather_blocks(kc, vc, ids, ko, vo)
            else:
                pd.paged_kv_scatter_blocks(ko, vo, ids, kc, vc)
        nbytes = 2 * 2 * n * bb + 4 * n
    else:
        live, bt, _ = wb.live_pool(nb, 64, live_frac=0.5, seed=1)
        t0 = time.perf_counter()
        for _ in range(10):
            pairs_h, remap_h, n_live = pd.paged_kv_compact_plan(live)
        res["host_plan_us"] = round((time.perf_counter() - t0) / 10 * 1e6, 1)
        pairs = pairs_h.cuda()
        remap = remap_h.cuda()
        table = torch.from_numpy(bt).cuda()
        n = int(pairs.shape[0])
        res.update({"live_blocks": n_live, "moved_blocks": n, "table_entries": table.numel()})

        def call(i):
            kc, vc = pools[i % 2]
            pd.paged_kv_copy_blocks(kc, vc, pairs)
            pd.paged_kv_remap_block_table(table, remap)
        nbytes = 2 * 2 * n * bb + 8 * n + 8 * table.numel() + 4 * nb
    kc0, vc0 = pools[0]
    if kind == "compact":
        before = (kc0.clone(), vc0.clone())
    call(0)
    torch.cuda.synchronize()

    def same(a, b):
        return bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))

    # oracle-free check of the first call: every moved block holds its
    # source's bytes (and the remapped table its new ids)
    if kind == "copy":
        src, dst = pairs[:, 0].long(), pairs[:, 1].long()
        res["check"] = {"blocks_copied_exactly": same(kc0[dst], kc0[src]) and
                        same(vc0[dst], vc0[src])}
    elif kind in ("gather", "scatter"):
        ko, vo = bufs[0]
        res["check"] = {"blocks_moved_exactly": same(kc0[ids.long()], ko) and
                        same(vc0[ids.long()], vo)}
    else:
        src, dst = pairs[:, 0].long(), pairs[:, 1].long()
        want = np.where(bt >= 0, remap_h.numpy()[np.maximum(bt, 0)], bt)
        res["check"] = {"blocks_copied_exactly": same(kc0[dst], before[0][src]) and
                        same(vc0[dst], before[1][src]),
                        "table_remapped": bool(np.array_equal(table.cpu().numpy(), want))}
        del before
    time_calls(call, iters, warmup, torch)
    st = sample_stats(time_samples(call, iters, 7, torch))
    gt = sample_stats(time_graph_samples(call, iters, 7, torch))
    ms, ms_g = st["median_us"] * 1e-3, gt["median_us"] * 1e-3
    res.update({"blocks": n, "us_per_call": round(ms * 1e3, 3),
                "us_per_call_graph": round(ms_g * 1e3, 3),
                "GBps_graph": round(nbytes / (ms_g * 1e-3) / 1e9, 1),
                "frac_of_peak_graph": round(nbytes / (ms_g * 1e-3) / 1e9 / PEAK_GBPS, 4),
                "algorithmic_bytes": nbytes,
                "samples": {"calls_per_sample": iters, "stream": st, "graph": gt}})
    del pools
    torch.cuda.empty_cache()
    return res


def _oracle_call(case, nseq: int, nthreads: int):
    """One oracle call on the first `nseq` sequences; (result, threads used)."""
    import oracle
    cl = case.context_lens[:nseq]
    if case.fp8:
        ref, _, used = oracle.attention_fp8(case.q[:nseq], case.k_cache, case.v_cache,
                                            case.block_table[:nseq], cl, scale=case.scale,
                                            dtype=case.dtype, k_scale=case.k_scale,
                                            v_scale=case.v_scale, nthreads=nthreads,
                                            return_threads=True)
    else:
        ref, _, used = oracle.attention(case.q[:nseq], case.k_cache, case.v_cache,
                                        case.block_table[:nseq], cl, scale=case.scale,
                                        dtype=case.dtype, nthreads=nthreads, return_threads=True)
    return ref, used


def oracle_threads() -> int:
    share = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, share or 1))


def oracle_parity(case, gpu_bits, nseq: int):
    """The parity gate of the oracle leg: one fp64 oracle call on the first
    `nseq` sequences, the GPU output of those sequences held to the parity
    tests' allclose gate. Returns (ok, errors, timing) where timing seeds the
    baseline's call times."""
    import numpy as np
    import oracle
    nthreads = oracle_threads()
    t0 = time.perf_counter()
    ref, used = _oracle_call(case, nseq, nthreads)
    first = time.perf_counter() - t0
    g = oracle.widen(gpu_bits[:nseq], case.dtype)
    err = np.abs(g - ref)
    ok = bool(np.all(np.isfinite(g)) and np.all(err <= 1e-2 + 1e-2 * np.abs(ref)))
    errs = {"sequences_checked": int(nseq), "max_abs": float(err.max()),
            "max_rel_gt_1e-2": float((err / np.maximum(np.abs(ref), 1e-2)).max())}
    return ok, errs, {"nseq": nseq, "nthreads": nthreads, "used": used, "times": [first]}


def cpu_baseline(case, timing, min_seconds: float = 10.0, max_calls: int = 25):
    """The oracle's timing: repeat the parity gate's call (same sequences,
    same threads) until at least `min_seconds` of calls have passed, report
    the median call, and add one single-thread call on a smaller sample."""
    nseq, nthreads, used = timing["nseq"], timing["nthreads"], timing["used"]
    times = list(timing["times"])
    while len(times) < max_calls and sum(times) < min_seconds:
        t0 = time.perf_counter()
        _, used = _oracle_call(case, nseq, nthreads)
        times.append(time.perf_counter() - t0)
    calls = len(times)
    times.sort()
    dt = times[calls // 2] if calls % 2 else 0.5 * (times[calls // 2 - 1] + times[calls // 2])
    sub_cl = case.context_lens[:nseq]
    nbytes = (2048 if case.fp8 else 4096) * int(sub_cl.astype("int64").sum()) + 16384 * nseq
    base = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(used),
            "kind": "oracle", "seconds_per_call": round(dt, 3), "calls": calls,
            "seconds_min": round(times[0], 3), "seconds_max": round(times[-1], 3),
            "sample": f"{nseq} of {case.B} sequences of the same workload (full contexts), "
                      f"median of {calls} oracle calls, fp64, {used} threads",
            "threads_used": int(used), **host_cpu()}
    # one single-thread call on a smaller sample of the same sequences
    n1 = max(1, min(nseq, 4))
    t1 = time.perf_counter()
    _oracle_call(case, n1, 1)
    dt1 = time.perf_counter() - t1
    b1 = (2048 if case.fp8 else 4096) * int(case.context_lens[:n1].astype("int64").sum()) + 16384 * n1
    base["single_thread"] = {"value": round(b1 / dt1 / 1e9, 4), "unit": "GB/s",
                             "seconds_per_call": round(dt1, 3), "sequences": n1}
    return base


def host_cpu() -> dict:
    """The host's CPU: model name, vendor, family/model/stepping (from
    /proc/cpuinfo), logical CPUs and physical cores in the machine, and the
    CPUs this process may run on."""
    info = {}
    phys = set()
    try:
        with open("/proc/cpuinfo") as f:
            cur = {}
            for line in f:
                if ":" not in line:
                    if cur:
                        phys.add((cur.get("physical id"), cur.get("core id")))
                    cur = {}
                    continue
                k, v = (x.strip() for x in line.split(":", 1))
                cur[k] = v
                if k in ("model name", "vendor_id", "cpu family", "model", "stepping") and \
                        k not in info:
                    info[k] = v
            if cur:
                phys.add((cur.get("physical id"), cur.get("core id")))
    except OSError:
        pass
    import platform
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"cpu_model": info.get("model name") or platform.processor() or platform.machine(),
            "cpu_vendor": info.get("vendor_id"),
            "cpu_family_model_stepping": [info.get("cpu family"), info.get("model"),
                                          info.get("stepping")],
            "cpu_core_family": _core_family(info.get("vendor_id"), info.get("cpu family")),
            "host_logical_cpus": os.cpu_count(),
            "host_physical_cores": len(phys) if phys and None not in next(iter(phys)) else None,
            "cpus_available_to_process": avail}


def _core_family(vendor, family):
    """AMD's published core family for its CPU family numbers (a virtual
    machine often reports only a generic model name)."""
    if vendor != "AuthenticAMD" or family is None:
        return None
    return {"23": "Zen / Zen 2 (family 17h)", "25": "Zen 3 / Zen 4 (family 19h)",
            "26": "Zen 5 (family 1Ah)"}.get(str(family))


def device_info(torch) -> dict:
    """The GPU the bench ran on and the software stack."""
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", None),
            "compute_units": pr.multi_processor_count,
            "memory_bytes": pr.total_memory, "hip": torch.version.hip, "torch": torch.__version__}


def launch_floor(torch, pd, iters=200):
    """Time per launch of the library's smallest kernel (its one-block fill of a
    256-byte workspace) on a stream and in a HIP graph: the per-call floor."""
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")

    def call(i):
        pd.paged_decode_workspace_init(ws)

    return {"kernel": "pd_zero_kernel (1 block)",
            "us_per_launch": round(time_calls(call, iters, 20, torch) * 1e3, 3),
            "us_per_launch_graph": round(time_graph(call, iters, torch) * 1e3, 3)}


def copy_roof(torch, nbytes=COPY_BYTES, iters=20):
    """Device-to-device copy of 1 GiB (torch's copy kernel): bytes read + written / time."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    ms = time_calls(lambda i: b.copy_(a), iters, 3, torch)
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * nbytes, "GBps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def load_traffic(workload: str):
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_sha():
        return None  # counters were taken on an older kernel
    return t


def read_pmc(path: str, counter: str, kernel_substr: str):
    """Per-dispatch values of `counter` for kernels whose name contains kernel_substr."""
    vals = []
    with open(path) as f:
        for row in csv.DictReader(f):
            if kernel_substr in row.get("Kernel_Name", "") and row.get("Counter_Name") == counter:
                vals.append(float(row["Counter_Value"]))
    return vals


def ingest_pmc(workload, fetch_csv, write_csv, cfetch_csv, cwrite_csv):
    import statistics
    f = read_pmc(fetch_csv, "FETCH_SIZE", DECODE_KERNEL)
    w = read_pmc(write_csv, "WRITE_SIZE", DECODE_KERNEL)
    cf = read_pmc(cfetch_csv, "FETCH_SIZE", "opy")
    cw = read_pmc(cwrite_csv, "WRITE_SIZE", "opy")
    if not (f and w and cf and cw):
        raise SystemExit("missing counter rows")
    # FETCH_SIZE / WRITE_SIZE are in KiB per dispatch; the copy moves COPY_BYTES each way
    kf = COPY_BYTES / (statistics.median(cf) * 1024.0)
    kw = COPY_BYTES / (statistics.median(cw) * 1024.0)
    fetch = statistics.median(f) * 1024.0 * kf
    write = statistics.median(w) * 1024.0 * kw
    doc = {"workload": workload, "kernel": DECODE_KERNEL, "kernel_sha": kernel_sha(),
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "traffic_bytes_per_launch": fetch + write,
           "copy_calibration": {"bytes": COPY_BYTES, "fetch_factor": kf, "write_factor": kw},
           "raw_median_kib": {"fetch": statistics.median(f), "write": statistics.median(w),
                              "copy_fetch": statistics.median(cf),
                              "copy_write": statistics.median(cw)},
           "dispatches": {"fetch": len(f), "write": len(w)}}
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"traffic_{workload}.json")
    with open(out, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")
    print(json.dumps(doc))


def calibrate_copy(torch, n=20):
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(n):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": COPY_BYTES, "copies": n}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--samples", type=int, default=7,
                    help="further timed blocks of --steps calls, stream and graph "
                         "(0: none, only the timed block)")
    ap.add_argument("--workload", default="large")
    ap.add_argument("--splits", type=int, default=None, help="force the split count")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=64)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--extras-only", action="store_true",
                    help="only the RoPE + KV write and block-movement tables (for profiling)")
    ap.add_argument("--ingest-pmc", nargs=4, metavar=("FETCH", "WRITE", "CFETCH", "CWRITE"))
    args = ap.parse_args()

    if args.ingest_pmc:
        ingest_pmc(args.workload, *args.ingest_pmc)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU; there is no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)
    if args.samples < 0 or args.steps < 1:
        print("bench.py: --steps must be at least 1 and --samples at least 0", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_gqa_decode_02_amd as pd
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    if args.extras_only:
        from workloads import rope as wrope
        table = pd.rope_cos_sin_table(32768, 128, wrope.QWEN_BASE)
        print(json.dumps({"rope_kv_write": {n: bench_rope(n, torch, pd, table) for n in ROPE_CASES},
                          "kv_block_moves": {n: bench_blocks(n, torch, pd) for n in BLOCK_CASES}}),
              flush=True)
        return

    case = make_workload(args.workload, args.seed)
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float16
    q, k, v, bt, cl = upload(case, torch)
    out = torch.empty_like(q)
    ws = pd.alloc_workspace(q, k, bt, args.splits)
    S, P = pd.paged_decode_plan(case.B, case.Hq, case.Hkv, case.D, case.max_blocks_per_seq,
                                case.block_size, dt, args.splits)

    def call(i):
        attend(pd, case, q, k, v, bt, cl, out, ws, args.splits)

    call(0)
    torch.cuda.synchronize()
    first = out.clone()
    ms = time_calls(call, args.steps, args.warmup, torch)
    torch.cuda.synchronize()
    stable = [bool(torch.equal(first.view(torch.int16), out.view(torch.int16)))]

    def same_bits():
        stable.append(bool(torch.equal(first.view(torch.int16), out.view(torch.int16))))

    # further samples of the same K calls, stream launches and then one graph
    # of K calls replayed, each sample followed by a bit comparison of `out`
    samp = None
    if args.samples > 0:
        samp = {"calls_per_sample": args.steps,
                "stream": sample_stats(time_samples(call, args.steps, args.samples, torch,
                                                    same_bits)),
                "graph": sample_stats(time_graph_samples(call, args.steps, args.samples, torch,
                                                         same_bits))}
    stable = all(stable)
    # correctness: the oracle leg checks the first call's output on the
    # sampled sequences (every later call gave the same bits, `stable`)
    ok, err, timing = None, {}, None
    if not args.no_cpu_baseline:
        bits = first.cpu().view(torch.int16).numpy().view("uint16")
        ok, err, timing = oracle_parity(case, bits, min(args.cpu_seqs, case.B))
        if not ok:
            print(json.dumps({"metric": METRIC, "error": "parity check failed", **err}))
            sys.exit(1)
    nbytes = case.algorithmic_bytes()
    gbps = nbytes / (ms * 1e-3) / 1e9

    traffic = load_traffic(args.workload)
    roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_GBPS, 4),
            "traffic": None if traffic is None else traffic["traffic_bytes_per_launch"],
            "kernel": DECODE_KERNEL,
            "algorithmic_bytes_per_launch": nbytes}

    res = {"metric": METRIC, "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
           "us_per_call": round(ms * 1e3, 3), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": case.dtype, "accumulate": "f32", "data": "synthetic",
           "config": {"workload": case.name, "batch": case.B, "context": int(case.context_lens.max()),
                      "Hq": case.Hq, "Hkv": case.Hkv, "head_dim": case.D,
                      "block_size": case.block_size, "splits": S, "partition_tokens": P,
                      "kv_dtype": "fp8_e4m3fn" if case.fp8 else case.dtype,
                      "algorithmic_bytes": nbytes, "overhead_bytes": overhead_bytes(case, S)},
           "parity": {"ok": ok, "bitwise_stable_over_timed_calls": stable,
                      **{k2: round(v2, 6) for k2, v2 in err.items()}},
           "roofline": roof, "samples": samp, "device": device_info(torch)}
    if not args.no_others:
        res["context"] = {"launch_floor": launch_floor(torch, pd), "d2d_copy_roof": copy_roof(torch)}
        others = {}
        for name in ("splitk_B8_L1024", "splitk_B8_L4096", "splitk_B32_L1024", "splitk_B64_L1024",
                     "splitk_B1_L1024", "ragged", "short_B32_L64_bf16_bs16",
                     "short_B32_L64_f16_bs32", "tiny", "large_fp8", "splitk_B32_L1024_fp8",
                     "splitk_B8_L1024_fp8", "ragged_fp8", "geom_14x2_D64_B32_L1024",
                     "geom_14x2_D64_B64_L4096", "geom_32x1_D128_B8_L4096",
                     "geom_32x1_D128_B64_L4096", "geom_32x1_D64_B64_L4096",
                     "geom_64x8_D128_B16_L4096", "geom_14x2_D64_B64_L4096_fp8"):
            others[name] = bench_other(name, torch, pd, samples=args.samples)
        res["others"] = others
        from workloads import rope as wrope
        table = pd.rope_cos_sin_table(32768, 128, wrope.QWEN_BASE)
        res["rope_kv_write"] = {n: bench_rope(n, torch, pd, table) for n in ROPE_CASES}
        res["kv_block_moves"] = {n: bench_blocks(n, torch, pd) for n in BLOCK_CASES}
    if timing is not None:  # the oracle's timing repeats run after the GPU's
        res["cpu_baseline"] = cpu_baseline(case, timing)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
