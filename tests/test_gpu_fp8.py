"""GPU parity of the FP8 (E4M3FN) KV-cache path against the fp64 oracle.

The FP8 cache is the next boundary the Loom Kernels home page lists ("Next
boundaries": FP8 KV-cache compression). Same workloads as the 16-bit path
with the caches stored as E4M3FN codes and one float32 scale per tensor; the
oracle decodes the codes exactly. Calls go through
paged_decode_attention_fp8 of the C ABI; the gates are those of helpers.py.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import check_case, compare, device_case, out_bits, run_library

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)


def test_tiny_fp8():
    c = workloads.tiny(0, kv_dtype="fp8")
    note(c.describe())
    check_case(c)


@pytest.mark.parametrize("case", list(workloads.short_cases(0, kv_dtype="fp8")),
                         ids=lambda c: c.name)
def test_short_context_sweep_fp8(case):
    note(case.describe())
    check_case(case)


@pytest.mark.parametrize("case", list(workloads.splitk_cases(0, kv_dtype="fp8")),
                         ids=lambda c: c.name)
def test_split_k_sweep_fp8(case):
    note(case.describe())
    check_case(case)


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 16])
def test_split_k_forced_split_counts_fp8(splits):
    c = workloads.splitk(4, 1000 - 3, seed=9, kv_dtype="fp8")
    note(f"{c.describe()} forced S={splits}")
    check_case(c, num_splits=splits, what=f"{c.name} S={splits}")


@pytest.mark.parametrize("splits", [None, 1, 4])
def test_ragged_batch_fp8(splits):
    c = workloads.ragged(0, kv_dtype="fp8")
    note(f"{c.describe()} S={splits}")
    check_case(c, num_splits=splits, what=f"{c.name} S={splits}")


def test_large_fp8_full_size():
    c = workloads.large(0, kv_dtype="fp8")
    note(c.describe())
    check_case(c)


@pytest.mark.parametrize("dtype,bs", [("bf16", 16), ("f16", 32)])
def test_odd_lengths_every_tail_fp8(dtype, bs):
    lens = list(range(1, 50)) + [255, 256, 257, 1023]
    c = workloads.make_case(f"tails_fp8_{dtype}_bs{bs}", len(lens), lens, dtype=dtype,
                            block_size=bs, seed=31, kv_dtype="fp8")
    note(c.describe())
    check_case(c)


def test_fp8_nan_codes_outside_the_valid_tokens_are_never_read():
    lens = [5, 16, 17, 100, 1]
    c = workloads.make_case("poison_fp8", len(lens), lens, dtype="bf16", block_size=16, seed=33,
                            max_blocks_per_seq=10, kv_dtype="fp8")
    clean = out_bits(run_library(c))
    live = set()
    for b, L in enumerate(lens):
        n = -(-L // 16)
        live.update(int(x) for x in c.block_table[b, :n])
        last = c.block_table[b, n - 1]
        c.k_cache[last, L - (n - 1) * 16:] = 0x7F
        c.v_cache[last, L - (n - 1) * 16:] = 0xFF
    dead = [i for i in range(c.num_blocks) if i not in live]
    assert dead
    for i in dead:
        c.k_cache[i] = 0x7F
        c.v_cache[i] = 0xFF
    for b, L in enumerate(lens):   # padding entries point at a NaN block (a valid id)
        c.block_table[b, -(-L // 16):] = dead[0]
    for s in (None, 1, 3):
        got = out_bits(run_library(c, num_splits=s))
        ref, _ = oracle.attention_case(c)
        compare(got, ref, "bf16", what=f"poison fp8 S={s}")
        if s is None:
            assert np.array_equal(got, clean)


def test_fp8_scales_are_applied_once_each():
    # the same codes with the scales doubled: scores change (k_scale), the
    # output doubles on top of that (v_scale); each against the oracle
    c = workloads.splitk(2, 300, seed=35, kv_dtype="fp8")
    dev = device_case(c)
    for ks, vs in ((c.k_scale, c.v_scale), (2 * c.k_scale, c.v_scale), (c.k_scale, 2 * c.v_scale)):
        c.k_scale, c.v_scale = float(np.float32(ks)), float(np.float32(vs))
        got = out_bits(run_library(c, dev=dev))
        ref, _ = oracle.attention_case(c)
        compare(got, ref, "bf16", what=f"scales {ks:.4g},{vs:.4g}")


def test_fp8_repeated_calls_and_graph_replay_are_bitwise_identical():
    import paged_gqa_decode_02_amd as pd
    c = workloads.splitk(8, 1024, seed=37, kv_dtype="fp8")
    q, k, v, bt, cl = device_case(c)
    ws = pd.alloc_workspace(q, k, bt)
    out = torch.empty_like(q)

    def call():
        pd.paged_decode_attention_fp8(q, k, v, bt, cl, out, k_scale=c.k_scale, v_scale=c.v_scale,
                                      scale=c.scale, workspace=ws)

    call()
    torch.cuda.synchronize()
    first = out_bits(out)
    ref, _ = oracle.attention_case(c)
    compare(first, ref, "bf16", what="fp8 first call")
    for _ in range(3):
        call()
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), first)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), first)


def test_fp8_binding_rejects_mismatched_inputs():
    import paged_gqa_decode_02_amd as pd
    c = workloads.tiny(0, kv_dtype="fp8")
    q, k, v, bt, cl = device_case(c)
    with pytest.raises(ValueError):
        pd.paged_decode_attention_fp8(q, k.view(torch.uint8).to(torch.int16), v, bt, cl,
                                      k_scale=1.0, v_scale=1.0)
    with pytest.raises(pd.PagedDecodeError) as e:
        pd.paged_decode_attention_fp8(q, k, v, bt, cl, k_scale=0.0, v_scale=1.0)
    assert e.value.code == 10


@pytest.mark.parametrize("Hq,Hkv,D", [(14, 2, 128), (32, 1, 128), (8, 8, 128), (64, 8, 128),
                                      (20, 1, 128), (14, 2, 64), (32, 8, 64), (32, 1, 64),
                                      (8, 8, 64), (21, 1, 64), (64, 1, 128), (128, 1, 64)])
@pytest.mark.parametrize("splits", [None, 3])
def test_fp8_other_group_sizes(Hq, Hkv, D, splits):
    # odd groups, MQA (two or three virtual KV heads), MHA, G = 8 and 20 at
    # D = 128, and the same kinds at D = 64 (the 14/2 D64 geometry included)
    lens = [1, 37, 700, 1024, 513, 0]
    c = workloads.make_case(f"fp8_{Hq}x{Hkv}_D{D}", len(lens), lens, dtype="bf16",
                            block_size=16, Hq=Hq, Hkv=Hkv, D=D, seed=90 + Hq + D,
                            scale=float(np.float32(1.0 / np.sqrt(D))), kv_dtype="fp8")
    note(f"{c.describe()} S={splits}")
    check_case(c, num_splits=splits, what=f"{c.name} S={splits}")


@pytest.mark.parametrize("dtype,bs", [("bf16", 16), ("f16", 32)])
def test_fp8_d64_every_tail(dtype, bs):
    lens = [1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 300]
    c = workloads.make_case(f"fp8_tails_D64_{dtype}_bs{bs}", len(lens), lens, dtype=dtype,
                            block_size=bs, Hq=14, Hkv=2, D=64, seed=97,
                            scale=float(np.float32(0.125)), kv_dtype="fp8")
    note(c.describe())
    for s in (None, 1, 2, 5):
        check_case(c, num_splits=s, what=f"{c.name} S={s}")


def test_fp8_d64_full_size():
    # the 14/2 D64 geometry at B64 x 4,096 tokens over an FP8 cache, planned,
    # every output against the oracle
    c = workloads.geometry(14, 2, 64, 64, 4096, seed=0, kv_dtype="fp8")
    note(c.describe())
    check_case(c)
