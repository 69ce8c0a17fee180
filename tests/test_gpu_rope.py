"""GPU parity of RoPE + paged KV-cache write (rope_paged_kv_write) and of the
cos/sin table (rope_cos_sin_table) against the fp64 oracle (oracle/rope.py).

Gates: the table within one float32 ulp of the oracle's rounded table; the
rotated q_out and cached keys within the decode path's gates (allclose
1e-2 + 1e-2|r| and one ulp of RNE(r)) of the unrounded fp64 rotation; the
cached values bit-exact; every cache slot the call does not name unchanged,
bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle import rope as orope
import paged_gqa_decode_02_amd as pd
import workloads
from workloads import rope as wrope

from helpers import compare, out_bits, run_library

pytestmark = pytest.mark.gpu

_TABLES = {}


def gpu_table(max_position, D, base):
    key = (max_position, D, base)
    if key not in _TABLES:
        _TABLES[key] = pd.rope_cos_sin_table(max_position, D, base)
        torch.cuda.synchronize()
    return _TABLES[key]


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(workloads.DTYPES[dtype]).cuda()


def run_write(case, *, packed=True, in_place=False, table=None):
    """Upload, call, return (q_out bits, k_cache bits, v_cache bits)."""
    qkv = to_dev(case.qkv, case.dtype)
    if packed:
        q, k, v = qkv[:, :case.Hq], qkv[:, case.Hq:case.Hq + case.Hkv], qkv[:, case.Hq + case.Hkv:]
    else:
        q, k, v = (to_dev(a, case.dtype) for a in (case.q, case.k, case.v))
    kc, vc = (to_dev(a, case.dtype) for a in (case.k_cache, case.v_cache))
    pos = torch.from_numpy(case.positions).cuda()
    slots = torch.from_numpy(case.slot_mapping).cuda()
    tab = table if table is not None else gpu_table(case.max_position, case.D, case.base)
    qo = pd.rope_paged_kv_write(q, k, v, pos, slots, tab, kc, vc, q_out=q if in_place else None)
    torch.cuda.synchronize()
    return out_bits(qo), out_bits(kc), out_bits(vc)


def check_write(case, got, table=None):
    qo, kc, vc = got
    tab = table if table is not None else orope.cos_sin_table_f32(case.max_position, case.D, case.base)
    q_rot, k_rot, kc_ref, vc_ref = orope.rope_kv_write(
        case.q, case.k, case.v, case.positions, case.slot_mapping, tab, case.k_cache,
        case.v_cache, dtype=case.dtype)
    rep = compare(qo, q_rot, case.dtype, what=f"{case.name} q_out")
    live = case.slot_mapping >= 0
    slots = case.slot_mapping[live].astype(np.int64)
    flat = kc.reshape(-1, case.Hkv, case.D)
    if live.any():
        compare(flat[slots], k_rot[live], case.dtype, what=f"{case.name} k_cache")
    assert np.array_equal(vc, vc_ref), f"{case.name}: v_cache differs"
    # the rotated keys at the named slots aside, the K cache is what it was
    untouched = np.ones(flat.shape[0], bool)
    untouched[slots] = False
    assert np.array_equal(flat[untouched], case.k_cache.reshape(-1, case.Hkv, case.D)[untouched])
    return rep


def test_table_matches_oracle():
    for max_pos, D, base in ((32768, 128, 1e6), (4096, 64, 10000.0), (2048, 256, 1e6)):
        g = gpu_table(max_pos, D, base).cpu().numpy()
        r = orope.cos_sin_table_f32(max_pos, D, base)
        gi, ri = g.view(np.int32).astype(np.int64), r.view(np.int32).astype(np.int64)
        # same sign everywhere that matters; distance in float32 ulps
        ulp = np.abs(gi - ri)
        zero = (g == 0) & (r == 0)
        ulp[zero] = 0
        assert int(ulp.max()) <= 1, (max_pos, D, base, int(ulp.max()))
        assert (ulp == 0).mean() > 0.999, (max_pos, D, base, float((ulp == 0).mean()))
        assert np.all(g[0, : D // 2] == 1.0) and np.all(g[0, D // 2:] == 0.0)


CASES = [
    # T, Hq, Hkv, D, dtype, bs, pad_every
    (1, 32, 8, 128, "bf16", 16, 0),
    (7, 32, 8, 128, "bf16", 32, 3),
    (64, 32, 8, 128, "f16", 16, 0),
    (300, 32, 8, 128, "bf16", 16, 5),
    (33, 14, 2, 64, "bf16", 16, 4),
    (40, 8, 1, 256, "f16", 32, 0),
    (17, 4, 4, 128, "f16", 16, 2),
]


@pytest.mark.parametrize("T,Hq,Hkv,D,dtype,bs,pad", CASES)
@pytest.mark.parametrize("packed", [True, False])
def test_scatter_write_matches_oracle(T, Hq, Hkv, D, dtype, bs, pad, packed):
    case = wrope.scatter(T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, block_size=bs, pad_every=pad,
                         max_position=32768, seed=T + D)
    print(case.describe(), "packed" if packed else "separate", flush=True)
    check_write(case, run_write(case, packed=packed))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_write_matches_oracle(dtype):
    case = wrope.prefill(2, 512, dtype=dtype, block_size=16, max_position=32768, seed=11)
    print(case.describe(), flush=True)
    check_write(case, run_write(case))


def test_in_place_q():
    case = wrope.scatter(50, dtype="bf16", seed=21)
    print(case.describe(), "in place", flush=True)
    check_write(case, run_write(case, packed=False, in_place=True))


def test_position_zero_leaves_q_and_k_unchanged():
    case = wrope.scatter(16, max_position=1, seed=4)
    assert np.all(case.positions == 0)
    qo, kc, _ = run_write(case)
    assert np.array_equal(qo, case.q)
    flat = kc.reshape(-1, case.Hkv, case.D)
    assert np.array_equal(flat[case.slot_mapping.astype(np.int64)], case.k)


def test_large_prefill_sampled():
    # 16,384 tokens at the decode geometry (the HBM-bound end of the range);
    # the oracle checks every 64th token and the caches' untouched slots
    case = wrope.prefill(4, 4096, dtype="bf16", block_size=16, max_position=32768, seed=5)
    print(case.describe(), flush=True)
    qo, kc, vc = run_write(case)
    sel = np.arange(0, case.T, 64)
    tab = orope.cos_sin_table_f32(case.max_position, case.D, case.base)
    sub = wrope.RopeCase(case.name + "_sample", len(sel), case.Hq, case.Hkv, case.D, case.dtype,
                         case.block_size, case.max_position, case.base, case.qkv[sel],
                         case.positions[sel], case.slot_mapping[sel], case.k_cache,
                         case.v_cache, case.seed)
    q_rot, k_rot, _, _ = orope.rope_kv_write(sub.q, sub.k, sub.v, sub.positions,
                                             sub.slot_mapping, tab, case.k_cache, case.v_cache,
                                             dtype="bf16")
    compare(qo[sel], q_rot, "bf16", what="q_out sample")
    slots = case.slot_mapping.astype(np.int64)
    flat_k = kc.reshape(-1, case.Hkv, case.D)
    flat_v = vc.reshape(-1, case.Hkv, case.D)
    compare(flat_k[slots[sel]], k_rot, "bf16", what="k_cache sample")
    assert np.array_equal(flat_v[slots], case.v)
    untouched = np.ones(flat_k.shape[0], bool)
    untouched[slots] = False
    assert np.array_equal(flat_k[untouched], case.k_cache.reshape(-1, case.Hkv, case.D)[untouched])
    assert np.array_equal(flat_v[untouched], case.v_cache.reshape(-1, case.Hkv, case.D)[untouched])


@pytest.mark.parametrize("bs", [16, 32])
def test_write_then_decode(bs):
    """The write feeds the decode: each sequence's new token goes to position
    L-1 through its block table, then paged decode attention reads it."""
    dec = workloads.make_case("feed", 8, [1, 16, 17, 100, 255, 256, 513, 1000], dtype="bf16",
                              block_size=bs, seed=7)
    case = wrope.decode_step(dec, seed=8)
    print(case.describe(), flush=True)
    qo, kc, vc = run_write(case, packed=True)
    tab = orope.cos_sin_table_f32(case.max_position, case.D, case.base)
    q_rot, _, kc_ref, vc_ref = orope.rope_kv_write(case.q, case.k, case.v, case.positions,
                                                   case.slot_mapping, tab, case.k_cache,
                                                   case.v_cache, dtype="bf16")
    # decode over the GPU-written cache with the GPU-rotated q, against the
    # oracle's decode over the oracle-written cache with its rotated q rounded
    # the same way the kernel rounds it
    q_bits = oracle.round_to_dtype(q_rot, "bf16")
    fed = workloads.Case(dec.name, dec.B, dec.Hq, dec.Hkv, dec.D, bs, "bf16", dec.scale, qo, kc,
                         vc, dec.block_table, dec.context_lens, dec.seed)
    out = run_library(fed)
    ref, _ = oracle.attention(q_bits, kc_ref, vc_ref, dec.block_table, dec.context_lens,
                              scale=dec.scale, dtype="bf16")
    # q_out and the cache may differ from the oracle's rounding by one ulp in
    # a few places, so the decode output is held to the allclose gate only
    g = oracle.widen(out_bits(out), "bf16")
    assert np.all(np.abs(g - ref) <= 1e-2 + 1e-2 * np.abs(ref))


def test_graph_replay_reads_positions_at_replay():
    case = wrope.scatter(32, seed=13)
    qkv = to_dev(case.qkv, "bf16")
    q, k, v = qkv[:, :32], qkv[:, 32:40], qkv[:, 40:]
    kc, vc = (to_dev(a, "bf16") for a in (case.k_cache, case.v_cache))
    pos = torch.from_numpy(case.positions).cuda()
    slots = torch.from_numpy(case.slot_mapping).cuda()
    tab = gpu_table(case.max_position, case.D, case.base)
    qo = torch.empty((32, 32, 128), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        pd.rope_paged_kv_write(q, k, v, pos, slots, tab, kc, vc, q_out=qo)  # warm up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pd.rope_paged_kv_write(q, k, v, pos, slots, tab, kc, vc, q_out=qo)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    for rep in range(3):
        new_pos = rng.integers(0, case.max_position, 32).astype(np.int32)
        pos.copy_(torch.from_numpy(new_pos))
        kc.copy_(to_dev(case.k_cache, "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        c2 = wrope.RopeCase(case.name, 32, 32, 8, 128, "bf16", 16, case.max_position, case.base,
                            case.qkv, new_pos, case.slot_mapping, case.k_cache, case.v_cache, 0)
        check_write(c2, (out_bits(qo), out_bits(kc), out_bits(vc)))


# ---------------------------------------------------------------------------
# the write into an FP8 cache: codes against the exact definition (nearest
# code of the fp64 value, or its neighbour across a midpoint the float32
# evaluation's error bound reaches), and bit for bit against a float32 model


def run_write_fp8(case, kc8, vc8, k_scale, v_scale, *, packed=True, table=None):
    """Upload, call rope_paged_kv_write_fp8 over caches holding the codes
    kc8/vc8 (with the given float32 host table as the cos/sin input, else
    the library's), return (q_out bits, k codes, v codes)."""
    qkv = to_dev(case.qkv, case.dtype)
    if packed:
        q, k, v = qkv[:, :case.Hq], qkv[:, case.Hq:case.Hq + case.Hkv], qkv[:, case.Hq + case.Hkv:]
    else:
        q, k, v = (to_dev(a, case.dtype) for a in (case.q, case.k, case.v))
    kc = torch.from_numpy(np.ascontiguousarray(kc8)).cuda().view(torch.float8_e4m3fn)
    vc = torch.from_numpy(np.ascontiguousarray(vc8)).cuda().view(torch.float8_e4m3fn)
    pos = torch.from_numpy(case.positions).cuda()
    slots = torch.from_numpy(case.slot_mapping).cuda()
    tab = gpu_table(case.max_position, case.D, case.base) if table is None else \
        torch.from_numpy(np.ascontiguousarray(table, np.float32)).cuda()
    qo = pd.rope_paged_kv_write_fp8(q, k, v, pos, slots, tab, kc, vc, k_scale=k_scale,
                                    v_scale=v_scale)
    torch.cuda.synchronize()
    return out_bits(qo), kc.view(torch.uint8).cpu().numpy(), vc.view(torch.uint8).cpu().numpy()


def random_codes(shape, seed):
    # any bytes but the two NaN codes, so untouched slots are checkable
    c = np.random.default_rng(seed).integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)


FP8_CASES = [
    # T, Hq, Hkv, D, dtype, bs, pad, k_scale, v_scale
    (64, 32, 8, 128, "bf16", 16, 0, 0.01, 0.01),
    (33, 32, 8, 128, "f16", 32, 4, 0.0078125, 0.015625),    # power-of-two scales
    (40, 14, 2, 64, "bf16", 16, 7, 0.02, 0.005),
    (16, 8, 4, 256, "f16", 16, 0, 0.03, 0.04),
    (128, 32, 8, 128, "bf16", 16, 9, 0.002, 0.003),          # many codes held at 448
]


def check_fp8_write(case, kc8, vc8, got_k, got_v, ks, vs, tab, what):
    """The FP8 write against its plain definition (oracle/rope.py
    rope_kv_write_fp8): at every written slot each code is the nearest
    E4M3FN code of the exact (fp64) key or value over its scale, or its
    neighbour across a midpoint within the float32 error bound of that exact
    value; every other byte unchanged. Returns the count of neighbour codes."""
    r = orope.rope_kv_write_fp8(case.q, case.k, case.v, case.positions, case.slot_mapping, tab,
                                kc8, vc8, dtype=case.dtype, k_scale=ks, v_scale=vs)
    s = r["slots"]
    H, D = case.Hkv, case.D
    written = np.zeros(got_k.reshape(-1, H, D).shape[0], bool)
    written[s] = True
    gk, gv = got_k.reshape(-1, H, D), got_v.reshape(-1, H, D)
    for name, g, c0 in (("K", gk, kc8), ("V", gv, vc8)):
        assert np.array_equal(g[~written], c0.reshape(-1, H, D)[~written]), \
            f"{what}: {name} bytes outside the written slots changed"
    ok_k, n_k = orope.fp8_codes_within_rounding(gk[s], r["k_exact"], r["k_eps"])
    ok_v, n_v = orope.fp8_codes_within_rounding(gv[s], r["v_exact"], r["v_eps"])
    for name, ok, ex, g in (("K", ok_k, r["k_exact"], gk[s]), ("V", ok_v, r["v_exact"], gv[s])):
        if not ok.all():
            i = np.unravel_index(np.argmin(ok), ok.shape)
            raise AssertionError(f"{what}: {name} code 0x{int(g[i]):02x} at {i} for exact "
                                 f"value {ex[i]!r} (nearest 0x{int(orope.fp8_encode_exact(ex[i])):02x})")
    print(f"{what}: {ok_k.size + ok_v.size} codes, {n_k} K and {n_v} V neighbour codes "
          f"across a midpoint", flush=True)
    return r, n_k + n_v


@pytest.mark.parametrize("T,Hq,Hkv,D,dtype,bs,pad,ks,vs", FP8_CASES)
@pytest.mark.parametrize("packed", [True, False])
def test_fp8_write_codes_against_the_exact_definition(T, Hq, Hkv, D, dtype, bs, pad, ks, vs,
                                                      packed):
    case = wrope.scatter(T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, block_size=bs, pad_every=pad,
                         max_position=32768, seed=T + D + 1)
    print(case.describe(), f"fp8 ks={ks} vs={vs}", "packed" if packed else "separate", flush=True)
    kc8 = random_codes(case.k_cache.shape, T)
    vc8 = random_codes(case.v_cache.shape, T + 1)
    tab = orope.cos_sin_table_f32(case.max_position, case.D, case.base)
    qo, kc, vc = run_write_fp8(case, kc8, vc8, ks, vs, packed=packed, table=tab)
    r, _ = check_fp8_write(case, kc8, vc8, kc, vc, ks, vs, tab, case.name)
    compare(qo, r["q_rot"], dtype, what=f"{case.name} q_out")
    if ks == 0.002:  # the case meant to hit the saturation
        assert np.count_nonzero((kc & 0x7F) == 0x7E) > 0


@pytest.mark.parametrize("T,Hq,Hkv,D,dtype,bs,pad,ks,vs", FP8_CASES)
def test_fp8_write_codes_match_the_float32_model_bit_for_bit(T, Hq, Hkv, D, dtype, bs, pad, ks,
                                                             vs):
    """Regression check: the kernel's codes equal, bit for bit, those of a
    float32 model of its evaluation order (oracle/rope.py
    rope_kv_write_fp8_f32_model), which the exact-definition test above
    bounds; a change in the kernel's arithmetic shows here first."""
    case = wrope.scatter(T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, block_size=bs, pad_every=pad,
                         max_position=32768, seed=T + D + 1)
    print(case.describe(), f"fp8 ks={ks} vs={vs} float32 model", flush=True)
    kc8 = random_codes(case.k_cache.shape, T)
    vc8 = random_codes(case.v_cache.shape, T + 1)
    tab = orope.cos_sin_table_f32(case.max_position, case.D, case.base)
    _, kc, vc = run_write_fp8(case, kc8, vc8, ks, vs, table=tab)
    _, kc_ref, vc_ref = orope.rope_kv_write_fp8_f32_model(
        case.q, case.k, case.v, case.positions, case.slot_mapping, tab, kc8, vc8, dtype=dtype,
        k_scale=ks, v_scale=vs)
    assert np.array_equal(kc, kc_ref), f"{case.name}: K codes differ at {np.argwhere(kc != kc_ref)[:4]}"
    assert np.array_equal(vc, vc_ref), f"{case.name}: V codes differ"


@pytest.mark.parametrize("bs", [16, 32])
def test_fp8_write_then_fp8_decode(bs):
    """The FP8 write feeds the FP8 decode: each sequence's new token goes to
    position L-1 through its block table, then paged decode attention reads
    the codes."""
    dec = workloads.make_case("feed8", 8, [1, 16, 17, 100, 255, 256, 513, 1000], dtype="bf16",
                              block_size=bs, seed=9, kv_dtype="fp8")
    case = wrope.decode_step(dec, seed=10)
    print(case.describe(), "fp8", flush=True)
    tab = orope.cos_sin_table_f32(case.max_position, case.D, case.base)
    qo, kc, vc = run_write_fp8(case, dec.k_cache, dec.v_cache, dec.k_scale, dec.v_scale,
                               table=tab)
    r, _ = check_fp8_write(case, dec.k_cache, dec.v_cache, kc, vc, dec.k_scale, dec.v_scale, tab,
                           "feed8")
    compare(qo, r["q_rot"], "bf16", what="feed8 q_out")
    # decode over the GPU-written codes with the GPU-rotated q, against the
    # oracle over the same bytes
    import dataclasses
    fed = dataclasses.replace(dec, q=qo, k_cache=kc, v_cache=vc)
    for s in (None, 1, 3):
        out = run_library(fed, num_splits=s)
        ref, _ = oracle.attention_fp8(qo, kc, vc, dec.block_table, dec.context_lens,
                                      scale=dec.scale, dtype="bf16", k_scale=dec.k_scale,
                                      v_scale=dec.v_scale)
        compare(out_bits(out), ref, "bf16", what=f"feed8 decode S={s}")


def test_positions_and_slots_outside_their_arrays_are_skipped():
    # the kernel's own bounds checks: a token whose position is outside the
    # table writes nothing (its q_out row keeps what it held, no K/V); one
    # whose slot is past the pool writes its rotated q but no K/V, as a
    # padding token does. Everything else matches the oracle run on the
    # tokens with valid positions, the bad slots taken as padding.
    case = wrope.scatter(40, max_position=4096, seed=77)
    print(case.describe(), "positions/slots out of range", flush=True)
    T = case.T
    nslots = case.k_cache.shape[0] * case.block_size
    bad_pos, bad_slot = np.array([3, 17, 30]), np.array([5, 22])
    pos, slots = case.positions.copy(), case.slot_mapping.copy()
    pos[bad_pos] = [case.max_position, -1, 2**31 - 1]
    slots[bad_slot] = [nslots, 2**31 - 1]
    qkv = to_dev(case.qkv, case.dtype)
    q, k, v = qkv[:, :case.Hq], qkv[:, case.Hq:case.Hq + case.Hkv], qkv[:, case.Hq + case.Hkv:]
    kc, vc = (to_dev(a, case.dtype) for a in (case.k_cache, case.v_cache))
    sentinel = np.full((T, case.Hq, case.D), 0x1234, np.uint16)
    qo = to_dev(sentinel, case.dtype)
    pd.rope_paged_kv_write(q, k, v, torch.from_numpy(pos).cuda(), torch.from_numpy(slots).cuda(),
                           gpu_table(case.max_position, case.D, case.base), kc, vc, q_out=qo)
    torch.cuda.synchronize()
    got_q, got_k, got_v = out_bits(qo), out_bits(kc), out_bits(vc)
    assert np.all(got_q[bad_pos] == 0x1234)
    keep = np.setdiff1d(np.arange(T), bad_pos)
    s2 = case.slot_mapping.copy()
    s2[bad_slot] = -1
    sub = dataclasses.replace(case, T=len(keep), qkv=case.qkv[keep], positions=case.positions[keep],
                              slot_mapping=s2[keep])
    check_write(sub, (got_q[keep], got_k, got_v))
