"""GPU parity of KV-cache block movement (paged_kv_copy_blocks, _gather_,
_scatter_, _compact_plan + _remap_block_table) against the oracle
(oracle/blocks.py): every byte of every cache and buffer bit-exact, and a
paged decode over a compacted cache bitwise equal to the one before."""
import numpy as np
import pytest
import torch

from oracle import blocks as ob
import paged_gqa_decode_02_amd as pd
import workloads
from workloads import blocks as wb

from helpers import out_bits

pytestmark = pytest.mark.gpu

GEOMS = [
    # num_blocks, block_size, Hkv, D, dtype: 32 KiB, 64 KiB, 4 KiB (one
    # 4 KiB chunk), 12 KiB and 48 KiB (3 and 12 chunks), 2 KiB (half a chunk)
    # and 6 KiB (a chunk and a half) blocks
    (512, 16, 8, 128, "bf16"),
    (256, 32, 8, 128, "f16"),
    (300, 16, 2, 64, "bf16"),
    (200, 16, 3, 128, "bf16"),
    (128, 16, 12, 128, "f16"),
    (256, 16, 1, 64, "bf16"),
    (96, 16, 3, 64, "f16"),
]


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(workloads.DTYPES[dtype]).cuda()


def host(t):
    return out_bits(t)


@pytest.mark.parametrize("nb,bs,hkv,d,dt", GEOMS)
@pytest.mark.parametrize("both", [True, False])
def test_copy_blocks(nb, bs, hkv, d, dt, both):
    case = wb.pool(nb, block_size=bs, Hkv=hkv, D=d, dtype=dt, seed=nb)
    pairs = wb.copy_pairs(nb, nb // 3, seed=bs)
    print(case.name, bs, hkv, d, dt, "pairs", len(pairs), "v" if both else "k only", flush=True)
    kc, vc = dev(case.k_cache, dt), dev(case.v_cache, dt)
    pd.paged_kv_copy_blocks(kc, vc if both else None, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(host(kc), ob.copy_blocks(case.k_cache, pairs))
    want_v = ob.copy_blocks(case.v_cache, pairs) if both else case.v_cache
    assert np.array_equal(host(vc), want_v)


def test_copy_fp8_cache_as_bytes():
    rng = np.random.default_rng(0)
    k = rng.integers(0, 256, size=(64, 16, 8, 128), dtype=np.uint8)
    v = rng.integers(0, 256, size=(64, 16, 8, 128), dtype=np.uint8)
    pairs = wb.copy_pairs(64, 20, seed=1)
    kc = torch.from_numpy(k).cuda().view(torch.float8_e4m3fn)
    vc = torch.from_numpy(v).cuda().view(torch.float8_e4m3fn)
    pd.paged_kv_copy_blocks(kc, vc, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(kc.view(torch.uint8).cpu().numpy(), ob.copy_blocks(k, pairs))
    assert np.array_equal(vc.view(torch.uint8).cpu().numpy(), ob.copy_blocks(v, pairs))


@pytest.mark.parametrize("nb,bs,hkv,d,dt", GEOMS)
def test_gather_scatter(nb, bs, hkv, d, dt):
    case = wb.pool(nb, block_size=bs, Hkv=hkv, D=d, dtype=dt, seed=nb + 1)
    ids = wb.block_ids(nb, nb // 2, seed=3)
    print(case.name, bs, hkv, d, dt, "ids", len(ids), flush=True)
    kc, vc = dev(case.k_cache, dt), dev(case.v_cache, dt)
    ids_d = torch.from_numpy(ids).cuda()
    ko, vo = pd.paged_kv_gather_blocks(kc, vc, ids_d)
    torch.cuda.synchronize()
    assert np.array_equal(host(ko), ob.gather_blocks(case.k_cache, ids))
    assert np.array_equal(host(vo), ob.gather_blocks(case.v_cache, ids))
    # scatter fresh blocks into the pool at the same ids
    other = wb.pool(len(ids), block_size=bs, Hkv=hkv, D=d, dtype=dt, seed=99)
    pd.paged_kv_scatter_blocks(dev(other.k_cache, dt), dev(other.v_cache, dt), ids_d, kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(host(kc), ob.scatter_blocks(case.k_cache, ids, other.k_cache))
    assert np.array_equal(host(vc), ob.scatter_blocks(case.v_cache, ids, other.v_cache))
    # gather K only
    ko2, vo2 = pd.paged_kv_gather_blocks(kc, None, ids_d)
    torch.cuda.synchronize()
    assert vo2 is None and np.array_equal(host(ko2), other.k_cache)


@pytest.mark.parametrize("seed,frac", [(0, 0.5), (1, 0.2), (2, 0.9), (3, 1.0), (4, 0.0)])
def test_compact_keeps_every_decode_bitwise(seed, frac):
    """Decode over the pool, compact it (plan, copy, remap), decode again:
    every output bit is the same, the caches match the oracle's compaction
    and the live blocks fill [0, n_live)."""
    nb, B = 1024, 8
    case = wb.pool(nb, seed=seed)
    live, bt, nper = wb.live_pool(nb, B, live_frac=frac, seed=seed)
    print(case.name, "live", int(live.sum()), "seqs", B, flush=True)
    ctx = np.minimum(nper.astype(np.int64) * 16, nper.astype(np.int64) * 16 - 3).clip(min=0)
    bt_dec = np.where(bt < 0, 0, bt).astype(np.int32)   # padding entries are never read
    q = workloads.normal_bits((B, 32, 128), "bf16", seed + 50)
    before = workloads.Case("c", B, 32, 8, 128, 16, "bf16", workloads.SCALE_D128, q,
                            case.k_cache, case.v_cache, bt_dec, ctx.astype(np.int32), seed)
    kc, vc = dev(case.k_cache, "bf16"), dev(case.v_cache, "bf16")
    bt_d = torch.from_numpy(bt_dec).cuda()
    cl_d = torch.from_numpy(before.context_lens).cuda()
    q_d = dev(q, "bf16")
    out0 = pd.paged_decode_attention(q_d, kc, vc, bt_d, cl_d, scale=before.scale)
    torch.cuda.synchronize()
    n, moved, _ = pd.paged_kv_compact(kc, vc, live, [bt_d])
    torch.cuda.synchronize()
    pairs, remap, n2 = ob.compact_plan(live.astype(bool))
    assert n == n2 and moved == len(pairs)
    want_k = ob.copy_blocks(case.k_cache, pairs) if len(pairs) else case.k_cache
    want_v = ob.copy_blocks(case.v_cache, pairs) if len(pairs) else case.v_cache
    assert np.array_equal(host(kc), want_k) and np.array_equal(host(vc), want_v)
    bt2 = bt_d.cpu().numpy()
    assert np.array_equal(bt2, ob.remap_block_table(bt_dec, remap))
    for b in range(B):
        assert np.all(bt2[b, :nper[b]] < n)
    out1 = pd.paged_decode_attention(q_d, kc, vc, bt_d, cl_d, scale=before.scale)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))


def test_remap_leaves_padding():
    remap = torch.tensor([5, 4, 3, 2, 1, 0], dtype=torch.int32).cuda()
    bt = torch.tensor([[0, 1, -1, 7], [5, 6, 2, -3]], dtype=torch.int32).cuda()
    pd.paged_kv_remap_block_table(bt, remap)
    torch.cuda.synchronize()
    assert bt.cpu().tolist() == [[5, 4, -1, 7], [0, 6, 3, -3]]


def test_copy_in_graph_reads_pairs_at_replay():
    case = wb.pool(256, seed=5)
    kc, vc = dev(case.k_cache, "bf16"), dev(case.v_cache, "bf16")
    pairs_d = torch.from_numpy(wb.copy_pairs(256, 40, seed=0)).cuda()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        pd.paged_kv_copy_blocks(kc, vc, pairs_d)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pd.paged_kv_copy_blocks(kc, vc, pairs_d)
    torch.cuda.synchronize()
    for rep in range(3):
        pairs = wb.copy_pairs(256, 40, seed=rep + 1)
        pairs_d.copy_(torch.from_numpy(pairs))
        kc.copy_(dev(case.k_cache, "bf16"))
        vc.copy_(dev(case.v_cache, "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(kc), ob.copy_blocks(case.k_cache, pairs))
        assert np.array_equal(host(vc), ob.copy_blocks(case.v_cache, pairs))
