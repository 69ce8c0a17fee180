"""GPU parity at the limits of the shapes the library takes.

The largest batch the grid allows (65,535 sequences, one workgroup row
each), outputs sampled across the whole batch against the oracle, planned
and split (the split's merge kernel then runs 65,535 x Hq workgroups). And
block ids more than 4 GiB into
the pool: the K/V addresses are 64-bit, so a case whose blocks sit past that
point gives the same bits as the same case in a small pool, for the decode,
the RoPE + KV write and the block moves.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import compare, device_case, out_bits, run_library

pytestmark = pytest.mark.gpu


def max_batch_case(Hq, Hkv, seed):
    B = 65535
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 21, size=B).astype(np.int32)   # 0 .. 2 blocks of 16
    need = int(sum(-(-int(L) // 16) for L in lens))
    return workloads.make_case(f"max_batch_{Hq}x{Hkv}", B, lens, dtype="bf16", block_size=16,
                               Hq=Hq, Hkv=Hkv, D=64, seed=seed, scale=float(np.float32(0.125)),
                               max_blocks_per_seq=2, pool_blocks=max(1, need))


def check_rows(c, got):
    # every 257th sequence, the last one and some empty ones, against the oracle
    lens = c.context_lens
    pick = np.unique(np.concatenate([np.arange(0, c.B, 257), [c.B - 1],
                                     np.nonzero(lens == 0)[0][:8]]))
    ref, _ = oracle.attention(c.q[pick], c.k_cache, c.v_cache, c.block_table[pick],
                              lens[pick], scale=c.scale, dtype=c.dtype)
    compare(got[pick], ref, c.dtype, what=f"{c.name} rows={len(pick)}")


def test_largest_batch_three_kv_heads():
    # the planned call has S = 1; a forced split runs the merge kernel over
    # 65,535 x 12 (sequence, query head) rows
    import paged_gqa_decode_02_amd as pd
    c = max_batch_case(12, 3, seed=41)
    print(c.describe(), flush=True)
    assert pd.paged_decode_plan(c.B, 12, 3, 64, 2, 16, torch.bfloat16)[0] == 1
    check_rows(c, out_bits(run_library(c)))
    check_rows(c, out_bits(run_library(c, num_splits=2)))


def test_largest_batch_split_one_kv_head():
    # 65,535 sequences x one KV head, split in two
    c = max_batch_case(8, 1, seed=43)
    print(c.describe(), flush=True)
    check_rows(c, out_bits(run_library(c, num_splits=2)))


@pytest.mark.parametrize("kv", ["", "fp8"])
def test_block_ids_past_4_gib_of_pool(kv):
    lens = [300, 17, 1024]
    c = workloads.make_case(f"far_blocks{'_' + kv if kv else ''}", len(lens), lens,
                            dtype="bf16", block_size=16, seed=42, kv_dtype=kv)
    print(c.describe(), flush=True)
    small = out_bits(run_library(c))
    q, k, v, bt, cl = device_case(c)
    block_bytes = k[0].numel() * k.element_size()       # 32 KiB (16-bit) or 16 KiB (FP8)
    base = (4 << 30) // block_bytes + 1000               # first far id: past 4 GiB
    nb = base + c.num_blocks
    kb = torch.zeros((nb,) + tuple(k.shape[1:]), dtype=k.dtype, device=k.device)
    vb = torch.zeros_like(kb)
    kb[base:] = k
    vb[base:] = v
    bt_far = bt + base
    import paged_gqa_decode_02_amd as pd
    if c.fp8:
        far = pd.paged_decode_attention_fp8(q, kb, vb, bt_far, cl, k_scale=c.k_scale,
                                            v_scale=c.v_scale, scale=c.scale)
    else:
        far = pd.paged_decode_attention(q, kb, vb, bt_far, cl, scale=c.scale)
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(far), small)
    ref, _ = oracle.attention_case(c)
    compare(small, ref, c.dtype, what=c.name)
    del kb, vb
    torch.cuda.empty_cache()


def far_pool(k, v, base):
    """Copies of (k, v) [NB, ...] at block ids base .. base + NB of a pool of
    zeros that size (the copies start past 4 GiB)."""
    nb = base + k.shape[0]
    kb = torch.zeros((nb,) + tuple(k.shape[1:]), dtype=k.dtype, device=k.device)
    vb = torch.zeros_like(kb)
    kb[base:] = k
    vb[base:] = v
    return kb, vb


def test_rope_write_to_slots_past_4_gib():
    from workloads import rope as wrope
    import paged_gqa_decode_02_amd as pd
    case = wrope.scatter(64, seed=44, pad_every=9)
    dt = workloads.DTYPES[case.dtype]
    qkv = case.torch_qkv().cuda()
    q, k, v = qkv[:, :case.Hq], qkv[:, case.Hq:case.Hq + case.Hkv], qkv[:, case.Hq + case.Hkv:]
    kc, vc = (t.cuda() for t in case.torch_caches())
    block_bytes = kc[0].numel() * 2
    base = (4 << 30) // block_bytes + 100
    kb, vb = far_pool(kc, vc, base)
    pos = torch.from_numpy(case.positions).cuda()
    slots = torch.from_numpy(case.slot_mapping).cuda()
    far_slots = torch.where(slots >= 0, slots + base * case.block_size, slots)
    table = pd.rope_cos_sin_table(case.max_position, case.D, case.base)
    q_small = pd.rope_paged_kv_write(q, k, v, pos, slots, table, kc, vc)
    q_far = pd.rope_paged_kv_write(q, k, v, pos, far_slots, table, kb, vb)
    torch.cuda.synchronize()
    assert torch.equal(q_small.view(torch.int16), q_far.view(torch.int16))
    assert torch.equal(kb[base:].view(torch.int16), kc.view(torch.int16))
    assert torch.equal(vb[base:].view(torch.int16), vc.view(torch.int16))
    assert not bool(kb[:base].view(torch.int16).any())   # nothing written below the copies
    del kb, vb
    torch.cuda.empty_cache()


def test_block_moves_past_4_gib():
    from workloads import blocks as wb
    import paged_gqa_decode_02_amd as pd
    case = wb.pool(96, seed=45)
    kc, vc = (t.cuda() for t in case.torch_caches())
    base = (4 << 30) // case.block_bytes + 100
    kb, vb = far_pool(kc, vc, base)
    pairs = torch.from_numpy(wb.copy_pairs(96, 30, seed=46)).cuda()
    ids = torch.from_numpy(wb.block_ids(96, 40, seed=47)).cuda()
    pd.paged_kv_copy_blocks(kc, vc, pairs)
    pd.paged_kv_copy_blocks(kb, vb, pairs + base)
    g_small = pd.paged_kv_gather_blocks(kc, vc, ids)
    g_far = pd.paged_kv_gather_blocks(kb, vb, ids + base)
    torch.cuda.synchronize()
    for a, b in zip(g_small, g_far):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(kb[base:].view(torch.int16), kc.view(torch.int16))
    assert torch.equal(vb[base:].view(torch.int16), vc.view(torch.int16))
    del kb, vb
    torch.cuda.empty_cache()
