"""Pins of the block-movement oracle (oracle/blocks.py): brute-force loops
and invariants that any correct copy, gather, scatter or compaction keeps."""
import itertools

import numpy as np
import pytest

from oracle import blocks as ob
from workloads import blocks as wb


def small_cache(nb=12, seed=0):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << 16, size=(nb, 2, 1, 4), dtype=np.uint16)


def test_copy_brute_force():
    c = small_cache()
    pairs = np.array([[0, 5], [0, 6], [3, 7], [11, 2]])
    out = ob.copy_blocks(c, pairs)
    for b in range(12):
        want = {5: 0, 6: 0, 7: 3, 2: 11}.get(b, b)
        assert np.array_equal(out[b], c[want])


def test_copy_rejects_unsafe_pairs():
    c = small_cache()
    with pytest.raises(ValueError):
        ob.copy_blocks(c, [[0, 5], [1, 5]])       # destination twice
    with pytest.raises(ValueError):
        ob.copy_blocks(c, [[0, 5], [5, 6]])       # 5 is read and written
    with pytest.raises(ValueError):
        ob.copy_blocks(c, [[0, 12]])              # outside the pool


def test_gather_then_scatter_round_trip():
    c = small_cache(seed=1)
    ids = np.array([9, 0, 4, 7])
    g = ob.gather_blocks(c, ids)
    assert g.shape == (4,) + c.shape[1:]
    for i, b in enumerate(ids):
        assert np.array_equal(g[i], c[b])
    # scatter into a zeroed pool puts each block back where it came from
    z = ob.scatter_blocks(np.zeros_like(c), ids, g)
    for b in range(12):
        assert np.array_equal(z[b], c[b] if b in ids else np.zeros_like(c[b]))
    with pytest.raises(ValueError):
        ob.scatter_blocks(c, [1, 1], g[:2])


def logical(cache, table, n):
    """What a sequence reads: its first n blocks through its table."""
    return np.stack([cache[table[i]] for i in range(n)]) if n else cache[:0]


@pytest.mark.parametrize("seed", range(6))
def test_compaction_keeps_what_every_sequence_reads(seed):
    nb = 40
    live, bt, nper = wb.live_pool(nb, 5, live_frac=0.45, seed=seed)
    c = small_cache(nb, seed)
    pairs, remap, n = ob.compact_plan(live)
    assert n == int(live.sum())
    c2 = ob.copy_blocks(c, pairs) if len(pairs) else c.copy()
    bt2 = ob.remap_block_table(bt, remap)
    used = set()
    for b in range(5):
        k = int(nper[b])
        assert np.array_equal(logical(c2, bt2[b], k), logical(c, bt[b], k))
        assert np.all(bt2[b, :k] < n)                 # live blocks now fill [0, n)
        assert np.all(bt2[b, k:] == -1)               # padding untouched
        used |= set(int(x) for x in bt2[b, :k])
    assert used == set(range(n))                      # a bijection onto [0, n)
    # fewest moves: exactly the live blocks at or above n move
    assert len(pairs) == int(live[n:].sum())
    assert np.all(pairs[:, 0] >= n) and np.all(pairs[:, 1] < n) if len(pairs) else True


def test_compaction_brute_force_minimal():
    # over every live set of 6 blocks: no plan that fills [0, n) moves fewer
    # blocks, and the plan's pairing is order-preserving (k-th mover to k-th hole)
    for bits in itertools.product([0, 1], repeat=6):
        live = np.array(bits, bool)
        pairs, remap, n = ob.compact_plan(live)
        movers = [b for b in range(6) if live[b] and b >= n]
        holes = [b for b in range(n) if not live[b]]
        assert [tuple(p) for p in pairs] == list(zip(movers, holes))
        assert sorted(remap[live]) == list(range(n))
        for b in range(6):
            if b not in movers:
                assert remap[b] == b


def test_workload_generators():
    p = wb.copy_pairs(64, 20, seed=3)
    assert p.shape == (20, 2) and len(set(p[:, 1])) == 20
    assert not set(p[:, 0]) & set(p[:, 1])
    ids = wb.block_ids(64, 30, seed=3)
    assert len(set(ids)) == 30 and ids.min() >= 0 and ids.max() < 64
    live, bt, nper = wb.live_pool(100, 7, seed=2)
    assert int(nper.sum()) == int(live.sum())
    assert sorted(x for x in bt.ravel() if x >= 0) == list(np.flatnonzero(live))
