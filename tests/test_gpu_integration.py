"""GPU integration checks of the call boundary: current-stream ordering,
what the call may write, buffer reuse, and HIP-graph capture/replay with the
paging metadata read at replay time (Loom Kernels benchmark page, "Validation
ladder": current-stream, mutation-schema and buffer-reuse tests, then graph
capture/replay)."""
import numpy as np
import pytest
import torch

import oracle
import paged_gqa_decode_02_amd as pd
import workloads
from helpers import compare, device_case, out_bits

pytestmark = pytest.mark.gpu


def test_call_is_ordered_on_a_non_default_stream():
    c = workloads.splitk(4, 512, seed=21)
    q, k, v, bt, cl = device_case(c)
    ref, _ = oracle.attention_case(c)
    s = torch.cuda.Stream()
    q_src = q.clone()
    q.zero_()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        # producer on the same stream, queued right before the call
        torch.cuda._sleep(2_000_000)
        q.copy_(q_src)
        out = pd.paged_decode_attention(q, k, v, bt, cl, scale=c.scale)
    s.synchronize()
    compare(out_bits(out), ref, "bf16", what="stream order")


def test_only_out_is_written_and_canaries_survive():
    c = workloads.splitk(2, 256, seed=22)
    q, k, v, bt, cl = device_case(c)
    before = [t.clone() for t in (q, k, v, bt, cl)]
    n = q.numel()
    buf = torch.full((n + 2 * 4096,), 1234.0, dtype=q.dtype, device="cuda")
    out = buf[4096:4096 + n].view_as(q)
    for s in (None, 1, 4):
        pd.paged_decode_attention(q, k, v, bt, cl, out, scale=c.scale, num_splits=s)
        torch.cuda.synchronize()
        assert torch.all(buf[:4096] == 1234.0) and torch.all(buf[4096 + n:] == 1234.0)
        for a, b in zip(before, (q, k, v, bt, cl)):
            assert torch.equal(a, b)
    ref, _ = oracle.attention_case(c)
    compare(out_bits(out), ref, "bf16", what="canary")


def test_out_and_workspace_reuse_across_shapes():
    out = None
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    pd.paged_decode_workspace_init(ws)
    for B, L in ((8, 1024), (1, 128), (8, 1024), (2, 512)):
        c = workloads.splitk(B, L, seed=23 + B + L)
        q, k, v, bt, cl = device_case(c)
        if out is None or out.shape != q.shape:
            out = torch.empty_like(q)
        pd.paged_decode_attention(q, k, v, bt, cl, out, scale=c.scale, workspace=ws)
        torch.cuda.synchronize()
        ref, _ = oracle.attention_case(c)
        compare(out_bits(out), ref, "bf16", what=f"reuse B{B} L{L}")


def test_graph_replay_reads_context_lens_at_replay_time():
    # one captured call, replayed with different context lengths written
    # between replays (all within max_blocks_per_seq * block_size)
    c = workloads.make_case("graph", 4, [700, 900, 1024, 513], dtype="bf16", block_size=16,
                            seed=24, max_blocks_per_seq=64)
    q, k, v, bt, cl = device_case(c)
    out = torch.empty_like(q)
    ws = pd.alloc_workspace(q, k, bt)
    # warm up on a side stream, as graph capture requires
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pd.paged_decode_attention(q, k, v, bt, cl, out, scale=c.scale, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pd.paged_decode_attention(q, k, v, bt, cl, out, scale=c.scale, workspace=ws)
    rng = np.random.default_rng(5)
    for rep in range(6):
        lens = rng.integers(0 if rep == 3 else 1, 1025, size=4).astype(np.int32)
        cl.copy_(torch.from_numpy(lens))
        g.replay()
        torch.cuda.synchronize()
        got = out_bits(out)
        # eager call on the same metadata must agree bitwise
        eager = out_bits(pd.paged_decode_attention(q, k, v, bt, cl, scale=c.scale,
                                                   workspace=pd.alloc_workspace(q, k, bt)))
        torch.cuda.synchronize()
        assert np.array_equal(got, eager), rep
        c.context_lens[:] = lens
        ref, _ = oracle.attention_case(c)
        compare(got, ref, "bf16", what=f"graph replay {rep}")


def test_wrong_dtype_and_shapes_are_rejected_by_the_binding():
    c = workloads.tiny(0)
    q, k, v, bt, cl = device_case(c)
    with pytest.raises(ValueError):
        pd.paged_decode_attention(q.float(), k, v, bt, cl)
    with pytest.raises(ValueError):
        pd.paged_decode_attention(q, k, v, bt.long(), cl)
    with pytest.raises(pd.PagedDecodeError) as e:
        pd.paged_decode_attention(q, k, v, bt, cl, q)  # out aliases q
    assert e.value.code == 5


@pytest.mark.parametrize("splits", [None, 2, 7, 32])
def test_split_workspace_needs_no_zeroing_and_partials_never_go_stale(splits):
    # a workspace filled with NaN bytes, never zeroed, then back-to-back
    # calls on it with different data and different context lengths (so
    # different partitions are live each time): each must match its own
    # oracle, whatever an earlier call left behind
    cases = [workloads.make_case("stale", 6, lens, dtype="bf16", block_size=16, seed=40 + i,
                                 max_blocks_per_seq=64)
             for i, lens in enumerate([[1024, 1000, 513, 64, 17, 1], [700, 1024, 1, 900, 333, 1024],
                                       [1, 2, 3, 1024, 1023, 512]])]
    S, _ = pd.paged_decode_plan(6, 32, 8, 128, 64, 16, torch.bfloat16, splits)
    assert S > 1
    ws = torch.full((pd.paged_decode_workspace_bytes(6, 32, 8, 128, 64, 16, torch.bfloat16,
                                                     splits) + 4096,), 0xFF, dtype=torch.uint8,
                    device="cuda")
    outs = []
    for c in cases * 2:
        q, k, v, bt, cl = device_case(c)
        outs.append((c, pd.paged_decode_attention(q, k, v, bt, cl, scale=c.scale, workspace=ws,
                                                  num_splits=splits)))
    torch.cuda.synchronize()
    for c, o in outs:
        ref, _ = oracle.attention_case(c)
        compare(out_bits(o), ref, "bf16", what=f"stale S={splits}")


def test_workspace_init_zeroes_the_whole_workspace():
    ws = torch.full((3 << 20,), 0xAB, dtype=torch.uint8, device="cuda")
    pd.paged_decode_workspace_init(ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws).item() == 0


@pytest.mark.parametrize("kv", ["", "fp8"])
def test_decode_step_graph_write_then_attend(kv):
    """A whole decode step captured in one HIP graph: the RoPE + KV write of
    each sequence's new token at position L - 1 (through its block table),
    then paged decode attention over the updated cache with the rotated q.
    Replayed four times with new q/k/v, positions, slots and lengths written
    between replays, each replay bitwise equal to the same two calls made
    eagerly on a second copy of the cache (out and every cache byte)."""
    fp8 = kv == "fp8"
    B, Hq, Hkv, D, bs, MB = 4, 32, 8, 128, 16, 64
    c = workloads.make_case(f"step{'_' + kv if kv else ''}", B, [300, 17, 1000, 64],
                            dtype="bf16", block_size=bs, seed=25, max_blocks_per_seq=MB,
                            kv_dtype=kv)
    ks, vs = (c.k_scale, c.v_scale) if fp8 else (1.0, 1.0)
    q0, k0, v0, bt, cl = device_case(c)
    tab = pd.rope_cos_sin_table(MB * bs, D, 1e6)
    lens = c.context_lens.astype(np.int64).copy()

    def step_inputs(rep):
        g = np.random.default_rng(100 + rep)
        qkv = torch.from_numpy(g.standard_normal((B, Hq + 2 * Hkv, D)).astype(np.float32))
        L = np.minimum(lens + 1, MB * bs)
        pos = (L - 1).astype(np.int32)
        slots = (c.block_table[np.arange(B), pos // bs].astype(np.int64) * bs + pos % bs)
        return qkv.to(torch.bfloat16).cuda(), torch.from_numpy(pos).cuda(), \
            torch.from_numpy(slots.astype(np.int32)).cuda(), torch.from_numpy(L.astype(np.int32)).cuda()

    def run_step(qkv, pos, slots, L, kc, vc, q_out, out, ws):
        q, k, v = qkv[:, :Hq], qkv[:, Hq:Hq + Hkv], qkv[:, Hq + Hkv:]
        if fp8:
            pd.rope_paged_kv_write_fp8(q, k, v, pos, slots, tab, kc, vc, q_out=q_out,
                                       k_scale=ks, v_scale=vs)
            pd.paged_decode_attention_fp8(q_out, kc, vc, bt, L, out, k_scale=ks, v_scale=vs,
                                          scale=c.scale, workspace=ws)
        else:
            pd.rope_paged_kv_write(q, k, v, pos, slots, tab, kc, vc, q_out=q_out)
            pd.paged_decode_attention(q_out, kc, vc, bt, L, out, scale=c.scale, workspace=ws)

    # the graph's state and the eager copy
    kc_g, vc_g = k0.clone(), v0.clone()
    kc_e, vc_e = k0.clone(), v0.clone()
    qkv_g, pos_g, slots_g, L_g = step_inputs(0)
    q_out_g = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    out_g = torch.empty_like(q_out_g)
    ws_g = pd.alloc_workspace(q_out_g, kc_g, bt)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on a side stream, as capture requires
        run_step(qkv_g, pos_g, slots_g, L_g, kc_g.clone(), vc_g.clone(), q_out_g, out_g, ws_g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_step(qkv_g, pos_g, slots_g, L_g, kc_g, vc_g, q_out_g, out_g, ws_g)
    for rep in range(4):
        qkv, pos, slots, L = step_inputs(rep)
        for dst, src in ((qkv_g, qkv), (pos_g, pos), (slots_g, slots), (L_g, L)):
            dst.copy_(src)
        graph.replay()
        q_out_e = torch.empty_like(q_out_g)
        out_e = torch.empty_like(out_g)
        run_step(qkv, pos, slots, L, kc_e, vc_e, q_out_e, out_e, pd.alloc_workspace(q_out_e, kc_e, bt))
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), rep
        assert torch.equal(kc_g.view(torch.uint8), kc_e.view(torch.uint8)), rep
        assert torch.equal(vc_g.view(torch.uint8), vc_e.view(torch.uint8)), rep
        assert bool(torch.isfinite(out_g.float()).all())
        lens = L.cpu().numpy().astype(np.int64)
