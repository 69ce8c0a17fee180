"""The Python binding refuses host tensors before anything reaches the
library: its entry points take device pointers only, and a host pointer in a
kernel argument would fault the GPU. Runs on the CPU (no GPU is needed to
see the refusal, which happens before any HIP call)."""
import pytest
import torch

import paged_gqa_decode_02_amd as pd

BF16 = torch.bfloat16


def decode_args(B=2, Hq=32, Hkv=8, D=128, bs=16, MB=4, cache_dtype=BF16):
    q = torch.zeros(B, Hq, D, dtype=BF16)
    k = torch.zeros(B * MB, bs, Hkv, D, dtype=cache_dtype)
    v = torch.zeros_like(k)
    bt = torch.arange(B * MB, dtype=torch.int32).reshape(B, MB)
    cl = torch.full((B,), 17, dtype=torch.int32)
    return q, k, v, bt, cl


def test_decode_refuses_host_tensors():
    with pytest.raises(ValueError, match="GPU"):
        pd.paged_decode_attention(*decode_args())
    with pytest.raises(ValueError, match="GPU"):
        pd.paged_decode_attention(*decode_args(), num_splits=2)


def test_fp8_decode_refuses_host_tensors():
    with pytest.raises(ValueError, match="GPU"):
        pd.paged_decode_attention_fp8(*decode_args(cache_dtype=torch.uint8), k_scale=1.0,
                                      v_scale=1.0)


def test_workspace_init_refuses_a_host_buffer():
    with pytest.raises(ValueError, match="GPU"):
        pd.paged_decode_workspace_init(torch.zeros(1024, dtype=torch.uint8))
    q, k, _, bt, _ = decode_args()
    with pytest.raises(ValueError, match="GPU"):
        pd.alloc_workspace(q, k, bt, num_splits=2)


def rope_args(T=3, Hq=4, Hkv=2, D=64, NB=4, bs=16, cache_dtype=BF16):
    q = torch.zeros(T, Hq, D, dtype=BF16)
    k = torch.zeros(T, Hkv, D, dtype=BF16)
    v = torch.zeros_like(k)
    pos = torch.arange(T, dtype=torch.int32)
    slots = torch.arange(T, dtype=torch.int32)
    cs = torch.zeros(16, D, dtype=torch.float32)
    kc = torch.zeros(NB, bs, Hkv, D, dtype=cache_dtype)
    return q, k, v, pos, slots, cs, kc, torch.zeros_like(kc)


def test_rope_write_refuses_host_tensors():
    with pytest.raises(ValueError, match="GPU"):
        pd.rope_paged_kv_write(*rope_args())
    with pytest.raises(ValueError, match="GPU"):
        pd.rope_paged_kv_write_fp8(*rope_args(cache_dtype=torch.uint8), k_scale=1.0, v_scale=1.0)
    with pytest.raises(ValueError, match="GPU"):
        pd.rope_cos_sin_table(16, 64, 10000.0, device="cpu")


def test_block_moves_refuse_host_tensors():
    kc = torch.zeros(8, 16, 2, 64, dtype=BF16)
    vc = torch.zeros_like(kc)
    ids = torch.tensor([1, 3], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        pd.paged_kv_copy_blocks(kc, vc, torch.tensor([[0, 1]], dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        pd.paged_kv_gather_blocks(kc, vc, ids)
    with pytest.raises(ValueError, match="GPU"):
        pd.paged_kv_scatter_blocks(kc[:2].clone(), vc[:2].clone(), ids, kc, vc)
    with pytest.raises(ValueError, match="GPU"):
        pd.paged_kv_remap_block_table(torch.zeros(4, dtype=torch.int32),
                                      torch.arange(8, dtype=torch.int32))


def test_the_compiled_binding_is_the_in_tree_one():
    # the per-step calls go through _lib/_pd_binding*.so, built in-tree and
    # linked to the library the package loaded
    import os
    lib_dir = os.path.dirname(pd.LIB_PATH)
    assert os.path.dirname(os.path.abspath(pd._b.__file__)) == lib_dir
    for name in ("decode", "rope", "workspace_init", "alloc_workspace_bytes"):
        assert callable(getattr(pd._b, name))
    with open("/proc/self/maps") as f:
        maps = f.read()
    assert maps.count(os.path.realpath(pd.LIB_PATH)) >= 1
    assert "libpaged_decode.so" not in maps.replace(os.path.realpath(pd.LIB_PATH), "")
