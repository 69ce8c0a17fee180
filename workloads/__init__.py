"""Seeded synthetic inputs for single-token paged GQA decode attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic. Both the fp64 CPU oracle (``oracle/``) and the HIP
library (``paged_gqa_decode_02_amd``) consume what it produces, and it imports
neither of them.

Workloads follow the sweeps of the Loom Kernels benchmark page ("Reproduce":
the paged-decode backend sweep over batches 1/8/32, contexts 16/32/64, f16 and
bf16, block sizes 16/32; and the split-K sweep over batches 1/2/4/8, contexts
128..1,024, bf16) and the Loom Kernels home page ("Supported now": paged
MQA/GQA decode with GQA packing and split-K/LSE), at Hq/Hkv = 32/8 and head
dim 128. The pages give no random-number recipe, so this module fixes one:

* Values are float32 draws from torch's default CPU generator (mt19937)
  seeded from ``seed``, multiplied by ``sigma`` and rounded
  to the 16-bit dtype with round-to-nearest-even (torch's CPU cast). The
  arrays handed out are the raw 16-bit patterns (``numpy.uint16``).
* Block tables come from a second generator seeded with ``seed + 1``:
  a random permutation of the physical pool dealt out row by row, so no
  physical block is shared between sequences.
* Ragged context lengths come from a third generator seeded with
  ``seed + 2``, uniform over the stated integer range.
* An FP8 cache (``kv_dtype="fp8"``, the OCP E4M3FN format) draws K and V the
  same way in float32, takes one float32 scale per tensor, amax / 448 (the
  largest finite code), and stores round-to-nearest-even(x / scale) as byte
  codes (torch's CPU cast); the value a code stands for is code * scale.

Layouts (row-major, contiguous):
  q, out       [B, Hq, D]
  k/v cache    [num_blocks, block_size, Hkv, D]
  block_table  int32 [B, max_blocks_per_seq]
  context_lens int32 [B]
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterator

import numpy as np
import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}
DTYPE_CODE = {"f16": 0, "bf16": 1}
FP8_MAX = 448.0  # largest finite E4M3FN value

# 1/sqrt(128) rounded to float32, the scale every workload uses.
SCALE_D128 = float(np.float32(1.0 / math.sqrt(128.0)))


@dataclasses.dataclass
class Case:
    """One generated decode call: raw 16-bit inputs plus paging metadata."""

    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    dtype: str
    scale: float
    q: np.ndarray            # uint16 [B, Hq, D]
    k_cache: np.ndarray      # uint16 (uint8 codes for an FP8 cache) [NB, bs, Hkv, D]
    v_cache: np.ndarray      # uint16 (uint8 codes for an FP8 cache) [NB, bs, Hkv, D]
    block_table: np.ndarray  # int32 [B, MB]
    context_lens: np.ndarray # int32 [B]
    seed: int
    q_sigma: float = 1.0
    kv_dtype: str = ""       # "" = the dtype of q; "fp8" = E4M3FN codes with scales
    k_scale: float = 1.0     # float32 scale of the FP8 K codes
    v_scale: float = 1.0     # float32 scale of the FP8 V codes

    @property
    def fp8(self) -> bool:
        return self.kv_dtype == "fp8"

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def dtype_code(self) -> int:
        return DTYPE_CODE[self.dtype]

    def algorithmic_bytes(self) -> int:
        """K+V over valid tokens, plus Q and O, in bytes."""
        es = 1 if self.fp8 else 2
        kv = 2 * self.Hkv * self.D * es * int(self.context_lens.astype(np.int64).sum())
        qo = 2 * self.B * self.Hq * self.D * 2
        return kv + qo

    def live_blocks(self) -> list[np.ndarray]:
        """Physical block ids each sequence actually reads, in logical order."""
        out = []
        for b in range(self.B):
            n = -(-int(self.context_lens[b]) // self.block_size)
            out.append(self.block_table[b, :n].copy())
        return out

    def torch_views(self):
        """(q, k_cache, v_cache) as CPU torch tensors: q in the 16-bit dtype, the
        caches in it too, or as float8_e4m3fn for an FP8 cache."""
        dt = DTYPES[self.dtype]
        q = torch.from_numpy(self.q.view(np.int16)).view(dt)
        if self.fp8:
            return (q,) + tuple(torch.from_numpy(a).view(torch.float8_e4m3fn)
                                for a in (self.k_cache, self.v_cache))
        return (q,) + tuple(torch.from_numpy(a.view(np.int16)).view(dt)
                            for a in (self.k_cache, self.v_cache))

    def describe(self) -> str:
        L = self.context_lens
        kv = f" kv=fp8(k_scale={self.k_scale:.6g},v_scale={self.v_scale:.6g})" if self.fp8 else ""
        return (f"{self.name}: B={self.B} Hq={self.Hq} Hkv={self.Hkv} D={self.D} "
                f"bs={self.block_size} {self.dtype}{kv} ctx[min={int(L.min())},max={int(L.max())}] "
                f"pool={self.num_blocks} MB={self.max_blocks_per_seq} seed={self.seed}")


def normal_bits(shape, dtype: str, seed: int, sigma: float = 1.0,
                chunk: int = 1 << 26) -> np.ndarray:
    """N(0, sigma^2) float32 draws rounded to ``dtype``, as uint16 bit patterns.

    Draws are made in chunks of ``chunk`` elements from one generator, so the
    result depends only on (shape, dtype, seed, sigma).
    """
    n = int(np.prod(shape))
    g = torch.Generator().manual_seed(int(seed))
    out = torch.empty(n, dtype=DTYPES[dtype])
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = torch.randn(e - s, generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        out[s:e] = x.to(DTYPES[dtype])
    return out.view(torch.int16).numpy().view(np.uint16).reshape(shape)


def normal_fp8(shape, seed: int, sigma: float = 1.0, chunk: int = 1 << 26):
    """N(0, sigma^2) float32 draws (the same stream as ``normal_bits``) stored
    as E4M3FN codes with one float32 scale, amax / 448: returns (uint8 codes,
    scale). Two passes over the stream, so no float32 copy is kept."""
    n = int(np.prod(shape))

    def draws():
        g = torch.Generator().manual_seed(int(seed))
        for s in range(0, n, chunk):
            x = torch.randn(min(n, s + chunk) - s, generator=g, dtype=torch.float32)
            if sigma != 1.0:
                x.mul_(sigma)
            yield s, x

    amax = 0.0
    for _, x in draws():
        amax = max(amax, float(x.abs().max()))
    scale = float(np.float32(amax / FP8_MAX)) if amax > 0 else 1.0
    out = torch.empty(n, dtype=torch.uint8)
    for s, x in draws():
        out[s:s + x.numel()] = (x / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    return out.numpy().reshape(shape), scale


def _perm(n: int, seed: int) -> np.ndarray:
    g = torch.Generator().manual_seed(int(seed))
    return torch.randperm(n, generator=g).numpy().astype(np.int32)


def make_case(name: str, B: int, ctx, *, dtype: str = "bf16", block_size: int = 16,
              Hq: int = 32, Hkv: int = 8, D: int = 128, seed: int = 0,
              pool_blocks: int | None = None, max_blocks_per_seq: int | None = None,
              q_sigma: float = 1.0, kv_sigma: float = 1.0,
              scale: float = SCALE_D128, kv_dtype: str = "") -> Case:
    """Build a case with per-sequence contexts ``ctx`` (int or sequence of ints).

    The physical pool defaults to twice the blocks the batch needs; block ids
    are a random permutation of the pool dealt out row by row (no reuse).
    Block-table entries past a sequence's last live block hold further
    (valid, unused) ids from the same permutation when the pool has them,
    else 0.
    """
    lens = np.full(B, ctx, dtype=np.int32) if np.isscalar(ctx) else np.asarray(ctx, dtype=np.int32)
    assert lens.shape == (B,)
    need = [-(-int(L) // block_size) for L in lens]
    MB = max_blocks_per_seq if max_blocks_per_seq is not None else max(1, max(need))
    assert MB >= max(need)
    total_need = sum(need)
    pool = pool_blocks if pool_blocks is not None else max(1, 2 * total_need)
    assert pool >= total_need
    perm = _perm(pool, seed + 1)
    bt = np.zeros((B, MB), dtype=np.int32)
    # live entries first, dealt out without overlap
    pos = 0
    for b in range(B):
        bt[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    # padding entries: remaining ids of the permutation, cycling; never read
    spare = perm[pos:] if pos < pool else perm[:1]
    j = 0
    for b in range(B):
        for i in range(need[b], MB):
            bt[b, i] = spare[j % len(spare)]
            j += 1
    q = normal_bits((B, Hq, D), dtype, seed * 7919 + 11, q_sigma)
    kshape = (pool, block_size, Hkv, D)
    if kv_dtype == "fp8":
        k, ks = normal_fp8(kshape, seed * 7919 + 12, kv_sigma)
        v, vs = normal_fp8(kshape, seed * 7919 + 13, kv_sigma)
        return Case(name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size,
                    dtype=dtype, scale=scale, q=q, k_cache=k, v_cache=v,
                    block_table=bt, context_lens=lens, seed=seed, q_sigma=q_sigma,
                    kv_dtype="fp8", k_scale=ks, v_scale=vs)
    assert kv_dtype in ("", dtype), kv_dtype
    k = normal_bits(kshape, dtype, seed * 7919 + 12, kv_sigma)
    v = normal_bits(kshape, dtype, seed * 7919 + 13, kv_sigma)
    return Case(name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size,
                dtype=dtype, scale=scale, q=q, k_cache=k, v_cache=v,
                block_table=bt, context_lens=lens, seed=seed, q_sigma=q_sigma)


# ---------------------------------------------------------------------------
# The five workloads.

def _suffix(kv_dtype: str) -> str:
    return "_fp8" if kv_dtype == "fp8" else ""


def tiny(seed: int = 0, kv_dtype: str = "") -> Case:
    """Batch 1, context 16 (one block of 16), bf16; pool of 4 blocks whose
    block-table row is a random permutation of {0..3}, only entry 0 live."""
    B, bs, pool = 1, 16, 4
    perm = _perm(pool, seed + 1)
    q = normal_bits((B, 32, 128), "bf16", seed * 7919 + 11)
    kw = {}
    if kv_dtype == "fp8":
        k, ks = normal_fp8((pool, bs, 8, 128), seed * 7919 + 12)
        v, vs = normal_fp8((pool, bs, 8, 128), seed * 7919 + 13)
        kw = dict(kv_dtype="fp8", k_scale=ks, v_scale=vs)
    else:
        k = normal_bits((pool, bs, 8, 128), "bf16", seed * 7919 + 12)
        v = normal_bits((pool, bs, 8, 128), "bf16", seed * 7919 + 13)
    return Case(name="tiny" + _suffix(kv_dtype), B=B, Hq=32, Hkv=8, D=128, block_size=bs,
                dtype="bf16", scale=SCALE_D128, q=q, k_cache=k, v_cache=v,
                block_table=perm.reshape(1, pool).copy(),
                context_lens=np.array([16], dtype=np.int32), seed=seed, **kw)


SHORT_BATCHES = (1, 8, 32)
SHORT_CONTEXTS = (16, 32, 64)
SHORT_DTYPES = ("f16", "bf16")
SHORT_BLOCKS = (16, 32)


def short(B: int, L: int, dtype: str, block_size: int, seed: int = 0,
          kv_dtype: str = "") -> Case:
    """Short-context route: all sequences of length L, pool twice the need."""
    return make_case(f"short_B{B}_L{L}_{dtype}_bs{block_size}{_suffix(kv_dtype)}", B, L,
                     dtype=dtype, block_size=block_size, seed=seed, kv_dtype=kv_dtype)


def short_cases(seed: int = 0, kv_dtype: str = "") -> Iterator[Case]:
    i = 0
    for B in SHORT_BATCHES:
        for L in SHORT_CONTEXTS:
            for dt in SHORT_DTYPES:
                for bs in SHORT_BLOCKS:
                    yield short(B, L, dt, bs, seed + 100 * i, kv_dtype)
                    i += 1


SPLITK_BATCHES = (1, 2, 4, 8)
SPLITK_CONTEXTS = (128, 256, 512, 1024)


def splitk(B: int, L: int, seed: int = 0, kv_dtype: str = "") -> Case:
    """Split-K/LSE sweep point: bf16, block size 16, pool twice the need."""
    return make_case(f"splitk_B{B}_L{L}{_suffix(kv_dtype)}", B, L, dtype="bf16", block_size=16,
                     seed=seed, kv_dtype=kv_dtype)


def splitk_cases(seed: int = 0, kv_dtype: str = "") -> Iterator[Case]:
    i = 0
    for B in SPLITK_BATCHES:
        for L in SPLITK_CONTEXTS:
            yield splitk(B, L, seed + 100 * i, kv_dtype)
            i += 1


def ragged(seed: int = 0, B: int = 32, max_ctx: int = 1024, q_sigma: float = math.sqrt(2.0),
           kv_dtype: str = "") -> Case:
    """Ragged batch: per-sequence contexts uniform in [1, max_ctx], bf16,
    block size 32, pool of B * max_ctx/32 blocks (one block-table row per
    sequence, no reuse), Q ~ N(0, 2) read as variance 2 (sigma = sqrt 2)."""
    g = torch.Generator().manual_seed(int(seed) + 2)
    lens = torch.randint(1, max_ctx + 1, (B,), generator=g).numpy().astype(np.int32)
    MB = max_ctx // 32
    return make_case("ragged_B32" + _suffix(kv_dtype), B, lens, dtype="bf16", block_size=32,
                     seed=seed, pool_blocks=B * MB, max_blocks_per_seq=MB, q_sigma=q_sigma,
                     kv_dtype=kv_dtype)


def large(seed: int = 0, B: int = 64, L: int = 4096, kv_dtype: str = "") -> Case:
    """Bandwidth-bound decode: batch 64, context 4096, bf16, block size 16;
    the pool is exactly the blocks needed and the block table is a random
    permutation of it (K+V = 1 GiB read per call)."""
    bs = 16
    MB = L // bs
    return make_case(f"large_B{B}_L{L}{_suffix(kv_dtype)}", B, L, dtype="bf16", block_size=bs,
                     seed=seed, pool_blocks=B * MB, max_blocks_per_seq=MB, kv_dtype=kv_dtype)


def geometry(Hq: int, Hkv: int, D: int, B: int, L: int, seed: int = 0, dtype: str = "bf16",
             block_size: int = 16, kv_dtype: str = "") -> Case:
    """B sequences of L tokens at another head geometry (the pages' 14/2 D64
    route, MQA 32/1, ...), N(0, 1) inputs, scale 1/sqrt(D) rounded to float32."""
    return make_case(f"geom_{Hq}x{Hkv}_D{D}_B{B}_L{L}{_suffix(kv_dtype)}", B, L, dtype=dtype,
                     block_size=block_size, Hq=Hq, Hkv=Hkv, D=D, seed=seed,
                     scale=float(np.float32(1.0 / math.sqrt(D))), kv_dtype=kv_dtype)
