"""The FP8 cache write's encoder against the oracle's, on the CPU.

`e4m3_code` (paged_gqa_decode_02_amd/csrc/pd_fp8_code.h) is the very source
the RoPE + KV write kernel includes; here it is compiled for the host with
g++ (tests/fp8_code_probe.cpp) and compared with the oracle's nearest-code
search (oracle/rope.py `fp8_encode`, written from the OCP E4M3FN definition:
nearest of the 127 finite magnitudes, ties to the even code, held at 448).

Coverage: every float32 whose magnitude lies in [2^-13, 2^11) (biased
exponents 114 to 137, both signs, all 2^23 fractions: 402,653,184 patterns,
which hold every code, every midpoint between codes and both float32
neighbours of each midpoint, the subnormal codes and the saturation at 448
and 464); and for every one of the 512 sign/exponent pairs a stratified set
of fractions (zero, one, all ones, each code-midpoint pattern and its two
neighbours, and a random sample), plus the infinities and NaNs."""
import ctypes
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from oracle import rope

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kernel_encoder(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    so = str(tmp_path_factory.mktemp("fp8") / "fp8_code_probe.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared",
                    os.path.join(ROOT, "tests", "fp8_code_probe.cpp"), "-o", so], check=True)
    lib = ctypes.CDLL(so)
    lib.pd_probe_e4m3.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]

    def enc(bits):
        bits = np.ascontiguousarray(bits, np.uint32)
        out = np.empty(bits.size, np.uint8)
        lib.pd_probe_e4m3(bits.ctypes.data, out.ctypes.data, bits.size)
        return out
    return enc


def oracle_codes(bits, pool):
    f = np.ascontiguousarray(bits, np.uint32).view(np.float32)
    parts = np.array_split(f, 8)
    return np.concatenate(list(pool.map(rope.fp8_encode, parts)))


def first_mismatch(bits, got, want):
    i = int(np.argmax(got != want))
    return f"bits 0x{int(bits[i]):08x}: kernel 0x{int(got[i]):02x}, oracle 0x{int(want[i]):02x}"


def test_every_float_of_the_coded_range(kernel_encoder):
    frac = np.arange(1 << 23, dtype=np.uint32)
    n = 0
    with ThreadPoolExecutor(8) as pool:
        for sign in (0, 1):
            for e in range(114, 138):
                bits = np.uint32((sign << 31) | (e << 23)) | frac
                got, want = kernel_encoder(bits), oracle_codes(bits, pool)
                assert np.array_equal(got, want), first_mismatch(bits, got, want)
                n += bits.size
    assert n == 402_653_184


def stratified_fractions(rng):
    f = [0, 1, (1 << 23) - 1]
    # the midpoint between two 3-bit fractions of a normal code sits at bit
    # 19; neighbours one float32 step either side
    for c in range(8):
        mid = (c << 20) | (1 << 19)
        f += [mid - 1, mid, mid + 1]
    f += rng.integers(0, 1 << 23, size=4096).tolist()
    return np.array(sorted(set(f)), dtype=np.uint32)


@pytest.mark.filterwarnings("ignore:invalid value encountered in cast")
def test_every_exponent_with_the_midpoint_neighbours(kernel_encoder):
    frac = stratified_fractions(np.random.default_rng(7))
    bits = (np.arange(512, dtype=np.uint32)[:, None] << np.uint32(23) | frac[None, :]).ravel()
    with ThreadPoolExecutor(8) as pool:
        want = oracle_codes(bits, pool)
    got = kernel_encoder(bits)
    assert np.array_equal(got, want), first_mismatch(bits, got, want)
    # the infinities saturate, every NaN gives the NaN code with its sign
    special = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF],
                       dtype=np.uint32)
    assert kernel_encoder(special).tolist() == [0x7E, 0xFE, 0x7F, 0xFF, 0x7F, 0xFF]
    assert rope.fp8_encode(special.view(np.float32)).tolist() == [0x7E, 0xFE, 0x7F, 0xFF, 0x7F,
                                                                  0xFF]
