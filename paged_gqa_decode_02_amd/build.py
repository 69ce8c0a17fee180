"""Build the in-tree HIP library ``_lib/libpaged_decode.so`` for gfx950.

    python paged_gqa_decode_02_amd/build.py

(run as a file: importing the package would load the library it rebuilds)

Compiles the kernels (``csrc/pd_kernels.hip``, ``csrc/pd_rope.hip``,
``csrc/pd_blocks.hip``, ``csrc/pd_scratch.hip``) and the host side
(``csrc/pd_api.cpp``, ``csrc/pd_kv_api.cpp``, ``csrc/pd_plan.cpp``) with hipcc
into one shared library exporting the C ABI of ``include/paged_decode.h`` and
``include/paged_kv.h``. Packed fp32 VALU instructions are disabled for the
device code.

Then compiles the Python binding of the per-step entry points
(``csrc/pd_binding.cpp``, argument checks and marshalling over torch
tensors) with g++ against torch's headers into ``_lib/_pd_binding*.so``,
linked to the library above.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIB_DIR, "libpaged_decode.so")
ARCH = "gfx950"

BINDING_SRC = "pd_binding.cpp"
SOURCES = ["pd_kernels.hip", "pd_rope.hip", "pd_blocks.hip", "pd_scratch.hip", "pd_api.cpp",
           "pd_kv_api.cpp", "pd_plan.cpp"]
HEADERS = ["pd_internal.h", "pd_fp8_code.h"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile the library (always) and return its path."""
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # the decode kernel's first arguments (block table, lengths, q and
           # the sizes and packed geometry their addresses need) arrive in
           # scalar registers
           "-mllvm", "-amdgpu-kernarg-preload-count=8",
           "-Wall", "-Wno-unused-function", "-Werror=float-conversion",
           "-Werror=implicit-int-float-conversion",
           "-I", os.path.join(ROOT, "include")]
    cmd += list(extra_flags or [])
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    # the binding names the library by this soname; the package loads it
    # by path first, and the loader then reuses that copy
    cmd += ["-Wl,-soname,libpaged_decode.so", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(x for x in res.stderr.splitlines() if noise not in x)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def binding_path() -> str:
    import sysconfig
    return os.path.join(LIB_DIR, "_pd_binding" + sysconfig.get_config_var("EXT_SUFFIX"))


def build_binding(verbose: bool = False) -> str:
    """Compile the Python binding (always) against the built library and
    torch's headers; return its path."""
    import sysconfig

    import torch.utils.cpp_extension as ce
    out = binding_path()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [shutil.which("g++") or "g++", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
           f"-D_GLIBCXX_USE_CXX11_ABI={int(torch_cxx11_abi())}",
           # torch's ROCm headers: HIP streams present themselves as CUDA ones
           "-D__HIP_PLATFORM_AMD__=1", "-DUSE_ROCM=1", "-DTORCH_EXTENSION_NAME=_pd_binding",
           "-I", os.path.join(ROOT, "include")]
    for inc in ce.include_paths() + [rocm_include(), sysconfig.get_paths()["include"]]:
        cmd += ["-isystem", inc]
    cmd += [os.path.join(CSRC, BINDING_SRC), "-o", tmp, "-L", LIB_DIR, "-lpaged_decode",
            "-Wl,-rpath,$ORIGIN"]
    for d in ce.library_paths():
        cmd += ["-L", d, "-Wl,-rpath," + d]
    cmd += ["-lc10", "-lc10_hip", "-ltorch", "-ltorch_cpu", "-ltorch_hip", "-ltorch_python"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ failed ({res.returncode}) building the binding:\n{res.stderr}")
    os.replace(tmp, out)
    return out


def torch_cxx11_abi() -> bool:
    import torch
    return bool(torch._C._GLIBCXX_USE_CXX11_ABI)


def rocm_include() -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(root, "include")


def build_all(verbose: bool = False) -> list[str]:
    """The library, then the binding linked to it."""
    return [build(verbose), build_binding(verbose)]


if __name__ == "__main__":
    print("\n".join(build_all(verbose=True)))
