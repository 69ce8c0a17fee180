"""Sanitizer lanes on the CPU (the sanitizer lanes of the vllm.cpp BENCHMARKS
page, ASan+UBSan and TSan, taken up for this library's host code and oracle).

* The C ABI's host logic (pd_api.cpp, pd_kv_api.cpp, pd_plan.cpp: argument
  checks, size arithmetic, planning, the compaction planner) built with g++
  under AddressSanitizer and UndefinedBehaviorSanitizer with stub launchers
  (tests/abi_sanitize.cpp), driven by a random sweep of valid and extreme
  arguments.
* The fp64 oracle (oracle/pd_oracle.c) built under ASan+UBSan and, since it
  runs on a pool of threads, under ThreadSanitizer; the oracle's pins
  (tests/test_oracle_pins.py) run against each build in a child process that
  preloads the sanitizer runtime.
* Each lane is shown to bite: a planted one-element overflow and a planted
  race in copies of the oracle are reported.

No GPU is involved; a lane whose sanitizer runtime the compiler lacks is
skipped."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_gqa_decode_02_amd", "csrc")
ORACLE_C = os.path.join(ROOT, "oracle", "pd_oracle.c")
SAN_ERRORS = ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer",
              "ERROR: LeakSanitizer")


def runtime(name):
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("gcc/g++ not found")
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not available")
    return path


def build_oracle(src, out, flags):
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                    "-fPIC", "-shared", "-pthread", *flags, src, "-o", out, "-lm"], check=True)


def run_child(cmd, env_extra, log_dir):
    env = dict(os.environ)
    env.update(env_extra)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    logs = ""
    for f in os.listdir(log_dir):
        with open(os.path.join(log_dir, f)) as fh:
            logs += fh.read()
    return res, res.stdout + res.stderr + logs


def asan_env(lib, log_dir):
    return {"LD_PRELOAD": runtime("libasan.so"), "PD_ORACLE_LIB": lib,
            "ASAN_OPTIONS": f"detect_leaks=0:abort_on_error=0:exitcode=97:"
                            f"log_path={log_dir}/asan",
            "UBSAN_OPTIONS": f"halt_on_error=1:print_stacktrace=1:log_path={log_dir}/ubsan"}


def tsan_env(lib, log_dir, supp):
    return {"LD_PRELOAD": runtime("libtsan.so"), "PD_ORACLE_LIB": lib,
            # torch's and numpy's own OpenMP threads are not instrumented:
            # keep them to one thread and leave their code out of the reports
            "OMP_NUM_THREADS": "1",
            "TSAN_OPTIONS": f"halt_on_error=1:exitcode=98:log_path={log_dir}/tsan:"
                            f"suppressions={supp}"}


def test_abi_host_logic_under_asan_and_ubsan(tmp_path):
    runtime("libasan.so")
    exe = str(tmp_path / "abi_sanitize")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "abi_sanitize.cpp"),
                    os.path.join(CSRC, "pd_api.cpp"), os.path.join(CSRC, "pd_kv_api.cpp"),
                    os.path.join(CSRC, "pd_plan.cpp"), "-o", exe], check=True)
    res = subprocess.run([exe, "200000"], capture_output=True, text=True, timeout=600,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert not any(e in out for e in SAN_ERRORS), out[-4000:]
    assert "0 failures" in out


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libpd_oracle_asan.so")
    build_oracle(ORACLE_C, lib, ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"])
    logs = tmp_path / "logs"
    logs.mkdir()
    res, out = run_child([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "tests/test_oracle_pins.py"], asan_env(lib, logs), str(logs))
    assert res.returncode == 0, out[-4000:]
    assert not any(e in out for e in SAN_ERRORS), out[-4000:]
    assert " passed" in res.stdout


def tsan_suppressions(tmp_path):
    supp = tmp_path / "tsan.supp"
    supp.write_text("race:libtorch_cpu.so\nrace:libgomp.so\nrace:_multiarray_umath\n")
    return str(supp)


def test_oracle_pins_under_tsan(tmp_path):
    lib = str(tmp_path / "libpd_oracle_tsan.so")
    build_oracle(ORACLE_C, lib, ["-fsanitize=thread"])
    logs = tmp_path / "logs"
    logs.mkdir()
    res, out = run_child([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "tests/test_oracle_pins.py"], tsan_env(lib, logs,
                                                                 tsan_suppressions(tmp_path)),
                         str(logs))
    assert res.returncode == 0, out[-4000:]
    assert not any(e in out for e in SAN_ERRORS), out[-4000:]
    assert " passed" in res.stdout


PROBE = """
import numpy as np, oracle, workloads
c = workloads.make_case("san", 4, [37, 64, 1, 50], dtype="bf16", block_size=16, seed=3,
                        max_blocks_per_seq=4)
out, lse = oracle.attention(c.q, c.k_cache, c.v_cache, c.block_table, c.context_lens,
                            scale=c.scale, dtype=c.dtype, nthreads=4)
print("probe done", float(np.abs(out).sum()))
"""


def mutant(tmp_path, old, new):
    src = open(ORACLE_C).read()
    assert src.count(old) == 1, old
    path = tmp_path / "pd_oracle_mutant.c"
    path.write_text(src.replace(old, new))
    return str(path)


def test_asan_lane_reports_a_planted_overflow_in_the_oracle(tmp_path):
    # the score buffer one element short: a context of full capacity (64
    # tokens here) writes one double past it
    src = mutant(tmp_path, "malloc(sizeof(double) * (size_t)(ctx_cap > 0 ? ctx_cap : 1))",
                 "malloc(sizeof(double) * (size_t)(ctx_cap > 1 ? ctx_cap - 1 : 1))")
    lib = str(tmp_path / "libmutant_asan.so")
    build_oracle(src, lib, ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"])
    logs = tmp_path / "logs"
    logs.mkdir()
    res, out = run_child([sys.executable, "-c", PROBE], asan_env(lib, logs), str(logs))
    assert res.returncode != 0 and "heap-buffer-overflow" in out, out[-3000:]


def test_tsan_lane_reports_a_planted_race_in_the_oracle(tmp_path):
    # every worker takes every (sequence, head) pair instead of its own
    # share, so two threads write the same output row
    src = mutant(tmp_path, "i < pairs && !err; i += J->nthreads", "i < pairs && !err; i += 1")
    lib = str(tmp_path / "libmutant_tsan.so")
    build_oracle(src, lib, ["-fsanitize=thread"])
    logs = tmp_path / "logs"
    logs.mkdir()
    res, out = run_child([sys.executable, "-c", PROBE],
                         tsan_env(lib, logs, tsan_suppressions(tmp_path)), str(logs))
    assert res.returncode != 0 and "WARNING: ThreadSanitizer: data race" in out, out[-3000:]
    assert "pd_oracle_mutant.c" in out
