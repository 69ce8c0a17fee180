"""The oracle's pins catch plausible mistakes in the oracle (CPU only).

Each case plants one mistake in a copy of oracle/pd_oracle.c (a dropped
term, a wrong sign, a wrong index or stride, a transposed operand, an
off-by-one), builds it with gcc and runs the pins of tests/test_oracle_pins.py
against that build (PD_ORACLE_LIB) in a child process: every mutant must make
at least one pin fail. A mutant the pins let through would be a mistake the
oracle could carry unseen into every parity test that trusts it.

The mistakes are planted in the C arithmetic of the decode (scores, softmax,
output, log-sum-exp, GQA grouping, paged addressing, partitions, the LSE
merge), in the exact widening of the 16-bit and FP8 formats and in the
rounding to 16 bits; and, in the same way, in the Python oracles of the RoPE
+ KV write (oracle/rope.py: frequencies, table, rotation, pairing, slots,
the E4M3FN encoder and its acceptance rule) and of the block moves
(oracle/blocks.py), against the pins of tests/test_oracle_rope.py and
tests/test_oracle_blocks.py."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "pd_oracle.c")

# (name, text in pd_oracle.c, replacement, replace every occurrence)
MUTANTS = [
    ("gqa_grouping_interleaved", "const int g = h / G;", "const int g = h % J->Hkv;", False),
    ("cache_layout_heads_before_tokens",
     "(((int64_t)blk * J->bs + t % J->bs) * J->Hkv + g) * D",
     "(((int64_t)blk * J->Hkv + g) * J->bs + t % J->bs) * D", True),
    ("block_table_row_stride", "J->bt[(int64_t)b * J->MB + t / J->bs]",
     "J->bt[(int64_t)b * J->bs + t / J->bs]", True),
    ("block_offset_off_by_one", "t % J->bs) * J->Hkv", "(t + 1) % J->bs) * J->Hkv", True),
    ("last_token_dropped", "err = attend(J, b, h, 0, L, s,", "err = attend(J, b, h, 0, L - 1, s,",
     False),
    ("scale_dropped", "s[t - t0] = J->scale * dot;", "s[t - t0] = dot;", False),
    ("softmax_sign_flipped", "exp(s[t - t0] - m)", "exp(m - s[t - t0])", True),
    ("normaliser_dropped", "for (int d = 0; d < D; ++d) o[d] /= Z;", "", False),
    ("lse_drops_the_max", "*lse = m + log(Z);", "*lse = log(Z);", False),
    ("lse_sign", "*lse = m + log(Z);", "*lse = m - log(Z);", False),
    ("v_read_from_k", "o[d] += w * widen(J->v[row + d], J->dtype);",
     "o[d] += w * widen(J->k[row + d], J->dtype);", False),
    ("q_index_transposed", "J->q + ((int64_t)b * J->Hq + h) * D",
     "J->q + ((int64_t)h * J->B + b) * D", False),
    ("empty_context_lse", "*lse = -INFINITY;\n        return 0;", "*lse = 0.0;\n        return 0;",
     False),
    ("partition_ignores_length", "int t1 = t0 + J->P < L ? t0 + J->P : L;", "int t1 = t0 + J->P;",
     False),
    ("partition_start_off_by_one", "int t0 = p * J->P;", "int t0 = p * J->P + (p > 0);", False),
    ("merge_weight_sign", "double w = exp(lse_part[i * S + p] - M);",
     "double w = exp(M - lse_part[i * S + p]);", False),
    ("merge_drops_ragged_partition", "int n = (L + P - 1) / P;", "int n = L / P;", False),
    ("merge_normaliser_dropped", "for (int d = 0; d < D; ++d) o[d] /= W;", "", False),
    ("bf16_exponent_bias", "ldexp((double)(128 + f), e - 134)", "ldexp((double)(128 + f), e - 133)",
     False),
    ("bf16_subnormal_scale", "ldexp((double)f, -133)", "ldexp((double)f, -134)", False),
    ("f16_exponent_bias", "ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)",
     False),
    ("f16_subnormal_scale", "ldexp((double)f, -24)", "ldexp((double)f, -25)", False),
    ("e4m3_exponent_bias", "ldexp((double)(8 + f), e - 10)", "ldexp((double)(8 + f), e - 9)", False),
    ("e4m3_subnormal_scale", "ldexp((double)f, -9)", "ldexp((double)f, -10)", False),
    ("e4m3_nan_code", "if (e == 15 && f == 7) return NAN;", "if (e == 15) return NAN;", False),
    ("fp8_key_takes_the_value_scale", "widen_e4m3(J->k8[row + d]) * J->k_scale",
     "widen_e4m3(J->k8[row + d]) * J->v_scale", False),
    ("fp8_value_scale_dropped", "widen_e4m3(J->v8[row + d]) * J->v_scale",
     "widen_e4m3(J->v8[row + d])", False),
    ("round_truncates", "double r = nearbyint(ldexp(a, -qe));", "double r = trunc(ldexp(a, -qe));",
     False),
    ("round_subnormal_quantum", "if (e < emin) e = emin;", "", False),
    ("round_carry_lost", "if (r >= ldexp(1.0, p)) { r = ldexp(1.0, fbits); qe += 1; }", "", False),
    ("round_overflow_not_infinite", "if (field >= expmax) return (uint16_t)(sign | (expmax << fbits));",
     "", False),
    ("block_id_bound_off_by_one", "if (blk < 0 || blk >= J->num_blocks) return -2;",
     "if (blk < 0 || blk > J->num_blocks) return -2;", False),
    ("length_bound_not_checked",
     "if (J->cl[b] < 0 || (int64_t)J->cl[b] > (int64_t)J->MB * J->bs) return -3;",
     "if (J->cl[b] < 0) return -3;", False),
]


def mutate(src: str, old: str, new: str, every: bool) -> str:
    n = src.count(old)
    assert n >= 1 and (every or n == 1), (old, n)
    return src.replace(old, new) if every else src.replace(old, new, 1)


def run_mutant(tmp_path, name, old, new, every):
    src = mutate(open(ORACLE_C).read(), old, new, every)
    c = tmp_path / f"{name}.c"
    c.write_text(src)
    lib = str(tmp_path / f"lib{name}.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-pthread", str(c), "-o", lib, "-lm"], check=True)
    env = dict(os.environ, PD_ORACLE_LIB=lib, OMP_NUM_THREADS="1",
               PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "tests/test_oracle_pins.py"], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=600)
    return name, res.returncode, res.stdout[-1500:]


def test_the_original_passes_its_pins():
    env = dict(os.environ, OMP_NUM_THREADS="1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "tests/test_oracle_pins.py"], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    if subprocess.run(["which", "gcc"], capture_output=True).returncode != 0:
        pytest.skip("gcc not found")
    workers = max(1, min(8, (os.cpu_count() or 2) // 2))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda m: run_mutant(tmp_path, *m), MUTANTS))
    survivors = [(name, out) for name, rc, out in results if rc == 0]
    assert not survivors, "mutants the pins let through: " + ", ".join(n for n, _ in survivors)
    # a failure must be a failing pin, not a crash of the test run itself
    for name, rc, out in results:
        assert rc == 1, (name, rc, out)


# Mistakes planted in the Python parts of the oracle: (name, file under
# oracle/, text, replacement). The pins of tests/test_oracle_rope.py and
# tests/test_oracle_blocks.py run against a copy of the package holding the
# mutant. (Two plausible edits are left out because they change nothing: in
# the FP8 acceptance rule the adjacency test is implied by the midpoint test
# while eps stays below a quarter of a code step, as it does by many orders
# of magnitude, since a code two or more steps from the nearest one lies that
# far from the midpoint between them; and a block-table remap that skips
# block 0 is the identity there, block 0 never moving in a compaction.)
PY_MUTANTS = [
    ("rope_frequency_exponent", "rope.py", "(-2.0 * i / rotary_dim)", "(-1.0 * i / rotary_dim)"),
    ("rope_table_columns_swapped", "rope.py", "[np.cos(ang), np.sin(ang)]",
     "[np.sin(ang), np.cos(ang)]"),
    ("rope_rotation_sign", "rope.py", "x1 * cos - x2 * sin", "x1 * cos + x2 * sin"),
    ("rope_interleaved_pairs", "rope.py", "x1, x2 = x[..., :h], x[..., h:]",
     "x1, x2 = x[..., 0::2], x[..., 1::2]"),
    ("rope_cos_sin_read_swapped", "rope.py",
     "cos, sin = tab[:, None, : D // 2], tab[:, None, D // 2:]",
     "sin, cos = tab[:, None, : D // 2], tab[:, None, D // 2:]"),
    ("rope_position_off_by_one", "rope.py", "tab = table.astype(np.float64)[pos]",
     "tab = table.astype(np.float64)[np.maximum(pos - 1, 0)]"),
    ("rope_values_rotated", "rope.py", "vc[slots[live]] = v[live]",
     "vc[slots[live]] = round_to_dtype(rotate(widen(v, dtype), cos, sin)[live], dtype)"),
    ("rope_slot_zero_is_padding", "rope.py", "    live = slots >= 0\n    if np.any",
     "    live = slots > 0\n    if np.any"),
    ("e4m3_subnormal_step", "rope.py", "f / 8.0 * 2.0 ** -6", "f / 8.0 * 2.0 ** -7"),
    ("e4m3_ties_to_odd", "rope.py", "(hi % 2 == 0)", "(hi % 2 == 1)"),
    ("e4m3_nan_code", "rope.py", "out = np.where(nan, 0x7F, code)", "out = np.where(nan, 0x7E, code)"),
    ("e4m3_value_sign", "rope.py", "return np.where(c & 0x80, -mag, mag)", "return mag"),
    ("fp8_key_scale_multiplies", "rope.py", "k_exact = k_rot[live] / np.float64(ks)",
     "k_exact = k_rot[live] * np.float64(ks)"),
    ("fp8_value_takes_the_key_scale", "rope.py",
     "v_exact = widen(np.asarray(v, np.uint16), dtype)[live] / np.float64(vs)",
     "v_exact = widen(np.asarray(v, np.uint16), dtype)[live] / np.float64(ks)"),
    ("fp8_bound_too_tight", "rope.py", "k_eps = ((2 * u + u * u) * ((1 + u) ** 2 + 1) + 1e-15)",
     "k_eps = ((u + u * u) * ((1 + u) ** 2 + 1) + 1e-15)"),
    ("fp8_rule_tolerance_loosened", "rope.py", "near = np.abs(exact - 0.5 * (gv + rv)) <= eps",
     "near = np.abs(exact - 0.5 * (gv + rv)) <= 2.5 * eps"),
    ("fp8_rule_ignores_the_midpoint", "rope.py", "ok = same | (adj & near)", "ok = same | adj"),
    ("copy_operands_swapped", "blocks.py", "        out[d] = cache[s]", "        out[s] = cache[d]"),
    ("gather_sorted", "blocks.py", "np.stack([cache[i] for i in ids])",
     "np.stack([cache[i] for i in sorted(ids)])"),
    ("scatter_reversed", "blocks.py", "        out[b] = src[i]",
     "        out[b] = src[len(ids) - 1 - i]"),
    ("compact_holes_reversed", "blocks.py", "for s, d in zip(movers, holes):",
     "for s, d in zip(movers, holes[::-1]):"),
    ("remap_skips_the_last_block", "blocks.py", "ok = (bt >= 0) & (bt < len(remap))",
     "ok = (bt >= 0) & (bt < len(remap) - 1)"),
]
PY_PINS = [os.path.join(ROOT, "tests", f) for f in ("test_oracle_rope.py", "test_oracle_blocks.py")]


def oracle_copy(tmp_path, tag):
    import shutil
    dst = tmp_path / tag / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("_build", "__pycache__", "*.so"))
    return dst


def real_oracle_lib(tmp_path):
    lib = str(tmp_path / "libpd_oracle_orig.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-pthread", ORACLE_C, "-o", lib, "-lm"], check=True)
    return lib


def run_py_mutant(tmp_path, lib, name, fname, old, new):
    pkg = oracle_copy(tmp_path, name)
    path = pkg / fname
    path.write_text(mutate(path.read_text(), old, new, False))
    # run from the copy's folder: it comes first on the child's path
    env = dict(os.environ, PD_ORACLE_LIB=lib, OMP_NUM_THREADS="1",
               PYTHONPATH=str(pkg.parent) + os.pathsep + ROOT)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          *PY_PINS], cwd=str(pkg.parent), env=env, capture_output=True, text=True,
                         timeout=600)
    return name, res.returncode, res.stdout[-1500:]


def test_every_planted_mistake_in_the_python_oracle_fails_a_pin(tmp_path):
    if subprocess.run(["which", "gcc"], capture_output=True).returncode != 0:
        pytest.skip("gcc not found")
    lib = real_oracle_lib(tmp_path)
    # the child processes import the copy, not the package in the tree
    pkg = oracle_copy(tmp_path, "probe")
    env = dict(os.environ, PD_ORACLE_LIB=lib,
               PYTHONPATH=str(pkg.parent) + os.pathsep + ROOT)
    where = subprocess.run([sys.executable, "-c", "import oracle, sys; print(oracle.__file__)"],
                           cwd=str(pkg.parent), env=env, capture_output=True, text=True, check=True)
    assert where.stdout.strip().startswith(str(pkg)), where.stdout
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *PY_PINS,
                          "-p", "no:randomly"], cwd=str(pkg.parent), env=env, capture_output=True,
                         text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:]   # the unmutated copy passes
    workers = max(1, min(8, (os.cpu_count() or 2) // 2))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda m: run_py_mutant(tmp_path, lib, *m), PY_MUTANTS))
    survivors = [name for name, rc, _ in results if rc == 0]
    assert not survivors, "mutants the pins let through: " + ", ".join(survivors)
    for name, rc, out in results:
        assert rc == 1, (name, rc, out)
