"""Write the regression fixture for the tiny workload.

The pages print no worked numeric example for paged decode, so this fixture is
a regression anchor, not an external pin: it records what the fp64 oracle
gives for the tiny workload (batch 1, Hq/Hkv 32/8, D 128, bf16, block size 16,
context 16, pool of 4 blocks) so that a change in the generator or the oracle
on another machine is caught. It calls only ``oracle`` and ``workloads``.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    seed = 0
    c = workloads.tiny(seed)
    out, lse = oracle.attention_case(c)
    doc = {
        "what": "fp64 oracle output for the tiny workload; regression anchor "
                "(the pages print no worked example)",
        "workload": c.describe(),
        "seed": seed,
        "block_table": c.block_table.tolist(),
        "out_hex": [float(x).hex() for x in out.reshape(-1)],
        "lse_hex": [float(x).hex() for x in lse.reshape(-1)],
        "out_bf16_bits": oracle.round_to_dtype(out, "bf16").reshape(-1).tolist(),
    }
    with open(os.path.join(HERE, "tiny_seed0.json"), "w") as f:
        json.dump(doc, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
