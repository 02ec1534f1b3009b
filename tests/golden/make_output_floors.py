"""Write output_floors.json: each bf16 workload's output-rounding floor, from the oracle alone.

    python tests/golden/make_output_floors.py [--workers N]

For the causal prefill (seed 3), split-KV decode (seed 4) and block-sparse
(seed 5) workloads, the fp64 oracle computes every output of the seeded
inputs (over a process pool, one head or block of rows per task), and the
floor max|bf16(O) - O| is taken over all of them: no bf16 output can be
closer to the exact result than that. A floor above the 1e-2 gate would make
the gate unattainable for that seed; the file records the floor, where it
occurs, and max|O|. Only ``oracle`` (through ``tests/full_oracle.py``, with
``workloads`` for the inputs) is called.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

sys.path.insert(0, os.path.join(ROOT, "tests"))
import full_oracle as F  # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workers", type=int, default=None)
    ap.add_argument("--only", default="prefill,decode,sparse")
    args = ap.parse_args()
    out_path = os.path.join(HERE, "output_floors.json")
    data = json.load(open(out_path)) if os.path.exists(out_path) else {}
    data["_about"] = ("Output-rounding floor max|bf16(O) - O| over every output of each bf16 workload's seeded "
                      "inputs, from the fp64 oracle (written by make_output_floors.py). No bf16 output can be "
                      "closer to the exact result than its floor.")
    for name in args.only.split(","):
        t0 = time.time()
        ref_o, _ = F.full_reference(name, args.workers)
        s = F.floor_summary(name, ref_o)
        s["oracle_wall_s_when_written"] = round(time.time() - t0, 1)
        data[name] = s
        print(json.dumps({name: s}), flush=True)
    with open(out_path, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
