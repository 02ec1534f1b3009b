"""Per-launch HBM traffic of each kernel from two rocprofv3 counter runs.

    python -m online_softmax_attention_pass_amd.traffic FETCH_CSV WRITE_CSV OUT_JSON

FETCH_CSV / WRITE_CSV are the ``*_counter_collection.csv`` files of two
``rocprofv3 --pmc FETCH_SIZE`` and ``rocprofv3 --pmc WRITE_SIZE`` runs of
``bench.py --workloads copy,...``. Both counters are read per dispatch in KiB
and averaged over the dispatches of each kernel. They are then scaled by the
ratio the same counter shows for the calibration copy (a torch elementwise
kernel over 1 GiB fp32: 2^30 bytes read and 2^30 bytes written per dispatch),
so the figures are HBM bytes in the units the copy defines.

The output maps each workload to its kernel's bytes per launch together with
the sha256 of the kernel source (and the headers it includes) it was measured on; bench.py reports the
figure only while that source is unchanged.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# (substring of the kernel name, workload, kernel source)
KERNELS = [
    ("softmax_rows", "softmax", "softmax_rows.hip"),
    ("layernorm_rows", "layernorm", "layernorm_rows.hip"),
    ("attention_bf16_sp_kernel<128, 4, 2, false>", "prefill", "attention_bf16.hip"),
    ("attention_bf16_sp_kernel<64, 2, 2, false>", "sparse", "attention_bf16.hip"),
    ("attention_bf16_sp_kernel<64, 2, 2, true>", "bitmap", "attention_bf16.hip"),
    ("decode_partial_kernel", "decode", "decode_splitkv.hip"),
    ("attention_f32", "attn_f32", "attention_f32.hip"),
]
COPY_KEY = "MulFunctor"
COPY_BYTES = float(1 << 30)


def source_sha(name: str, csrc: str = CSRC) -> str:
    """sha256[:16] over a kernel source and, in include order, every local
    header it pulls in (``#include "..."``, followed recursively)."""
    h = hashlib.sha256()
    seen = set()

    def add(fname):
        if fname in seen:
            return
        seen.add(fname)
        text = open(os.path.join(csrc, fname), "rb").read()
        h.update(text)
        for inc in re.findall(rb'^#include "([^"]+)"', text, re.M):
            add(inc.decode())

    add(name)
    return h.hexdigest()[:16]


def per_kernel_kib(path: str, counter: str) -> dict:
    """Mean counter value (KiB) per dispatch, keyed by kernel name."""
    acc = defaultdict(lambda: [0.0, 0])
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            a = acc[row["Kernel_Name"]]
            a[0] += float(row["Counter_Value"])
            a[1] += 1
    return {k: v[0] / v[1] for k, v in acc.items() if v[1]}


def find(table: dict, key: str):
    hits = [v for k, v in table.items() if key in k]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {key!r}, found {len(hits)}")
    return hits[0]


def main(argv):
    if len(argv) != 3:
        raise SystemExit(__doc__)
    fetch = per_kernel_kib(argv[0], "FETCH_SIZE")
    write = per_kernel_kib(argv[1], "WRITE_SIZE")
    f_scale = COPY_BYTES / find(fetch, COPY_KEY)
    w_scale = COPY_BYTES / find(write, COPY_KEY)
    out = {"calibration": {"copy_bytes_each_way": COPY_BYTES, "fetch_bytes_per_kib": f_scale,
                           "write_bytes_per_kib": w_scale}}
    for key, workload, src in KERNELS:
        fb = find(fetch, key) * f_scale
        wb = find(write, key) * w_scale
        out[workload] = {"kernel": key, "source_sha": source_sha(src), "fetch_bytes": round(fb),
                         "write_bytes": round(wb), "bytes_per_launch": round(fb + wb)}
    with open(argv[2], "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main(sys.argv[1:])
