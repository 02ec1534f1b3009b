"""Per-launch HBM traffic of each kernel from rocprofv3 counter runs.

    python -m online_softmax_attention_pass_amd.traffic OUT_JSON RUN [RUN ...]
    RUN = WORKLOADS:FETCH_CSV:WRITE_CSV

Each RUN is one ``bench.py --workloads WORKLOADS`` invocation profiled twice,
with ``rocprofv3 --pmc FETCH_SIZE`` and with ``--pmc WRITE_SIZE``; FETCH_CSV and
WRITE_CSV are the two ``*_counter_collection.csv`` files. Both counters are
read per dispatch in KiB and averaged over the dispatches of each kernel, then
scaled by the ratio the same counter shows for the calibration copy (a torch
elementwise kernel over 1 GiB fp32: 2^30 bytes read and 2^30 bytes written per
dispatch), which the first run must include (workload ``copy``). Workloads
that share a kernel instance go in different runs: within a run, a kernel is
attributed to the one listed workload that uses it.

The output maps each workload to its kernel's bytes per launch together with
the sha256 of the kernel source (and the headers it includes) it was measured
on; bench.py reports the figure only while that source is unchanged.
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

# workload -> (substring of its dominant kernel's name, kernel source)
KERNELS = {
    "softmax": ("softmax_rows", "softmax_rows.hip"),
    "layernorm": ("layernorm_rows", "layernorm_rows.hip"),
    "prefill": ("attention_bf16_sp_kernel<128, 4, 2, false, false, 0, false>", "attention_bf16.hip"),
    "sparse": ("attention_bf16_sp_kernel<64, 2, 2, false, false, 0, true>", "attention_bf16.hip"),
    "bitmap": ("attention_bf16_sp_kernel<64, 2, 2, true, false, 0, true>", "attention_bf16.hip"),
    "decode": ("decode_partial_kernel", "decode_splitkv.hip"),
    "attn_f32": ("attention_f32", "attention_f32.hip"),
    "gqa": ("attention_bf16_sp_kernel<128, 1, 1, false, true, 0, false>", "attention_bf16.hip"),
    "mla": ("attention_bf16_sp_kernel<128, 4, 2, false, true, 0, false>", "attention_bf16.hip"),
    "alibi": ("attention_bf16_sp_kernel<128, 4, 2, false, false, 1, false>", "attention_bf16.hip"),
    "window": ("attention_bf16_sp_kernel<128, 4, 2, false, false, 1, false>", "attention_bf16.hip"),
    "softcap": ("attention_bf16_sp_kernel<128, 4, 2, false, false, 2, false>", "attention_bf16.hip"),
    "moe": ("moe_route_heads_kernel", "moe_route.hip"),
    "bigbird": ("attention_rowwise_kernel", "attention_rowwise.hip"),
}
COPY_KEY = "MulFunctor"
COPY_BYTES = float(1 << 30)


# Launcher declarations only: they cannot change a kernel's code.
HASH_SKIP = {"launch.h"}


def code_only(text: bytes) -> bytes:
    """A source with its comments removed and its whitespace collapsed: what the
    compiler sees of it (a comment edit does not change the kernel)."""
    text = re.sub(rb"/\*.*?\*/", b" ", text, flags=re.S)
    text = re.sub(rb"//[^\n]*", b" ", text)
    return b" ".join(text.split())


def source_sha(name: str, csrc: str = CSRC) -> str:
    """sha256[:16] over the code (comments and whitespace aside) of a kernel
    source and, in include order, of every local header it pulls in
    (``#include "..."``, followed recursively), except the launcher
    declarations."""
    h = hashlib.sha256()
    seen = set(HASH_SKIP)

    def add(fname):
        if fname in seen:
            return
        seen.add(fname)
        text = open(os.path.join(csrc, fname), "rb").read()
        h.update(code_only(text))
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
    if len(argv) < 2:
        raise SystemExit(__doc__)
    out_path, runs = argv[0], []
    for spec in argv[1:]:
        wl, fcsv, wcsv = spec.split(":")
        runs.append(([w for w in wl.split(",") if w], per_kernel_kib(fcsv, "FETCH_SIZE"),
                     per_kernel_kib(wcsv, "WRITE_SIZE")))
    names0, fetch0, write0 = runs[0]
    if "copy" not in names0:
        raise SystemExit("the first run must include the copy calibration")
    f_scale = COPY_BYTES / find(fetch0, COPY_KEY)
    w_scale = COPY_BYTES / find(write0, COPY_KEY)
    out = {"calibration": {"copy_bytes_each_way": COPY_BYTES, "fetch_bytes_per_kib": f_scale,
                           "write_bytes_per_kib": w_scale}}
    for names, fetch, write in runs:
        for workload in names:
            if workload == "copy":
                continue
            if workload not in KERNELS:
                raise SystemExit(f"unknown workload {workload!r}")
            shared = [w for w in names if w != workload and KERNELS.get(w, ("",))[0] == KERNELS[workload][0]]
            if shared:
                raise SystemExit(f"{workload} shares its kernel with {shared} in one run")
            key, src = KERNELS[workload]
            fb = find(fetch, key) * f_scale
            wb = find(write, key) * w_scale
            out[workload] = {"kernel": key, "source_sha": source_sha(src), "fetch_bytes": round(fb),
                             "write_bytes": round(wb), "bytes_per_launch": round(fb + wb)}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main(sys.argv[1:])
