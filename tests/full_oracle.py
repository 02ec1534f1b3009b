"""Every output of a workload from the fp64 oracle, computed on the host's cores.

Test infrastructure: the full-output parity tests and
``golden/make_output_floors.py`` call it. The oracle runs unchanged, one head
or one block of query rows per task, over a pool of
``oracle.pool.workers_available()`` forked processes (each with a one-thread
BLAS, none touching the GPU);
the inputs of each task are drawn by ``workloads`` from the workload's seed,
exactly as the device inputs are.
"""
from __future__ import annotations

import numpy as np

import oracle as O
import workloads as W
from oracle import pool

# Query rows per task: 1024 (a 1024 x Lk fp64 score block is 32 to 64 MiB per
# worker; whole 4096-row heads run several times slower per row, mostly in
# page faults on their larger temporaries).
ROW_BLOCK = {"attn_f32": 128, "prefill": 1024, "sparse": 1024}
SOFTMAX_ROWS_PER_TASK = 64
DECODE_HEADS_PER_TASK = 16


def attention_tasks(name):
    c = W.CONFIGS[name]
    rb = ROW_BLOCK[name]
    return [(name, b, h, r0, min(r0 + rb, c["Lq"])) for b in range(c["B"]) for h in range(c["H"])
            for r0 in range(0, c["Lq"], rb)]


def decode_tasks(name):
    c = W.CONFIGS[name]
    n = c["B"] * c["H"]
    return [(name, i, min(i + DECODE_HEADS_PER_TASK, n)) for i in range(0, n, DECODE_HEADS_PER_TASK)]


def softmax_tasks(name):
    c = W.CONFIGS[name]
    return [(name, r, min(r + SOFTMAX_ROWS_PER_TASK, c["rows"])) for r in range(0, c["rows"], SOFTMAX_ROWS_PER_TASK)]


def full_reference(name, workers=None):
    """(ref_o, ref_lse) over every output of an attention or decode workload:
    O [B, H, Lq, d] and LSE [B, H, Lq] (decode: [B, H, 1, d] and [B, H])."""
    c = W.CONFIGS[name]
    if c["kind"] == "decode":
        tasks = decode_tasks(name)
        ref_o = np.empty((c["B"] * c["H"], c["d"]))
        ref_l = np.empty(c["B"] * c["H"])
        for (_, i0, i1), (o, l) in zip(tasks, pool.imap_tasks("decode", tasks, workers)):
            ref_o[i0:i1], ref_l[i0:i1] = o, l
        return ref_o.reshape(c["B"], c["H"], 1, c["d"]), ref_l.reshape(c["B"], c["H"])
    tasks = attention_tasks(name)
    ref_o = np.empty((c["B"], c["H"], c["Lq"], c["d"]))
    ref_l = np.empty((c["B"], c["H"], c["Lq"]))
    for (_, b, h, r0, r1), (o, l) in zip(tasks, pool.imap_tasks("attention", tasks, workers)):
        ref_o[b, h, r0:r1], ref_l[b, h, r0:r1] = o, l
    return ref_o, ref_l


def softmax_reference_blocks(name, workers=None):
    """Yield (r0, r1, y_ref) row blocks of the softmax workload, in order."""
    tasks = softmax_tasks(name)
    for (_, r0, r1), y in zip(tasks, pool.imap_tasks("softmax", tasks, workers)):
        yield r0, r1, y


def floor_summary(name, ref_o):
    """The output-rounding floor max|bf16(O) - O| over all outputs, where it
    occurs, and how many outputs alone exceed the 1e-2 gate."""
    c = W.CONFIGS[name]
    gap = np.abs(O.round_to_bf16(ref_o) - ref_o)
    at = np.unravel_index(int(np.argmax(gap)), gap.shape)
    return {"workload": c["name"], "seed": c["seed"], "outputs": int(ref_o.size), "floor": float(gap.max()),
            "floor_at": [int(i) for i in at], "o_at_floor": float(ref_o[at]),
            "max_abs_o": float(np.abs(ref_o).max()), "elements_with_floor_above_1e-2": int((gap > 1e-2).sum())}


def check_bf16_gates(name, got_o, got_l, ref_o, ref_l, gate_o=1e-2, gate_l=1e-3):
    """Max abs error over every output against the bf16 gates (O 1e-2, LSE 1e-3).

    An output whose exact value is more than gate_o from every bf16 number (its
    own rounding floor |bf16(O) - O| exceeds the gate) cannot meet the gate in
    any bf16 output; the seed is kept and such an element is reported by name.
    For it the check is the tightest one a bf16 output allows: the result is
    one of the two bf16 neighbours of the exact value (it errs by less than one
    bf16 spacing there). Every other output must be within gate_o. Raises
    AssertionError naming the elements that fail; returns the figures."""
    gap = np.abs(O.round_to_bf16(ref_o) - ref_o)
    err = np.abs(got_o - ref_o)
    assert not np.isnan(got_o).any() and not np.isnan(got_l).any(), f"{name}: NaN in the output"
    unatt = gap > gate_o
    lines = []
    for ix in np.argwhere(unatt):
        ix = tuple(int(i) for i in ix)
        nearest = float(O.round_to_bf16(np.array([ref_o[ix]]))[0])
        lines.append(f"gate unattainable at {ix}: exact O {ref_o[ix]:.6f}, nearest bf16 {nearest:.6f} "
                     f"(floor {gap[ix]:.3e}); kernel {got_o[ix]:.6f} (error {err[ix]:.3e})")
    spacing = np.ldexp(1.0, np.frexp(np.abs(ref_o))[1] - 8)       # bf16 spacing at |O|
    assert np.all(err[unatt] < spacing[unatt]), f"{name}: not a bf16 neighbour of the exact value:\n" + \
        "\n".join(lines)
    e_gated = float(err[~unatt].max()) if (~unatt).any() else 0.0
    if e_gated > gate_o:
        bad = np.argwhere((err > gate_o) & ~unatt)[:20]
        raise AssertionError(f"{name}: max|dO| {e_gated:.3e} > {gate_o:g} at\n" + "\n".join(
            f"{tuple(int(i) for i in ix)}: got {got_o[tuple(ix)]:.6f} ref {ref_o[tuple(ix)]:.6f} "
            f"floor {gap[tuple(ix)]:.3e}" for ix in bad))
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(got_l), fin) and np.array_equal(got_l[~fin], ref_l[~fin]), \
        f"{name}: LSE infinities differ"
    e_l = float(np.abs(got_l[fin] - ref_l[fin]).max()) if fin.any() else 0.0
    assert e_l <= gate_l, f"{name}: max|dLSE| {e_l:.3e} > {gate_l:g}"
    return {"max_err_o": float(err.max()), "max_err_o_gated": e_gated, "max_err_lse": e_l,
            "gated_outputs": int((~unatt).sum()), "unattainable": lines}
