#!/usr/bin/env python3
"""Throughput of the online-softmax attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads softmax,prefill,decode,...]

One JSON line is printed. Its headline (``value``) is the row-softmax
workload, fp32 4096 x 32768, in GB/s of algorithmic HBM traffic (one read and
one write per element); every workload that ran is also reported under
``workloads`` with its own time, throughput and roofline: causal bf16 prefill
(B4 H32 L4096 d128, TFLOP/s), split-KV bf16 decode (B64 H32 Lk32768 d128, 16
splits, GB/s), block-sparse bf16 attention (B2 H16 L8192 d64, TFLOP/s on
active tiles) and single-head fp32 attention (B1 H1 L128 d64, microseconds;
its few-microsecond calls are paced by the host's call rate in a plain loop,
so the leg also times them captured in one HIP graph, ``graph_replay``).
Extension workloads: element bitmaps in partial tiles (B2 H16 L8192 d64,
TFLOP/s), row layer normalisation (fp32 4096 x 32768, GB/s), and decode with
grouped queries at Lk 32768, d 128: 8 query heads per key/value head (B64 Hq64
Hkv8, 4 splits) and 128 query heads on one cache (B64 Hq128 Hkv1, 8 splits),
in GB/s with TFLOP/s alongside; and the score modifications on the causal
prefill shape (B4 H32 L4096 d128): ALiBi bias, tanh softcap 50, and a
1024-key sliding window (TFLOP/s); and mixture-of-experts routing of 131072
tokens over 256 experts, top 8 (GB/s).

Timing: every leg's inputs are made resident in HBM first; then, once,
leg after leg, back to back: 50 ms of untimed calls while the clock settles
after the change of load (reported per leg as ``settle``), then exactly W
untimed warm-up calls, then K calls between one pair of HIP events recorded on
the stream the kernels run on (the mean per call), then K more, each bracketed
by its own events (their median, p10 and p90); device syncs bracket each region. No call finds its
operands in the 256 MB Infinity Cache left by earlier calls: the softmax and
layer-norm workloads (1 GiB per call) alternate two buffer sets, the
block-sparse and bitmap workloads (about 135 MB) rotate three, the MoE and
BigBird workloads two; the prefill-shape workloads (512 MiB of q, k, v, o),
the decodes (1 to 32 GiB) exceed the cache by themselves.
The split-KV and grouped-query decodes' roofline is over the whole call (the
partial kernel plus the merge); the partial kernel alone is reported beside
it, labelled.
CPU baseline: after the GPU legs, the fp64 oracle as it stands, on a bounded
sample of each workload, over all of this host's cores (one forked process
per core, at most 16, BLAS one thread each), in each leg's own unit. A pilot
pass over the sample sets how many times it is run, so that the timed part
spends about 16 s of CPU time summed over the processes.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published

KERNEL_SOURCES = {
    "copy": None, "softmax": "softmax_rows.hip", "prefill": "attention_bf16.hip", "decode": "decode_splitkv.hip",
    "sparse": "attention_bf16.hip", "attn_f32": "attention_f32.hip", "bitmap": "attention_bf16.hip",
    "layernorm": "layernorm_rows.hip", "gqa": "attention_bf16.hip", "mla": "attention_bf16.hip",
    "alibi": "attention_bf16.hip", "softcap": "attention_bf16.hip", "window": "attention_bf16.hip",
    "moe": "moe_route.hip", "bigbird": "attention_rowwise.hip",
}


def source_sha(name: str) -> str:
    from online_softmax_attention_pass_amd.traffic import source_sha as sha
    return sha(name, os.path.join(ROOT, "online_softmax_attention_pass_amd", "csrc"))


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was
    taken on the kernel source as it is now; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p)).get(workload)
    except (OSError, ValueError):
        return None
    if not t or KERNEL_SOURCES.get(workload) is None or t.get("source_sha") != source_sha(KERNEL_SOURCES[workload]):
        return None
    return t.get("bytes_per_launch")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timer:
    """HIP events on the current stream: one pair around all the timed calls
    (the launches queue back to back, so the mean is the kernels' own time),
    then one pair per call in a second pass for the spread."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, steps):
        torch = self.torch
        stream = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        mean_ms = a.elapsed_time(b) / steps
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for x, y in ev:
            x.record(stream)
            fn()
            y.record(stream)
        torch.cuda.synchronize()
        per = [x.elapsed_time(y) for x, y in ev]
        return mean_ms, per, wall


SETTLE_MS = 50.0  # untimed calls of each leg before its warm-up calls
CPU_BASELINE_CPU_S = 16.0  # CPU seconds (summed over the pool) of each leg's timed oracle sample


def warm_up(torch, fn, calls):
    """Exactly `calls` untimed calls."""
    for _ in range(calls):
        fn()
    torch.cuda.synchronize()
    return calls


def settle(torch, fn, ms):
    """Untimed calls for `ms` milliseconds before a leg's warm-up calls. On this
    chip the clock moves for several milliseconds after the load changes (from
    idle, or from another leg's kind of work): a fresh run of causal-prefill
    calls starts near 0.61 ms per call, slows to about 0.78 ms and comes back
    to 0.60 ms over about 20 calls. Timing that transient would understate the
    steady rate, so each leg first settles, and the record says how long."""
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()   # pace the host to the GPU so elapsed time is GPU time
    torch.cuda.synchronize()
    return n


def graph_replay_ms(torch, fn, outputs, steps):
    """Per-call GPU time of `steps` calls captured in one HIP graph and replayed:
    a call of a few microseconds is otherwise paced by the host's call rate
    (argument checks and the ctypes call take about 10 us in Python). The
    replay's outputs must equal the eager call's."""
    try:
        fn()
        torch.cuda.synchronize()
        want = [t.clone() for t in outputs]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):   # torch wants a non-default stream for capture
            fn()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                fn()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        same = all(torch.equal(x, y) for x, y in zip(outputs, want))
        return {"ms_per_call": round(a.elapsed_time(b) / steps, 5), "calls_per_replay": steps,
                "outputs_equal_eager": bool(same)}
    except Exception as e:  # noqa: BLE001 - a capture failure is reported, not fatal
        return {"error": f"{type(e).__name__}: {e}"}


def roofline(bound, achieved, peak, unit, traffic):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def setup_softmax(rf, torch, W):
    """Two input/output sets (2 GiB), used alternately, so that no call finds
    its operands in the 256 MB Infinity Cache left by the previous one."""
    c = W.CONFIGS["softmax"]
    x = W.softmax_rows_input(c["seed"], c["rows"], c["cols"])
    sets = []
    for _ in range(2):
        xd = torch.from_numpy(x).cuda()
        sets.append((xd, torch.empty_like(xd)))
    nbytes = 2 * x.size * 4
    turn = [0]

    def call():
        xd, yd = sets[turn[0]]
        turn[0] ^= 1
        rf.rf_softmax_rows(xd, out=yd)
    return dict(fn=call, work=nbytes, unit="GB/s", bound="hbm", keep=sets, cfg=c,
                extra={"buffer_sets": 2})


def setup_prefill(rf, torch, W):
    c = W.CONFIGS["prefill"]
    q, k, v = (torch.from_numpy(W.normal_tensor(c["seed"], t, c["B"], c["H"], c["Lq"], c["d"], "bf16").view(np.int16))
               .view(torch.bfloat16).cuda() for t in (W.TID_Q, W.TID_K, W.TID_V))
    o = torch.empty_like(q)
    lse = torch.empty((c["B"], c["H"], c["Lq"]), dtype=torch.float32, device="cuda")
    flops = 4 * c["B"] * c["H"] * c["Lq"] * c["Lk"] * c["d"] / 2   # causal: half of the dense score matrix
    return dict(fn=lambda: rf.rf_attention_fwd(q, k, v, scale=c["scale"], causal=True, out=o, lse=lse),
                work=flops, unit="TFLOP/s", bound="mfma", keep=(q, k, v, o, lse), cfg=c)


def _setup_score_mod(rf, torch, W, kind):
    c = W.EXTENSION_CONFIGS["score_mod"]
    B, H, L, d = c["B"], c["H"], c["Lq"], c["d"]
    q, k, v = (torch.from_numpy(W.normal_tensor(c["seed"], t, B, H, L, d, "bf16").view(np.int16))
               .view(torch.bfloat16).cuda() for t in (W.TID_Q, W.TID_K, W.TID_V))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    kw = {"alibi": dict(alibi_slopes=torch.from_numpy(W.alibi_slopes(H)).cuda()),
          "softcap": dict(softcap=c["softcap"]), "window": dict(window=c["window"])}[kind]
    if kind == "window":   # visible (row, key) pairs of a causal window, 4 d flop each
        Wn = c["window"]
        pairs = Wn * (Wn + 1) // 2 + (L - Wn) * Wn
    else:                  # the causal convention of the prefill workload
        pairs = L * L / 2
    cfg = dict(c, name=f"{kind}_causal_bf16_B{B}_H{H}_L{L}_d{d}")
    return dict(fn=lambda: rf.rf_attention_fwd_mod(q, k, v, scale=c["scale"], causal=True, out=o, lse=lse, **kw),
                work=4 * B * H * pairs * d, unit="TFLOP/s", bound="mfma", keep=(q, k, v, o, lse, kw), cfg=cfg)


def setup_alibi(rf, torch, W):
    return _setup_score_mod(rf, torch, W, "alibi")


def setup_softcap(rf, torch, W):
    return _setup_score_mod(rf, torch, W, "softcap")


def setup_window(rf, torch, W):
    return _setup_score_mod(rf, torch, W, "window")


N_SETS_SMALL = 3   # buffer sets for workloads whose operands (~135 MB) would fit the 256 MB Infinity Cache


def _rotating_sets(torch, make, n):
    """n independent copies of a workload's device buffers, used in turn, so
    that no call finds its operands in the 256 MB Infinity Cache left by the
    previous calls (n x the working set > 256 MB)."""
    sets = [make() for _ in range(n)]
    state = {"i": 0}

    def next_set():
        x = sets[state["i"] % n]
        state["i"] += 1
        return x
    return sets, next_set


def setup_sparse(rf, torch, W):
    c = W.CONFIGS["sparse"]
    q, k, v = (torch.from_numpy(W.normal_tensor(c["seed"], t, c["B"], c["H"], c["Lq"], c["d"], "bf16").view(np.int16))
               .view(torch.bfloat16).cuda() for t in (W.TID_Q, W.TID_K, W.TID_V))
    bm = W.config_block_mask("sparse")
    bmd = torch.from_numpy(bm).cuda()
    lse_shape = (c["B"], c["H"], c["Lq"])
    sets, next_set = _rotating_sets(torch, lambda: (q.clone(), k.clone(), v.clone(), torch.empty_like(q),
                                                    torch.empty(lse_shape, dtype=torch.float32, device="cuda")),
                                    N_SETS_SMALL)
    del q, k, v
    flops = 4 * 64 * 64 * c["d"] * int(bm.sum()) * c["B"] * c["H"]   # active 64x64 tiles, counted whole

    def fn():
        q, k, v, o, lse = next_set()
        rf.rf_attention_fwd(q, k, v, scale=c["scale"], causal=True, block_mask=bmd, out=o, lse=lse)
    return dict(fn=fn, work=flops, unit="TFLOP/s", bound="mfma", keep=(sets, bmd), cfg=c,
                extra={"active_tiles_per_head": int(bm.sum()), "tiles_per_head": int(bm.size),
                       "buffer_sets": N_SETS_SMALL})


def setup_layernorm(rf, torch, W):
    """Extension workload: row layer normalisation of fp32 4096 x 32768 (the
    softmax shape), two alternating buffer sets like the softmax workload."""
    c = W.EXTENSION_CONFIGS["layernorm"]
    x = W.softmax_rows_input(c["seed"], c["rows"], c["cols"])
    g, b = W.layernorm_affine(c["seed"], c["cols"])
    gd, bd = torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda()
    sets = []
    for _ in range(2):
        xd = torch.from_numpy(x).cuda()
        sets.append((xd, torch.empty_like(xd), torch.empty(c["rows"], device="cuda"),
                     torch.empty(c["rows"], device="cuda")))
    turn = [0]

    def call():
        xd, yd, md, rd = sets[turn[0]]
        turn[0] ^= 1
        rf.rf_layernorm_rows(xd, gd, bd, eps=c["eps"], out=yd, mean=md, rstd=rd)
    nbytes = 2 * x.size * 4 + 2 * c["cols"] * 4 + 2 * c["rows"] * 4   # x, y, gamma, beta, mean, rstd
    return dict(fn=call, work=nbytes, unit="GB/s", bound="hbm", keep=(sets, gd, bd), cfg=c,
                extra={"buffer_sets": 2})


def setup_bitmap(rf, torch, W):
    """Extension workload: element bitmaps inside partial tiles (a 512-key
    element-level causal window plus random tiles), at the block-sparse shape."""
    c = W.EXTENSION_CONFIGS["bitmap"]
    seed = c["seed"]
    q, k, v = (torch.from_numpy(W.normal_tensor(seed, t, c["B"], c["H"], c["Lq"], c["d"], "bf16").view(np.int16))
               .view(torch.bfloat16).cuda() for t in (W.TID_Q, W.TID_K, W.TID_V))
    kinds, bits = W.extension_bitmap_mask()
    kd = torch.from_numpy(kinds).cuda()
    bd = torch.from_numpy(bits.view(np.int64)).cuda()
    lse_shape = (c["B"], c["H"], c["Lq"])
    sets, next_set = _rotating_sets(torch, lambda: (q.clone(), k.clone(), v.clone(), torch.empty_like(q),
                                                    torch.empty(lse_shape, dtype=torch.float32, device="cuda")),
                                    N_SETS_SMALL)
    del q, k, v
    active = int((kinds != 0).sum())
    flops = 4 * 64 * 64 * c["d"] * active * c["B"] * c["H"]   # active 64x64 tiles, counted whole
    n_full = int((kinds == 1).sum())
    n_vis_part = int(sum(bin(int(w)).count("1") for w in bits[kinds == 2].ravel()))
    visible = n_full * 64 * 64 + n_vis_part

    def fn():
        q, k, v, o, lse = next_set()
        rf.rf_attention_fwd_bitmap(q, k, v, kd, bd, scale=c["scale"], causal=c["causal"], out=o, lse=lse)
    return dict(fn=fn, work=flops, unit="TFLOP/s", bound="mfma", keep=(sets, kd, bd), cfg=c,
                extra={"active_tiles_per_head": active, "partial_tiles_per_head": int((kinds == 2).sum()),
                       "visible_fraction_of_active": round(visible / (active * 64 * 64), 4),
                       "buffer_sets": N_SETS_SMALL})


def setup_bigbird(rf, torch, W):
    """Extension workload: the row kernel on a chunk of 256 queries over 16384
    keys under a BigBird-style element mask (the kernel the analytic choice
    picks there); the tile kernel on the same call is timed beside it.
    Algorithmic bytes: q, o and lse, the K and V rows of every key some query
    row of the head sees (each once), and the mask words the rows read."""
    c = W.EXTENSION_CONFIGS["bigbird_chunk"]
    B, H, Lq, Lk, d = c["B"], c["H"], c["Lq"], c["Lk"], c["d"]
    # two sets of q, k, v (about 176 MB of touched K/V each), alternated so no
    # call is served from the Infinity Cache
    sets = []
    for i in range(2):
        q = torch.from_numpy(W.normal_tensor(c["seed"] + i, W.TID_Q, B, H, Lq, d, "bf16").view(np.int16)).view(
            torch.bfloat16).cuda()
        k, v = (torch.from_numpy(W.normal_tensor(c["seed"] + i, t, B, H, Lk, d, "bf16").view(np.int16)).view(
            torch.bfloat16).cuda() for t in (W.TID_K, W.TID_V))
        sets.append((q, k, v))
    vis = W.bigbird_chunk_mask(c["seed"], Lq, Lk, c["n_global"], c["window"], c["n_random"])
    kinds, bits = W.element_mask_tiles(vis)
    plan = rf.rf_attention_plan(kinds, bits, B, H, Lq, Lk, d, c["causal"])
    kd = torch.from_numpy(kinds).cuda()
    bd = torch.from_numpy(bits.view(np.int64)).cuda()
    o = torch.empty_like(sets[0][0])
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    keys = int(vis.any(axis=0).sum())
    mask_bytes = kinds.size + 8 * Lq * int((kinds == 2).sum(axis=1).max(initial=0))
    nbytes = B * H * (2 * Lq * d * 2 + Lq * 4 + keys * 2 * d * 2) + mask_bytes
    state = {"i": 0}

    def call(entry):
        q, k, v = sets[state["i"] % 2]
        state["i"] += 1
        entry(q, k, v, kd, bd, scale=c["scale"], causal=c["causal"], out=o, lse=lse)
    return dict(fn=lambda: call(rf.rf_attention_fwd_rowwise),
                alternatives={"tile_kernel": lambda: call(rf.rf_attention_fwd_bitmap)},
                work=nbytes, unit="GB/s", bound="hbm", keep=(sets, kd, bd, o, lse), cfg=c,
                extra={"visible_per_row": int(vis.sum(axis=1).max()), "keys_seen_per_head": keys,
                       "plan": {k_: (round(v_, 1) if isinstance(v_, float) else v_) for k_, v_ in plan.items()}})


def setup_decode(rf, torch, W):
    c = W.CONFIGS["decode"]
    B, H, Lk, d, S = c["B"], c["H"], c["Lk"], c["d"], c["num_splits"]

    def up(t, L):
        a = W.normal_tensor(c["seed"], t, B, H, L, d, "bf16")
        x = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        del a
        return x
    log("decode: generating 32 GiB of K/V on the host")
    q = up(W.TID_Q, 1)
    k = up(W.TID_K, Lk)
    v = up(W.TID_V, Lk)
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws_bytes = rf.rf_attention_decode_splitkv_workspace_size(B, H, d, S)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    nbytes = 2 * B * H * Lk * d * 2 + B * H * d * 2 * 2 + B * H * 4
    # the merge alone, on the same workspace layout, to split the two launches' times
    n = B * H
    o_parts = ws[: n * S * d * 4].view(torch.float32).view(n, S, d)
    lse_off = -(-n * S * d * 4 // 256) * 256
    lse_parts = ws[lse_off: lse_off + n * S * 4].view(torch.float32).view(n, S)
    o2 = o.view(n, d)
    lse2 = lse.view(n)
    merge = lambda: rf.rf_lse_merge(o_parts, lse_parts, out_dtype=torch.bfloat16, out=o2, lse=lse2)
    return dict(fn=lambda: rf.rf_attention_decode_splitkv(q, k, v, scale=c["scale"], num_splits=S, workspace=ws,
                                                          out=o, lse=lse),
                work=nbytes, unit="GB/s", bound="hbm", keep=(q, k, v, o, lse, ws), cfg=c, subtract=merge,
                extra={"workspace_bytes_round_trip": int(2 * n * S * (d + 1) * 4)})


def _setup_gqa(rf, torch, W, name):
    c = W.EXTENSION_CONFIGS[name]
    B, Hq, Hkv, Lk, d, S = c["B"], c["Hq"], c["Hkv"], c["Lk"], c["d"], c["num_splits"]
    log(f"{name}: generating {2 * B * Hkv * Lk * d * 2 / 2**30:.1f} GiB of K/V on the host")
    up = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    qh, kh, vh = W.gqa_inputs(c)
    q, k, v = up(qh), up(kh), up(vh)
    del qh, kh, vh
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws_bytes = rf.rf_attention_decode_gqa_workspace_size(B, Hq, d, S)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    nbytes = 2 * B * Hkv * Lk * d * 2 + 2 * B * Hq * d * 2 + B * Hq * 4
    n = B * Hq
    o_parts = ws[: n * S * d * 4].view(torch.float32).view(n, S, d)
    lse_off = -(-n * S * d * 4 // 256) * 256
    lse_parts = ws[lse_off: lse_off + n * S * 4].view(torch.float32).view(n, S)
    merge = lambda: rf.rf_lse_merge(o_parts, lse_parts, out_dtype=torch.bfloat16, out=o.view(n, d), lse=lse.view(n))
    return dict(fn=lambda: rf.rf_attention_decode_gqa(q, k, v, scale=c["scale"], num_splits=S, workspace=ws,
                                                      out=o, lse=lse),
                work=nbytes, unit="GB/s", bound="hbm", keep=(q, k, v, o, lse, ws), cfg=c, subtract=merge,
                flops=4 * B * Hq * Lk * d, extra={"workspace_bytes_round_trip": int(2 * n * S * (d + 1) * 4)})


def setup_gqa_decode(rf, torch, W):
    return _setup_gqa(rf, torch, W, "gqa_decode")


def setup_mla_decode(rf, torch, W):
    return _setup_gqa(rf, torch, W, "mla_decode")


def setup_moe(rf, torch, W):
    c = W.EXTENSION_CONFIGS["moe"]
    T, E, k = c["T"], c["E"], c["k"]
    # two sets of logits (128 MiB each), alternated so no call is served from the Infinity Cache
    sets = [torch.from_numpy(W.moe_logits(c["seed"] + i, T, E)).cuda() for i in range(2)]
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    state = {"i": 0}

    def fn():
        x = sets[state["i"] % 2]
        state["i"] += 1
        rf.rf_moe_route(x, k, c["renorm"], out_idx=idx, out_w=w)
    return dict(fn=fn, work=T * E * 4 + T * k * 8, unit="GB/s", bound="hbm", keep=(sets, idx, w), cfg=c)


def setup_attn_f32(rf, torch, W):
    c = W.CONFIGS["attn_f32"]
    q, k, v = (torch.from_numpy(W.normal_tensor(c["seed"], t, 1, 1, 128, 64, "f32")).cuda()
               for t in (W.TID_Q, W.TID_K, W.TID_V))
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 128), dtype=torch.float32, device="cuda")
    flops = 4 * 128 * 128 * 64
    return dict(fn=lambda: rf.rf_attention_fwd(q, k, v, scale=c["scale"], out=o, lse=lse), work=flops,
                unit="TFLOP/s", bound="alu", keep=(q, k, v, o, lse), cfg=c, graph=(o, lse))


def setup_copy(rf, torch, W):
    """Counter calibration only (not run by default): a plain torch elementwise
    copy of 1 GiB fp32, whose HBM traffic is known (one read, one write)."""
    n = 1 << 28
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    return dict(fn=lambda: torch.mul(x, 1.0, out=y), work=2 * n * 4, unit="GB/s", bound="hbm", keep=(x, y),
                cfg={"name": "calibration_copy_f32_1GiB", "dtype": "f32"})


SETUPS = {"copy": setup_copy, "bitmap": setup_bitmap, "layernorm": setup_layernorm, "softmax": setup_softmax, "prefill": setup_prefill, "decode": setup_decode, "sparse": setup_sparse, "gqa": setup_gqa_decode, "mla": setup_mla_decode,
          "alibi": setup_alibi, "bigbird": setup_bigbird, "softcap": setup_softcap, "window": setup_window, "moe": setup_moe,
          "attn_f32": setup_attn_f32}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample of each workload,
# over the host's cores (one forked process per core, BLAS one thread each)
# ---------------------------------------------------------------------------

def _cycle(items, n):
    return [items[i % len(items)] for i in range(n)]


def cpu_baseline_plan(name, W, workers):
    """(task kind, tasks, algorithmic work of the tasks in the workload's unit
    base, unit, sample description): each process gets a few tasks, and the
    work is counted as the GPU leg counts it."""
    C, X = W.CONFIGS, W.EXTENSION_CONFIGS
    if name in ("softmax", "layernorm"):
        c = C["softmax"] if name == "softmax" else X["layernorm"]
        per = 10 if name == "softmax" else 30
        blocks = [(name, r, r + 64) for r in range(0, c["rows"], 64)]
        tasks = _cycle(blocks, workers * per)
        rows = 64 * len(tasks)
        return (name, tasks, 2 * rows * c["cols"] * 4, "GB/s",
                f"{rows} rows of {c['cols']} (64-row blocks, cycling over the {c['rows']} rows)")
    if name in ("prefill", "sparse", "attn_f32"):
        c = C[name]
        if name == "prefill":
            # one block of 1024 query rows per process, spread over heads and row ranges;
            # work = 4 d flops per visible (row, key) pair, row i seeing i + 1 keys
            blocks = [(name, b, h, r, r + 1024) for b in range(c["B"]) for h in range(c["H"])
                      for r in range(0, c["Lq"], 1024)]
            tasks = blocks[:workers]            # whole heads' row blocks, in order: an even mix
            work = sum(4 * c["d"] * (r1 * (r1 + 1) - r0 * (r0 + 1)) / 2 for _, _, _, r0, r1 in tasks)
            return ("attention", tasks, work, "TFLOP/s",
                    f"{len(tasks)} blocks of 1024 query rows (of {len(blocks)} over the {c['B'] * c['H']} heads); "
                    "work = the causal pairs of those rows")
        if name == "attn_f32":
            tasks = [(name, 0, 0, 0, c["Lq"])] * (workers * 1000)
            return ("attention", tasks, len(tasks) * 4 * c["Lq"] * c["Lk"] * c["d"], "TFLOP/s",
                    f"the whole workload (one head) {len(tasks)} times")
        bm = W.config_block_mask(name)
        blocks = [(name, b, h, r, r + 1024) for b in range(c["B"]) for h in range(c["H"])
                  for r in range(0, c["Lq"], 1024)]
        tasks = blocks[:workers * 4]
        work = sum(4 * 64 ** 3 * int(bm[r0 // 64:r1 // 64].sum()) for _, _, _, r0, r1 in tasks)
        return ("attention", tasks, work, "TFLOP/s",
                f"{len(tasks)} blocks of 1024 query rows (of {len(blocks)} over the {c['B'] * c['H']} heads); "
                "work = active 64x64 tiles in those rows")
    if name == "decode":
        c = C[name]
        n = c["B"] * c["H"]
        tasks = _cycle([(name, i, i + 8) for i in range(0, n, 8)], workers)
        per_head = 2 * c["Lk"] * c["d"] * 2 + 2 * c["d"] * 2 + 4
        return ("decode", tasks, 8 * len(tasks) * per_head, "GB/s",
                f"{8 * len(tasks)} of the {n} heads, all {c['Lk']} keys each (unsplit)")
    if name in ("bitmap", "bigbird"):
        key = "bitmap" if name == "bitmap" else "bigbird_chunk"
        c = X[key]
        if name == "bitmap":
            kinds, _ = W.extension_bitmap_mask()
            blocks = [(key, "", b, h, r, r + 1024) for b in range(c["B"]) for h in range(c["H"])
                      for r in range(0, c["Lq"], 1024)]
            tasks = blocks[:workers * 4]
            work = sum(4 * 64 ** 3 * int((kinds[t[4] // 64:t[5] // 64] != 0).sum()) for t in tasks)
            return ("ext_attention", tasks, work, "TFLOP/s",
                    f"{len(tasks)} blocks of 1024 query rows (of {len(blocks)}); "
                    "work = active 64x64 tiles in those rows")
        vis = W.bigbird_chunk_mask(c["seed"], c["Lq"], c["Lk"], c["n_global"], c["window"], c["n_random"])
        kinds, _ = W.element_mask_tiles(vis)
        keys = int(vis.any(axis=0).sum())
        mask_bytes = kinds.size + 8 * c["Lq"] * int((kinds == 2).sum(axis=1).max(initial=0))
        per_head = 2 * c["Lq"] * c["d"] * 2 + c["Lq"] * 4 + keys * 2 * c["d"] * 2 + mask_bytes / c["H"]
        heads = [(key, "", 0, h, 0, c["Lq"]) for h in range(c["H"])]
        tasks = _cycle(heads, workers * 8)
        return ("ext_attention", tasks, per_head * len(tasks), "GB/s", f"{len(tasks)} heads (cycling over {c['H']})")
    if name in ("alibi", "softcap", "window"):
        c = X["score_mod"]
        per = {"alibi": 2, "softcap": 1, "window": 2}[name]
        heads = [("score_mod", name, b, h, 0, c["Lq"]) for b in range(c["B"]) for h in range(c["H"])]
        tasks = _cycle(heads, workers * per)
        L, Wn = c["Lq"], c["window"]
        pairs = Wn * (Wn + 1) // 2 + (L - Wn) * Wn if name == "window" else L * L / 2
        return ("ext_attention", tasks, 4 * pairs * c["d"] * len(tasks), "TFLOP/s",
                f"{len(tasks)} of the {len(heads)} heads, every row")
    if name in ("gqa", "mla"):
        key = "gqa_decode" if name == "gqa" else "mla_decode"
        c = X[key]
        G = c["Hq"] // c["Hkv"]
        units = [(key, b, j) for b in range(c["B"]) for j in range(c["Hkv"])]
        tasks = _cycle(units, workers * (2 if name == "gqa" else 1))
        per_unit = 2 * c["Lk"] * c["d"] * 2 + 2 * G * c["d"] * 2 + G * 4
        return ("gqa", tasks, per_unit * len(tasks), "GB/s",
                f"{len(tasks)} of the {len(units)} key/value heads, each with its {G} query heads")
    if name == "moe":
        c = X["moe"]
        blocks = [("moe", t, t + 4096) for t in range(0, c["T"], 4096)]
        tasks = _cycle(blocks, workers * 20)
        return ("moe", tasks, len(tasks) * 4096 * (c["E"] * 4 + c["k"] * 8), "GB/s",
                f"{4096 * len(tasks)} tokens (4096-token blocks, cycling over the {c['T']})")
    return None


def cpu_baseline(name, W):
    """The fp64 oracle on a bounded sample of workload `name`, timed over the
    host's cores, in the GPU leg's unit (the oracle is never tuned for this)."""
    from oracle import pool
    workers = pool.workers_available()
    plan = cpu_baseline_plan(name, W, workers)
    if plan is None:
        return None
    kind, tasks, work, unit, sample = plan
    # A pilot pass sizes the timed run: the sample's tasks are run as many
    # times as it takes to spend about CPU_BASELINE_CPU_S of CPU time.
    pilot = pool.timed_run(kind, tasks, workers)
    repeat = max(1, min(200, math.ceil(CPU_BASELINE_CPU_S / max(pilot["cpu_s"], 1e-3))))
    r = pool.timed_run(kind, tasks, workers, repeat=repeat)
    scale = 1e9 if unit == "GB/s" else 1e12
    return {"value": round(work * repeat / r["wall_s"] / scale, 6), "unit": unit, "cores": r["workers"],
            "kind": "oracle",
            "sample": f"{sample}, run {repeat} times; fp64 NumPy oracle, {r['wall_s']:.2f} s wall and "
                      f"{r['cpu_s']:.1f} s CPU on {r['workers']} processes (BLAS one thread each; input drawing "
                      f"{r['input_gen_s']:.1f} s and a {pilot['wall_s']:.2f} s pilot pass, not timed)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workloads",
                    default="softmax,prefill,decode,sparse,attn_f32,bitmap,layernorm,gqa,mla,alibi,softcap,window,moe,bigbird")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="milliseconds of untimed calls of each leg before its --warmup calls (the clock settles)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (no sharding, no collectives). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import online_softmax_attention_pass_amd as rf
    import workloads as W
    rf.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    wanted = [w.strip() for w in args.workloads.split(",") if w.strip()]
    # Every leg's inputs go to the GPU first, so that the legs then run back to
    # back: the GPU does not idle (and its clock does not drop) between them.
    legs = {}
    for name in wanted:
        log(f"{name}: setup")
        legs[name] = SETUPS[name](rf, torch, W)

    results = {}
    cfgs = {}
    timer = Timer(torch)
    for name in wanted:
        s = legs[name]
        n_settle = settle(torch, s["fn"], args.settle_ms)
        n_warm = warm_up(torch, s["fn"], args.warmup)
        log(f"{name}: timing {args.steps} calls (after {n_settle} settle and {n_warm} warm-up calls)")
        call_ms, per, wall = timer.run(s["fn"], args.steps)
        thr = s["work"] / (call_ms * 1e-3) / (1e9 if s["unit"] == "GB/s" else 1e12)
        peak = {"hbm": HBM_PEAK_GBS, "mfma": BF16_PEAK_TFLOPS, "alu": FP32_VALU_PEAK_TFLOPS}[s["bound"]]
        r = {"workload": s["cfg"]["name"], "value": round(thr, 3), "unit": s["unit"],
             "ms_per_call": round(call_ms, 5), "ms_p10": round(float(np.percentile(per, 10)), 5),
             "ms_median": round(float(np.median(per)), 5),
             "ms_p90": round(float(np.percentile(per, 90)), 5), "wall_s": round(wall, 4),
             "roofline": roofline(s["bound"], thr, peak, s["unit"], measured_traffic(name)),
             "warmup_calls": n_warm, "settle": {"ms": args.settle_ms, "calls": n_settle}}
        if "subtract" in s:
            # The call is the partial kernel plus the merge; the roofline above
            # is over the whole call. The partial kernel alone, labelled as such:
            # the call time minus the merge timed on its own.
            warm_up(torch, s["subtract"], args.warmup)
            merge_ms = timer.run(s["subtract"], args.steps)[0]
            kern_ms = call_ms - merge_ms
            kthr = s["work"] / (kern_ms * 1e-3) / (1e9 if s["unit"] == "GB/s" else 1e12)
            r["merge_ms"] = round(merge_ms, 5)
            r["partial_kernel_only"] = {"ms": round(kern_ms, 5), "achieved": round(kthr, 3),
                                        "frac": round(kthr / peak, 4)}
        if "graph" in s:
            r["graph_replay"] = graph_replay_ms(torch, s["fn"], s["graph"], args.steps)
        for alt, fn in s.get("alternatives", {}).items():
            warm_up(torch, fn, args.warmup)
            r[f"{alt}_ms"] = round(timer.run(fn, args.steps)[0], 5)
        if "flops" in s:
            r["tflops"] = round(s["flops"] / (call_ms * 1e-3) / 1e12, 3)
        r.update(s.get("extra", {}))
        results[name] = r
        cfgs[name] = s["cfg"]
        log(f"{name}: {r['value']} {r['unit']} ({call_ms:.4f} ms/call, frac {r['roofline']['frac']})")
    del legs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        for name in wanted:
            log(f"{name}: cpu baseline (fp64 oracle on a sample, over the host's cores)")
            cb = cpu_baseline(name, W)
            if cb is not None:
                results[name]["cpu_baseline"] = cb

    head = "softmax" if "softmax" in results else wanted[0]
    h = results[head]
    hc = cfgs[head]
    out = {
        "metric": "fused attention TFLOP/s (% bf16 MFMA peak); softmax/decode GB/s (% HBM peak)",
        "value": h["value"], "unit": h["unit"], "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": h["ms_per_call"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if hc["dtype"] == "f32" else "bf16", "data": "synthetic",
        "config": {"workload": hc["name"], **{k: v for k, v in hc.items() if k in
                                              ("rows", "cols", "B", "H", "Lq", "Lk", "d", "num_splits")}},
        "roofline": h["roofline"],
        "settle_ms_per_leg": args.settle_ms,
        "workloads": results,
    }
    if "cpu_baseline" in h:
        out["cpu_baseline"] = h["cpu_baseline"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
