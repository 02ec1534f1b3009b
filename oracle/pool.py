"""The fp64 oracle spread over the host's cores, one head or one block of rows per task.

TEST INFRASTRUCTURE ONLY (the full-output parity tests and the benchmark's
CPU-baseline leg use it). Nothing here adds arithmetic: every task draws its
inputs with ``workloads`` (the same seeded per-head / per-row generators the
device inputs come from) and calls one oracle function unchanged on one head,
or on a block of query rows of one head. Rows of attention and of a softmax
are independent by definition (each output row depends only on its own query
row or input row), so splitting the work this way changes no arithmetic; only
the BLAS may sum a dot product in another order for another block height
(about 1e-16 apart).

Workers are forked (no new program is started: a process that has already
initialised the GPU must not exec one) and never touch the GPU; each limits
its BLAS to one thread, so N workers use N cores, and leaves with os._exit,
running no exit handlers of the parent's libraries.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time

import numpy as np

from . import oracle as O

# Workers on a host: all the cores this process may run on, at most 16 (the
# CPU share of one GPU on the machines the benchmark runs on).
MAX_WORKERS = 16


def workers_available(cap: int = MAX_WORKERS) -> int:
    return max(1, min(cap, len(os.sched_getaffinity(0))))


# ---------------------------------------------------------------------------
# Task kinds. prepare(args) draws the inputs (not part of the oracle's work);
# compute(inputs) is the oracle call itself.
# ---------------------------------------------------------------------------

def _cfg(name):
    import workloads as W
    return W.CONFIGS[name] if name in W.CONFIGS else W.EXTENSION_CONFIGS[name]


def _prep_attention(name, b, h, r0, r1):
    """Inputs of query rows [r0, r1) of head (b, h) of an attention workload."""
    import workloads as W
    c = _cfg(name)
    q = W.normal_head(c["seed"], W.TID_Q, b, h, c["Lq"], c["d"], c["dtype"])
    k = W.normal_head(c["seed"], W.TID_K, b, h, c["Lk"], c["d"], c["dtype"])
    v = W.normal_head(c["seed"], W.TID_V, b, h, c["Lk"], c["d"], c["dtype"])
    if c["dtype"] == "bf16":
        q, k, v = (O.bf16_bits_to_f64(a) for a in (q, k, v))
    mask = W.config_block_mask(name) if name in W.CONFIGS else None
    return (q[None, None], k[None, None], v[None, None], c["scale"], bool(c["causal"]), mask,
            np.arange(r0, r1))


def _run_attention(inp):
    q, k, v, scale, causal, mask, rows = inp
    o, lse = O.attention(q, k, v, scale, causal, mask, q_rows=rows)
    return o[0, 0], lse[0, 0]


def _prep_decode(name, bh0, bh1):
    """Inputs of decode heads bh0 .. bh1 - 1 (flat b * H + h): one query token each."""
    import workloads as W
    c = _cfg(name)
    out = []
    for bh in range(bh0, bh1):
        b, h = divmod(bh, c["H"])
        q = W.normal_head(c["seed"], W.TID_Q, b, h, 1, c["d"], "bf16")
        k = W.normal_head(c["seed"], W.TID_K, b, h, c["Lk"], c["d"], "bf16")
        v = W.normal_head(c["seed"], W.TID_V, b, h, c["Lk"], c["d"], "bf16")
        # held as float32 (exact for bf16 values) until the oracle widens them
        out.append(tuple(O.bf16_bits_to_f64(a).astype(np.float32)[None, None] for a in (q, k, v)))
    return out, c["scale"]


def _run_decode(inp):
    heads, scale = inp
    os_, ls = [], []
    for q, k, v in heads:
        o, lse = O.attention(q, k, v, scale)          # unsplit: the definition over all keys
        os_.append(o[0, 0, 0])
        ls.append(lse[0, 0, 0])
    return np.stack(os_), np.array(ls)


def _prep_softmax(name, r0, r1):
    import workloads as W
    c = _cfg(name)
    return W.softmax_rows_input(c["seed"], r1 - r0, c["cols"], row_ids=range(r0, r1))


def _run_softmax(x):
    return O.softmax_rows(x)


def _prep_ext_attention(name, variant, b, h, r0, r1):
    """Inputs of query rows [r0, r1) of head (b, h) of an extension attention
    workload: element bitmaps ("bitmap", "bigbird_chunk") or one score
    modification ("score_mod" with variant "alibi", "softcap" or "window")."""
    import workloads as W
    c = _cfg(name)
    q, k, v = (O.bf16_bits_to_f64(W.normal_head(c["seed"], t, b, h, L, c["d"], "bf16"))[None, None]
               for t, L in ((W.TID_Q, c["Lq"]), (W.TID_K, c["Lk"]), (W.TID_V, c["Lk"])))
    rows = np.arange(r0, r1)
    if name == "score_mod":
        kw = {"alibi": {"alibi_slopes": W.alibi_slopes(c["H"])[h:h + 1]}, "softcap": {"softcap": c["softcap"]},
              "window": {"window": c["window"]}}[variant]
        return ("mod", q, k, v, c["scale"], bool(c["causal"]), kw, rows)
    if name == "bitmap":
        kinds, bits = W.extension_bitmap_mask()
    else:
        kinds, bits = W.element_mask_tiles(W.bigbird_chunk_mask(c["seed"], c["Lq"], c["Lk"], c["n_global"],
                                                                c["window"], c["n_random"]))
    return ("bits", q, k, v, c["scale"], bool(c["causal"]), {"block_mask": kinds, "tile_bits": bits}, rows)


def _run_ext_attention(inp):
    what, q, k, v, scale, causal, kw, rows = inp
    if what == "mod":
        o, lse = O.attention_score_mod(q, k, v, scale, causal, q_rows=rows, **kw)
    else:
        o, lse = O.attention(q, k, v, scale, causal, kw["block_mask"], q_rows=rows, tile_bits=kw["tile_bits"])
    return o[0, 0], lse[0, 0]


def _prep_layernorm(name, r0, r1):
    import workloads as W
    c = _cfg(name)
    x = W.softmax_rows_input(c["seed"], r1 - r0, c["cols"], row_ids=range(r0, r1))
    g, b = W.layernorm_affine(c["seed"], c["cols"])
    return x, g, b, c["eps"]


def _run_layernorm(inp):
    x, g, b, eps = inp
    return O.layernorm_rows(x, g, b, eps)


def _prep_gqa(name, b, j):
    """Inputs of key/value head j of batch entry b of a grouped-query decode
    workload, with the G query tokens that read it (query heads j G .. j G + G - 1)."""
    import workloads as W
    c = _cfg(name)
    G = c["Hq"] // c["Hkv"]
    q = np.stack([W.normal_head(c["seed"], W.TID_Q, b, hq, 1, c["d"], "bf16")[0] for hq in range(j * G, j * G + G)])
    k = W.normal_head(c["seed"], W.TID_K, b, j, c["Lk"], c["d"], "bf16")[None]
    v = W.normal_head(c["seed"], W.TID_V, b, j, c["Lk"], c["d"], "bf16")[None]
    return tuple(O.bf16_bits_to_f64(a).astype(np.float32)[None] for a in (q, k, v)) + (c["scale"],)


def _run_gqa(inp):
    q, k, v, scale = inp
    return O.decode_gqa(q, k, v, scale)


def _prep_moe(name, t0, t1):
    import workloads as W
    c = _cfg(name)
    return W.moe_logits_block(c["seed"], t0, t1, c["E"]).astype(np.float64), c["k"], c["renorm"]


def _run_moe(inp):
    x, k, renorm = inp
    return O.moe_route(x, k, renorm)


TASKS = {
    "attention": (_prep_attention, _run_attention),
    "decode": (_prep_decode, _run_decode),
    "softmax": (_prep_softmax, _run_softmax),
    "ext_attention": (_prep_ext_attention, _run_ext_attention),
    "layernorm": (_prep_layernorm, _run_layernorm),
    "gqa": (_prep_gqa, _run_gqa),
    "moe": (_prep_moe, _run_moe),
}


# ---------------------------------------------------------------------------
# Pool machinery
# ---------------------------------------------------------------------------

def _limit_blas():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:          # no control available: the BLAS keeps its own setting
        pass


def _worker_init(root):
    import sys
    if root not in sys.path:
        sys.path.insert(0, root)
    _limit_blas()


def _one(task):
    kind, args = task
    prep, run = TASKS[kind]
    return run(prep(*args))


def _root():
    return os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def imap_tasks(kind: str, args_list, workers: int | None = None):
    """Yield the oracle's result of each task, in order, computed over a
    pool of forked workers (results stream back, so the caller can compare
    block by block)."""
    workers = workers_available() if workers is None else workers
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_worker_init, initargs=(_root(),)) as pool:
        for r in pool.imap(_one, [(kind, tuple(a)) for a in args_list], chunksize=1):
            yield r


def map_tasks(kind: str, args_list, workers: int | None = None):
    return list(imap_tasks(kind, args_list, workers))


def _timed_worker(kind, my_tasks, repeat, barrier, out_q, root):
    _worker_init(root)
    prep, run = TASKS[kind]
    t_gen0 = time.perf_counter()
    inputs = [prep(*a) for a in my_tasks]
    t_gen = time.perf_counter() - t_gen0
    barrier.wait(timeout=900)                        # every worker starts the oracle together
    c0 = time.process_time()
    t0 = time.perf_counter()
    for _ in range(repeat):
        for x in inputs:
            run(x)
    t1 = time.perf_counter()
    out_q.put((t0, t1, t_gen, time.process_time() - c0))


def timed_run(kind: str, args_list, workers: int | None = None, repeat: int = 1) -> dict:
    """Time the oracle on the given tasks over `workers` processes (one process
    per core, BLAS one thread each). Every process first draws the inputs of
    its share of the tasks; then all start together, run their share `repeat`
    times, and the wall clock runs from that start to the last process's end
    (input drawing excluded, and reported separately). `cpu_s` is the
    processes' summed CPU time over the timed part."""
    workers = workers_available() if workers is None else workers
    workers = max(1, min(workers, len(args_list)))
    shares = [args_list[i::workers] for i in range(workers)]
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(workers)
    out_q = ctx.Queue()
    procs = [ctx.Process(target=_timed_worker, args=(kind, [tuple(a) for a in s], repeat, barrier, out_q, _root()))
             for s in shares]
    for p in procs:
        p.start()
    res = [out_q.get(timeout=1800) for _ in procs]
    for p in procs:
        p.join()
        if p.exitcode != 0:
            raise RuntimeError(f"oracle worker exited with {p.exitcode}")
    t0 = min(r[0] for r in res)
    t1 = max(r[1] for r in res)
    return {"wall_s": t1 - t0, "workers": workers, "input_gen_s": max(r[2] for r in res), "tasks": len(args_list),
            "repeat": repeat, "cpu_s": sum(r[3] for r in res)}
