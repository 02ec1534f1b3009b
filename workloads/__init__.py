"""Seeded synthetic inputs shared by the fp64 oracle and the GPU path.

This module only *draws* inputs. It contains none of the arithmetic of the
method (no max, no exponential, no normalisation, no contraction): both the
oracle and the device path consume exactly the arrays produced here, and each
side interprets them on its own.

Every tensor slice is a pure function of (config seed, tensor id, slice
index): a NumPy ``Generator(PCG64(SeedSequence([seed, tensor_id, *index])))``
draws it. So any single attention head, or any single softmax row, can be
regenerated on any machine without materialising the whole tensor, which is
what lets the oracle check sampled heads of a 32 GiB decode cache.

Value distributions follow the workloads the pages describe: i.i.d. N(0, 1)
queries, keys and values; softmax rows of N(0, 2^2) plus a per-row offset
uniform in [-50, 50]; block masks of the causal / sliding-window / random
kinds that the STOF page (Accelerating Sparse Transformer Inference on GPU,
Résumé technique, Énoncé du problème) lists as the sparsity patterns that
matter.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

# Tensor ids inside one config's seed space.
TID_Q, TID_K, TID_V, TID_X, TID_MASK, TID_U = 0, 1, 2, 3, 4, 5
TID_GAMMA, TID_BETA = 6, 7

MASK_TILE = 64  # granularity of the block mask, in tokens, on both axes

# The five workloads. Sizes are the ones the throughput figures are quoted on.
CONFIGS = {
    "attn_f32": dict(seed=1, name="attn_f32_B1_H1_L128_d64", kind="attention", dtype="f32",
            B=1, H=1, Lq=128, Lk=128, d=64, scale=1.0 / math.sqrt(64),
            causal=False, mask=None),
    "softmax": dict(seed=2, name="softmax_f32_4096x32768", kind="softmax", dtype="f32",
            rows=4096, cols=32768),
    "prefill": dict(seed=3, name="causal_prefill_bf16_B4_H32_L4096_d128", kind="attention",
            dtype="bf16", B=4, H=32, Lq=4096, Lk=4096, d=128,
            scale=1.0 / math.sqrt(128), causal=True, mask=None),
    "decode": dict(seed=4, name="splitkv_decode_bf16_B64_H32_Lk32768_d128_s16",
            kind="decode", dtype="bf16", B=64, H=32, Lk=32768, d=128,
            scale=1.0 / math.sqrt(128), num_splits=16),
    "sparse": dict(seed=5, name="block_sparse_bf16_B2_H16_L8192_d64", kind="attention",
            dtype="bf16", B=2, H=16, Lq=8192, Lk=8192, d=64,
            scale=1.0 / math.sqrt(64), causal=True, mask="window512_rand10"),
}


def rng(seed: int, tensor_id: int, *index: int) -> np.random.Generator:
    """The one generator every slice comes from."""
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id)] + [int(i) for i in index])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the raw uint16 bits.

    Input preparation only: the draws are float32, the bf16 workloads store
    the rounded bit patterns, and both sides widen those bits themselves.
    """
    b = np.array(x, dtype=np.float32, copy=True).reshape(-1).view(np.uint32)
    nan = np.isnan(b.view(np.float32))
    t = b >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    b += t
    out = b.view(np.uint16)[1::2].copy()       # little-endian: the high half of each word
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out.reshape(np.shape(x))


def normal_head(seed: int, tensor_id: int, b: int, h: int, L: int, d: int, dtype: str) -> np.ndarray:
    """One [L, d] head of i.i.d. N(0, 1): float32, or bf16 bits (uint16) when dtype == 'bf16'."""
    z = rng(seed, tensor_id, b, h).standard_normal((L, d), dtype=np.float32)
    return f32_to_bf16_bits(z) if dtype == "bf16" else z


_SHARED = {}


def _fill_heads(args):
    key, seed, tensor_id, B, H, L, d, dtype, lo, hi = args
    arr = _SHARED[key]
    for bh in range(lo, hi):
        arr[bh] = normal_head(seed, tensor_id, bh // H, bh % H, L, d, dtype)
    return hi - lo


def normal_tensor(seed: int, tensor_id: int, B: int, H: int, L: int, d: int, dtype: str,
                  workers: int | None = None) -> np.ndarray:
    """A [B, H, L, d] tensor assembled from per-head draws.

    Large tensors are filled by a pool of forked workers writing straight into
    an anonymous shared mapping, which the returned array keeps alive (no copy).
    """
    npdt = np.uint16 if dtype == "bf16" else np.float32
    n_heads = B * H
    nbytes = n_heads * L * d * np.dtype(npdt).itemsize
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    if nbytes < (64 << 20) or workers <= 1 or n_heads < 2:
        out = np.empty((n_heads, L, d), dtype=npdt)
        for bh in range(n_heads):
            out[bh] = normal_head(seed, tensor_id, bh // H, bh % H, L, d, dtype)
        return out.reshape(B, H, L, d)
    import mmap
    from multiprocessing import get_context
    mm = mmap.mmap(-1, nbytes, flags=mmap.MAP_SHARED | mmap.MAP_ANONYMOUS)
    arr = np.frombuffer(mm, dtype=npdt).reshape(n_heads, L, d)
    key = id(arr)
    _SHARED[key] = arr          # inherited by the forked workers
    try:
        step = max(1, math.ceil(n_heads / (workers * 8)))
        jobs = [(key, seed, tensor_id, B, H, L, d, dtype, lo, min(n_heads, lo + step))
                for lo in range(0, n_heads, step)]
        with ProcessPoolExecutor(max_workers=workers, mp_context=get_context("fork")) as ex:
            done = sum(ex.map(_fill_heads, jobs))
        assert done == n_heads
    finally:
        del _SHARED[key]
    return arr.reshape(B, H, L, d)


def softmax_row(seed: int, r: int, cols: int) -> np.ndarray:
    """Row r of the softmax workload: float32(2 z + u_r), z ~ N(0, 1), u_r ~ U[-50, 50]."""
    z = rng(seed, TID_X, r).standard_normal(cols, dtype=np.float32)
    u = rng(seed, TID_U, r).uniform(-50.0, 50.0)
    return (2.0 * z.astype(np.float64) + u).astype(np.float32)


def softmax_rows_input(seed: int, rows: int, cols: int, row_ids=None) -> np.ndarray:
    ids = range(rows) if row_ids is None else row_ids
    return np.stack([softmax_row(seed, int(r), cols) for r in ids]) if len(ids) else \
        np.zeros((0, cols), np.float32)


def window_random_block_mask(seed: int, n_tiles: int, window_tiles: int = 8,
                             frac: float = 0.10) -> np.ndarray:
    """uint8 [n_tiles, n_tiles] tile mask: a causal sliding window plus random lower tiles.

    Tile (I, J) is active when I - window_tiles < J <= I (the window, diagonal
    included), plus exactly round(frac * N) tiles drawn uniformly without
    replacement from the N tiles strictly below the window (J <= I - window_tiles).
    """
    m = np.zeros((n_tiles, n_tiles), dtype=np.uint8)
    for i in range(n_tiles):
        m[i, max(0, i - window_tiles + 1): i + 1] = 1
    cand_i, cand_j = np.nonzero(np.tril(np.ones((n_tiles, n_tiles), bool), k=-window_tiles))
    n_pick = int(round(frac * len(cand_i)))
    if n_pick:
        pick = rng(seed, TID_MASK).choice(len(cand_i), size=n_pick, replace=False)
        m[cand_i[pick], cand_j[pick]] = 1
    return m


def window_bitmap_mask(seed: int, L: int, window: int = 512, frac: float = 0.10):
    """Tile kinds uint8 [n, n] and row bitmaps uint64 [n, n, 64] (n = ceil(L / 64)).

    Row i sees key j when i - window < j <= i (an element-level causal sliding
    window), plus every key of exactly round(frac * N) 64x64 tiles drawn
    uniformly without replacement from the N tiles wholly below the window's
    tile band (J <= I - window / 64 - 1). Tiles whose elements are all visible
    get kind 1, none kind 0, the rest kind 2 with word r of the tile holding
    row r's visibility of its 64 keys (bit j).
    """
    n = math.ceil(L / MASK_TILE)
    wt = window // MASK_TILE
    kinds = np.zeros((n, n), dtype=np.uint8)
    bits = np.zeros((n, n, MASK_TILE), dtype=np.uint64)
    r = np.arange(MASK_TILE)[:, None]
    c = np.arange(MASK_TILE)[None, :]
    weights = (np.uint64(1) << np.arange(MASK_TILE, dtype=np.uint64))
    for I in range(n):
        for J in range(max(0, I - wt), I + 1):
            i = I * MASK_TILE + r
            j = J * MASK_TILE + c
            vis = (j <= i) & (j > i - window) & (i < L) & (j < L)
            if vis.all():
                kinds[I, J] = 1
            elif vis.any():
                kinds[I, J] = 2
                bits[I, J] = (vis.astype(np.uint64) * weights).sum(axis=1, dtype=np.uint64)
    cand_i, cand_j = np.nonzero(np.tril(np.ones((n, n), bool), k=-(wt + 1)))
    n_pick = int(round(frac * len(cand_i)))
    if n_pick:
        pick = rng(seed, TID_MASK).choice(len(cand_i), size=n_pick, replace=False)
        kinds[cand_i[pick], cand_j[pick]] = 1
    return kinds, bits


# Extension beyond the five specified workloads: element-level sparsity inside
# partial tiles (the STOF two-level format), at the block-sparse shape.
EXTENSION_CONFIGS = {
    "bitmap": dict(name="bitmap_sparse_bf16_B2_H16_L8192_d64", kind="attention", dtype="bf16",
                   B=2, H=16, Lq=8192, Lk=8192, d=64, scale=1.0 / math.sqrt(64), causal=True,
                   mask="window512_elem_rand10", seed=6),
    # Row layer normalisation (mean and variance as one fused reduction), at the
    # softmax workload's shape; rows are drawn as the softmax rows are.
    "layernorm": dict(name="layernorm_f32_4096x32768", kind="layernorm", dtype="f32", rows=4096, cols=32768,
                      eps=1e-5, seed=7),
    # Decode with grouped queries at the decode workload's cache length: 8 query
    # heads per key/value head (grouped-query attention), and every query head
    # on one shared cache (the MLA sharing pattern). q is drawn as [B, Hq, 1, d],
    # k and v as [B, Hkv, Lk, d], per head like every other tensor.
    "gqa_decode": dict(name="gqa_decode_bf16_B64_Hq64_Hkv8_Lk32768_d128_s4", kind="decode_gqa", dtype="bf16",
                       B=64, Hq=64, Hkv=8, Lk=32768, d=128, scale=1.0 / math.sqrt(128), num_splits=4, seed=8),
    "mla_decode": dict(name="shared_kv_decode_bf16_B64_Hq128_Hkv1_Lk32768_d128_s8", kind="decode_gqa",
                       dtype="bf16", B=64, Hq=128, Hkv=1, Lk=32768, d=128, scale=1.0 / math.sqrt(128),
                       num_splits=8, seed=9),
    # Score modifications (the FlexAttention variants) on the causal prefill
    # shape: one set of q, k, v for three variants, each on top of causal: an
    # ALiBi bias with the geometric slopes, a tanh softcap of 50, and an
    # element-level sliding window of 1024 keys.
    "score_mod": dict(name="score_mod_bf16_B4_H32_L4096_d128", kind="attention", dtype="bf16", B=4, H=32,
                      Lq=4096, Lk=4096, d=128, scale=1.0 / math.sqrt(128), causal=True, softcap=50.0,
                      window=1024, seed=10),
    # A chunk of 256 queries at the end of a 16384-key context under a
    # BigBird-style element mask (STOF's mask family): 64 global keys, a causal
    # local window of 256 keys, and 64 keys per row drawn uniformly at random
    # from the rest of the row's past: the highly sparse, short-query regime.
    "bigbird_chunk": dict(name="bigbird_chunk_bf16_B1_H32_Lq256_Lk16384_d128", kind="attention", dtype="bf16",
                          B=1, H=32, Lq=256, Lk=16384, d=128, scale=1.0 / math.sqrt(128), causal=True,
                          n_global=64, window=256, n_random=64, seed=12),
    # Mixture-of-experts routing: router logits of 131072 tokens over 256
    # experts, top 8 renormalised (a large-expert-count layer).
    "moe": dict(name="moe_route_f32_T131072_E256_k8", kind="moe", dtype="f32", T=131072, E=256, k=8, renorm=True,
                seed=11),
}

TID_LOGITS = 8


MOE_DRAW_BLOCK = 4096   # tokens per generator: block t0 .. t0 + 4095 comes from rng(seed, TID_LOGITS, t0)


def moe_logits_block(seed: int, t0: int, t1: int, E: int) -> np.ndarray:
    """Tokens [t0, t1) of the router logits (t0 a multiple of MOE_DRAW_BLOCK)."""
    assert t0 % MOE_DRAW_BLOCK == 0
    x = np.empty((t1 - t0, E), np.float32)
    for b in range(t0, t1, MOE_DRAW_BLOCK):
        n = min(t1, b + MOE_DRAW_BLOCK) - b
        x[b - t0:b - t0 + n] = 2.0 * rng(seed, TID_LOGITS, b).standard_normal((n, E), dtype=np.float32)
    return x


def moe_logits(seed: int, T: int, E: int, quantum: float = 0.0) -> np.ndarray:
    """Router logits [T, E] float32 ~ N(0, 2^2), drawn in blocks of 4096 tokens;
    quantum > 0 rounds them to multiples of it (many exact ties)."""
    x = moe_logits_block(seed, 0, T, E)
    if quantum > 0:
        x = (np.round(x / quantum) * quantum).astype(np.float32)
    return x


def alibi_slopes(H: int) -> np.ndarray:
    """The geometric ALiBi slopes 2^(-8 (h + 1) / H), h = 0 .. H - 1 (float32)."""
    return (2.0 ** (-8.0 * (np.arange(H) + 1) / H)).astype(np.float32)


def gqa_inputs(cfg: dict, Lk: int | None = None):
    """q [B, Hq, d], k and v [B, Hkv, Lk, d] of a grouped-query decode config
    (raw bf16 bits as uint16), drawn per head."""
    Lk = cfg["Lk"] if Lk is None else Lk
    q = normal_tensor(cfg["seed"], TID_Q, cfg["B"], cfg["Hq"], 1, cfg["d"], cfg["dtype"])[:, :, 0]
    k = normal_tensor(cfg["seed"], TID_K, cfg["B"], cfg["Hkv"], Lk, cfg["d"], cfg["dtype"])
    v = normal_tensor(cfg["seed"], TID_V, cfg["B"], cfg["Hkv"], Lk, cfg["d"], cfg["dtype"])
    return q, k, v


def layernorm_affine(seed: int, cols: int):
    """gamma ~ 1 + 0.1 N(0, 1) and beta ~ 0.1 N(0, 1), float32 [cols]."""
    g = (1.0 + 0.1 * rng(seed, TID_GAMMA).standard_normal(cols)).astype(np.float32)
    b = (0.1 * rng(seed, TID_BETA).standard_normal(cols)).astype(np.float32)
    return g, b


def extension_bitmap_mask():
    c = EXTENSION_CONFIGS["bitmap"]
    return window_bitmap_mask(c["seed"], c["Lq"], window=512, frac=0.10)


def config_block_mask(name: str):
    c = CONFIGS[name]
    if c.get("mask") != "window512_rand10":
        return None
    n = math.ceil(c["Lq"] / MASK_TILE)
    return window_random_block_mask(c["seed"], n, window_tiles=512 // MASK_TILE, frac=0.10)


def element_mask_tiles(vis: np.ndarray):
    """Tile kinds uint8 [nI, nJ] and row bitmaps uint64 [nI, nJ, 64] of a
    boolean element mask vis [Lq, Lk] (True = visible): kind 0 for a tile with
    no visible element, 1 for one whose elements inside [Lq, Lk] are all
    visible, 2 otherwise, with word r holding row r's 64 keys (bit j)."""
    Lq, Lk = vis.shape
    nI, nJ = math.ceil(Lq / MASK_TILE), math.ceil(Lk / MASK_TILE)
    pad = np.zeros((nI * MASK_TILE, nJ * MASK_TILE), bool)
    pad[:Lq, :Lk] = vis
    inside = np.zeros_like(pad)
    inside[:Lq, :Lk] = True
    t = pad.reshape(nI, MASK_TILE, nJ, MASK_TILE).transpose(0, 2, 1, 3)
    tin = inside.reshape(nI, MASK_TILE, nJ, MASK_TILE).transpose(0, 2, 1, 3)
    anyv = t.any(axis=(2, 3))
    allv = (t | ~tin).all(axis=(2, 3))
    kinds = np.where(allv & anyv, 1, np.where(anyv, 2, 0)).astype(np.uint8)
    weights = np.uint64(1) << np.arange(MASK_TILE, dtype=np.uint64)
    bits = (t.astype(np.uint64) * weights).sum(axis=3, dtype=np.uint64)
    bits[kinds != 2] = 0
    return np.ascontiguousarray(kinds), np.ascontiguousarray(bits)


def bigbird_chunk_mask(seed: int, Lq: int, Lk: int, n_global: int, window: int, n_random: int) -> np.ndarray:
    """Boolean element mask [Lq, Lk] for Lq queries at positions Lk - Lq + i:
    keys j < n_global, keys in (p - window, p], and n_random keys per row drawn
    without replacement from [n_global, p - window] (all of them if fewer)."""
    vis = np.zeros((Lq, Lk), bool)
    for i in range(Lq):
        p = Lk - Lq + i
        vis[i, :min(n_global, p + 1)] = True
        vis[i, max(0, p - window + 1):p + 1] = True
        lo, hi = n_global, p - window + 1
        if hi > lo:
            pick = rng(seed, TID_MASK, i).choice(hi - lo, size=min(n_random, hi - lo), replace=False)
            vis[i, lo + pick] = True
    return vis
