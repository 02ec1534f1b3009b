"""Plain, unfused, multi-pass fp64 reference of what the hot path computes.

TEST INFRASTRUCTURE ONLY — see the package docstring. Nothing here is tiled,
fused or reordered beyond what each definition states; rows are independent
by definition, so selecting a subset of query rows changes no arithmetic.

Sources (the pages are web summaries of three papers):

* RedFuser page (French), "Résumé technique", 1. Problématique and
  2. Méthodologie: safe softmax is a cascaded reduction, d_i = ⊕ F_i(X[l], D_i):
  a max reduction, then a sum of exponentials that depends on that max, then
  a normalisation; attention appends a GEMM. The Korean page of the same
  paper spells the chain out as max → exponential sum → normalise
  (기술 요약, 1. 문제 정의) and states the fusion conditions (2. 방법론, 가):
  F_i = G_i ⊗ H_i, ⊗ a commutative monoid, ⊕ distributive over ⊗.
* RedFuser page, 3. Contributions clés: the single-segment strategy keeps the
  whole reduction in one block in incremental form; the multi-segment
  strategy partitions the reduction axis and merges partial results
  (FlashDecoding is the special case).
* FLASHLIGHT page (Italian), Metodologia, item 3: the online form keeps a
  running max and a running sum and rescales the sum whenever the max
  changes, via e^{x-y} = e^x / e^y.
* STOF page (French), Résumé technique: causal / sliding-window / random
  block masks, with masked tiles skipped instead of computed and reset.
* RedFuser page, 1. Problématique: normalisation layers are cascaded
  reductions too (the mean, then the squared deviations from it); the Korean
  page reports variance as one of its workloads.

Readings where the pages are silent (each also listed in the design notes):

* causal masking is bottom-right aligned: key j is visible to query i iff
  j <= i + (Lk - Lq);
* the block mask has 64 x 64 tiles and is broadcast over batch and heads;
* a query row with no visible key yields O = 0 and LSE = -inf (the identity
  of the merge monoid);
* LSE uses the natural logarithm; scores are s = scale * (q . k) before the max;
* a split-KV decode splits Lk into contiguous chunks of ceil(Lk / S) keys.

Pins: every function here is checked in ``tests/test_oracle.py`` against
closed forms, invariants, SciPy, and pure-Python brute force on tiny inputs.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# number formats (oracle-side, independent of the device code)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bit patterns (uint16) to float64 exactly.

    A bfloat16 is the upper 16 bits of an IEEE binary32, so shifting the bits
    into the top half of a 32-bit word reconstructs the value exactly.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values directly to the nearest bfloat16 (ties to even), as float64.

    Used only to report the output-quantisation floor max|bf16(O) - O|: a
    bf16 output cannot be closer to the exact result than this. bfloat16
    keeps 8 significant bits and the binary32 exponent range.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])                     # x = f * 2**e, 0.5 <= |f| < 1
    e = np.maximum(e, -125)                     # below 2**-126 the spacing is fixed
    quantum = np.ldexp(1.0, e - 8)
    r = np.rint(x[fin] / quantum) * quantum     # rint: half to even
    r[np.abs(r) > 3.3895313892515355e38] = np.inf * np.sign(r[np.abs(r) > 3.3895313892515355e38])
    out[fin] = r
    return out


# ---------------------------------------------------------------------------
# safe softmax over rows: the three-pass cascaded reduction
# ---------------------------------------------------------------------------

def softmax_rows(x: np.ndarray) -> np.ndarray:
    """y = exp(x - max) / sum(exp(x - max)) along the last axis, in three passes.

    Pass 1 (first reduction): m = max_j x_j.
    Pass 2 (second reduction, depends on m): l = sum_j exp(x_j - m).
    Pass 3 (elementwise, depends on m and l): y_j = exp(x_j - m) / l.
    A row that is entirely -inf has no defined softmax and yields NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    l = np.sum(np.exp(x - m), axis=-1, keepdims=True)
    return np.exp(x - m) / l


def logsumexp_rows(x: np.ndarray) -> np.ndarray:
    """ln sum_j exp(x_j) along the last axis, via the same max-shifted passes."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        safe = np.where(np.isfinite(m), m, 0.0)
        l = np.sum(np.exp(x - safe[..., None]), axis=-1)
        return np.where(np.isfinite(m), safe + np.log(l), m)


# ---------------------------------------------------------------------------
# layer normalisation of rows: a cascade of two reductions, then a normalise
# ---------------------------------------------------------------------------

def layernorm_rows(x: np.ndarray, gamma=None, beta=None, eps: float = 1e-5):
    """Row-wise layer normalisation in fp64, three passes.

    RedFuser page, 1. Problématique (normalisation layers are cascaded
    reductions) and the Korean page's results (variance as a workload): the
    mean is one reduction, the sum of squared deviations from it a second
    that depends on the first, and the output a normalisation by both.

      pass 1: mean_r = (1/n) sum_j x_rj
      pass 2: var_r  = (1/n) sum_j (x_rj - mean_r)^2       (population variance)
      pass 3: y_rj   = (x_rj - mean_r) / sqrt(var_r + eps) * gamma_j + beta_j

    gamma, beta: [cols] or None (1 and 0). Returns (y, mean, rstd) with
    rstd_r = 1 / sqrt(var_r + eps).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    mean = x.sum(axis=-1) / n                                   # pass 1
    dev = x - mean[..., None]
    var = (dev * dev).sum(axis=-1) / n                          # pass 2
    rstd = 1.0 / np.sqrt(var + eps)
    y = dev * rstd[..., None]                                   # pass 3
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        y = y + np.asarray(beta, dtype=np.float64)
    return y, mean, rstd


# ---------------------------------------------------------------------------
# attention: scores, the masked safe softmax, then the P·V GEMM
# ---------------------------------------------------------------------------

def element_mask(Lq: int, Lk: int, causal: bool, block_mask=None, tile: int = 64,
                 q_rows=None, tile_bits=None) -> np.ndarray:
    """Boolean [rows, Lk]: which keys each query row may attend to.

    visible(i, j) = (not causal or j <= i + Lk - Lq)
                    and (block_mask is None or block_mask[i // tile, j // tile] != 0)

    With ``tile_bits`` (uint64 [n_row_tiles, n_col_tiles, 64]; STOF page,
    Méthodologie 1, two-level storage format: "full" and "partial" outer tiles,
    64-bit element bitmaps inside the partial ones) the kind block_mask[I, J]
    decides: 1 = full tile, 0 = empty, any other value = partial, where row i
    sees key j iff bit (j mod 64) of word tile_bits[I, J, i mod 64] is set (the
    64 words of a tile are its rows; the page groups the same 4096 bits by 8x8
    blocks).
    """
    i = np.arange(Lq) if q_rows is None else np.asarray(q_rows)
    i = i[:, None]
    j = np.arange(Lk)[None, :]
    vis = np.ones((i.shape[0], Lk), dtype=bool)
    if causal:
        vis &= j <= i + (Lk - Lq)
    if block_mask is not None:
        bm = np.asarray(block_mask)
        kind = bm[i // tile, j // tile]
        if tile_bits is None:
            vis &= kind != 0
        else:
            words = np.asarray(tile_bits, dtype=np.uint64)[i // tile, j // tile, i % tile]
            bit = (words >> (j % tile).astype(np.uint64)) & np.uint64(1)
            vis &= (kind == 1) | ((kind != 0) & (bit == 1))
    return vis


def _attention_head(q, k, v, scale, visible):
    """One head: S = scale Q K^T, masked; three-pass softmax on rows; O = P V."""
    S = scale * (q @ k.T)                                  # explicit GEMM in fp64
    S = np.where(visible, S, NEG_INF)
    m = S.max(axis=1) if S.shape[1] else np.full(S.shape[0], NEG_INF)   # pass 1
    has_key = np.isfinite(m)
    m_safe = np.where(has_key, m, 0.0)
    E = np.exp(S - m_safe[:, None])                       # exp(-inf) = 0 where masked
    l = E.sum(axis=1)                                      # pass 2
    l_safe = np.where(has_key, l, 1.0)
    P = E / l_safe[:, None]                                # pass 3
    O = P @ v                                              # explicit GEMM in fp64
    O[~has_key] = 0.0
    lse = np.where(has_key, m_safe + np.log(l_safe), NEG_INF)
    return O, lse


def attention(q, k, v, scale: float, causal: bool = False, block_mask=None,
              tile: int = 64, q_rows=None, tile_bits=None):
    """Multi-head attention with the masked safe softmax, in fp64.

    q: [B, H, Lq, d]; k, v: [B, H, Lk, d] (any real dtype; widened to fp64).
    Returns (O [B, H, rows, d], LSE [B, H, rows]); rows = Lq, or the selected
    global query rows ``q_rows`` (the mask uses their global indices).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    rows = np.arange(Lq) if q_rows is None else np.asarray(q_rows)
    vis = element_mask(Lq, Lk, causal, block_mask, tile, rows, tile_bits)
    O = np.zeros((B, H, len(rows), v.shape[3]))
    LSE = np.full((B, H, len(rows)), NEG_INF)
    for b in range(B):
        for h in range(H):
            O[b, h], LSE[b, h] = _attention_head(q[b, h, rows], k[b, h], v[b, h], scale, vis)
    return O, LSE


def attention_score_mod(q, k, v, scale: float, causal: bool = False, block_mask=None, window: int = 0,
                        alibi_slopes=None, softcap: float = 0.0, q_rows=None):
    """Attention with score modifications, in fp64: the FlexAttention variants
    the FLASHLIGHT page benchmarks (Risultati: ALiBi, Softcap, Causal, Sliding
    Window; the Softcap attention of LLaMa-3.2-1B under vLLM).

    q: [B, H, Lq, d]; k, v: [B, H, Lk, d]. For head h, query row i at position
    p_i = i + Lk - Lq (bottom-right, as the causal rule) and key j:
      s = scale * (q_i . k_j)
      softcap > 0     : s <- softcap * tanh(s / softcap)
      alibi_slopes [H]: s <- s + slope_h * (j - p_i)
      visible(i, j)   = element_mask(...)  and  (window == 0  or  j > p_i - window)
    then the masked softmax in three passes and O = P V, LSE = m + ln l; a row
    with no visible key gives O = 0, LSE = -inf. Returns (O, LSE) for the rows
    q_rows (all rows by default).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    rows = np.arange(Lq) if q_rows is None else np.asarray(q_rows)
    pos = rows[:, None] + (Lk - Lq)                        # query positions
    j = np.arange(Lk)[None, :]
    vis = element_mask(Lq, Lk, causal, block_mask, q_rows=rows)
    if window:
        vis &= j > pos - window
    O = np.zeros((B, H, len(rows), v.shape[3]))
    LSE = np.full((B, H, len(rows)), NEG_INF)
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h, rows] @ k[b, h].T)         # explicit GEMM
            if softcap > 0:
                S = softcap * np.tanh(S / softcap)
            if alibi_slopes is not None:
                S = S + float(alibi_slopes[h]) * (j - pos)
            S = np.where(vis, S, NEG_INF)
            m = S.max(axis=1) if Lk else np.full(len(rows), NEG_INF)    # pass 1
            live = np.isfinite(m)
            m0 = np.where(live, m, 0.0)
            E = np.exp(S - m0[:, None])
            l = E.sum(axis=1)                                  # pass 2
            l1 = np.where(live, l, 1.0)
            O[b, h] = np.where(live[:, None], (E / l1[:, None]) @ v[b, h], 0.0)   # pass 3, P V
            LSE[b, h] = np.where(live, m0 + np.log(l1), NEG_INF)
    return O, LSE


def moe_route(logits, k: int, renorm: bool):
    """Mixture-of-experts routing, in fp64: the softmax over each token's expert
    logits, then its k largest probabilities (RedFuser page, 1. Problématique:
    MoE routing as a cascaded reduction; 4. Résultats Expérimentaux).

    logits: [T, E]. The softmax is monotone, so the selected experts are the k
    largest logits, taken largest first, equal logits by lower expert index (a
    stable sort of the exact inputs: no rounding decides the choice). Weights:
      p_e = exp(x_e - m) / sum_j exp(x_j - m)           (three passes)
      w_r = p_{idx_r}, or p_{idx_r} / sum_{r'} p_{idx_r'} with renorm.
    Returns (idx int32 [T, k], w float64 [T, k]).
    """
    x = np.asarray(logits, dtype=np.float64)
    idx = np.argsort(-x, axis=-1, kind="stable")[:, :k].astype(np.int32)
    p = softmax_rows(x)
    w = np.take_along_axis(p, idx, axis=-1)
    if renorm:
        w = w / w.sum(axis=-1, keepdims=True)
    return idx, w


def decode_gqa(q, k, v, scale: float):
    """Decode with grouped queries, in fp64: one token per query head, and
    query heads that share key/value heads (RedFuser page, 4. Résultats
    Expérimentaux: the MHA and MLA workloads).

    q: [B, Hq, d]; k, v: [B, Hkv, Lk, d] with Hq = G * Hkv. Query head hq reads
    key/value head hq // G (G consecutive query heads per key/value head; Hkv = 1
    is the MLA sharing pattern). Per query head, unmasked:
      s_j = scale * (q . k_j);  m = max_j s_j;  l = sum_j exp(s_j - m);
      o = sum_j exp(s_j - m) v_j / l;  lse = m + ln l.
    Lk = 0 gives o = 0 and lse = -inf. Returns (o [B, Hq, d], lse [B, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    o = np.zeros((B, Hq, v.shape[3]))
    lse = np.full((B, Hq), NEG_INF)
    if Lk == 0:
        return o, lse
    for b in range(B):
        for hq in range(Hq):
            kh, vh = k[b, hq // G], v[b, hq // G]
            s_ = scale * (kh @ q[b, hq])                  # scores, one per key
            m = s_.max()                                   # pass 1
            e = np.exp(s_ - m)
            l = e.sum()                                    # pass 2
            o[b, hq] = (e @ vh) / l                        # pass 3 and the P.V product
            lse[b, hq] = m + np.log(l)
    return o, lse


# ---------------------------------------------------------------------------
# multi-segment split and the log-sum-exp merge
# ---------------------------------------------------------------------------

def split_ranges(Lk: int, num_splits: int):
    """Contiguous chunks of ceil(Lk / S) keys; trailing chunks may be short or empty."""
    chunk = -(-Lk // num_splits) if Lk > 0 else 0
    return [(min(Lk, s * chunk), min(Lk, (s + 1) * chunk)) for s in range(num_splits)]


def decode_splitkv_partials(q, k, v, scale: float, num_splits: int):
    """Per chunk s: the normalised partial output O_s and its lse_s (chunk attention).

    q: [B, H, 1, d]; k, v: [B, H, Lk, d]. Returns O_parts [B, H, S, d] and
    lse_parts [B, H, S]; an empty chunk gives (0, -inf).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, _, d = q.shape
    Lk = k.shape[2]
    o_parts = np.zeros((B, H, num_splits, v.shape[3]))
    lse_parts = np.full((B, H, num_splits), NEG_INF)
    for s, (lo, hi) in enumerate(split_ranges(Lk, num_splits)):
        if hi > lo:
            o, lse = attention(q, k[:, :, lo:hi], v[:, :, lo:hi], scale)
            o_parts[:, :, s] = o[:, :, 0]
            lse_parts[:, :, s] = lse[:, :, 0]
    return o_parts, lse_parts


def lse_merge(o_parts, lse_parts):
    """Merge normalised partials: M = max lse_s, w_s = exp(lse_s - M), W = sum w_s,
    O = sum_s w_s O_s / W, LSE = M + ln W. All-empty input gives (0, -inf).

    o_parts: [..., S, d]; lse_parts: [..., S]. A part with lse_s = -inf has
    weight exactly zero and its O_s is never read (it may hold anything).
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=-1)
    has = np.isfinite(M)
    M_safe = np.where(has, M, 0.0)
    live = np.isfinite(lse_parts)
    with np.errstate(invalid="ignore"):
        shifted = np.where(live, lse_parts - M_safe[..., None], NEG_INF)
    w = np.exp(shifted)                      # exactly 0 for parts with lse = -inf
    W = w.sum(axis=-1)
    contrib = np.where(live[..., None], w[..., None] * np.where(live[..., None], o_parts, 0.0), 0.0)
    W_safe = np.where(has, W, 1.0)
    O = contrib.sum(axis=-2) / W_safe[..., None]
    O = np.where(has[..., None], O, 0.0)
    LSE = np.where(has, M_safe + np.log(W_safe), NEG_INF)
    return O, LSE


# ---------------------------------------------------------------------------
# the incremental (online) form — used only to pin "online == three-pass"
# ---------------------------------------------------------------------------

def online_softmax_stats(x_row: np.ndarray, tile: int):
    """Walk one row in tiles keeping (m, l): m' = max(m, max tile),
    l <- l * exp(m - m') + sum exp(x - m'). Returns the final (m, l)."""
    x_row = np.asarray(x_row, dtype=np.float64)
    m, l = NEG_INF, 0.0
    for lo in range(0, len(x_row), tile):
        blk = x_row[lo:lo + tile]
        m_new = max(m, float(blk.max()))
        if m_new == NEG_INF:
            continue
        alpha = 1.0 if m == NEG_INF else math.exp(m - m_new)
        l = l * alpha + float(np.exp(blk - m_new).sum())
        m = m_new
    return m, l


def online_attention(q_row, k, v, scale: float, tile: int, visible=None):
    """One query row, keys walked in tiles with the running (m, l, acc) rescale.

    For each tile: m' = max(m, max_j s_j); alpha = exp(m - m') (1 while m = -inf);
    l <- alpha l + sum_j exp(s_j - m'); acc <- alpha acc + sum_j exp(s_j - m') v_j.
    Finally O = acc / l and LSE = m + ln l (O = 0, LSE = -inf with no key).
    """
    q_row = np.asarray(q_row, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lk = k.shape[0]
    vis = np.ones(Lk, bool) if visible is None else np.asarray(visible, bool)
    m, l = NEG_INF, 0.0
    acc = np.zeros(v.shape[1])
    for lo in range(0, Lk, tile):
        hi = min(Lk, lo + tile)
        s = scale * (k[lo:hi] @ q_row)
        s = np.where(vis[lo:hi], s, NEG_INF)
        m_new = max(m, float(s.max()))
        if m_new == NEG_INF:
            continue
        alpha = 1.0 if m == NEG_INF else math.exp(m - m_new)
        p = np.exp(s - m_new)
        l = alpha * l + float(p.sum())
        acc = alpha * acc + p @ v[lo:hi]
        m = m_new
    if m == NEG_INF:
        return np.zeros(v.shape[1]), NEG_INF
    return acc / l, m + math.log(l)
