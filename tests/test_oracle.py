"""Pins for the fp64 oracle: closed forms, invariants, library cross-checks and
pure-Python brute force, plus planted mistakes that each pin must catch.

Nothing here needs a GPU. The pins are chosen so that a plausible slip
anywhere in the oracle (a dropped term, a wrong sign or index, a transposed
operand, a missing normalisation) fails at least one of them; the ``mutant``
tests plant exactly such slips in copies of the oracle and assert that.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle as O
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
NEG_INF = -math.inf


def _golden():
    with open(os.path.join(HERE, "golden", "closed_forms.json")) as f:
        g = json.load(f)

    def conv(v):
        if isinstance(v, list):
            return [conv(x) for x in v]
        if v == "-inf":
            return NEG_INF
        return v
    return {k: [{kk: conv(vv) for kk, vv in case.items()} for case in cases]
            for k, cases in g.items() if not k.startswith("_")}


GOLD = _golden()


# ---------------------------------------------------------------------------
# pin predicates: each takes an implementation and says whether it holds
# ---------------------------------------------------------------------------

def pin_softmax_sums_to_one(softmax_fn):
    r = np.random.default_rng(11)
    x = r.normal(0, 3, size=(16, 1000)) + r.uniform(-50, 50, size=(16, 1))
    y = softmax_fn(x)
    return bool(np.all(np.isfinite(y)) and np.max(np.abs(y.sum(-1) - 1)) < 1e-13)


def pin_softmax_shift_invariance(softmax_fn):
    r = np.random.default_rng(12)
    x = r.normal(0, 2, size=(8, 257))
    base = softmax_fn(x)
    for c in (50.0, -50.0, 1000.0, -1000.0):
        y = softmax_fn(x + c)
        if not np.all(np.isfinite(y)) or np.max(np.abs(y - base)) > 1e-12:
            return False
    return True


def pin_softmax_golden(softmax_fn):
    return all(np.allclose(softmax_fn(np.array([c["x"]]))[0], c["y"], rtol=0, atol=1e-15)
               for c in GOLD["softmax"])


def _vis_fn(Lq, Lk, causal, bm, tile):
    def visible(i, j):
        ok = True
        if causal:
            ok = ok and (j <= i + (Lk - Lq))   # bottom-right aligned causal reading
        if bm is not None:
            ok = ok and bm[i // tile][j // tile] != 0
        return ok
    return visible


def brute_attention(q, k, v, scale, visible):
    """Pure-Python loops with math.exp / math.fsum; no NumPy arithmetic."""
    Lq, d = len(q), len(q[0])
    Lk, dv = len(k), len(v[0])
    out, lses = [], []
    for i in range(Lq):
        keys = [j for j in range(Lk) if visible(i, j)]
        if not keys:
            out.append([0.0] * dv)
            lses.append(NEG_INF)
            continue
        s = {j: scale * math.fsum(q[i][e] * k[j][e] for e in range(d)) for j in keys}
        mx = max(s.values())
        ex = {j: math.exp(s[j] - mx) for j in keys}
        den = math.fsum(ex.values())
        out.append([math.fsum(ex[j] * v[j][e] for j in keys) / den for e in range(dv)])
        lses.append(mx + math.log(den))
    return out, lses


BRUTE_CASES = [
    # (Lq, Lk, d, dv, causal, block mask (tile 2) or None, scale)
    (4, 4, 4, 4, False, None, 0.5),
    (4, 4, 4, 4, True, None, 0.5),
    (3, 5, 4, 2, True, None, 0.7),                      # Lq != Lk: bottom-right alignment
    (4, 4, 4, 4, False, [[1, 0], [1, 1]], 0.5),
    (4, 6, 3, 4, True, [[0, 1, 1], [1, 0, 1]], 1.3),
    (4, 4, 4, 4, True, [[0, 0], [1, 1]], 0.5),          # rows 0-1 have no visible key
    (1, 7, 4, 4, True, None, 0.5),                      # decode-shaped
]


def pin_attention_bruteforce(attn_fn):
    r = np.random.default_rng(13)
    for (Lq, Lk, d, dv, causal, bm, scale) in BRUTE_CASES:
        q = r.normal(size=(1, 1, Lq, d))
        k = r.normal(size=(1, 1, Lk, d))
        v = r.normal(size=(1, 1, Lk, dv))
        bmm = None if bm is None else np.array(bm, dtype=np.uint8)
        o, lse = attn_fn(q, k, v, scale, causal, bmm, 2)
        bo, blse = brute_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), scale,
                                   _vis_fn(Lq, Lk, causal, bm, 2))
        if not np.allclose(o[0, 0], np.array(bo), rtol=0, atol=1e-13):
            return False
        bl = np.array(blse)
        fin = np.isfinite(bl)
        if not np.array_equal(fin, np.isfinite(lse[0, 0])):
            return False
        if not np.allclose(lse[0, 0][fin], bl[fin], rtol=0, atol=1e-13):
            return False
        if np.any(lse[0, 0][~fin] != NEG_INF):
            return False
    return True


def pin_attention_uniform_query(attn_fn):
    """q = 0: every visible key gets the same weight, so O is the mean of the
    visible V rows and LSE = ln(number of visible keys)."""
    r = np.random.default_rng(14)
    for (Lq, Lk, causal) in [(6, 6, True), (3, 9, True), (5, 5, False)]:
        q = np.zeros((1, 1, Lq, 8))
        k = r.normal(size=(1, 1, Lk, 8))
        v = r.normal(size=(1, 1, Lk, 3))
        o, lse = attn_fn(q, k, v, 0.3, causal, None, 64)
        for i in range(Lq):
            n = (i + 1 + Lk - Lq) if causal else Lk
            if abs(lse[0, 0, i] - math.log(n)) > 1e-13:
                return False
            if not np.allclose(o[0, 0, i], v[0, 0, :n].mean(0), rtol=0, atol=1e-13):
                return False
    return True


def pin_attention_identity_values(attn_fn):
    """V = I (Lk = d): O is the softmax matrix itself; compare with SciPy."""
    r = np.random.default_rng(15)
    q = r.normal(size=(2, 2, 5, 6))
    k = r.normal(size=(2, 2, 6, 6))
    v = np.broadcast_to(np.eye(6), (2, 2, 6, 6)).copy()
    o, lse = attn_fn(q, k, v, 0.4, False, None, 64)
    s = 0.4 * np.einsum("bhqd,bhkd->bhqk", q, k)
    return bool(np.allclose(o, scipy.special.softmax(s, axis=-1), rtol=0, atol=1e-14)
                and np.allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=0, atol=1e-13))


def pin_attention_single_key(attn_fn):
    """Lk = 1: O = v_0 and LSE = s_00, exactly; causal row 0 of a square problem likewise."""
    r = np.random.default_rng(16)
    q = r.normal(size=(1, 1, 3, 4))
    k = r.normal(size=(1, 1, 1, 4))
    v = r.normal(size=(1, 1, 1, 4))
    o, lse = attn_fn(q, k, v, 0.9, False, None, 64)
    if not np.array_equal(o[0, 0], np.repeat(v[0, 0], 3, axis=0)):
        return False
    if not np.allclose(lse[0, 0], 0.9 * (q[0, 0] @ k[0, 0, 0]), rtol=0, atol=1e-15):
        return False
    k2 = r.normal(size=(1, 1, 3, 4))
    v2 = r.normal(size=(1, 1, 3, 4))
    o2, lse2 = attn_fn(q, k2, v2, 0.9, True, None, 64)
    return bool(np.array_equal(o2[0, 0, 0], v2[0, 0, 0])
                and abs(lse2[0, 0, 0] - 0.9 * q[0, 0, 0] @ k2[0, 0, 0]) < 1e-15)


def pin_attention_key_permutation(attn_fn):
    """Without a mask, permuting keys together with their values changes nothing."""
    r = np.random.default_rng(17)
    q = r.normal(size=(1, 2, 4, 5))
    k = r.normal(size=(1, 2, 9, 5))
    v = r.normal(size=(1, 2, 9, 3))
    perm = r.permutation(9)
    o1, l1 = attn_fn(q, k, v, 0.6, False, None, 64)
    o2, l2 = attn_fn(q, k[:, :, perm], v[:, :, perm], 0.6, False, None, 64)
    return bool(np.allclose(o1, o2, rtol=0, atol=1e-14) and np.allclose(l1, l2, rtol=0, atol=1e-14))


def pin_merge_golden(merge_fn):
    for c in GOLD["lse_merge"]:
        o, lse = merge_fn(np.array(c["o_parts"]), np.array(c["lse_parts"]))
        if not np.allclose(o, c["o"], rtol=0, atol=1e-15):
            return False
        if c["lse"] == NEG_INF:
            if lse != NEG_INF:
                return False
        elif abs(lse - c["lse"]) > 1e-15:
            return False
    return True


def pin_merge_monoid(merge_fn):
    """Associativity, commutativity, identity, at lse magnitudes where exp overflows."""
    r = np.random.default_rng(18)
    for offset in (0.0, 800.0, -800.0):
        parts = [(r.normal(size=4), r.normal() * 5 + offset) for _ in range(3)]

        def m2(a, b):
            o, l = merge_fn(np.stack([a[0], b[0]]), np.array([a[1], b[1]]))
            return (o, float(l))
        ab_c = m2(m2(parts[0], parts[1]), parts[2])
        a_bc = m2(parts[0], m2(parts[1], parts[2]))
        flat = merge_fn(np.stack([p[0] for p in parts]), np.array([p[1] for p in parts]))
        ba = m2(parts[1], parts[0])
        ab = m2(parts[0], parts[1])
        ident = m2(parts[0], (np.full(4, np.nan), NEG_INF))
        for x, y in ((ab_c, a_bc), (ab_c, (flat[0], float(flat[1]))), (ab, ba), (ident, parts[0])):
            if not (np.all(np.isfinite(x[0])) and np.allclose(x[0], y[0], rtol=0, atol=1e-13)
                    and abs(x[1] - y[1]) <= 1e-13 * max(1.0, abs(y[1]))):
                return False
    return True


def pin_split_merge_equals_unsplit(partials_fn, merge_fn, attn_fn):
    """The multi-segment strategy: split the keys, attend per chunk, merge == unsplit."""
    r = np.random.default_rng(19)
    for (Lk, S) in [(37, 4), (5, 8), (64, 1), (100, 7)]:      # includes empty chunks
        q = r.normal(size=(2, 3, 1, 8))
        k = r.normal(size=(2, 3, Lk, 8))
        v = r.normal(size=(2, 3, Lk, 6))
        op, lp = partials_fn(q, k, v, 0.35, S)
        o, lse = merge_fn(op, lp)
        ref_o, ref_lse = attn_fn(q, k, v, 0.35, False, None, 64)
        if not (np.allclose(o, ref_o[:, :, 0], rtol=0, atol=1e-13)
                and np.allclose(lse, ref_lse[:, :, 0], rtol=0, atol=1e-12)):
            return False
    return True


# ---------------------------------------------------------------------------
# the oracle satisfies every pin
# ---------------------------------------------------------------------------

def _oracle_attn(q, k, v, scale, causal, bm, tile):
    return O.attention(q, k, v, scale, causal, bm, tile)


def test_softmax_pins():
    assert pin_softmax_sums_to_one(O.softmax_rows)
    assert pin_softmax_shift_invariance(O.softmax_rows)
    assert pin_softmax_golden(O.softmax_rows)


def test_softmax_naive_form_overflows():
    """The +1000 shift pin has teeth: the unshifted exp overflows even in fp64."""
    x = np.array([[1000.0, 999.0, 998.0]])
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(x) / np.exp(x).sum(-1, keepdims=True)
    assert np.isnan(naive).all()
    assert np.allclose(O.softmax_rows(x), scipy.special.softmax(x, axis=-1), rtol=0, atol=1e-15)


def test_softmax_vs_scipy_on_workload_rows():
    x = W.softmax_rows_input(2, 6, 32768)
    ref = scipy.special.softmax(x.astype(np.float64), axis=-1)
    assert np.max(np.abs(O.softmax_rows(x) - ref)) < 1e-14


def test_logsumexp_golden_and_scipy():
    for c in GOLD["logsumexp"]:
        assert abs(O.logsumexp_rows(np.array(c["x"])) - c["lse"]) < 1e-13
    r = np.random.default_rng(3)
    x = r.normal(0, 10, size=(5, 77))
    assert np.allclose(O.logsumexp_rows(x), scipy.special.logsumexp(x, axis=-1), rtol=0, atol=1e-12)
    assert O.logsumexp_rows(np.array([NEG_INF, NEG_INF])) == NEG_INF


@pytest.mark.parametrize("tile", [1, 7, 64, 1000, 5000])
def test_online_stats_equal_three_pass(tile):
    r = np.random.default_rng(tile)
    x = r.normal(0, 2, 1000) + r.uniform(-50, 50)
    # make the running max change in almost every tile (monotone ramp)
    x[::3] += np.linspace(0, 30, len(x[::3]))
    m, l = O.online_softmax_stats(x, tile)
    assert m == x.max()
    ref_l = np.exp(x - x.max()).sum()
    assert abs(l - ref_l) <= 1e-12 * ref_l


@pytest.mark.parametrize("tile", [1, 7, 64, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_online_attention_equals_three_pass(tile, causal):
    r = np.random.default_rng(100 + tile)
    Lq, Lk, d = 5, 300, 16
    q = r.normal(size=(1, 1, Lq, d))
    k = r.normal(size=(1, 1, Lk, d)) + np.linspace(0, 3, Lk)[:, None]   # rising scores
    v = r.normal(size=(1, 1, Lk, 8))
    bm = (r.uniform(size=(1, 5)) < 0.6).astype(np.uint8)
    bm[0, 0] = 1
    ref_o, ref_lse = O.attention(q, k, v, 0.25, causal, bm, 64)
    vis = O.element_mask(Lq, Lk, causal, bm, 64)
    for i in range(Lq):
        o, lse = O.online_attention(q[0, 0, i], k[0, 0], v[0, 0], 0.25, tile, vis[i])
        assert np.allclose(o, ref_o[0, 0, i], rtol=1e-12, atol=1e-13)
        assert abs(lse - ref_lse[0, 0, i]) <= 1e-12 * max(1, abs(lse))


def test_attention_pins():
    assert pin_attention_bruteforce(_oracle_attn)
    assert pin_attention_uniform_query(_oracle_attn)
    assert pin_attention_identity_values(_oracle_attn)
    assert pin_attention_single_key(_oracle_attn)
    assert pin_attention_key_permutation(_oracle_attn)


def test_fully_masked_rows_and_empty_keys():
    r = np.random.default_rng(4)
    q = r.normal(size=(1, 1, 4, 4))
    k = r.normal(size=(1, 1, 4, 4))
    v = r.normal(size=(1, 1, 4, 4))
    bm = np.array([[0]], dtype=np.uint8)
    o, lse = O.attention(q, k, v, 0.5, False, bm, 64)
    assert np.array_equal(o, np.zeros_like(o)) and np.all(lse == NEG_INF)
    o, lse = O.attention(q, k[:, :, :0], v[:, :, :0], 0.5, False)
    assert np.array_equal(o, np.zeros((1, 1, 4, 4))) and np.all(lse == NEG_INF)


def test_causal_single_query_sees_every_key():
    """Bottom-right alignment: a one-row query attends its whole key range."""
    r = np.random.default_rng(5)
    q = r.normal(size=(2, 2, 1, 8))
    k = r.normal(size=(2, 2, 50, 8))
    v = r.normal(size=(2, 2, 50, 8))
    a = O.attention(q, k, v, 0.3, True)
    b = O.attention(q, k, v, 0.3, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_q_rows_subset_matches_full():
    r = np.random.default_rng(6)
    q = r.normal(size=(1, 2, 130, 8))
    k = r.normal(size=(1, 2, 140, 8))
    v = r.normal(size=(1, 2, 140, 8))
    bm = (r.uniform(size=(3, 3)) < 0.5).astype(np.uint8)
    full = O.attention(q, k, v, 0.3, True, bm)
    rows = [0, 63, 64, 129]
    sub = O.attention(q, k, v, 0.3, True, bm, q_rows=rows)
    assert np.array_equal(sub[0], full[0][:, :, rows]) and np.array_equal(sub[1], full[1][:, :, rows])


def test_merge_pins():
    assert pin_merge_golden(O.lse_merge)
    assert pin_merge_monoid(O.lse_merge)
    assert pin_split_merge_equals_unsplit(O.decode_splitkv_partials, O.lse_merge, _oracle_attn)


def test_split_ranges():
    assert O.split_ranges(32768, 16) == [(2048 * s, 2048 * (s + 1)) for s in range(16)]
    assert O.split_ranges(5, 8) == [(0, 1), (1, 2), (2, 3), (3, 4), (4, 5), (5, 5), (5, 5), (5, 5)]
    assert O.split_ranges(0, 3) == [(0, 0)] * 3


def test_bf16_widening_known_bits():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x4049, 0x0000, 0x8000], dtype=np.uint16)
    want = [1.0, -2.0, math.inf, -math.inf, 2.0 ** -133, 3.140625, 0.0, -0.0]
    got = O.bf16_bits_to_f64(bits)
    assert all(g == w for g, w in zip(got.tolist(), want))
    assert math.copysign(1, got[-1]) == -1


def test_bf16_rounding_ties_and_cross_check():
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.0, 1 + 2 ** -8 + 2 ** -30])
    assert O.round_to_bf16(x).tolist() == [1.0, 1 + 2 ** -6, -1.0, 3.0, 1 + 2 ** -7]
    # two independent implementations agree on float32-representable values
    r = np.random.default_rng(7)
    f = (r.normal(size=20000) * np.exp2(r.integers(-20, 20, 20000))).astype(np.float32)
    via_bits = O.bf16_bits_to_f64(W.f32_to_bf16_bits(f))
    assert np.array_equal(via_bits, O.round_to_bf16(f.astype(np.float64)))


def test_workload_generators_are_pure_functions_of_the_seed():
    a = W.normal_head(3, W.TID_Q, 1, 2, 16, 8, "bf16")
    b = W.normal_head(3, W.TID_Q, 1, 2, 16, 8, "bf16")
    c = W.normal_head(3, W.TID_Q, 1, 3, 16, 8, "bf16")
    assert a.dtype == np.uint16 and np.array_equal(a, b) and not np.array_equal(a, c)
    t = W.normal_tensor(3, W.TID_Q, 2, 3, 16, 8, "bf16")
    assert np.array_equal(t[1, 2], a)
    x = W.softmax_rows_input(2, 3, 100, row_ids=[5, 9, 5])
    assert np.array_equal(x[0], x[2]) and np.array_equal(x[0], W.softmax_row(2, 5, 100))


def test_config5_mask_counts():
    m = W.config_block_mask("sparse")
    assert m.shape == (128, 128)
    window = sum(min(i + 1, 8) for i in range(128))
    assert window == 996
    assert int(m.sum()) == 996 + 726
    assert np.all(np.triu(m, 1) == 0)                    # nothing above the diagonal
    assert np.all(np.diag(m) == 1)


# ---------------------------------------------------------------------------
# planted mistakes: every mutant must fail at least one pin
# ---------------------------------------------------------------------------

def _softmax_no_shift(x):
    e = np.exp(np.asarray(x, np.float64))
    return e / e.sum(-1, keepdims=True)


def _softmax_divides_by_max(x):
    x = np.asarray(x, np.float64)
    m = x.max(-1, keepdims=True)
    return np.exp(x - m) / np.exp(x - m).max(-1, keepdims=True)


def _softmax_wrong_sign(x):
    x = np.asarray(x, np.float64)
    m = x.max(-1, keepdims=True)
    return np.exp(m - x) / np.exp(m - x).sum(-1, keepdims=True)


@pytest.mark.parametrize("mutant", [_softmax_no_shift, _softmax_divides_by_max, _softmax_wrong_sign])
def test_softmax_mutants_are_caught(mutant):
    with np.errstate(all="ignore"):
        caught = not (pin_softmax_sums_to_one(mutant) and pin_softmax_shift_invariance(mutant)
                      and pin_softmax_golden(mutant))
    assert caught


def _attn_mutant(kind):
    def fn(q, k, v, scale, causal, bm, tile):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        B, H, Lq, d = q.shape
        Lk = k.shape[2]
        i = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        vis = np.ones((Lq, Lk), bool)
        if causal:
            if kind == "causal_top_left":
                vis &= j <= i
            elif kind == "causal_flipped":
                vis &= j >= i + (Lk - Lq)
            else:
                vis &= j <= i + (Lk - Lq)
        if bm is not None:
            if kind == "mask_transposed":
                vis &= np.asarray(bm)[(j // tile) % bm.shape[0], (i // tile) % bm.shape[1]] != 0
            else:
                vis &= np.asarray(bm)[i // tile, j // tile] != 0
        Oo = np.zeros((B, H, Lq, v.shape[3]))
        L = np.full((B, H, Lq), NEG_INF)
        for b in range(B):
            for h in range(H):
                sc = 1.0 if kind == "no_scale" else scale
                if kind == "transposed_operand" and Lq == Lk:
                    S = sc * (k[b, h] @ q[b, h].T)
                else:
                    S = sc * (q[b, h] @ k[b, h].T)
                S = np.where(vis, S, NEG_INF)
                m = S.max(1)
                has = np.isfinite(m)
                ms = np.where(has, m, 0.0)
                E = np.exp(S - ms[:, None])
                l = E.sum(1)
                ls = np.where(has, l, 1.0)
                P = E if kind == "no_normalise" else E / ls[:, None]
                Oo[b, h] = P @ v[b, h]
                Oo[b, h][~has] = 0
                L[b, h] = np.where(has, (np.log(ls) if kind == "lse_no_max" else ms + np.log(ls)), NEG_INF)
        return Oo, L
    return fn


@pytest.mark.parametrize("kind", ["no_scale", "transposed_operand", "causal_top_left", "causal_flipped",
                                  "mask_transposed", "no_normalise", "lse_no_max"])
def test_attention_mutants_are_caught(kind):
    fn = _attn_mutant(kind)
    with np.errstate(all="ignore"):
        ok = (pin_attention_bruteforce(fn) and pin_attention_uniform_query(fn)
              and pin_attention_identity_values(fn) and pin_attention_single_key(fn)
              and pin_attention_key_permutation(fn))
    assert not ok
    # the same skeleton without a planted mistake passes (the mutant harness is sound)
    assert pin_attention_bruteforce(_attn_mutant("none"))


def _merge_mutant(kind):
    def fn(o_parts, lse_parts):
        o_parts = np.asarray(o_parts, np.float64)
        lse_parts = np.asarray(lse_parts, np.float64)
        M = lse_parts.max(-1)
        has = np.isfinite(M)
        Ms = np.where(has, M, 0.0)
        live = np.isfinite(lse_parts)
        if kind == "no_max_shift":
            w = np.where(live, np.exp(np.where(live, lse_parts, 0.0)), 0.0)
        else:
            w = np.where(live, np.exp(np.where(live, lse_parts, 0.0) - Ms[..., None]), 0.0)
        Wt = w.sum(-1)
        c = np.where(live[..., None], w[..., None] * np.where(live[..., None], o_parts, 0.0), 0.0).sum(-2)
        Ws = np.where(has, Wt, 1.0)
        Oo = c if kind == "no_divide" else c / Ws[..., None]
        Oo = np.where(has[..., None], Oo, 0.0)
        if kind == "lse_no_log":
            L = np.where(has, Ms + Ws, NEG_INF)
        elif kind == "no_max_shift":
            L = np.where(has, np.log(Ws), NEG_INF)
        else:
            L = np.where(has, Ms + np.log(Ws), NEG_INF)
        return Oo, L
    return fn


@pytest.mark.parametrize("kind", ["no_max_shift", "no_divide", "lse_no_log"])
def test_merge_mutants_are_caught(kind):
    fn = _merge_mutant(kind)
    with np.errstate(all="ignore"):
        ok = (pin_merge_golden(fn) and pin_merge_monoid(fn)
              and pin_split_merge_equals_unsplit(O.decode_splitkv_partials, fn, _oracle_attn))
    assert not ok
    assert pin_merge_golden(_merge_mutant("none")) and pin_merge_monoid(_merge_mutant("none"))


# ---------------------------------------------------------------------------
# element bitmaps inside partial tiles (STOF two-level format)
# ---------------------------------------------------------------------------

def _bitmap_case(seed, Lq=130, Lk=200):
    r = np.random.default_rng(seed)
    nI, nJ = -(-Lq // 64), -(-Lk // 64)
    kinds = r.choice(np.array([0, 1, 2, 7], np.uint8), size=(nI, nJ))   # 7: any other nonzero kind is partial
    bits = r.integers(0, 2 ** 63, size=(nI, nJ, 64), dtype=np.uint64) * np.uint64(2) + \
        r.integers(0, 2, size=(nI, nJ, 64), dtype=np.uint64)
    return kinds, bits


def _decode_python(Lq, Lk, causal, kinds, bits):
    """The bitmap definition written out with Python integers, element by element."""
    out = np.zeros((Lq, Lk), dtype=bool)
    for i in range(Lq):
        for j in range(Lk):
            kind = int(kinds[i // 64][j // 64])
            if kind == 0:
                vis = False
            elif kind == 1:
                vis = True
            else:
                word = int(bits[i // 64][j // 64][i % 64])
                vis = (word >> (j % 64)) & 1 == 1
            if causal and j > i + (Lk - Lq):
                vis = False
            out[i, j] = vis
    return out


def pin_bitmap_bruteforce(mask_fn):
    for seed, causal in ((21, False), (22, True)):
        kinds, bits = _bitmap_case(seed)
        if not np.array_equal(mask_fn(130, 200, causal, kinds, bits), _decode_python(130, 200, causal, kinds, bits)):
            return False
    return True


def pin_bitmap_all_ones_is_full(mask_fn):
    kinds, _ = _bitmap_case(23)
    ones = np.full(kinds.shape + (64,), np.uint64(2 ** 64 - 1))
    full = np.where(kinds != 0, 1, 0).astype(np.uint8)
    return bool(np.array_equal(mask_fn(130, 200, False, kinds, ones), mask_fn(130, 200, False, full, ones)))


def pin_bitmap_causal_diagonal(mask_fn):
    """Lower-triangular bitmaps on the diagonal tiles, full tiles below, empty above:
    without the causal flag this is exactly the causal mask."""
    n = 4
    kinds = np.tril(np.ones((n, n), np.uint8)) + np.eye(n, dtype=np.uint8)     # 1 below, 2 on the diagonal
    tri = np.array([(1 << (r + 1)) - 1 for r in range(64)], dtype=np.uint64)   # row r sees keys 0..r
    bits = np.zeros((n, n, 64), np.uint64)
    for t in range(n):
        bits[t, t] = tri
    got = mask_fn(256, 256, False, kinds, bits)
    return bool(np.array_equal(got, O.element_mask(256, 256, True)))


def pin_bitmap_single_bit(mask_fn):
    kinds = np.full((3, 3), 2, np.uint8)
    bits = np.zeros((3, 3, 64), np.uint64)
    bits[1, 2, 5] = np.uint64(1) << np.uint64(9)
    got = mask_fn(192, 192, False, kinds, bits)
    want = np.zeros((192, 192), bool)
    want[64 + 5, 128 + 9] = True
    return bool(np.array_equal(got, want))


def _oracle_mask(Lq, Lk, causal, kinds, bits):
    return O.element_mask(Lq, Lk, causal, kinds, 64, None, bits)


def test_bitmap_mask_pins():
    assert pin_bitmap_bruteforce(_oracle_mask)
    assert pin_bitmap_all_ones_is_full(_oracle_mask)
    assert pin_bitmap_causal_diagonal(_oracle_mask)
    assert pin_bitmap_single_bit(_oracle_mask)


def test_bitmap_attention_matches_python_masked_attention():
    """Attention under a bitmap mask against pure-Python loops over the
    decoded element mask (exp via math.exp, sums via math.fsum)."""
    Lq, Lk, d = 70, 90, 3
    r = np.random.default_rng(24)
    kinds, bits = _bitmap_case(25, Lq, Lk)
    kinds[0, 0] = 2
    q, k, v = r.normal(size=(1, 1, Lq, d)), r.normal(size=(1, 1, Lk, d)), r.normal(size=(1, 1, Lk, d))
    o, lse = O.attention(q, k, v, 0.4, True, kinds, tile_bits=bits)
    vis = _decode_python(Lq, Lk, True, kinds, bits)
    for i in range(Lq):
        s = [0.4 * math.fsum(q[0, 0, i, e] * k[0, 0, j, e] for e in range(d)) for j in range(Lk) if vis[i, j]]
        js = [j for j in range(Lk) if vis[i, j]]
        if not s:
            assert lse[0, 0, i] == NEG_INF and np.all(o[0, 0, i] == 0)
            continue
        m = max(s)
        w = [math.exp(x - m) for x in s]
        W_ = math.fsum(w)
        ref = [math.fsum(wi * v[0, 0, j, e] for wi, j in zip(w, js)) / W_ for e in range(d)]
        assert np.allclose(o[0, 0, i], ref, rtol=1e-12, atol=1e-13)
        assert abs(lse[0, 0, i] - (m + math.log(W_))) <= 1e-12


def _mask_mutant(kind):
    def fn(Lq, Lk, causal, kinds, bits):
        i = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        vis = np.ones((Lq, Lk), bool)
        if causal:
            vis &= j <= i + (Lk - Lq)
        kk = np.asarray(kinds)[i // 64, j // 64]
        if kind == "transposed_words":
            words = np.asarray(bits, np.uint64)[i // 64, j // 64, j % 64]
            bit = (words >> (i % 64).astype(np.uint64)) & np.uint64(1)
        elif kind == "bit_off_by_one":
            words = np.asarray(bits, np.uint64)[i // 64, j // 64, i % 64]
            bit = (words >> ((j + 1) % 64).astype(np.uint64)) & np.uint64(1)
        elif kind == "msb_first":
            words = np.asarray(bits, np.uint64)[i // 64, j // 64, i % 64]
            bit = (words >> (63 - j % 64).astype(np.uint64)) & np.uint64(1)
        else:
            words = np.asarray(bits, np.uint64)[i // 64, j // 64, i % 64]
            bit = (words >> (j % 64).astype(np.uint64)) & np.uint64(1)
        if kind == "partial_as_full":
            vis &= kk != 0
        elif kind == "only_kind_two_partial":
            vis &= (kk == 1) | ((kk == 2) & (bit == 1))
        elif kind == "full_uses_bits":
            vis &= (kk != 0) & (bit == 1)
        else:
            vis &= (kk == 1) | ((kk != 0) & (bit == 1))
        return vis
    return fn


@pytest.mark.parametrize("kind", ["transposed_words", "bit_off_by_one", "msb_first", "partial_as_full",
                                  "only_kind_two_partial", "full_uses_bits"])
def test_bitmap_mutants_are_caught(kind):
    fn = _mask_mutant(kind)
    ok = (pin_bitmap_bruteforce(fn) and pin_bitmap_all_ones_is_full(fn) and pin_bitmap_causal_diagonal(fn)
          and pin_bitmap_single_bit(fn))
    assert not ok
    none = _mask_mutant("none")
    assert pin_bitmap_bruteforce(none) and pin_bitmap_causal_diagonal(none) and pin_bitmap_single_bit(none)


def test_bitmap_workload_mask():
    """The extension workload's mask: every row sees exactly its 512-key causal
    window, plus whole random tiles strictly below the window's tile band."""
    kinds, bits = W.extension_bitmap_mask()
    n = kinds.shape[0]
    wt = 8
    n_cand = sum(max(0, I - wt) for I in range(n))
    random_tiles = int(((kinds == 1) & np.tril(np.ones((n, n), bool), k=-(wt + 1))).sum())
    assert random_tiles == round(0.10 * n_cand)
    assert int((kinds == 2).sum()) == n + (n - wt)           # diagonal tiles + the window's lower-edge tiles
    # full and empty tiles carry no bits; partial tiles have some but not all
    assert not bits[kinds != 2].any()
    part = bits[kinds == 2]
    assert np.all(part.any(axis=-1)) and not np.all(part == np.uint64(2 ** 64 - 1))
    rows = [0, 63, 64, 511, 512, 1000, 8191]
    vis = O.element_mask(8192, 8192, False, kinds, 64, rows, bits)
    for i, vr in zip(rows, vis):
        window = set(range(max(0, i - 511), i + 1))
        got = set(np.nonzero(vr)[0].tolist())
        assert window <= got
        assert all(kinds[i // 64, j // 64] == 1 and j // 64 <= i // 64 - wt - 1 for j in got - window)


# ---------------------------------------------------------------------------
# layer normalisation rows (the mean / variance cascade)
# ---------------------------------------------------------------------------

def pin_ln_bruteforce(ln):
    r = np.random.default_rng(31)
    x = r.normal(2, 3, size=(5, 37))
    g, b = r.normal(1, 0.2, 37), r.normal(0, 0.3, 37)
    y, mean, rstd = ln(x, g, b, 1e-3)
    for i in range(5):
        row = [float(t) for t in x[i]]
        m = math.fsum(row) / 37
        v = math.fsum((t - m) ** 2 for t in row) / 37
        rs = 1 / math.sqrt(v + 1e-3)
        if abs(mean[i] - m) > 1e-13 or abs(rstd[i] - rs) > 1e-12 * rs:
            return False
        if max(abs(y[i, j] - ((row[j] - m) * rs * g[j] + b[j])) for j in range(37)) > 1e-12:
            return False
    return True


def pin_ln_closed_forms(ln):
    # two elements a, b: mean (a+b)/2, variance ((a-b)/2)^2, outputs +-(a-b)/2 * rstd
    y, mean, rstd = ln(np.array([[3.0, -1.0]]), None, None, 0.0)
    if abs(mean[0] - 1.0) > 1e-15 or abs(rstd[0] - 0.5) > 1e-15 or np.max(np.abs(y - [[1.0, -1.0]])) > 1e-15:
        return False
    # a constant row has zero variance: y = beta exactly, rstd = 1/sqrt(eps)
    beta = np.arange(6.0)
    y, mean, rstd = ln(np.full((1, 6), 7.25), np.full(6, 3.0), beta, 0.25)
    return bool(mean[0] == 7.25 and rstd[0] == 2.0 and np.array_equal(y[0], beta))


def pin_ln_invariances(ln):
    r = np.random.default_rng(32)
    x = r.normal(0, 1.5, size=(8, 300))
    y0, _, _ = ln(x, None, None, 0.0)
    for c in (1000.0, -1000.0, 50.0):                       # shift invariance
        if np.max(np.abs(ln(x + c, None, None, 0.0)[0] - y0)) > 1e-9:
            return False
    if np.max(np.abs(ln(4.0 * x, None, None, 0.0)[0] - y0)) > 1e-12:   # scale invariance (eps = 0)
        return False
    # normalised rows: mean 0, mean square var / (var + eps)
    y, _, rstd = ln(x, None, None, 0.5)
    var = x.var(axis=1)
    return bool(np.max(np.abs(y.mean(1))) < 1e-13 and
                np.max(np.abs((y * y).mean(1) - var / (var + 0.5))) < 1e-12)


def pin_ln_numpy(ln):
    r = np.random.default_rng(33)
    x = r.normal(-3, 2, size=(6, 1000))
    g, b = r.normal(1, 0.1, 1000), r.normal(0, 0.1, 1000)
    y, mean, rstd = ln(x, g, b, 1e-5)
    want = (x - x.mean(1, keepdims=True)) / np.sqrt(x.var(1, keepdims=True) + 1e-5) * g + b
    return bool(np.max(np.abs(y - want)) < 1e-12 and np.max(np.abs(mean - x.mean(1))) < 1e-13)


def test_layernorm_pins():
    assert pin_ln_bruteforce(O.layernorm_rows)
    assert pin_ln_closed_forms(O.layernorm_rows)
    assert pin_ln_invariances(O.layernorm_rows)
    assert pin_ln_numpy(O.layernorm_rows)


def _ln_mutant(kind):
    def fn(x, gamma=None, beta=None, eps=1e-5):
        x = np.asarray(x, np.float64)
        n = x.shape[-1]
        mean = x.sum(-1) / n
        dev = x - mean[..., None]
        var = (dev * dev).sum(-1) / (n - 1 if kind == "sample_variance" and n > 1 else n)
        if kind == "eps_outside_sqrt":
            rstd = 1.0 / (np.sqrt(var) + eps)
        elif kind == "no_sqrt":
            rstd = 1.0 / (var + eps)
        else:
            rstd = 1.0 / np.sqrt(var + eps)
        y = (x if kind == "no_centering" else dev) * rstd[..., None]
        g = None if gamma is None else np.asarray(gamma, np.float64)
        b = None if beta is None else np.asarray(beta, np.float64)
        if kind == "gamma_beta_swapped":
            g, b = b, g
        if g is not None:
            y = y * g
        if b is not None:
            y = y + b
        return y, mean, rstd
    return fn


@pytest.mark.parametrize("kind", ["sample_variance", "eps_outside_sqrt", "no_sqrt", "no_centering",
                                  "gamma_beta_swapped"])
def test_layernorm_mutants_are_caught(kind):
    fn = _ln_mutant(kind)
    with np.errstate(all="ignore"):
        ok = pin_ln_bruteforce(fn) and pin_ln_closed_forms(fn) and pin_ln_invariances(fn) and pin_ln_numpy(fn)
    assert not ok
    none = _ln_mutant("none")
    assert pin_ln_bruteforce(none) and pin_ln_closed_forms(none) and pin_ln_invariances(none) and pin_ln_numpy(none)


# ---------------------------------------------------------------------------
# grouped-query decode (query heads sharing key/value heads)
# ---------------------------------------------------------------------------

def _gqa_inputs(seed, B, Hq, Hkv, Lk, d):
    r = np.random.default_rng(seed)
    return r.normal(size=(B, Hq, d)), r.normal(size=(B, Hkv, Lk, d)), r.normal(size=(B, Hkv, Lk, d))


def pin_gqa_bruteforce(fn):
    """Pure Python (math.exp, math.fsum) on B = 2, Hq = 6, Hkv = 2 (G = 3), Lk = 5, d = 3."""
    B, Hq, Hkv, Lk, d, sc = 2, 6, 2, 5, 3, 0.7
    q, k, v = _gqa_inputs(41, B, Hq, Hkv, Lk, d)
    o, lse = fn(q, k, v, sc)
    G = Hq // Hkv
    for b in range(B):
        for hq in range(Hq):
            j = hq // G
            s = [sc * math.fsum(float(q[b, hq, t]) * float(k[b, j, i, t]) for t in range(d)) for i in range(Lk)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            l = math.fsum(e)
            want = [math.fsum(e[i] * float(v[b, j, i, t]) for i in range(Lk)) / l for t in range(d)]
            if max(abs(o[b, hq, t] - want[t]) for t in range(d)) > 1e-13:
                return False
            if abs(lse[b, hq] - (m + math.log(l))) > 1e-13:
                return False
    return True


def pin_gqa_is_mha_with_repeated_kv(fn):
    """Equal to the (separately pinned) multi-head attention oracle at Lq = 1 with
    each key/value head repeated for its G consecutive query heads."""
    for i, (B, Hq, Hkv, Lk, d) in enumerate(((1, 8, 2, 40, 16), (2, 4, 4, 17, 8), (1, 5, 1, 33, 4))):
        q, k, v = _gqa_inputs(42 + i, B, Hq, Hkv, Lk, d)
        o, lse = fn(q, k, v, 0.3)
        G = Hq // Hkv
        ro, rl = O.attention(q[:, :, None], np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.3)
        if np.max(np.abs(o - ro[:, :, 0])) > 1e-13 or np.max(np.abs(lse - rl[:, :, 0])) > 1e-13:
            return False
    return True


def pin_gqa_closed_forms(fn):
    q, k, v = _gqa_inputs(45, 2, 6, 3, 11, 4)
    # q = 0: every key weighs the same, o = mean of the head's value rows, lse = ln Lk
    o, lse = fn(np.zeros_like(q), k, v, 1.0)
    want = np.repeat(v.mean(axis=2), 2, axis=1)
    if np.max(np.abs(o - want)) > 1e-14 or np.max(np.abs(lse - math.log(11))) > 1e-14:
        return False
    # one key: o = v_0 exactly, lse = the single score
    o, lse = fn(q, k[:, :, :1], v[:, :, :1], 0.5)
    if not np.array_equal(o, np.repeat(v[:, :, 0], 2, axis=1)):
        return False
    s0 = 0.5 * np.einsum("bhd,bhd->bh", q, np.repeat(k[:, :, 0], 2, axis=1))
    if np.max(np.abs(lse - s0)) > 1e-14:
        return False
    # no keys: (0, -inf)
    o, lse = fn(q, k[:, :, :0], v[:, :, :0], 0.5)
    return bool(np.all(o == 0) and np.all(lse == -np.inf))


def test_gqa_pins():
    assert pin_gqa_bruteforce(O.decode_gqa)
    assert pin_gqa_is_mha_with_repeated_kv(O.decode_gqa)
    assert pin_gqa_closed_forms(O.decode_gqa)


def _gqa_mutant(kind):
    def fn(q, k, v, scale):
        q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
        B, Hq, d = q.shape
        Hkv, Lk = k.shape[1], k.shape[2]
        G = Hq // Hkv
        o = np.zeros((B, Hq, v.shape[3]))
        lse = np.full((B, Hq), -np.inf)
        if Lk == 0:
            return o, lse
        for b in range(B):
            for hq in range(Hq):
                j = hq % Hkv if kind == "interleaved_heads" else hq // G
                kh = k[b, j]
                vh = kh if kind == "values_from_keys" else v[b, j]
                s_ = (1.0 if kind == "no_scale" else scale) * (kh @ q[b, hq])
                m = s_.max()
                e = np.exp(s_ - m)
                l = e.sum()
                o[b, hq] = (e @ vh) / (1.0 if kind == "unnormalised" else l)
                lse[b, hq] = (0.0 if kind == "lse_without_max" else m) + np.log(l)
        return o, lse
    return fn


@pytest.mark.parametrize("kind", ["interleaved_heads", "values_from_keys", "no_scale", "unnormalised",
                                  "lse_without_max"])
def test_gqa_mutants_are_caught(kind):
    fn = _gqa_mutant(kind)
    assert not (pin_gqa_bruteforce(fn) and pin_gqa_is_mha_with_repeated_kv(fn) and pin_gqa_closed_forms(fn))
    none = _gqa_mutant("none")
    assert pin_gqa_bruteforce(none) and pin_gqa_is_mha_with_repeated_kv(none) and pin_gqa_closed_forms(none)


# ---------------------------------------------------------------------------
# score modifications: softcap, ALiBi bias, element-level sliding window
# ---------------------------------------------------------------------------

def _mod_inputs(seed, B, H, Lq, Lk, d, qscale=1.0):
    r = np.random.default_rng(seed)
    return qscale * r.normal(size=(B, H, Lq, d)), r.normal(size=(B, H, Lk, d)), r.normal(size=(B, H, Lk, d))


def pin_mod_bruteforce(fn):
    """Pure Python (math.tanh, math.exp, math.fsum): causal with Lq < Lk, window 3,
    two ALiBi slopes and a softcap that bends the scores (|s| up to ~6 vs cap 2)."""
    B, H, Lq, Lk, d, sc, cap, W = 1, 2, 3, 6, 4, 0.9, 2.0, 3
    slopes = [0.5, 0.25]
    q, k, v = _mod_inputs(51, B, H, Lq, Lk, d, qscale=2.0)
    o, lse = fn(q, k, v, sc, causal=True, window=W, alibi_slopes=np.array(slopes), softcap=cap)
    for h in range(H):
        for i in range(Lq):
            p = i + Lk - Lq
            keys = [j for j in range(Lk) if j <= p and j > p - W]
            s = []
            for j in keys:
                x = sc * math.fsum(float(q[0, h, i, t]) * float(k[0, h, j, t]) for t in range(d))
                s.append(cap * math.tanh(x / cap) + slopes[h] * (j - p))
            m = max(s)
            e = [math.exp(x - m) for x in s]
            l = math.fsum(e)
            for t in range(d):
                want = math.fsum(e[n] * float(v[0, h, keys[n], t]) for n in range(len(keys))) / l
                if abs(o[0, h, i, t] - want) > 1e-13:
                    return False
            if abs(lse[0, h, i] - (m + math.log(l))) > 1e-13:
                return False
    return True


def pin_mod_reductions(fn):
    """No modification equals the (separately pinned) attention oracle; a huge
    softcap, zero slopes and a window covering every key change nothing; a
    window equals the same mask given as element bitmaps (the oracle's
    bitmap decoding, a separate code path)."""
    q, k, v = _mod_inputs(52, 1, 2, 70, 150, 8)
    ref = O.attention(q, k, v, 0.4, True)
    for kw in (dict(), dict(softcap=1e7), dict(alibi_slopes=np.zeros(2)), dict(window=150)):
        got = fn(q, k, v, 0.4, causal=True, **kw)
        if np.max(np.abs(got[0] - ref[0])) > 1e-9 or np.max(np.abs(got[1] - ref[1])) > 1e-9:
            return False
    W = 37
    Lq, Lk = 70, 150
    i = np.arange(Lq)[:, None] + (Lk - Lq)
    j = np.arange(Lk)[None, :]
    vis = (j <= i) & (j > i - W)
    nI, nJ = -(-Lq // 64), -(-Lk // 64)
    pad = np.zeros((nI * 64, nJ * 64), bool)
    pad[:Lq, :Lk] = vis
    tiles = pad.reshape(nI, 64, nJ, 64).transpose(0, 2, 1, 3)
    bits = (tiles.astype(np.uint64) << np.arange(64, dtype=np.uint64)).sum(axis=-1, dtype=np.uint64)
    kinds = np.full((nI, nJ), 2, np.uint8)
    ref = O.attention(q, k, v, 0.4, False, kinds, tile_bits=bits)
    got = fn(q, k, v, 0.4, causal=True, window=W)
    return bool(np.max(np.abs(got[0] - ref[0])) < 1e-12 and np.max(np.abs(got[1] - ref[1])) < 1e-12)


def pin_mod_closed_forms(fn):
    Lq = Lk = 40
    d = Lk
    # ALiBi with q = 0, causal: P_ij = e^{-a (p - j)} / sum_{t=0}^{p} e^{-a t}; with V = I, O is P itself
    a = 0.3
    q = np.zeros((1, 1, Lq, d))
    k = np.random.default_rng(53).normal(size=(1, 1, Lk, d))
    v = np.eye(Lk)[None, None]
    o, lse = fn(q, k, v, 1.0, causal=True, alibi_slopes=np.array([a]))
    for i in (0, 1, 17, Lq - 1):
        z = (1 - math.exp(-a * (i + 1))) / (1 - math.exp(-a))
        want = np.zeros(d)
        want[:i + 1] = np.exp(-a * (i - np.arange(i + 1))) / z
        if np.max(np.abs(o[0, 0, i] - want)) > 1e-14 or abs(lse[0, 0, i] - math.log(z)) > 1e-14:
            return False
    # window 1, causal: only the diagonal key, O = v_p exactly, LSE = its score
    q, k, v = _mod_inputs(54, 1, 2, 5, 9, 4)
    o, lse = fn(q, k, v, 0.7, causal=True, window=1)
    p = np.arange(5) + 4
    if not np.array_equal(o[0], v[0][:, p]):
        return False
    s = 0.7 * np.einsum("hid,hid->hi", q[0], k[0][:, p])
    if np.max(np.abs(lse[0] - s)) > 1e-14:
        return False
    # a softcap bounds every logit: |s'| < cap, so P stays within e^{2 cap} of uniform
    q, k, v = _mod_inputs(55, 1, 1, 4, 30, 8, qscale=5.0)
    cap = 0.1
    o, lse = fn(q, k, v, 1.0, softcap=cap)
    dev = np.abs(o[0, 0] - v[0, 0].mean(axis=0))
    return bool(np.all(dev <= (math.exp(2 * cap) - 1) * np.abs(v).max()) and
                np.all(np.abs(lse - math.log(30)) <= cap))


def test_score_mod_pins():
    assert pin_mod_bruteforce(O.attention_score_mod)
    assert pin_mod_reductions(O.attention_score_mod)
    assert pin_mod_closed_forms(O.attention_score_mod)


def _mod_mutant(kind):
    def fn(q, k, v, scale, causal=False, block_mask=None, window=0, alibi_slopes=None, softcap=0.0, q_rows=None):
        q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
        B, H, Lq, d = q.shape
        Lk = k.shape[2]
        pos = np.arange(Lq)[:, None] + (Lk - Lq)
        j = np.arange(Lk)[None, :]
        vis = O.element_mask(Lq, Lk, causal, block_mask)
        if window:
            vis &= (j >= pos - window) if kind == "window_off_by_one" else (j > pos - window)
        o = np.zeros((B, H, Lq, d))
        lse = np.full((B, H, Lq), -np.inf)
        for h in range(H):
            S = q[0, h] @ k[0, h].T
            if softcap > 0:
                if kind == "softcap_before_scale":
                    S = scale * softcap * np.tanh(S / softcap)
                elif kind == "softcap_clamp":
                    S = np.clip(scale * S, -softcap, softcap)
                else:
                    S = softcap * np.tanh(scale * S / softcap)
            else:
                S = scale * S
            if alibi_slopes is not None:
                hh = H - 1 - h if kind == "slopes_reversed" else h
                rel = (j - np.arange(Lq)[:, None]) if kind == "alibi_top_left" else (j - pos)
                S = S + (-1 if kind == "alibi_sign" else 1) * float(alibi_slopes[hh]) * rel
            S = np.where(vis, S, -np.inf)
            m = S.max(axis=1)
            live = np.isfinite(m)
            m0 = np.where(live, m, 0.0)
            E = np.exp(S - m0[:, None])
            l = np.where(live, E.sum(axis=1), 1.0)
            o[0, h] = np.where(live[:, None], (E / l[:, None]) @ v[0, h], 0.0)
            lse[0, h] = np.where(live, m0 + np.log(l), -np.inf)
        return o, lse
    return fn


@pytest.mark.parametrize("kind", ["softcap_before_scale", "softcap_clamp", "alibi_sign", "alibi_top_left",
                                  "slopes_reversed", "window_off_by_one"])
def test_score_mod_mutants_are_caught(kind):
    fn = _mod_mutant(kind)
    with np.errstate(all="ignore"):
        assert not (pin_mod_bruteforce(fn) and pin_mod_reductions(fn) and pin_mod_closed_forms(fn))
    none = _mod_mutant("none")
    assert pin_mod_bruteforce(none) and pin_mod_reductions(none) and pin_mod_closed_forms(none)


# ---------------------------------------------------------------------------
# mixture-of-experts routing: softmax over experts, then the top k
# ---------------------------------------------------------------------------

def pin_moe_bruteforce(fn):
    """Pure Python: sort by (-x, index), math.exp / math.fsum probabilities."""
    r = np.random.default_rng(61)
    x = r.normal(0, 2, size=(7, 13))
    x[3, 5] = x[3, 9] = x[3].max() + 1.0            # a tie at the top
    for k in (1, 4, 13):
        for renorm in (False, True):
            idx, w = fn(x, k, renorm)
            for t in range(7):
                row = [float(v) for v in x[t]]
                order = sorted(range(13), key=lambda e: (-row[e], e))[:k]
                m = max(row)
                z = math.fsum(math.exp(v - m) for v in row)
                p = [math.exp(row[e] - m) / z for e in order]
                if renorm:
                    s = math.fsum(p)
                    p = [v / s for v in p]
                if list(idx[t]) != order or max(abs(w[t, i] - p[i]) for i in range(k)) > 1e-15:
                    return False
    return True


def pin_moe_closed_forms(fn):
    # logits ln 1, ln 2, ln 3, ln 2: probabilities 1/8, 2/8, 3/8, 2/8
    x = np.log(np.array([[1.0, 2.0, 3.0, 2.0]]))
    idx, w = fn(x, 3, False)
    if idx.tolist() != [[2, 1, 3]] or np.max(np.abs(w - [[3 / 8, 2 / 8, 2 / 8]])) > 1e-15:
        return False
    idx, w = fn(x, 2, True)                            # renormalised over the two kept
    if idx.tolist() != [[2, 1]] or np.max(np.abs(w - [[0.6, 0.4]])) > 1e-15:
        return False
    # equal logits: the lowest indices, each 1/E (or 1/k renormalised); k = 1 renormalised weighs exactly 1
    x = np.full((2, 6), 0.25)
    idx, w = fn(x, 3, False)
    if idx.tolist() != [[0, 1, 2]] * 2 or np.max(np.abs(w - 1 / 6)) > 1e-15:
        return False
    idx, w = fn(x, 3, True)
    if np.max(np.abs(w - 1 / 3)) > 1e-15:
        return False
    idx, w = fn(np.random.default_rng(62).normal(size=(5, 9)), 1, True)
    return bool(np.all(w == 1.0))


def pin_moe_invariances(fn):
    r = np.random.default_rng(63)
    x = r.normal(0, 3, size=(6, 40))
    for k, renorm in ((8, False), (8, True), (40, False)):
        idx0, w0 = fn(x, k, renorm)
        if k == 40 and not renorm and abs(float(w0.sum(axis=1).max()) - 1) > 1e-14:   # every expert: sums to 1
            return False
        for c in (1000.0, -1000.0):                   # shift invariance (the naive form overflows at +1000)
            idx, w = fn(x + c, k, renorm)
            if not np.array_equal(idx, idx0) or not np.all(np.abs(w - w0) <= 1e-12):   # NaN fails too
                return False
    return True


def test_moe_route_pins():
    assert pin_moe_bruteforce(O.moe_route)
    assert pin_moe_closed_forms(O.moe_route)
    assert pin_moe_invariances(O.moe_route)


def _moe_mutant(kind):
    def fn(logits, k, renorm):
        x = np.asarray(logits, np.float64)
        if kind == "ascending":
            idx = np.argsort(x, axis=-1, kind="stable")[:, :k]
        elif kind == "ties_high_index":
            idx = (x.shape[1] - 1 - np.argsort(-x[:, ::-1], axis=-1, kind="stable"))[:, :k]
        else:
            idx = np.argsort(-x, axis=-1, kind="stable")[:, :k]
        if kind == "no_shift":
            with np.errstate(all="ignore"):
                e = np.exp(x)
                p = e / e.sum(axis=-1, keepdims=True)
        else:
            p = O.softmax_rows(x)
        w = np.take_along_axis(p, idx, axis=-1)
        if renorm and kind != "renorm_ignored":
            w = w / w.sum(axis=-1, keepdims=True)
        if kind == "always_renorm" and not renorm:
            w = w / w.sum(axis=-1, keepdims=True)
        return idx.astype(np.int32), w
    return fn


@pytest.mark.parametrize("kind", ["ascending", "ties_high_index", "no_shift", "renorm_ignored", "always_renorm"])
def test_moe_route_mutants_are_caught(kind):
    fn = _moe_mutant(kind)
    with np.errstate(all="ignore"):
        assert not (pin_moe_bruteforce(fn) and pin_moe_closed_forms(fn) and pin_moe_invariances(fn))
    none = _moe_mutant("none")
    assert pin_moe_bruteforce(none) and pin_moe_closed_forms(none) and pin_moe_invariances(none)


# ---------------------------------------------------------------------------
# The oracle's process pool (full-output parity and the CPU baseline) splits
# work by head and by block of rows only: its results equal the serial
# oracle's exactly.
# ---------------------------------------------------------------------------

def test_pool_attention_row_blocks_equal_serial():
    from oracle import pool
    import workloads as W
    c = W.CONFIGS["attn_f32"]
    blocks = [(0, 50), (50, 51), (51, 128)]
    got = pool.map_tasks("attention", [("attn_f32", 0, 0, r0, r1) for r0, r1 in blocks], workers=3)
    q, k, v = (W.normal_tensor(c["seed"], t, 1, 1, 128, 64, "f32") for t in (W.TID_Q, W.TID_K, W.TID_V))
    ro, rl = O.attention(q, k, v, c["scale"])
    # the BLAS may block a 50-row and a 128-row product differently: the
    # summation order of a dot product, and only that, may change
    assert np.abs(np.concatenate([g[0] for g in got]) - ro[0, 0]).max() <= 1e-14
    assert np.abs(np.concatenate([g[1] for g in got]) - rl[0, 0]).max() <= 1e-14


def test_pool_masked_bf16_head_rows_equal_serial():
    from oracle import pool
    import workloads as W
    c = W.CONFIGS["sparse"]
    rows = (4000, 4100)
    (go, gl), = pool.map_tasks("attention", [("sparse", 1, 7, *rows)], workers=1)
    q, k, v = (O.bf16_bits_to_f64(W.normal_head(c["seed"], t, 1, 7, c["Lq"], c["d"], "bf16"))[None, None]
               for t in (W.TID_Q, W.TID_K, W.TID_V))
    ro, rl = O.attention(q, k, v, c["scale"], True, W.config_block_mask("sparse"), q_rows=np.arange(*rows))
    assert np.array_equal(go, ro[0, 0]) and np.array_equal(gl, rl[0, 0])   # same rows, same calls


def test_pool_softmax_and_decode_equal_serial():
    from oracle import pool
    import workloads as W
    got = pool.map_tasks("softmax", [("softmax", 0, 3), ("softmax", 4090, 4096)], workers=2)
    c = W.CONFIGS["softmax"]
    want = O.softmax_rows(W.softmax_rows_input(c["seed"], 6, c["cols"], row_ids=[0, 1, 2, 4093, 4094, 4095][:3]))
    assert np.array_equal(got[0], want)
    assert got[1].shape == (6, c["cols"])
    c = W.CONFIGS["decode"]
    (go, gl), = pool.map_tasks("decode", [("decode", 65, 67)], workers=1)
    for i, bh in enumerate((65, 66)):
        b, h = divmod(bh, c["H"])
        q, k, v = (O.bf16_bits_to_f64(W.normal_head(c["seed"], t, b, h, L, c["d"], "bf16"))[None, None]
                   for t, L in ((W.TID_Q, 1), (W.TID_K, c["Lk"]), (W.TID_V, c["Lk"])))
        ro, rl = O.attention(q, k, v, c["scale"])
        assert np.array_equal(go[i], ro[0, 0, 0]) and gl[i] == rl[0, 0, 0]


def test_pool_timed_run_reports_workers():
    from oracle import pool
    r = pool.timed_run("attention", [("attn_f32", 0, 0, 0, 64), ("attn_f32", 0, 0, 64, 128)], workers=2)
    assert r["workers"] == 2 and r["tasks"] == 2 and r["wall_s"] > 0 and r["repeat"] == 1 and r["cpu_s"] > 0
    r3 = pool.timed_run("attention", [("attn_f32", 0, 0, 0, 64), ("attn_f32", 0, 0, 64, 128)], workers=2, repeat=3)
    assert r3["repeat"] == 3 and r3["cpu_s"] > 0 and r3["wall_s"] > 0   # (times of tiny tasks are noise)


# ---------------------------------------------------------------------------
# The full-output bf16 gate: planted mistakes in a copy of an oracle result
# ---------------------------------------------------------------------------

def test_bf16_gate_accepts_rounded_and_flags_planted_errors():
    import full_oracle as F
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((2, 3, 50, 8))
    ref[0, 1, 7, 5] = -4.139159435727643          # its nearest bf16 is 0.01416 away: gate unattainable
    lse = rng.standard_normal((2, 3, 50))
    lse[1, 2, 0] = -np.inf
    good = O.round_to_bf16(ref)
    r = F.check_bf16_gates("t", good, lse.copy(), ref, lse)
    assert r["max_err_o"] > 1e-2 and r["max_err_o_gated"] <= 2.0 ** -7 and len(r["unattainable"]) == 1
    other = good.copy()
    other[0, 1, 7, 5] = -4.15625                   # the other bf16 neighbour: still accepted
    F.check_bf16_gates("t", other, lse, ref, lse)
    for mutate in (lambda o, l: o.__setitem__((1, 0, 3, 2), o[1, 0, 3, 2] + 0.011),     # one element off
                   lambda o, l: o.__setitem__((0, 1, 7, 5), -4.1875),                   # two spacings off
                   lambda o, l: l.__setitem__((0, 0, 4), l[0, 0, 4] + 2e-3),            # LSE off
                   lambda o, l: l.__setitem__((1, 2, 0), 0.0),                          # -inf lost
                   lambda o, l: o.__setitem__((0, 0, 0, 0), np.nan)):
        o2, l2 = good.copy(), lse.copy()
        mutate(o2, l2)
        with pytest.raises(AssertionError):
            F.check_bf16_gates("t", o2, l2, ref, lse)
