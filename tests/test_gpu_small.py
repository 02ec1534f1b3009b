"""GPU parity against the fp64 oracle on small and edge-case shapes.

Sizes span several tiles and ragged tails; every call goes through the C ABI
(via the binding). Tolerances: fp32 outputs 1e-5 max abs, bf16 outputs 1e-2
max abs, LSE 1e-3 max abs (tighter where the arithmetic allows it).
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, dev_bf16, dev_f32, host_f64, note

pytestmark = pytest.mark.gpu


def _normal(seed, tid, shape, dtype):
    z = W.rng(seed, tid).standard_normal(shape, dtype=np.float32)
    return W.f32_to_bf16_bits(z) if dtype == "bf16" else z


def _widen(a, dtype):
    return O.bf16_bits_to_f64(a) if dtype == "bf16" else a.astype(np.float64)


def _dev(a, dtype):
    return dev_bf16(a) if dtype == "bf16" else dev_f32(a)


# ---------------------------------------------------------------------------
# softmax rows
# ---------------------------------------------------------------------------

SOFTMAX_SHAPES = [(1, 1), (3, 7), (5, 100), (4, 1024), (3, 4095), (2, 4096), (2, 32768), (2, 65536),
                  (2, 65540), (2, 70001), (300, 33)]


@pytest.mark.parametrize("rows,cols", SOFTMAX_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_softmax_rows_small(rf_gpu, rows, cols, dtype):
    r = W.rng(100, rows, cols)
    x = (r.standard_normal((rows, cols)) * 2 + r.uniform(-50, 50, (rows, 1))).astype(np.float32)
    xs = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    note(f"softmax {rows}x{cols} {dtype}")
    y = rf_gpu.rf_softmax_rows(_dev(xs, dtype))
    ref = O.softmax_rows(_widen(xs, dtype))
    if dtype == "f32":
        assert_close(host_f64(y), ref, 1e-5, "softmax f32")
    else:
        got = host_f64(y)
        # bf16 output: within one rounding of the exact value (half an ulp, 2^-9 relative) plus fp32 noise
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)


@pytest.mark.parametrize("offset", [1000.0, -1000.0, 80.0])
def test_softmax_large_offsets(rf_gpu, offset):
    """exp(x) alone overflows here even in fp64; only the max-shifted form survives."""
    r = W.rng(101, int(abs(offset)))
    x = (r.standard_normal((8, 5000)) * 2 + offset).astype(np.float32)
    note(f"softmax offset {offset}")
    y = rf_gpu.rf_softmax_rows(dev_f32(x))
    assert_close(host_f64(y), O.softmax_rows(x), 1e-5, "softmax offset")


def test_softmax_special_values(rf_gpu):
    x = np.zeros((4, 300), np.float32)
    x[0] = -np.inf                       # all -inf: NaN, as the definition gives
    x[1, ::2] = -np.inf                  # half masked
    x[2, 7] = 5.0
    x[2, 100:] = -np.inf
    x[3] = np.linspace(-30, 30, 300)
    note("softmax special values")
    y = host_f64(rf_gpu.rf_softmax_rows(dev_f32(x)))
    assert np.isnan(y[0]).all()
    with np.errstate(invalid="ignore"):
        ref = O.softmax_rows(x[1:])
    assert_close(y[1:], ref, 1e-6, "softmax special")


def test_softmax_deterministic(rf_gpu):
    x = dev_f32(W.softmax_rows_input(2, 16, 32768))
    note("softmax determinism")
    a = rf_gpu.rf_softmax_rows(x)
    b = rf_gpu.rf_softmax_rows(x)
    assert bool((a == b).all())


# ---------------------------------------------------------------------------
# LSE merge
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,S,d", [(1, 1, 1), (7, 3, 5), (64, 16, 128), (33, 5, 64), (10, 1024, 4), (5, 2, 130)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_lse_merge(rf_gpu, n, S, d, out):
    import torch
    r = W.rng(102, n, S, d)
    o_parts = r.standard_normal((n, S, d)).astype(np.float32)
    lse_parts = (r.standard_normal((n, S)) * 3 + r.uniform(-20, 20, (n, 1))).astype(np.float32)
    dead = r.uniform(size=(n, S)) < 0.25
    lse_parts[dead] = -np.inf
    o_parts[dead] = np.nan                 # must never be read
    lse_parts[0] = -np.inf                 # a row with no live part
    note(f"lse_merge n={n} S={S} d={d} out={out}")
    o, lse = rf_gpu.rf_lse_merge(dev_f32(o_parts), dev_f32(lse_parts),
                                 out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    ref_o, ref_lse = O.lse_merge(np.where(dead[..., None], 0.0, o_parts), lse_parts)
    assert_close(host_f64(o), ref_o, 1e-5 if out == "f32" else 1e-2, "merged O")
    assert_close(host_f64(lse), ref_lse, 1e-5, "merged LSE")


# ---------------------------------------------------------------------------
# split-KV decode
# ---------------------------------------------------------------------------

DECODE_CASES = [  # B, H, Lk, d, splits
    (1, 1, 1, 128, 1), (2, 3, 100, 128, 3), (2, 2, 37, 64, 16), (1, 2, 4096, 128, 16),
    (2, 1, 5000, 64, 7), (1, 1, 33, 128, 64), (3, 2, 2048, 128, 1), (1, 1, 0, 128, 4),
]


@pytest.mark.parametrize("B,H,Lk,d,S", DECODE_CASES)
def test_decode_splitkv(rf_gpu, B, H, Lk, d, S):
    q = _normal(103, 0, (B, H, 1, d), "bf16")
    k = _normal(103, 1, (B, H, Lk, d), "bf16")
    v = _normal(103, 2, (B, H, Lk, d), "bf16")
    scale = 1 / math.sqrt(d)
    note(f"decode B={B} H={H} Lk={Lk} d={d} S={S}")
    o, lse = rf_gpu.rf_attention_decode_splitkv(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=scale, num_splits=S)
    ref_o, ref_lse = O.attention(O.bf16_bits_to_f64(q), O.bf16_bits_to_f64(k), O.bf16_bits_to_f64(v), scale)
    assert_close(host_f64(o), ref_o, 1e-2, "decode O")
    assert_close(host_f64(lse), ref_lse[:, :, 0], 1e-3, "decode LSE")


def test_decode_workspace_fully_written(rf_gpu):
    """NaN-filled workspace: every partial must be overwritten (else NaN leaks out)."""
    import torch
    B, H, Lk, d, S = 2, 2, 1000, 128, 16
    q, k, v = (_normal(104, i, (B, H, L, d), "bf16") for i, L in ((0, 1), (1, Lk), (2, Lk)))
    ws = torch.full((rf_gpu.rf_attention_decode_splitkv_workspace_size(B, H, d, S) // 4,), float("nan"),
                    device="cuda")
    note("decode NaN workspace")
    o, lse = rf_gpu.rf_attention_decode_splitkv(dev_bf16(q), dev_bf16(k), dev_bf16(v), num_splits=S,
                                                workspace=ws.view(torch.uint8))
    ref_o, ref_lse = O.attention(O.bf16_bits_to_f64(q), O.bf16_bits_to_f64(k), O.bf16_bits_to_f64(v),
                                 1 / math.sqrt(d))
    assert_close(host_f64(o), ref_o, 1e-2, "decode O")
    assert_close(host_f64(lse), ref_lse[:, :, 0], 1e-3, "decode LSE")


# ---------------------------------------------------------------------------
# attention forward (fp32 and bf16)
# ---------------------------------------------------------------------------

ATT_CASES = [  # B, H, Lq, Lk, causal, mask density (None = dense)
    (1, 1, 1, 1, False, None), (1, 2, 64, 64, False, None), (2, 2, 200, 200, True, None),
    (1, 1, 300, 257, True, None), (1, 2, 100, 300, True, None), (1, 1, 300, 100, True, None),
    (1, 1, 130, 77, False, None), (2, 1, 256, 256, True, 0.5), (1, 2, 333, 321, False, 0.4),
    (1, 1, 192, 448, True, 0.3), (1, 1, 64, 0, False, None), (1, 3, 513, 513, True, None),
]


def _mask(seed, Lq, Lk, density):
    if density is None:
        return None
    r = W.rng(seed, 4, Lq, Lk)
    m = (r.uniform(size=(math.ceil(Lq / 64), math.ceil(Lk / 64))) < density).astype(np.uint8)
    m[0, 0] = 1
    return m


def _check_attention(rf_gpu, dtype, d, B, H, Lq, Lk, causal, density, seed, tol_o):
    import torch
    q = _normal(seed, 0, (B, H, Lq, d), dtype)
    k = _normal(seed, 1, (B, H, Lk, d), dtype)
    v = _normal(seed, 2, (B, H, Lk, d), dtype)
    bm = _mask(seed, Lq, Lk, density)
    scale = 1 / math.sqrt(d)
    note(f"attention {dtype} d={d} B={B} H={H} Lq={Lq} Lk={Lk} causal={causal} mask={density}")
    o, lse = rf_gpu.rf_attention_fwd(_dev(q, dtype), _dev(k, dtype), _dev(v, dtype), scale=scale, causal=causal,
                                     block_mask=None if bm is None else torch.from_numpy(bm).cuda())
    ref_o, ref_lse = O.attention(_widen(q, dtype), _widen(k, dtype), _widen(v, dtype), scale, causal, bm)
    e_o = assert_close(host_f64(o), ref_o, tol_o, "O")
    e_l = assert_close(host_f64(lse), ref_lse, 1e-3 if dtype == "bf16" else 1e-5, "LSE")
    return e_o, e_l


@pytest.mark.parametrize("B,H,Lq,Lk,causal,density", ATT_CASES)
@pytest.mark.parametrize("d", [64, 128])
def test_attention_bf16(rf_gpu, d, B, H, Lq, Lk, causal, density):
    _check_attention(rf_gpu, "bf16", d, B, H, Lq, Lk, causal, density, 105, 1e-2)


@pytest.mark.parametrize("B,H,Lq,Lk,causal,density", ATT_CASES)
@pytest.mark.parametrize("d", [1, 17, 64, 100, 128])
def test_attention_f32(rf_gpu, d, B, H, Lq, Lk, causal, density):
    _check_attention(rf_gpu, "f32", d, B, H, Lq, Lk, causal, density, 106, 1e-5)


# fp32 with d <= 64 runs on a one-row-per-wavefront kernel while the 16-row
# kernel would have fewer than 512 workgroups; these shapes (512 and more
# 16-row tiles) keep the 16-row kernel covered at small d as well.
F32_TILED_CASES = [(2, 4, 1024, 300, True, None), (1, 8, 1100, 517, False, 0.5), (4, 2, 1030, 1030, True, 0.3)]


@pytest.mark.parametrize("B,H,Lq,Lk,causal,density", F32_TILED_CASES)
@pytest.mark.parametrize("d", [17, 64])
def test_attention_f32_tiled_path_small_d(rf_gpu, d, B, H, Lq, Lk, causal, density):
    _check_attention(rf_gpu, "f32", d, B, H, Lq, Lk, causal, density, 109, 1e-5)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_scale_sign_and_zero(rf_gpu, dtype):
    for scale in (-0.3, 0.0, 2.5):
        q = _normal(107, 0, (1, 2, 150, 64), dtype)
        k = _normal(107, 1, (1, 2, 130, 64), dtype)
        v = _normal(107, 2, (1, 2, 130, 64), dtype)
        note(f"attention {dtype} scale={scale}")
        o, lse = rf_gpu.rf_attention_fwd(_dev(q, dtype), _dev(k, dtype), _dev(v, dtype), scale=scale, causal=True)
        ref_o, ref_lse = O.attention(_widen(q, dtype), _widen(k, dtype), _widen(v, dtype), scale, True)
        # fp32: the d-term dot product carries d roundings of relative size 2^-24, which add
        # like a random walk, so a score s = scale q.k is off by about 2^-24 sqrt(d) |s|. A
        # relative error e in every weight moves O = sum_j w_j v_j by at most
        # e sum_j w_j |v_j - O| <= 2 e max|v|. So the bound is 2 2^-24 sqrt(d) max|s| max|v|,
        # from this test's own inputs (scale 2.5: max|s| about 80, bound about 3e-4), and the
        # 1e-5 gate where that is smaller (the configured scale 1/sqrt(d)).
        s_max = abs(scale) * float(np.abs(_widen(q, dtype)[0] @ np.swapaxes(_widen(k, dtype)[0], 1, 2)).max())
        tol32 = max(1e-5, 2 * 2.0 ** -24 * math.sqrt(64) * s_max * float(np.abs(_widen(v, dtype)).max()))
        assert_close(host_f64(o), ref_o, 1e-2 if dtype == "bf16" else tol32, f"O scale={scale}")
        assert_close(host_f64(lse), ref_lse, 1e-3 if dtype == "bf16" else tol32, f"LSE scale={scale}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_masked_tiles_are_skipped_not_reset(rf_gpu, dtype):
    """NaN-poison every K/V row of key tiles that no query row may see: the
    output must stay finite and exact, so those tiles were never loaded."""
    import torch
    B, H, L, d = 1, 2, 512, 64
    q = _normal(108, 0, (B, H, L, d), dtype)
    k = _normal(108, 1, (B, H, L, d), dtype)
    v = _normal(108, 2, (B, H, L, d), dtype)
    bm = np.tril(np.ones((8, 8), np.uint8))
    bm[:, 2] = 0
    bm[:, 5] = 0
    ref_o, ref_lse = O.attention(_widen(q, dtype), _widen(k, dtype), _widen(v, dtype), 0.125, True, bm)
    kp, vp = k.copy(), v.copy()
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    for tile in (2, 5):
        kp[:, :, tile * 64:(tile + 1) * 64] = nan
        vp[:, :, tile * 64:(tile + 1) * 64] = nan
    note(f"NaN-poisoned masked tiles {dtype}")
    o, lse = rf_gpu.rf_attention_fwd(_dev(q, dtype), _dev(kp, dtype), _dev(vp, dtype), scale=0.125, causal=True,
                                     block_mask=torch.from_numpy(bm).cuda())
    assert_close(host_f64(o), ref_o, 1e-2 if dtype == "bf16" else 1e-5, "O")
    assert_close(host_f64(lse), ref_lse, 1e-3 if dtype == "bf16" else 1e-5, "LSE")


def test_attention_bf16_rising_scores(rf_gpu):
    """Scores that rise along the keys move the running max in every tile."""
    d, L = 128, 640
    q = np.ones((1, 1, L, d), np.float32) * 0.1
    k = (np.linspace(0, 4, L)[:, None] * np.ones((1, d))).astype(np.float32)[None, None]
    v = _normal(109, 2, (1, 1, L, d), "f32")
    qb, kb, vb = (W.f32_to_bf16_bits(a) for a in (q, k, v))
    note("rising scores")
    o, lse = rf_gpu.rf_attention_fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), causal=True)
    ref_o, ref_lse = O.attention(*(O.bf16_bits_to_f64(a) for a in (qb, kb, vb)), 1 / math.sqrt(d), True)
    assert_close(host_f64(o), ref_o, 1e-2, "O")
    assert_close(host_f64(lse), ref_lse, 1e-3, "LSE")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_bf16_jumps_inside_tiles(rf_gpu, d, causal):
    """Scores that jump by far more than the rescale slack (2^8) in the second
    32-key half of a tile, in the first half of the next one, and in the last
    tile: the reference must move after part of a tile is already in O."""
    L = 256
    q = np.full((1, 2, L, d), 0.5, np.float32)
    k = np.zeros((1, 2, L, d), np.float32)
    k[:, :, 96:128] = 2.0      # tile 1, keys 32..63 of the tile
    k[:, :, 128:160] = 4.0     # tile 2, keys 0..31
    k[:, :, 224:256] = 6.0     # tile 3 (last), keys 32..63
    v = _normal(112, 2, (1, 2, L, d), "f32")
    qb, kb, vb = (W.f32_to_bf16_bits(a) for a in (q, k, v))
    note(f"jumps inside tiles d={d} causal={causal}")
    o, lse = rf_gpu.rf_attention_fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), causal=causal)
    ref_o, ref_lse = O.attention(*(O.bf16_bits_to_f64(a) for a in (qb, kb, vb)), 1 / math.sqrt(d), causal)
    assert_close(host_f64(o), ref_o, 1e-2, "O")
    assert_close(host_f64(lse), ref_lse, 1e-3, "LSE")


@pytest.mark.parametrize("d", [64, 128])
def test_attention_bf16_reference_from_a_later_tile(rf_gpu, d):
    """A wave whose first visited key tile is hidden by its block-mask row has no
    exponent reference yet; its next tile's scores (about -220 in log2 units)
    would all underflow against a zero reference. Rows 0..63 see only key tile
    1, whose keys are identical: O is the mean of those V rows."""
    import torch
    L = 256
    q = np.ones((1, 1, L, d), np.float32)
    k = np.ones((1, 1, L, d), np.float32)
    k[:, :, 64:128] = -1.2 * 128 / d
    v = _normal(113, 2, (1, 1, L, d), "f32")
    bm = np.zeros((4, 4), np.uint8)
    bm[0, 1] = 1
    bm[1, 0] = bm[1, 1] = 1
    bm[2, 2] = bm[3, 3] = 1
    qb, kb, vb = (W.f32_to_bf16_bits(a) for a in (q, k, v))
    note(f"reference from a later tile d={d}")
    o, lse = rf_gpu.rf_attention_fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), scale=1.0,
                                     block_mask=torch.from_numpy(bm).cuda())
    ref_o, ref_lse = O.attention(*(O.bf16_bits_to_f64(a) for a in (qb, kb, vb)), 1.0, False, bm)
    assert np.all(np.isfinite(ref_lse)) and ref_lse[0, 0, 0] < -100
    assert_close(host_f64(o), ref_o, 1e-2, "O")
    assert_close(host_f64(lse), ref_lse, 1e-3, "LSE")


def test_attention_bf16_deterministic(rf_gpu):
    q, k, v = (dev_bf16(_normal(110, i, (2, 4, 700, 128), "bf16")) for i in range(3))
    note("attention determinism")
    o1, l1 = rf_gpu.rf_attention_fwd(q, k, v, causal=True)
    o2, l2 = rf_gpu.rf_attention_fwd(q, k, v, causal=True)
    assert bool((o1.view(dtype=__import__("torch").int16) == o2.view(dtype=__import__("torch").int16)).all())
    assert bool((l1 == l2).all())


def test_output_canaries(rf_gpu):
    """Writes stay inside the outputs: guard regions around O and LSE keep their bytes."""
    import torch
    B, H, Lq, Lk, d = 1, 2, 200, 190, 128
    q, k, v = (dev_bf16(_normal(111, i, (B, H, L, d), "bf16")) for i, L in ((0, Lq), (1, Lk), (2, Lk)))
    pad = 4096
    ob = torch.full((pad + B * H * Lq * d + pad,), 12345, dtype=torch.int16, device="cuda")
    lb = torch.full((pad + B * H * Lq + pad,), 7.0, dtype=torch.float32, device="cuda")
    o = ob[pad:pad + B * H * Lq * d].view(torch.bfloat16).view(B, H, Lq, d)
    lse = lb[pad:pad + B * H * Lq].view(B, H, Lq)
    note("canaries")
    rf_gpu.rf_attention_fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((ob[:pad] == 12345).all()) and bool((ob[-pad:] == 12345).all())
    assert bool((lb[:pad] == 7.0).all()) and bool((lb[-pad:] == 7.0).all())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Lq,Lk,causal", [(1, 2, 300, 300, True), (2, 1, 200, 333, True), (1, 1, 130, 700, False),
                                              (1, 3, 64, 64, True), (1, 1, 257, 129, True)])
def test_attention_bf16_mask_free_equals_all_ones_mask(rf_gpu, d, B, H, Lq, Lk, causal):
    """A call without a block mask runs the mask-free kernel instance, one with
    an all-ones mask the masked instance: the same tiles in the same order with
    the same arithmetic, so the outputs must be identical bit for bit (plain,
    softcap and window; ALiBi walks the tiles in another order without a mask)."""
    import torch
    q, k, v = (dev_bf16(_normal(109, t, (B, H, L, d), "bf16")) for t, L in ((0, Lq), (1, Lk), (2, Lk)))
    ones = torch.ones((-(-Lq // 64), -(-Lk // 64)), dtype=torch.uint8, device="cuda")
    note(f"mask-free vs all-ones mask d={d} B={B} H={H} Lq={Lq} Lk={Lk} causal={causal}")
    for kw in ({}, {"softcap": 30.0}, {"window": 100}):
        if kw:
            a = rf_gpu.rf_attention_fwd_mod(q, k, v, causal=causal, **kw)
            b = rf_gpu.rf_attention_fwd_mod(q, k, v, causal=causal, block_mask=ones, **kw)
        else:
            a = rf_gpu.rf_attention_fwd(q, k, v, causal=causal)
            b = rf_gpu.rf_attention_fwd(q, k, v, causal=causal, block_mask=ones)
        for x, y, name in zip(a, b, ("O", "LSE")):
            assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                               y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)), (kw, name)


@pytest.mark.parametrize("cols", [5, 255, 257, 1023, 4097, 8191, 16385, 32767, 32769, 50257, 65533, 65535])
def test_softmax_ragged_widths(rf_gpu, cols):
    """fp32 rows whose width is not a multiple of 4 (rows then start only 4-byte
    aligned, and each row's last 16-byte vector straddles its end), at every
    register-table boundary: against the oracle, and the elements past a row's
    end never touched (the next row is intact)."""
    rows = 3
    x = W.softmax_rows_input(2, rows, cols)
    note(f"softmax ragged cols={cols}")
    y = host_f64(rf_gpu.rf_softmax_rows(dev_f32(x)))
    ref = O.softmax_rows(x.astype(np.float64))
    assert_close(y, ref, 1e-5, f"y cols={cols}")
    assert np.allclose(y.sum(axis=1), 1.0, atol=1e-5)


@pytest.mark.parametrize("cols", [6, 250, 1022, 4094, 16386, 32766, 50258, 65534])
def test_softmax_ragged_even_widths_bf16(rf_gpu, cols):
    """bf16 rows of even width not a multiple of 8: 16-byte vectors, the last
    one straddling the row's end on a dword boundary; against the oracle on
    the bf16 inputs (output rounded to bf16)."""
    rows = 3
    x = W.f32_to_bf16_bits(W.softmax_rows_input(2, rows, cols))
    note(f"softmax bf16 ragged cols={cols}")
    y = host_f64(rf_gpu.rf_softmax_rows(dev_bf16(x)))
    ref = O.softmax_rows(O.bf16_bits_to_f64(x))
    assert_close(y, ref, 1e-2, f"y cols={cols}")


# ---------------------------------------------------------------------------
# streams: every call is enqueued on torch's current stream
# ---------------------------------------------------------------------------

def test_calls_run_on_the_current_stream(rf_gpu):
    """Under a side stream, the calls' results are complete once that stream
    alone is synchronised, while the default stream is still busy with a spin
    kernel queued before them: they were enqueued on the side stream."""
    import torch
    if not hasattr(torch.cuda, "_sleep"):
        pytest.skip("torch.cuda._sleep is not available")
    q, k, v = (_normal(131, t, (1, 2, 300, 128), "bf16") for t in (0, 1, 2))
    x = _normal(132, 3, (64, 5000), "f32")
    qd, kd, vd, xd = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f32(x)
    ref_o, ref_l = rf_gpu.rf_attention_fwd(qd, kd, vd, causal=True)
    ref_y = rf_gpu.rf_softmax_rows(xd)
    torch.cuda.synchronize()
    o, l, y = torch.empty_like(ref_o), torch.empty_like(ref_l), torch.empty_like(ref_y)
    side = torch.cuda.Stream()
    note("attention and softmax on a side stream behind a busy default stream")
    torch.cuda._sleep(200_000_000)          # about 0.1 s of spinning on the default stream
    with torch.cuda.stream(side):
        rf_gpu.rf_attention_fwd(qd, kd, vd, causal=True, out=o, lse=l)
        rf_gpu.rf_softmax_rows(xd, out=y)
    side.synchronize()
    assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(l, ref_l) and torch.equal(y, ref_y)
    torch.cuda.synchronize()
