"""GPU parity of attention with element bitmaps inside partial tiles.

Every call goes through rf_attention_fwd_bitmap; the oracle is the fp64
masked attention with the same tile kinds and row bitmaps. Gates: bf16 O
1e-2, fp32 O 1e-5, LSE 1e-3 (bf16) / 1e-5 (fp32), max abs.
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


def _random_bitmaps(seed, Lq, Lk, p_full=0.3, p_part=0.4):
    r = W.rng(seed, 4, Lq, Lk)
    nI, nJ = math.ceil(Lq / 64), math.ceil(Lk / 64)
    u = r.uniform(size=(nI, nJ))
    kinds = np.where(u < p_full, 1, np.where(u < p_full + p_part, 2, 0)).astype(np.uint8)
    kinds[(u >= p_full) & (u < p_full + p_part / 4)] = 7      # another partial kind value
    kinds[0, 0] = 2
    density = r.uniform(0.2, 0.9, size=(nI, nJ, 1))
    bitsel = r.uniform(size=(nI, nJ, 64, 64)) < density[..., None]
    weights = np.uint64(1) << np.arange(64, dtype=np.uint64)
    bits = (bitsel.astype(np.uint64) * weights).sum(axis=-1, dtype=np.uint64)
    return kinds, bits


def _run(rf_gpu, dtype, d, B, H, Lq, Lk, causal, kinds, bits, seed, kv=None):
    import torch
    q = _normal(seed, 0, (B, H, Lq, d), dtype)
    k, v = kv if kv is not None else (_normal(seed, 1, (B, H, Lk, d), dtype), _normal(seed, 2, (B, H, Lk, d), dtype))
    scale = 1 / math.sqrt(d)
    note(f"bitmap attention {dtype} d={d} B={B} H={H} Lq={Lq} Lk={Lk} causal={causal}")
    o, lse = rf_gpu.rf_attention_fwd_bitmap(_dev(q, dtype), _dev(k, dtype), _dev(v, dtype),
                                            torch.from_numpy(kinds).cuda(),
                                            torch.from_numpy(bits.view(np.int64)).cuda(), scale=scale, causal=causal)
    return o, lse, q, k, v, scale


def _check(rf_gpu, dtype, d, B, H, Lq, Lk, causal, kinds, bits, seed):
    o, lse, q, k, v, scale = _run(rf_gpu, dtype, d, B, H, Lq, Lk, causal, kinds, bits, seed)
    ref_o, ref_lse = O.attention(_widen(q, dtype), _widen(k, dtype), _widen(v, dtype), scale, causal, kinds,
                                 tile_bits=bits)
    assert_close(host_f64(o), ref_o, 1e-2 if dtype == "bf16" else 1e-5, "O")
    assert_close(host_f64(lse), ref_lse, 1e-3 if dtype == "bf16" else 1e-5, "LSE")


BITMAP_CASES = [  # B, H, Lq, Lk, causal
    (1, 2, 200, 300, False), (1, 1, 130, 77, True), (2, 1, 256, 256, True), (1, 1, 64, 640, False),
    (1, 2, 333, 321, True), (1, 1, 1, 200, False),
]


@pytest.mark.parametrize("B,H,Lq,Lk,causal", BITMAP_CASES)
@pytest.mark.parametrize("d", [64, 128])
def test_bitmap_bf16(rf_gpu, d, B, H, Lq, Lk, causal):
    kinds, bits = _random_bitmaps(130, Lq, Lk)
    _check(rf_gpu, "bf16", d, B, H, Lq, Lk, causal, kinds, bits, 131)


@pytest.mark.parametrize("B,H,Lq,Lk,causal", BITMAP_CASES)
@pytest.mark.parametrize("d", [17, 64, 128])
def test_bitmap_f32(rf_gpu, d, B, H, Lq, Lk, causal):
    kinds, bits = _random_bitmaps(132, Lq, Lk)
    _check(rf_gpu, "f32", d, B, H, Lq, Lk, causal, kinds, bits, 133)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_bitmap_element_window(rf_gpu, dtype, d):
    """The element-level 512-key causal window plus random tiles, at L = 1024."""
    kinds, bits = W.window_bitmap_mask(134, 1024, window=512, frac=0.3)
    _check(rf_gpu, dtype, d, 1, 2, 1024, 1024, False, kinds, bits, 135)


@pytest.mark.parametrize("d", [64, 128])
def test_bitmap_rows_of_one_workgroup_differ(rf_gpu, d):
    """128 query rows span two mask rows: tile 1 is partial for the first and
    full for the second, tile 2 empty for the first and partial for the
    second, tile 3 partial for both; some rows see nothing in a partial tile."""
    Lq, Lk = 128, 256
    kinds = np.array([[1, 2, 0, 2], [1, 1, 2, 2]], np.uint8)
    r = W.rng(136, 4)
    bits = r.integers(0, 2 ** 63, size=(2, 4, 64), dtype=np.uint64) * np.uint64(2)
    bits[0, 1, :7] = 0                  # rows 0..6 see no key of tile 1
    bits[1, 3, 60:] = np.uint64(2 ** 64 - 1)
    _check(rf_gpu, "bf16", d, 1, 2, Lq, Lk, False, kinds, bits, 137)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bitmap_empty_tiles_are_never_loaded(rf_gpu, dtype):
    """NaN-poison every key/value row of the empty tiles: the result stays exact."""
    B, H, L, d = 1, 2, 512, 64
    kinds, bits = _random_bitmaps(138, L, L, p_full=0.4, p_part=0.4)
    kinds[:, 3] = 0
    kinds[:, 6] = 0
    k = _normal(139, 1, (B, H, L, d), dtype)
    v = _normal(139, 2, (B, H, L, d), dtype)
    q = _normal(139, 0, (B, H, L, d), dtype)
    ref_o, ref_lse = O.attention(_widen(q, dtype), _widen(k, dtype), _widen(v, dtype), 1 / math.sqrt(d), False,
                                 kinds, tile_bits=bits)
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    for t in (3, 6):
        k[:, :, 64 * t:64 * (t + 1)] = nan
        v[:, :, 64 * t:64 * (t + 1)] = nan
    o, lse, *_ = _run(rf_gpu, dtype, d, B, H, L, L, False, kinds, bits, 139, kv=(k, v))
    assert_close(host_f64(o), ref_o, 1e-2 if dtype == "bf16" else 1e-5, "O")
    assert_close(host_f64(lse), ref_lse, 1e-3 if dtype == "bf16" else 1e-5, "LSE")
