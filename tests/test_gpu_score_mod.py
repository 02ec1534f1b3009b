"""GPU parity of attention with score modifications (rf_attention_fwd_mod):
softcap, ALiBi bias and element-level sliding window, alone and together.

The oracle is the fp64 oracle.attention_score_mod. Gates: bf16 O 1e-2 and
LSE 1e-3; fp32 O 1e-5 and LSE 1e-5 (max abs).
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, dev_bf16, dev_f32, host_f64, note

pytestmark = pytest.mark.gpu


def _normal(seed, tid, shape, dtype, s=1.0):
    z = (s * W.rng(seed, tid, *shape).standard_normal(shape)).astype(np.float32)
    return W.f32_to_bf16_bits(z) if dtype == "bf16" else z


def _widen(a, dtype):
    return O.bf16_bits_to_f64(a) if dtype == "bf16" else a.astype(np.float64)


def _dev(a, dtype):
    return dev_bf16(a) if dtype == "bf16" else dev_f32(a)


def _run_check(rf_gpu, dtype, d, B, H, Lq, Lk, causal, window, alibi, softcap, seed, scale=None, block_mask=None,
               qs=1.0, kv=None):
    import torch
    q = _normal(seed, 0, (B, H, Lq, d), dtype, qs)
    k, v = kv if kv is not None else (_normal(seed, 1, (B, H, Lk, d), dtype), _normal(seed, 2, (B, H, Lk, d), dtype))
    scale = 1 / math.sqrt(d) if scale is None else scale
    slopes = W.alibi_slopes(H) if alibi else None
    note(f"score mod {dtype} d={d} B={B} H={H} Lq={Lq} Lk={Lk} causal={causal} window={window} alibi={alibi} "
         f"softcap={softcap} scale={scale}")
    o, lse = rf_gpu.rf_attention_fwd_mod(
        _dev(q, dtype), _dev(k, dtype), _dev(v, dtype), scale=scale, causal=causal,
        block_mask=None if block_mask is None else torch.from_numpy(block_mask).cuda(), window=window,
        alibi_slopes=None if slopes is None else torch.from_numpy(slopes).cuda(), softcap=softcap)
    ref_o, ref_lse = O.attention_score_mod(_widen(q, dtype), _widen(k, dtype), _widen(v, dtype), scale, causal,
                                           block_mask, window, None if slopes is None else slopes.astype(np.float64),
                                           softcap)
    assert_close(host_f64(o), ref_o, 1e-2 if dtype == "bf16" else 1e-5, "O")
    assert_close(host_f64(lse), ref_lse, 1e-3 if dtype == "bf16" else 1e-5, "LSE")


MOD_CASES = [  # B, H, Lq, Lk, causal, window, alibi, softcap
    (1, 2, 200, 300, True, 0, True, 0.0),       # ALiBi, causal, Lq < Lk
    (1, 2, 200, 300, False, 0, True, 0.0),      # ALiBi without causal: positive bias for later keys
    (1, 2, 333, 321, True, 0, False, 2.0),      # a softcap that bends the scores
    (2, 1, 256, 256, True, 100, False, 0.0),    # window not aligned to tiles
    (1, 2, 130, 700, True, 64, True, 30.0),     # all three, Lq < Lk
    (1, 1, 300, 300, True, 1, False, 0.0),      # window 1: the diagonal key only
    (1, 2, 500, 500, False, 300, False, 0.0),   # window without causal (lower edge only)
    (1, 1, 64, 640, True, 700, True, 5.0),      # window wider than the keys
    (1, 1, 1, 200, True, 50, True, 0.0),        # one query row
    (1, 3, 257, 257, True, 65, True, 1.0),      # ragged everything
]


@pytest.mark.parametrize("B,H,Lq,Lk,causal,window,alibi,softcap", MOD_CASES)
@pytest.mark.parametrize("d", [64, 128])
def test_score_mod_bf16(rf_gpu, d, B, H, Lq, Lk, causal, window, alibi, softcap):
    _run_check(rf_gpu, "bf16", d, B, H, Lq, Lk, causal, window, alibi, softcap, 160)


@pytest.mark.parametrize("B,H,Lq,Lk,causal,window,alibi,softcap", MOD_CASES)
@pytest.mark.parametrize("d", [17, 64, 128])
def test_score_mod_f32(rf_gpu, d, B, H, Lq, Lk, causal, window, alibi, softcap):
    _run_check(rf_gpu, "f32", d, B, H, Lq, Lk, causal, window, alibi, softcap, 161)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.9])
def test_score_mod_scale_sign_and_zero(rf_gpu, dtype, d, scale):
    _run_check(rf_gpu, dtype, d, 1, 2, 150, 190, True, 80, True, 3.0, 162, scale=scale)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 32)])
def test_score_mod_with_block_mask(rf_gpu, dtype, d):
    L = 512
    bm = (W.rng(163, 4).uniform(size=(8, 8)) < 0.6).astype(np.uint8)
    np.fill_diagonal(bm, 1)
    _run_check(rf_gpu, dtype, d, 1, 2, L, L, True, 150, True, 10.0, 164, block_mask=bm)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_window_tiles_before_every_row_are_never_loaded(rf_gpu, dtype, d):
    """64 query rows at the end of 2048 keys, window 64: keys 0..1919 are before
    every row's window. They are NaN in K and V; a loaded and masked value tile
    would still leak NaN through 0 * NaN in P V."""
    B, H, Lq, Lk, W_ = 1, 2, 64, 2048, 64
    k = _normal(165, 1, (B, H, Lk, d), dtype)
    v = _normal(165, 2, (B, H, Lk, d), dtype)
    q = _normal(165, 0, (B, H, Lq, d), dtype)
    ref_o, ref_lse = O.attention_score_mod(_widen(q, dtype), _widen(k, dtype), _widen(v, dtype), 1 / math.sqrt(d),
                                           True, None, W_)
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    k[:, :, :1920] = nan
    v[:, :, :1920] = nan
    note(f"score mod window skip {dtype} d={d}")
    o, lse = rf_gpu.rf_attention_fwd_mod(_dev(q, dtype), _dev(k, dtype), _dev(v, dtype), causal=True, window=W_)
    assert_close(host_f64(o), ref_o, 1e-2 if dtype == "bf16" else 1e-5, "O")
    assert_close(host_f64(lse), ref_lse, 1e-3 if dtype == "bf16" else 1e-5, "LSE")
