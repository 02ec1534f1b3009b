"""GPU parity of decode with grouped queries (rf_attention_decode_gqa).

Query head hq reads key/value head hq // G; the oracle is the fp64
oracle.decode_gqa. Gates: bf16 O 1e-2 max abs, LSE 1e-3.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, dev_bf16, host_f64, note

pytestmark = pytest.mark.gpu


def _inputs(seed, B, Hq, Hkv, Lk, d):
    r = W.rng(seed, B, Hq, Hkv, Lk, d)
    f = lambda *s: W.f32_to_bf16_bits(r.standard_normal(s, dtype=np.float32))
    return f(B, Hq, d), f(B, Hkv, Lk, d), f(B, Hkv, Lk, d)


def _run(rf_gpu, q, k, v, scale, S, workspace=None):
    return rf_gpu.rf_attention_decode_gqa(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=scale, num_splits=S,
                                          workspace=workspace)


def _check(rf_gpu, B, Hq, Hkv, Lk, d, S, seed, scale=None):
    q, k, v = _inputs(seed, B, Hq, Hkv, Lk, d)
    scale = 1 / math.sqrt(d) if scale is None else scale
    note(f"gqa decode B={B} Hq={Hq} Hkv={Hkv} Lk={Lk} d={d} S={S} scale={scale}")
    o, lse = _run(rf_gpu, q, k, v, scale, S)
    ref_o, ref_lse = O.decode_gqa(*(O.bf16_bits_to_f64(a) for a in (q, k, v)), scale)
    assert_close(host_f64(o), ref_o, 1e-2, "O")
    assert_close(host_f64(lse), ref_lse, 1e-3, "LSE")


GQA_CASES = [  # B, Hq, Hkv, Lk, d, S
    (1, 8, 1, 200, 64, 1),
    (2, 8, 2, 1000, 128, 4),
    (1, 16, 2, 4097, 128, 7),      # ragged last tile, uneven splits
    (2, 32, 32, 333, 64, 3),       # G = 1: plain multi-head decode
    (1, 128, 1, 3000, 128, 16),    # every query head on one cache: one full 128-row tile
    (1, 130, 1, 700, 128, 5),      # G = 130: two query tiles of one key/value head
    (1, 130, 2, 700, 64, 2),       # G = 65 at d = 64 (64-row tiles): two query tiles
    (3, 6, 3, 65, 64, 64),         # more splits than key tiles: empty splits
    (1, 4, 4, 1, 128, 2),          # one key
    (1, 12, 4, 64, 64, 1),         # exactly one tile, written directly
    (2, 24, 3, 2049, 128, 1),      # G = 8, no split
    (1, 32, 1, 1500, 128, 3),      # G = 32: one full 32-row tile
    (2, 16, 8, 777, 128, 5),       # G = 2
    (1, 16, 2, 999, 64, 3),        # G = 8 at d = 64
    (2, 16, 4, 5000, 64, 6),       # G = 4 at d = 64
    (1, 66, 2, 1100, 128, 4),      # G = 33: a 64-row tile, ragged
    (1, 64, 1, 900, 128, 2),       # G = 64: one full 64-row tile
    (1, 65, 1, 700, 128, 3),       # G = 65: a 128-row tile
]


@pytest.mark.parametrize("B,Hq,Hkv,Lk,d,S", GQA_CASES)
def test_gqa_decode(rf_gpu, B, Hq, Hkv, Lk, d, S):
    _check(rf_gpu, B, Hq, Hkv, Lk, d, S, 150)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.5])
@pytest.mark.parametrize("S", [1, 3])
def test_gqa_decode_scale_sign_and_zero(rf_gpu, scale, S):
    _check(rf_gpu, 2, 16, 4, 300, 128, S, 151, scale=scale)


@pytest.mark.parametrize("S", [1, 4])
def test_gqa_decode_no_keys(rf_gpu, S):
    import torch
    q, k, v = _inputs(152, 2, 8, 2, 0, 64)
    note(f"gqa decode Lk=0 S={S}")
    o, lse = _run(rf_gpu, q, k, v, 0.125, S)
    torch.cuda.synchronize()
    assert np.all(host_f64(o) == 0) and np.all(host_f64(lse) == -np.inf)


def test_gqa_decode_ignores_workspace_contents(rf_gpu):
    """The workspace is NaN-filled before the call: every partial is written
    (empty splits too) before the merge reads it."""
    import torch
    B, Hq, Hkv, Lk, d, S = 2, 16, 2, 500, 128, 12          # 8 key tiles, 12 splits: 4 empty
    q, k, v = _inputs(153, B, Hq, Hkv, Lk, d)
    ws = torch.full((rf_gpu.rf_attention_decode_gqa_workspace_size(B, Hq, d, S) // 4,), float("nan"),
                    device="cuda").view(torch.uint8)
    note("gqa decode NaN workspace")
    o, lse = _run(rf_gpu, q, k, v, 1 / math.sqrt(d), S, workspace=ws)
    ref_o, ref_lse = O.decode_gqa(*(O.bf16_bits_to_f64(a) for a in (q, k, v)), 1 / math.sqrt(d))
    assert_close(host_f64(o), ref_o, 1e-2, "O")
    assert_close(host_f64(lse), ref_lse, 1e-3, "LSE")


def test_gqa_decode_is_deterministic(rf_gpu):
    import torch
    q, k, v = _inputs(154, 2, 32, 4, 3000, 128)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    note("gqa decode determinism")
    a = rf_gpu.rf_attention_decode_gqa(qd, kd, vd, num_splits=5)
    b = rf_gpu.rf_attention_decode_gqa(qd, kd, vd, num_splits=5)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
