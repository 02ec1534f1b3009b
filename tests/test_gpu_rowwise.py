"""GPU parity of the row-wise masked attention kernel (rf_attention_fwd_rowwise)
against the fp64 masked attention oracle. Gates: bf16 O 1e-2, LSE 1e-3 (max abs)."""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, dev_bf16, host_f64, note

pytestmark = pytest.mark.gpu


def _normal(seed, tid, shape):
    return W.f32_to_bf16_bits(W.rng(seed, tid, *shape).standard_normal(shape, dtype=np.float32))


def _masks(seed, Lq, Lk, p_full, p_part, density=(0.2, 0.9)):
    r = W.rng(seed, 4, Lq, Lk)
    nI, nJ = -(-Lq // 64), -(-Lk // 64)
    u = r.uniform(size=(nI, nJ))
    kinds = np.where(u < p_full, 1, np.where(u < p_full + p_part, 2, 0)).astype(np.uint8)
    kinds[(u >= p_full) & (u < p_full + p_part / 4)] = 9
    dens = r.uniform(*density, size=(nI, nJ, 1))
    sel = r.uniform(size=(nI, nJ, 64, 64)) < dens[..., None]
    bits = (sel.astype(np.uint64) << np.arange(64, dtype=np.uint64)).sum(axis=-1, dtype=np.uint64)
    return kinds, bits


def _run(rf_gpu, d, B, H, Lq, Lk, causal, kinds, bits, seed, scale=None, kv=None):
    import torch
    q = _normal(seed, 0, (B, H, Lq, d))
    k, v = kv if kv is not None else (_normal(seed, 1, (B, H, Lk, d)), _normal(seed, 2, (B, H, Lk, d)))
    scale = 1 / math.sqrt(d) if scale is None else scale
    note(f"rowwise d={d} B={B} H={H} Lq={Lq} Lk={Lk} causal={causal} kinds={kinds is not None} "
         f"bits={bits is not None} scale={scale}")
    o, lse = rf_gpu.rf_attention_fwd_rowwise(
        dev_bf16(q), dev_bf16(k), dev_bf16(v), None if kinds is None else torch.from_numpy(kinds).cuda(),
        None if bits is None else torch.from_numpy(bits.view(np.int64)).cuda(), scale=scale, causal=causal)
    return o, lse, q, k, v, scale


def _check(rf_gpu, d, B, H, Lq, Lk, causal, kinds, bits, seed, scale=None):
    o, lse, q, k, v, scale = _run(rf_gpu, d, B, H, Lq, Lk, causal, kinds, bits, seed, scale)
    ref_o, ref_lse = O.attention(*(O.bf16_bits_to_f64(a) for a in (q, k, v)), scale, causal, kinds, tile_bits=bits)
    assert_close(host_f64(o), ref_o, 1e-2, "O")
    assert_close(host_f64(lse), ref_lse, 1e-3, "LSE")


CASES = [  # B, H, Lq, Lk, causal
    (1, 2, 200, 300, False), (1, 1, 130, 77, True), (2, 1, 256, 256, True), (1, 1, 64, 640, False),
    (1, 2, 333, 321, True), (1, 1, 1, 200, False), (1, 1, 70, 4097, True),
]


@pytest.mark.parametrize("B,H,Lq,Lk,causal", CASES)
@pytest.mark.parametrize("d", [64, 128])
def test_rowwise_bitmaps(rf_gpu, d, B, H, Lq, Lk, causal):
    kinds, bits = _masks(180, Lq, Lk, 0.3, 0.4)
    _check(rf_gpu, d, B, H, Lq, Lk, causal, kinds, bits, 181)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_rowwise_dense_and_block_mask(rf_gpu, d, causal):
    _check(rf_gpu, d, 1, 2, 190, 260, causal, None, None, 182)
    kinds, _ = _masks(183, 190, 260, 0.5, 0.0)
    kinds[:, 0] = 1
    _check(rf_gpu, d, 1, 2, 190, 260, causal, kinds, None, 184)


@pytest.mark.parametrize("d", [64, 128])
def test_rowwise_element_window(rf_gpu, d):
    kinds, bits = W.window_bitmap_mask(185, 1024, window=512, frac=0.3)
    _check(rf_gpu, d, 1, 2, 1024, 1024, False, kinds, bits, 186)


@pytest.mark.parametrize("d", [64, 128])
def test_rowwise_very_sparse_rows(rf_gpu, d):
    """A handful of keys per row scattered over 8192 keys; some rows see nothing."""
    Lq, Lk = 130, 8192
    kinds, bits = _masks(187, Lq, Lk, 0.0, 0.05, density=(0.01, 0.05))
    bits[0, :, 3] = 0                                  # row 3 sees no key at all
    _check(rf_gpu, d, 1, 2, Lq, Lk, False, kinds, bits, 188)


@pytest.mark.parametrize("scale", [-0.3, 0.0])
def test_rowwise_scale_sign_and_zero(rf_gpu, scale):
    kinds, bits = _masks(189, 150, 200, 0.3, 0.5)
    _check(rf_gpu, 128, 1, 1, 150, 200, True, kinds, bits, 190, scale=scale)


@pytest.mark.parametrize("d", [64, 128])
def test_rowwise_loads_visible_keys_only(rf_gpu, d):
    """Every key that no row sees (empty tiles, and clear bits inside partial
    tiles) is NaN in K and V: the row kernel never loads it."""
    B, H, L = 1, 2, 512
    kinds, bits = _masks(191, L, L, 0.2, 0.5)
    q = _normal(192, 0, (B, H, L, d))
    k = _normal(192, 1, (B, H, L, d))
    v = _normal(192, 2, (B, H, L, d))
    ref_o, ref_lse = O.attention(*(O.bf16_bits_to_f64(a) for a in (q, k, v)), 1 / math.sqrt(d), False, kinds,
                                 tile_bits=bits)
    seen = O.element_mask(L, L, False, kinds, tile_bits=bits).any(axis=0)
    k[:, :, ~seen] = np.uint16(0x7FC0)
    v[:, :, ~seen] = np.uint16(0x7FC0)
    o, lse, *_ = _run(rf_gpu, d, B, H, L, L, False, kinds, bits, 192, kv=(k, v))
    assert_close(host_f64(o), ref_o, 1e-2, "O")
    assert_close(host_f64(lse), ref_lse, 1e-3, "LSE")


def _timed_us(fn, n=10):
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / n * 1e3


@pytest.mark.parametrize("d,Lq,Lk,causal,p_tile,bit_d", [
    (128, 1024, 1024, True, 1.0, 0.5),     # dense-ish causal square mask: tile kernel
    (128, 64, 16384, False, 0.3, 0.01),    # one query block over long keys, ~1% of keys: row kernel
    (64, 64, 16384, False, 0.3, 0.01),
])
def test_plan_picks_the_faster_kernel(rf_gpu, d, Lq, Lk, causal, p_tile, bit_d):
    """The analytic choice (STOF page, Méthodologie 1) against measured calls of
    both kernels, on masks where the two differ by about 3x: the pick must not
    be the slower one by more than 25%."""
    import torch
    B, H = 1, 16
    r = W.rng(181, 4, Lq, Lk)
    nI, nJ = Lq // 64, Lk // 64
    kinds = np.where(r.uniform(size=(nI, nJ)) < p_tile, 2, 0).astype(np.uint8)
    sel = r.uniform(size=(nI, nJ, 64, 64)) < bit_d
    bits = (sel.astype(np.uint64) << np.arange(64, dtype=np.uint64)).sum(axis=-1, dtype=np.uint64)
    q = dev_bf16(_normal(181, 0, (B, H, Lq, d)))
    k, v = dev_bf16(_normal(181, 1, (B, H, Lk, d))), dev_bf16(_normal(181, 2, (B, H, Lk, d)))
    kd, bd = torch.from_numpy(kinds).cuda(), torch.from_numpy(bits.view(np.int64)).cuda()
    note(f"plan d={d} Lq={Lq} Lk={Lk} causal={causal} p_tile={p_tile} bit_d={bit_d}")
    plan = rf_gpu.rf_attention_plan(kinds, bits, B, H, Lq, Lk, d, causal)
    t = {"tile": _timed_us(lambda: rf_gpu.rf_attention_fwd_bitmap(q, k, v, kd, bd, causal=causal)),
         "row": _timed_us(lambda: rf_gpu.rf_attention_fwd_rowwise(q, k, v, kd, bd, causal=causal))}
    note(f"  measured {t}, estimated tile {plan['est_tile_us']:.1f} row {plan['est_row_us']:.1f}, "
         f"pick {plan['kernel']}")
    assert t[plan["kernel"]] <= 1.25 * min(t.values())
