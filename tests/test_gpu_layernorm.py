"""GPU parity of the row layer normalisation against the fp64 oracle.

Gates: fp32 y 1e-5 max abs; bf16 y within one bf16 rounding of the exact
value (2^-8 relative) plus 1e-5; mean and rstd (fp32) 1e-6 relative + 1e-6.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, dev_bf16, dev_f32, host_f64, note

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (3, 7), (5, 100), (4, 1024), (3, 4095), (2, 4096), (2, 32768), (2, 65536), (2, 65540),
          (2, 70001), (300, 33), (3, 16389), (3, 16383), (2, 32776)]


def _rows(seed, rows, cols, offset_scale=50.0):
    r = W.rng(seed, rows, cols)
    return (r.standard_normal((rows, cols)) * 2 + r.uniform(-offset_scale, offset_scale, (rows, 1))).astype(np.float32)


def _check(rf_gpu, x, dtype, gamma, beta, eps, tag):
    import torch
    xs = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    xd = dev_bf16(xs) if dtype == "bf16" else dev_f32(xs)
    g = None if gamma is None else torch.from_numpy(gamma).cuda()
    b = None if beta is None else torch.from_numpy(beta).cuda()
    note(f"layernorm {tag} {x.shape} {dtype}")
    y, mean, rstd = rf_gpu.rf_layernorm_rows(xd, g, b, eps=eps)
    xw = O.bf16_bits_to_f64(xs) if dtype == "bf16" else xs.astype(np.float64)
    ry, rm, rr = O.layernorm_rows(xw, gamma, beta, eps)
    got = host_f64(y)
    if dtype == "f32":
        assert_close(got, ry, 1e-5, f"layernorm y {tag}")
    else:
        assert np.all(np.abs(got - ry) <= np.abs(ry) * 2.0 ** -8 + 1e-5), f"layernorm bf16 y {tag}"
    for name, g_, r_ in (("mean", host_f64(mean), rm), ("rstd", host_f64(rstd), rr)):
        assert np.all(np.abs(g_ - r_) <= 1e-6 * np.abs(r_) + 1e-6), f"layernorm {name} {tag}"


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layernorm_rows(rf_gpu, rows, cols, dtype):
    x = _rows(140, rows, cols)
    g, b = W.layernorm_affine(141, cols)
    _check(rf_gpu, x, dtype, g, b, 1e-5, "affine")


@pytest.mark.parametrize("rows,cols", [(4, 1024), (3, 70001), (7, 33)])
def test_layernorm_without_affine(rf_gpu, rows, cols):
    _check(rf_gpu, _rows(142, rows, cols), "f32", None, None, 1e-3, "no affine")


@pytest.mark.parametrize("offset", [1000.0, -1000.0, 80.0])
def test_layernorm_large_offsets(rf_gpu, offset):
    """Rows far from zero: the statistics must not lose the spread."""
    r = W.rng(143, int(abs(offset)))
    x = (r.standard_normal((6, 5000)) + offset).astype(np.float32)
    g, b = W.layernorm_affine(144, 5000)
    _check(rf_gpu, x, "f32", g, b, 1e-5, f"offset {offset}")


def test_layernorm_constant_rows(rf_gpu):
    """Zero variance: y = beta exactly, rstd = 1/sqrt(eps)."""
    import torch
    x = np.full((3, 4096), 7.25, np.float32)
    x[1] = -3.5
    g, b = W.layernorm_affine(145, 4096)
    note("layernorm constant rows")
    y, mean, rstd = rf_gpu.rf_layernorm_rows(dev_f32(x), torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda(),
                                             eps=0.25)
    assert np.array_equal(host_f64(y), np.broadcast_to(b.astype(np.float64), (3, 4096)))
    assert np.allclose(host_f64(rstd), 2.0, rtol=0, atol=1e-6)
    assert np.allclose(host_f64(mean), [7.25, -3.5, 7.25], rtol=0, atol=1e-6)


@pytest.mark.parametrize("cols", [5, 255, 257, 1023, 4097, 8191, 16385, 32767])
def test_layernorm_ragged_widths(rf_gpu, cols):
    """fp32 rows whose width is not a multiple of 4 (16-byte vectors with the
    last one straddling the row's end; rows start only 4-byte aligned), at
    every register-table boundary, with gamma and beta: against the oracle."""
    import torch
    rows = 3
    x = W.softmax_rows_input(7, rows, cols)
    g, b = W.layernorm_affine(7, cols)
    note(f"layernorm ragged cols={cols}")
    y, mean, rstd = rf_gpu.rf_layernorm_rows(dev_f32(x), torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda(),
                                             eps=1e-5)
    ry, rm, rr = O.layernorm_rows(x.astype(np.float64), g, b, 1e-5)
    assert_close(host_f64(y), ry, 1e-5, f"y cols={cols}")
    assert np.all(np.abs(host_f64(mean) - rm) <= 1e-6 * np.abs(rm) + 1e-6)
    assert np.all(np.abs(host_f64(rstd) - rr) <= 1e-6 * np.abs(rr) + 1e-6)


@pytest.mark.parametrize("cols", [6, 250, 1022, 4094, 16386, 32766])
def test_layernorm_ragged_even_widths_bf16(rf_gpu, cols):
    """bf16 rows of even width not a multiple of 8 (16-byte vectors, the last
    one straddling the row's end on a dword boundary), with gamma and beta."""
    g, b = W.layernorm_affine(7, cols)
    _check(rf_gpu, _rows(7, 3, cols), "bf16", g, b, 1e-5, f"ragged bf16 cols={cols}")
