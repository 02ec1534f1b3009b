"""GPU parity of mixture-of-experts routing (rf_moe_route) against the fp64
oracle.moe_route. The chosen experts are decided on the exact input logits
(the softmax is monotone), so indices must match exactly; weights (fp32) are
gated at 1e-5 max abs."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import dev_bf16, dev_f32, note

pytestmark = pytest.mark.gpu


def _check(rf_gpu, x, k, renorm, dtype, tag):
    import torch
    xs = W.f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)
    xd = dev_bf16(xs) if dtype == "bf16" else dev_f32(xs)
    note(f"moe route {tag} T={x.shape[0]} E={x.shape[1]} k={k} renorm={renorm} {dtype}")
    idx, w = rf_gpu.rf_moe_route(xd, k, renorm)
    torch.cuda.synchronize()
    xw = O.bf16_bits_to_f64(xs) if dtype == "bf16" else xs.astype(np.float64)
    ref_idx, ref_w = O.moe_route(xw, k, renorm)
    got_idx = idx.cpu().numpy()
    assert np.array_equal(got_idx, ref_idx), f"{tag}: {int((got_idx != ref_idx).sum())} indices differ"
    err = np.abs(w.cpu().numpy().astype(np.float64) - ref_w)
    assert np.all(err <= 1e-5), f"{tag}: weight error {err.max():.3e}"


CASES = [  # T, E, k, renorm, dtype
    (1000, 8, 2, True, "f32"), (777, 8, 8, False, "f32"), (500, 16, 4, True, "bf16"), (300, 33, 5, False, "f32"),
    (257, 64, 8, True, "f32"), (100, 100, 7, True, "f32"), (1000, 256, 8, True, "f32"), (200, 257, 32, False, "f32"),
    (50, 1024, 32, True, "bf16"), (3, 1, 1, True, "f32"), (5000, 160, 6, False, "bf16"), (64, 512, 1, False, "f32"),
]


@pytest.mark.parametrize("T,E,k,renorm,dtype", CASES)
def test_moe_route(rf_gpu, T, E, k, renorm, dtype):
    _check(rf_gpu, W.moe_logits(170, T, E), k, renorm, dtype, "random")


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (256, 8), (300, 16)])
def test_moe_route_ties_go_to_the_lower_expert(rf_gpu, E, k):
    """Logits rounded to multiples of 1/4: many exact ties inside the top k."""
    _check(rf_gpu, W.moe_logits(171, 2000, E, quantum=0.25), k, True, "f32", "ties")


@pytest.mark.parametrize("E,k", [(16, 4), (200, 8)])
def test_moe_route_masked_experts(rf_gpu, E, k):
    """Experts at -inf weigh 0; with fewer finite logits than k the rest are the
    lowest-index masked experts."""
    x0 = W.moe_logits(172, 512, E)
    x = x0.copy()
    r = W.rng(172, 99)
    x[r.uniform(size=x.shape) < 0.5] = -np.inf
    x[:, E - 1] = x0[:, E - 1]                        # no row entirely -inf (its weights would be NaN)
    x[:8, :] = -np.inf
    x[:8, :2] = 1.0                                   # two finite experts only
    _check(rf_gpu, x, k, False, "f32", "masked")


@pytest.mark.parametrize("offset", [1000.0, -1000.0])
def test_moe_route_large_offsets(rf_gpu, offset):
    _check(rf_gpu, W.moe_logits(173, 300, 128) + np.float32(offset), 8, True, "f32", f"offset {offset}")


def test_moe_route_is_deterministic(rf_gpu):
    import torch
    xd = dev_f32(W.moe_logits(174, 4096, 256))
    note("moe route determinism")
    a = rf_gpu.rf_moe_route(xd, 8, True)
    b = rf_gpu.rf_moe_route(xd, 8, True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", [8, 16])
def test_moe_route_top_experts_in_one_block(rf_gpu, dtype, k):
    """The k largest logits sit in one contiguous block of 16 experts, then in a
    block of experts 64 apart: each lane group that holds them must give up
    more of them than it keeps sorted at once (the rebuild path of E <= 256)."""
    x = W.moe_logits(175, 600, 256)
    x[:300, :16] += np.float32(20.0)
    x[300:, ::64] += np.float32(20.0)
    x[300:, 1::64] += np.float32(19.0)
    x[300:, 2::64] += np.float32(18.0)
    x[300:, 3::64] += np.float32(17.0)
    _check(rf_gpu, x, k, True, dtype, "one block")
