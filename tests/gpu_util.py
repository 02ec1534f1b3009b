"""Helpers shared by the GPU parity tests: device upload of the seeded inputs
and element-wise comparison against the fp64 oracle."""
import sys

import numpy as np

import oracle as O


def note(msg: str):
    """Name the case before a GPU step, flushed, so a crash still says which case ran."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host_f64(t) -> np.ndarray:
    """Exact fp64 copy of a device fp32 / bf16 tensor."""
    import torch
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.float().cpu().numpy().astype(np.float64)


def max_abs_err(got: np.ndarray, want: np.ndarray) -> float:
    """Max |got - want|; infinities must match exactly, NaN anywhere is an error."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    if np.isnan(got).any() or np.isnan(want).any():
        return float("inf")
    inf_g, inf_w = np.isinf(got), np.isinf(want)
    if not np.array_equal(inf_g, inf_w) or not np.array_equal(got[inf_g], want[inf_w]):
        return float("inf")
    fin = ~inf_g
    return float(np.max(np.abs(got[fin] - want[fin]))) if fin.any() else 0.0


def assert_close(got, want, tol, what):
    err = max_abs_err(got, want)
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"
    return err
