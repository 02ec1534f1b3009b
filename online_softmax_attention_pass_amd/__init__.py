"""Python binding of librf, the MI355X online-softmax attention library.

Argument marshalling only: each function checks tensor shapes, dtypes and
devices, then passes device pointers, sizes and the current HIP stream to the
C entry point of the same name declared in ``include/rf.h``. Every step of
the computation runs in the HIP kernels; there is no fallback of any kind, and
a missing ``librf.so`` is an error.

Build the library with ``python -m online_softmax_attention_pass_amd.build``.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "RF_F32", "RF_BF16", "RFError", "load", "library_path",
    "rf_softmax_rows", "rf_layernorm_rows", "rf_attention_fwd", "rf_attention_fwd_bitmap", "rf_attention_fwd_mod",
    "rf_attention_decode_splitkv", "rf_attention_decode_splitkv_noalloc",
    "rf_attention_decode_splitkv_workspace_size", "rf_attention_decode_gqa", "rf_attention_decode_gqa_workspace_size",
    "rf_lse_merge", "rf_moe_route", "rf_attention_fwd_rowwise", "rf_attention_plan", "rf_abi_version",
]

RF_F32, RF_BF16 = 0, 1
RF_OK, RF_ERR_INVALID_ARG, RF_ERR_UNSUPPORTED, RF_ERR_WORKSPACE, RF_ERR_HIP = 0, 1, 2, 3, 4
MASK_TILE = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def library_path() -> str:
    return os.environ.get("RF_LIBRARY", os.path.join(_HERE, "librf.so"))


class RFError(RuntimeError):
    def __init__(self, status: int, fn: str, message: str):
        self.status = status
        super().__init__(f"{fn} failed with {status}: {message}")


def load():
    """Load librf.so and declare its C signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"librf.so not found at {path}; build it with "
                           f"`python -m online_softmax_attention_pass_amd.build`")
    # One HIP runtime per process: torch ships its own libamdhip64 and
    # libhsa-runtime64, under the same sonames as the system's. Loaded first,
    # torch's copies satisfy librf's dependencies by soname; loaded after
    # librf, they would come in as a second runtime beside the system's, and
    # librf's calls would then find no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "rf_softmax_rows": ([P, P, I64, I64, I, P], I),
        "rf_layernorm_rows": ([P, P, P, P, P, P, I64, I64, F, I, P], I),
        "rf_attention_fwd": ([P, P, P, P, P, I, I, I, I, I, F, I, P, I, P], I),
        "rf_attention_fwd_bitmap": ([P, P, P, P, P, I, I, I, I, I, F, I, P, P, I, P], I),
        "rf_attention_fwd_mod": ([P, P, P, P, P, I, I, I, I, I, F, I, P, I, P, F, I, P], I),
        "rf_attention_decode_splitkv_workspace_size": ([I, I, I, I], SZ),
        "rf_attention_decode_splitkv": ([P, P, P, P, P, I, I, I, I, F, I, P, SZ, I, P], I),
        "rf_attention_decode_splitkv_noalloc": ([P, P, P, P, P, I, I, I, I, F, I, I, P], I),
        "rf_attention_decode_gqa_workspace_size": ([I, I, I, I], SZ),
        "rf_attention_decode_gqa": ([P, P, P, P, P, I, I, I, I, I, F, I, P, SZ, I, P], I),
        "rf_lse_merge": ([P, P, P, P, I64, I, I, I, P], I),
        "rf_moe_route": ([P, P, P, I64, I, I, I, I, P], I),
        "rf_attention_fwd_rowwise": ([P, P, P, P, P, I, I, I, I, I, F, I, P, P, I, P], I),
        "rf_attention_plan": ([P, P, I, I, I, I, I, I, P, P, P, P, P], I),
        "rf_status_string": ([I], ctypes.c_char_p),
        "rf_last_error_message": ([], ctypes.c_char_p),
        "rf_abi_version": ([], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int, fn: str):
    if status != RF_OK:
        lib = load()
        raise RFError(status, fn, lib.rf_last_error_message().decode())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return RF_F32
    if t.dtype == torch.bfloat16:
        return RF_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _dev(*ts):
    """The index of the one GPU all given tensors are on (None entries are skipped)."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        i = t.get_device()
        if dev is None:
            dev = i
        elif i != dev:
            raise ValueError("all tensors must be on one device")
    return dev


_raw_stream = None


def _stream(dev: int):
    """torch's current stream on device index dev, as the raw hipStream_t value.
    (The raw query skips building a Stream object: small calls are paced by this
    host path.)"""
    global _raw_stream
    if _raw_stream is None:
        torch = _torch()
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None) or \
            (lambda i: torch.cuda.current_stream(i).cuda_stream)
    return _raw_stream(dev)


def _ptr(t):
    """Device address of a tensor's data, or None (NULL) for a missing or empty tensor."""
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _check_out(o, shape, dtype, what="out"):
    """A caller-supplied output must have the exact shape and dtype the kernel writes:
    the C ABI sees only a pointer, so a smaller or narrower tensor would be overrun."""
    if tuple(o.shape) != tuple(shape) or o.dtype != dtype:
        raise ValueError(f"{what} must be {dtype} {tuple(shape)}, got {o.dtype} {tuple(o.shape)}")


def _check_same_dtype(q, *ts):
    for t in ts:
        if t.dtype != q.dtype:
            raise ValueError("q, k, v must share a dtype")


def rf_abi_version() -> int:
    return load().rf_abi_version()


def rf_softmax_rows(x, out=None):
    """Safe softmax over the last dimension of a contiguous fp32 / bf16 tensor."""
    torch = _torch()
    lib = load()
    if x.dim() < 1 or x.shape[-1] < 1:
        raise ValueError("x needs a non-empty last dimension")
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    dev = _dev(x, y)
    cols = x.shape[-1]
    rows = x.numel() // cols
    _check(lib.rf_softmax_rows(_ptr(x), _ptr(y), rows, cols, _dtype_code(x), _stream(dev)), "rf_softmax_rows")
    return y


def rf_layernorm_rows(x, gamma=None, beta=None, eps=1e-5, out=None, mean=None, rstd=None, want_stats=True):
    """Row layer normalisation of x [rows, cols] (fp32 or bf16); gamma, beta fp32 [cols] or None.

    Returns (y, mean, rstd): y like x; mean and rstd fp32 [rows] (None if want_stats is False).
    """
    torch = _torch()
    lib = load()
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [rows, cols] tensor")
    rows, cols = x.shape
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (cols,) or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous fp32 [{cols}]")
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous():
        raise ValueError("out must match x")
    if want_stats:
        mean = torch.empty(rows, dtype=torch.float32, device=x.device) if mean is None else mean
        rstd = torch.empty(rows, dtype=torch.float32, device=x.device) if rstd is None else rstd
    for name, t in (("mean", mean), ("rstd", rstd)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (rows,)):
            raise ValueError(f"{name} must be fp32 [{rows}]")
    dev = _dev(x, gamma, beta, y, mean, rstd)
    st = lib.rf_layernorm_rows(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd), rows, cols,
                               float(eps), _dtype_code(x), _stream(dev))
    _check(st, "rf_layernorm_rows")
    return y, mean, rstd


def rf_attention_fwd(q, k, v, scale=None, causal=False, block_mask=None, out=None, lse=None, want_lse=True):
    """Attention forward. q [B,H,Lq,d]; k, v [B,H,Lk,d]; block_mask uint8 [ceil(Lq/64), ceil(Lk/64)] or None.

    Returns (o, lse) with o like q and lse fp32 [B,H,Lq] (None if want_lse is False).
    """
    torch = _torch()
    lib = load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if k.shape != (B, H, Lk, d) or v.shape != (B, H, Lk, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    if block_mask is not None:
        want = (math.ceil(Lq / MASK_TILE), math.ceil(Lk / MASK_TILE))
        if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != want:
            raise ValueError(f"block_mask must be uint8 {want}")
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is None and want_lse:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, Lq) or lse.dtype != torch.float32):
        raise ValueError("lse must be fp32 [B, H, Lq]")
    dev = _dev(q, k, v, o, lse, block_mask)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.rf_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Lq, Lk, d, float(scale),
                              1 if causal else 0, _ptr(block_mask), _dtype_code(q), _stream(dev))
    _check(st, "rf_attention_fwd")
    return o, lse


def rf_attention_fwd_mod(q, k, v, scale=None, causal=False, block_mask=None, window=0, alibi_slopes=None, softcap=0.0,
                         out=None, lse=None, want_lse=True):
    """Attention with score modifications: softcap (tanh), ALiBi bias (alibi_slopes fp32 [H] on the GPU),
    element-level sliding window of `window` keys. Shapes and outputs as rf_attention_fwd."""
    torch = _torch()
    lib = load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if k.shape != (B, H, Lk, d) or v.shape != (B, H, Lk, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    if block_mask is not None:
        want = (math.ceil(Lq / MASK_TILE), math.ceil(Lk / MASK_TILE))
        if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != want:
            raise ValueError(f"block_mask must be uint8 {want}")
    if alibi_slopes is not None and (alibi_slopes.dtype != torch.float32 or tuple(alibi_slopes.shape) != (H,)):
        raise ValueError(f"alibi_slopes must be fp32 [{H}]")
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is None and want_lse:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_out(lse, (B, H, Lq), torch.float32, "lse")
    dev = _dev(q, k, v, o, lse, block_mask, alibi_slopes)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.rf_attention_fwd_mod(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Lq, Lk, d, float(scale),
                                  1 if causal else 0, _ptr(block_mask), int(window), _ptr(alibi_slopes),
                                  float(softcap), _dtype_code(q), _stream(dev))
    _check(st, "rf_attention_fwd_mod")
    return o, lse


def rf_attention_fwd_bitmap(q, k, v, tile_kind, tile_bits, scale=None, causal=False, out=None, lse=None,
                            want_lse=True):
    """Attention forward with element bitmaps inside partial tiles.

    tile_kind uint8 [ceil(Lq/64), ceil(Lk/64)] (0 empty, 1 full, other = partial);
    tile_bits int64 or uint64 [ceil(Lq/64), ceil(Lk/64), 64]: word r of a tile is
    query row r's visibility of the tile's 64 keys (bit j). Returns (o, lse).
    """
    torch = _torch()
    lib = load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if k.shape != (B, H, Lk, d) or v.shape != (B, H, Lk, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    want = (math.ceil(Lq / MASK_TILE), math.ceil(Lk / MASK_TILE))
    if tile_kind.dtype != torch.uint8 or tuple(tile_kind.shape) != want:
        raise ValueError(f"tile_kind must be uint8 {want}")
    if tile_bits.dtype not in (torch.int64, getattr(torch, "uint64", torch.int64)) or \
            tuple(tile_bits.shape) != want + (MASK_TILE,) or not tile_bits.is_contiguous():
        raise ValueError(f"tile_bits must be contiguous 64-bit {want + (MASK_TILE,)}")
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is None and want_lse:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, Lq) or lse.dtype != torch.float32):
        raise ValueError("lse must be fp32 [B, H, Lq]")
    dev = _dev(q, k, v, o, lse, tile_kind, tile_bits)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.rf_attention_fwd_bitmap(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Lq, Lk, d, float(scale),
                                     1 if causal else 0, _ptr(tile_kind), _ptr(tile_bits), _dtype_code(q),
                                     _stream(dev))
    _check(st, "rf_attention_fwd_bitmap")
    return o, lse


def rf_attention_decode_splitkv_workspace_size(B: int, H: int, d: int, num_splits: int) -> int:
    return int(load().rf_attention_decode_splitkv_workspace_size(B, H, d, num_splits))


def rf_attention_decode_splitkv(q, k, v, scale=None, num_splits=16, workspace=None, out=None, lse=None,
                                want_lse=True):
    """Split-KV decode. q [B,H,1,d]; k, v [B,H,Lk,d] (bf16). Returns (o [B,H,1,d], lse [B,H])."""
    torch = _torch()
    lib = load()
    if q.dim() != 4 or q.shape[2] != 1:
        raise ValueError("q must be [B, H, 1, d]")
    B, H, _, d = q.shape
    Lk = k.shape[2]
    if k.shape != (B, H, Lk, d) or v.shape != (B, H, Lk, d):
        raise ValueError("k, v must be [B, H, Lk, d] matching q")
    _check_same_dtype(q, k, v)
    ws_bytes = rf_attention_decode_splitkv_workspace_size(B, H, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q) if out is None else out
    _check_out(o, q.shape, q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_out(lse, (B, H), torch.float32, "lse")
    dev = _dev(q, k, v, o, lse, workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = workspace.numel() * workspace.element_size()
    st = lib.rf_attention_decode_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Lk, d,
                                         float(scale), num_splits, _ptr(workspace), nbytes, _dtype_code(q),
                                         _stream(dev))
    _check(st, "rf_attention_decode_splitkv")
    return o, lse


def rf_attention_decode_splitkv_noalloc(q, k, v, scale=None, num_splits=16, out=None, lse=None, want_lse=True):
    """Split-KV decode with the partials in the library's own device scratch (no
    workspace, nothing allocated by the library). Same result as
    rf_attention_decode_splitkv. Calls that overlap on one GPU race."""
    torch = _torch()
    lib = load()
    if q.dim() != 4 or q.shape[2] != 1:
        raise ValueError("q must be [B, H, 1, d]")
    B, H, _, d = q.shape
    Lk = k.shape[2]
    if k.shape != (B, H, Lk, d) or v.shape != (B, H, Lk, d):
        raise ValueError("k, v must be [B, H, Lk, d] matching q")
    _check_same_dtype(q, k, v)
    o = torch.empty_like(q) if out is None else out
    _check_out(o, q.shape, q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_out(lse, (B, H), torch.float32, "lse")
    dev = _dev(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.rf_attention_decode_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Lk, d,
                                                 float(scale), num_splits, _dtype_code(q), _stream(dev))
    _check(st, "rf_attention_decode_splitkv_noalloc")
    return o, lse


def rf_attention_decode_gqa_workspace_size(B: int, Hq: int, d: int, num_splits: int) -> int:
    return int(load().rf_attention_decode_gqa_workspace_size(B, Hq, d, num_splits))


def rf_attention_decode_gqa(q, k, v, scale=None, num_splits=1, workspace=None, out=None, lse=None, want_lse=True):
    """Grouped-query decode. q [B,Hq,d]; k, v [B,Hkv,Lk,d] (bf16), Hq a multiple of Hkv.
    Returns (o [B,Hq,d], lse [B,Hq])."""
    torch = _torch()
    lib = load()
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and k, v [B, Hkv, Lk, d]")
    B, Hq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Lk, d) or v.shape != (B, Hkv, Lk, d):
        raise ValueError("k, v must be [B, Hkv, Lk, d] matching q")
    _check_same_dtype(q, k, v)
    ws_bytes = rf_attention_decode_gqa_workspace_size(B, Hq, d, num_splits)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q) if out is None else out
    _check_out(o, q.shape, q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_out(lse, (B, Hq), torch.float32, "lse")
    dev = _dev(q, k, v, o, lse, workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.rf_attention_decode_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Lk, d,
                                     float(scale), num_splits, _ptr(workspace), nbytes, _dtype_code(q),
                                     _stream(dev))
    _check(st, "rf_attention_decode_gqa")
    return o, lse


def rf_lse_merge(o_parts, lse_parts, out_dtype=None, out=None, lse=None, want_lse=True):
    """Merge normalised partials: o_parts fp32 [n, S, d], lse_parts fp32 [n, S] -> (o [n, d], lse [n])."""
    torch = _torch()
    lib = load()
    n, S, d = o_parts.shape
    if lse_parts.shape != (n, S):
        raise ValueError("lse_parts must be [n, S]")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("partials must be fp32")
    out_dtype = (torch.float32 if out is None else out.dtype) if out_dtype is None else out_dtype
    o = torch.empty((n, d), dtype=out_dtype, device=o_parts.device) if out is None else out
    _check_out(o, (n, d), out_dtype)
    if lse is None and want_lse:
        lse = torch.empty((n,), dtype=torch.float32, device=o_parts.device)
    if lse is not None:
        _check_out(lse, (n,), torch.float32, "lse")
    dev = _dev(o_parts, lse_parts, o, lse)
    st = lib.rf_lse_merge(_ptr(o_parts), _ptr(lse_parts), _ptr(o), _ptr(lse), n, S, d, _dtype_code(o),
                          _stream(dev))
    _check(st, "rf_lse_merge")
    return o, lse


def rf_moe_route(logits, k, renorm=True, out_idx=None, out_w=None):
    """Mixture-of-experts routing of logits [T, E] (fp32 or bf16): the k most probable experts of each
    token under the softmax. Returns (idx int32 [T, k], w fp32 [T, k])."""
    torch = _torch()
    lib = load()
    if logits.dim() != 2:
        raise ValueError("logits must be [T, E]")
    T, E = logits.shape
    idx = torch.empty((T, k), dtype=torch.int32, device=logits.device) if out_idx is None else out_idx
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device) if out_w is None else out_w
    if idx.shape != (T, k) or idx.dtype != torch.int32 or w.shape != (T, k) or w.dtype != torch.float32:
        raise ValueError("out_idx must be int32 [T, k] and out_w fp32 [T, k]")
    dev = _dev(logits, idx, w)
    st = lib.rf_moe_route(_ptr(logits), _ptr(idx), _ptr(w), T, E, int(k), 1 if renorm else 0, _dtype_code(logits),
                          _stream(dev))
    _check(st, "rf_moe_route")
    return idx, w


def rf_attention_fwd_rowwise(q, k, v, tile_kind=None, tile_bits=None, scale=None, causal=False, out=None, lse=None,
                             want_lse=True):
    """Row-wise masked attention (bf16): the result of rf_attention_fwd_bitmap by the row kernel.
    tile_kind uint8 [ceil(Lq/64), ceil(Lk/64)] and tile_bits int64/uint64 [.., .., 64] on the GPU, or None."""
    torch = _torch()
    lib = load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if k.shape != (B, H, Lk, d) or v.shape != (B, H, Lk, d):
        raise ValueError("k, v must be [B, H, Lk, d] matching q")
    nI, nJ = math.ceil(Lq / MASK_TILE), math.ceil(Lk / MASK_TILE)
    if tile_kind is not None and (tile_kind.dtype != torch.uint8 or tuple(tile_kind.shape) != (nI, nJ)):
        raise ValueError(f"tile_kind must be uint8 {(nI, nJ)}")
    if tile_bits is not None and (tile_bits.element_size() != 8 or tuple(tile_bits.shape) != (nI, nJ, MASK_TILE)):
        raise ValueError(f"tile_bits must be 64-bit {(nI, nJ, MASK_TILE)}")
    _check_same_dtype(q, k, v)
    o = torch.empty_like(q) if out is None else out
    _check_out(o, q.shape, q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_out(lse, (B, H, Lq), torch.float32, "lse")
    dev = _dev(q, k, v, o, lse, tile_kind, tile_bits)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.rf_attention_fwd_rowwise(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Lq, Lk, d, float(scale),
                                      1 if causal else 0, _ptr(tile_kind), _ptr(tile_bits), _dtype_code(q),
                                      _stream(dev))
    _check(st, "rf_attention_fwd_rowwise")
    return o, lse


def rf_attention_plan(tile_kind, tile_bits, B, H, Lq, Lk, d, causal):
    """The analytic kernel choice from HOST (numpy) copies of a mask (either may be None).
    Returns dict(kernel="tile"|"row", est_tile_us, est_row_us, tile_work, row_batches)."""
    import numpy as np
    lib = load()
    kinds = None if tile_kind is None else np.ascontiguousarray(tile_kind, dtype=np.uint8)
    bits = None if tile_bits is None else np.ascontiguousarray(tile_bits).view(np.uint64)
    kern, et, er = ctypes.c_int(0), ctypes.c_double(0), ctypes.c_double(0)
    tw, rg = ctypes.c_int64(0), ctypes.c_int64(0)
    hp = lambda a: ctypes.c_void_p(0) if a is None else a.ctypes.data_as(ctypes.c_void_p)
    st = lib.rf_attention_plan(hp(kinds), hp(bits), B, H, Lq, Lk, d, 1 if causal else 0, ctypes.byref(kern),
                               ctypes.byref(et), ctypes.byref(er), ctypes.byref(tw), ctypes.byref(rg))
    _check(st, "rf_attention_plan")
    return dict(kernel="row" if kern.value == 1 else "tile", est_tile_us=et.value, est_row_us=er.value,
                tile_work=tw.value, row_batches=rg.value)
