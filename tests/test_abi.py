"""C-ABI checks that need no GPU: the library loads, exports every function
``include/rf.h`` declares, and rejects bad arguments before any HIP call.

Every call here either fails validation or has no work (rows = 0, B = 0, ...),
so nothing reaches the HIP runtime.
"""
import ctypes
import os
import re

import pytest

import online_softmax_attention_pass_amd as rf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rf.h")

OK, INVALID, UNSUP, WS = rf.RF_OK, rf.RF_ERR_INVALID_ARG, rf.RF_ERR_UNSUPPORTED, rf.RF_ERR_WORKSPACE
F32, BF16 = rf.RF_F32, rf.RF_BF16
P = ctypes.c_void_p
FAKE = P(0x10000)            # a non-NULL, 256-byte-aligned address that is never dereferenced
NUL = P(0)


@pytest.fixture(scope="module")
def lib():
    return rf.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rf_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"rf_softmax_rows", "rf_attention_fwd", "rf_attention_decode_splitkv", "rf_lse_merge"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"librf.so does not export {n}"


def test_exports_no_cxx_names_for_the_abi(lib):
    # the entry points are plain C symbols (no mangling)
    out = os.popen(f"nm -D --defined-only {rf.library_path()}").read()
    for n in declared_functions():
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_abi_version(lib):
    assert lib.rf_abi_version() == 7


def test_status_strings(lib):
    assert lib.rf_status_string(OK) == b"RF_OK"
    assert lib.rf_status_string(INVALID) == b"RF_ERR_INVALID_ARG"
    assert lib.rf_status_string(UNSUP) == b"RF_ERR_UNSUPPORTED"
    assert lib.rf_status_string(WS) == b"RF_ERR_WORKSPACE"
    assert lib.rf_status_string(rf.RF_ERR_HIP) == b"RF_ERR_HIP"
    assert lib.rf_status_string(99) == b"RF_UNKNOWN_STATUS"


def _msg(lib):
    return lib.rf_last_error_message().decode()


@pytest.mark.parametrize("args,code", [
    ((NUL, NUL, 4, 8, F32), INVALID),          # NULL with work
    ((FAKE, FAKE, -1, 8, F32), INVALID),       # rows < 0
    ((FAKE, FAKE, 4, 0, F32), INVALID),        # cols < 1
    ((FAKE, FAKE, 4, 8, 7), INVALID),          # dtype
    ((FAKE, FAKE, 1 << 40, 1 << 40, F32), INVALID),   # overflow
    ((FAKE, P(0x10001), 4, 8, F32), INVALID),  # misaligned fp32
    ((NUL, NUL, 0, 8, F32), OK),               # no rows: nothing to do
    ((NUL, NUL, 0, 8, BF16), OK),
])
def test_softmax_validation(lib, args, code):
    assert lib.rf_softmax_rows(*args, NUL) == code
    assert (_msg(lib) == "") == (code == OK)


@pytest.mark.parametrize("args,code", [
    ((NUL, NUL, NUL, NUL, NUL, NUL, 4, 8, 1e-5, F32), INVALID),        # NULL x, y with work
    ((FAKE, NUL, NUL, FAKE, NUL, NUL, -1, 8, 1e-5, F32), INVALID),     # rows < 0
    ((FAKE, NUL, NUL, FAKE, NUL, NUL, 4, 0, 1e-5, F32), INVALID),      # cols < 1
    ((FAKE, NUL, NUL, FAKE, NUL, NUL, 4, 8, -1.0, F32), INVALID),      # eps < 0
    ((FAKE, NUL, NUL, FAKE, NUL, NUL, 4, 8, float("nan"), F32), INVALID),
    ((FAKE, NUL, NUL, FAKE, NUL, NUL, 4, 8, 1e-5, 9), INVALID),        # dtype
    ((FAKE, NUL, NUL, FAKE, NUL, NUL, 1 << 40, 1 << 40, 1e-5, F32), INVALID),
    ((FAKE, P(0x10002), NUL, FAKE, NUL, NUL, 4, 8, 1e-5, F32), INVALID),   # misaligned gamma
    ((P(0x10001), NUL, NUL, FAKE, NUL, NUL, 4, 8, 1e-5, BF16), INVALID),   # misaligned bf16 x
    ((NUL, NUL, NUL, NUL, NUL, NUL, 0, 8, 1e-5, F32), OK),             # no rows
])
def test_layernorm_validation(lib, args, code):
    assert lib.rf_layernorm_rows(*args, NUL) == code
    assert (_msg(lib) == "") == (code == OK)
    if code != OK:
        assert "rf_layernorm_rows" in _msg(lib)


ATT = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=2, H=3, Lq=100, Lk=90, d=128, scale=0.1, causal=1,
           mask=NUL, dtype=BF16)


def att(lib, **kw):
    a = dict(ATT, **kw)
    return lib.rf_attention_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Lq"], a["Lk"],
                                a["d"], a["scale"], a["causal"], a["mask"], a["dtype"], NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), INVALID),
    (dict(B=-1), INVALID), (dict(H=-2), INVALID), (dict(Lq=-1), INVALID), (dict(Lk=-5), INVALID),
    (dict(d=0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(d=96), UNSUP), (dict(d=32), UNSUP), (dict(d=256), UNSUP),
    (dict(dtype=F32, d=129), UNSUP),
    (dict(q=NUL), INVALID), (dict(o=NUL), INVALID), (dict(k=NUL), INVALID), (dict(v=NUL), INVALID),
    (dict(q=P(0x10008)), UNSUP),                       # bf16 path needs 16-byte rows
    (dict(dtype=F32, d=33, q=P(0x10002)), INVALID),     # fp32 misaligned
    (dict(B=0), OK), (dict(H=0), OK), (dict(Lq=0), OK),
    (dict(B=0, q=NUL, k=NUL, v=NUL, o=NUL), OK),
    (dict(B=1 << 20, H=1 << 20, Lq=1 << 20), INVALID),  # overflow
    (dict(Lk=1 << 23), UNSUP),                           # one bf16 K head beyond 2^31 bytes
    (dict(Lk=(1 << 23) - 1, B=0), OK),
])
def test_attention_validation(lib, kw, code):
    assert att(lib, **kw) == code
    if code != OK:
        assert "rf_attention_fwd" in _msg(lib)


def att_mod(lib, **kw):
    a = dict(ATT, window=0, slopes=NUL, cap=0.0)
    a.update(kw)
    return lib.rf_attention_fwd_mod(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Lq"], a["Lk"],
                                    a["d"], a["scale"], a["causal"], a["mask"], a["window"], a["slopes"], a["cap"],
                                    a["dtype"], NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(window=-1), INVALID), (dict(cap=-1.0), INVALID), (dict(cap=float("nan")), INVALID),
    (dict(cap=float("inf")), INVALID), (dict(slopes=P(0x10002)), INVALID),
    (dict(dtype=7), INVALID), (dict(d=96), UNSUP), (dict(q=NUL), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(B=0, window=16, cap=30.0), OK), (dict(Lq=0, slopes=FAKE), OK),
])
def test_attention_mod_validation(lib, kw, code):
    assert att_mod(lib, **kw) == code
    if code != OK:
        assert "rf_attention_fwd_mod" in _msg(lib)


def att_bitmap(lib, **kw):
    a = dict(ATT, kinds=FAKE, bits=FAKE)
    a.update(kw)
    return lib.rf_attention_fwd_bitmap(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Lq"], a["Lk"],
                                       a["d"], a["scale"], a["causal"], a["kinds"], a["bits"], a["dtype"], NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(bits=NUL), INVALID), (dict(kinds=NUL), INVALID),
    (dict(bits=P(0x10008)), INVALID),                     # bitmaps must be 16-byte aligned
    (dict(dtype=5), INVALID), (dict(d=96), UNSUP), (dict(q=NUL), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(Lq=1 << 18, Lk=1 << 18), UNSUP),                # 4096 x 4096 tiles x 512 B > 2^32 bytes
    (dict(B=0), OK), (dict(B=0, q=NUL, k=NUL, v=NUL, o=NUL, kinds=NUL, bits=NUL), OK),
    (dict(Lq=0, bits=NUL), OK),
])
def test_attention_bitmap_validation(lib, kw, code):
    assert att_bitmap(lib, **kw) == code
    if code != OK:
        assert "rf_attention_fwd_bitmap" in _msg(lib)


def test_library_usable_after_error(lib):
    assert att(lib, d=96) == UNSUP
    assert _msg(lib) != ""
    assert att(lib, B=0) == OK
    assert _msg(lib) == ""


def test_decode_workspace_size(lib):
    B, H, d, S = 64, 32, 128, 16
    n = B * H * S
    want = -(-n * d * 4 // 256) * 256 + -(-n * 4 // 256) * 256
    assert lib.rf_attention_decode_splitkv_workspace_size(B, H, d, S) == want
    assert lib.rf_attention_decode_splitkv_workspace_size(1, 1, 64, 3) == 768 + 256
    assert lib.rf_attention_decode_splitkv_workspace_size(1, 1, 64, 5) == 1280 + 256
    assert lib.rf_attention_decode_splitkv_workspace_size(-1, 1, 64, 3) == 0
    assert lib.rf_attention_decode_splitkv_workspace_size(1, 1, 64, 0) == 0
    assert lib.rf_attention_decode_splitkv_workspace_size(1, 1, 64, 1025) == 0


DEC = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=4, H=2, Lk=1000, d=128, scale=0.1, S=16, ws=FAKE,
           ws_bytes=1 << 30, dtype=BF16)


def dec(lib, **kw):
    a = dict(DEC, **kw)
    return lib.rf_attention_decode_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Lk"],
                                           a["d"], a["scale"], a["S"], a["ws"], a["ws_bytes"], a["dtype"], NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=9), INVALID), (dict(B=-1), INVALID), (dict(Lk=-1), INVALID), (dict(d=0), INVALID),
    (dict(S=0), INVALID), (dict(S=1025), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(dtype=F32), UNSUP), (dict(d=96), UNSUP),
    (dict(q=NUL), INVALID), (dict(o=NUL), INVALID), (dict(k=NUL), INVALID),
    (dict(ws=NUL), WS), (dict(ws_bytes=100), WS), (dict(ws=P(0x10010)), WS),
    (dict(q=P(0x10008)), UNSUP),
    (dict(B=0), OK), (dict(H=0, ws=NUL, ws_bytes=0), OK),
])
def test_decode_validation(lib, kw, code):
    assert dec(lib, **kw) == code


def test_gqa_workspace_size(lib):
    B, Hq, d, S = 64, 64, 128, 4
    assert lib.rf_attention_decode_gqa_workspace_size(B, Hq, d, S) == \
        lib.rf_attention_decode_splitkv_workspace_size(B, Hq, d, S)
    assert lib.rf_attention_decode_gqa_workspace_size(B, Hq, d, 1) == 0      # written directly
    assert lib.rf_attention_decode_gqa_workspace_size(-1, Hq, d, 4) == 0
    assert lib.rf_attention_decode_gqa_workspace_size(1, 1, 64, 1025) == 0


GQA = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=4, Hq=16, Hkv=2, Lk=1000, d=128, scale=0.1, S=8, ws=FAKE,
           ws_bytes=1 << 30, dtype=BF16)


def gqa(lib, **kw):
    a = dict(GQA, **kw)
    return lib.rf_attention_decode_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Lk"],
                                       a["d"], a["scale"], a["S"], a["ws"], a["ws_bytes"], a["dtype"], NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=9), INVALID), (dict(B=-1), INVALID), (dict(Hq=-2), INVALID), (dict(Lk=-1), INVALID),
    (dict(Hkv=0), INVALID), (dict(Hkv=3), INVALID), (dict(Hkv=32), INVALID), (dict(d=0), INVALID),
    (dict(S=0), INVALID), (dict(S=1025), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(dtype=F32), UNSUP), (dict(d=96), UNSUP), (dict(Lk=1 << 23), UNSUP), (dict(B=1 << 27), UNSUP),
    (dict(q=NUL), INVALID), (dict(o=NUL), INVALID), (dict(k=NUL), INVALID), (dict(v=NUL), INVALID),
    (dict(lse=P(0x10002)), INVALID),
    (dict(ws=NUL), WS), (dict(ws_bytes=100), WS), (dict(ws=P(0x10010)), WS),
    (dict(k=P(0x10008)), UNSUP), (dict(o=P(0x10004)), UNSUP),
    (dict(B=0), OK), (dict(Hq=0, ws=NUL, ws_bytes=0), OK),
])
def test_gqa_validation(lib, kw, code):
    assert gqa(lib, **kw) == code
    if code != OK:
        assert "rf_attention_decode_gqa" in _msg(lib)


@pytest.mark.parametrize("args,code", [
    ((FAKE, FAKE, FAKE, FAKE, 10, 4, 128, 5), INVALID),      # out dtype
    ((FAKE, FAKE, FAKE, FAKE, -1, 4, 128, F32), INVALID),
    ((FAKE, FAKE, FAKE, FAKE, 10, 0, 128, F32), INVALID),
    ((FAKE, FAKE, FAKE, FAKE, 10, 1025, 128, F32), INVALID),
    ((FAKE, FAKE, FAKE, FAKE, 10, 4, 0, F32), INVALID),
    ((NUL, FAKE, FAKE, FAKE, 10, 4, 128, F32), INVALID),
    ((FAKE, NUL, FAKE, FAKE, 10, 4, 128, F32), INVALID),
    ((FAKE, FAKE, NUL, FAKE, 10, 4, 128, F32), INVALID),
    ((FAKE, FAKE, FAKE, FAKE, 1 << 50, 1000, 1000, F32), INVALID),
    ((NUL, NUL, NUL, NUL, 0, 4, 128, BF16), OK),
])
def test_lse_merge_validation(lib, args, code):
    assert lib.rf_lse_merge(*args, NUL) == code


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib
    monkeypatch.setenv("RF_LIBRARY", str(tmp_path / "missing.so"))
    mod = importlib.reload(rf)
    try:
        with pytest.raises(RuntimeError, match="librf.so not found"):
            mod.load()
    finally:
        monkeypatch.delenv("RF_LIBRARY")
        importlib.reload(rf)


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "online_softmax_attention_pass_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\bimport\s+oracle|\bfrom\s+oracle\b|oracle/", text), f


@pytest.mark.parametrize("args,code", [
    ((FAKE, FAKE, FAKE, 100, 64, 8, 1, 7), INVALID),            # dtype
    ((FAKE, FAKE, FAKE, -1, 64, 8, 1, F32), INVALID),
    ((FAKE, FAKE, FAKE, 100, 0, 1, 1, F32), INVALID),
    ((FAKE, FAKE, FAKE, 100, 64, 0, 1, F32), INVALID),
    ((FAKE, FAKE, FAKE, 100, 4, 5, 1, F32), INVALID),           # k > E
    ((FAKE, FAKE, FAKE, 100, 2048, 8, 1, F32), UNSUP),          # E > 1024
    ((FAKE, FAKE, FAKE, 100, 256, 33, 1, F32), UNSUP),          # k > 32
    ((NUL, FAKE, FAKE, 100, 64, 8, 1, F32), INVALID),
    ((FAKE, NUL, FAKE, 100, 64, 8, 1, BF16), INVALID),
    ((FAKE, FAKE, NUL, 100, 64, 8, 0, F32), INVALID),
    ((P(0x10002), FAKE, FAKE, 100, 64, 8, 1, F32), INVALID),    # fp32 logits misaligned
    ((FAKE, FAKE, FAKE, 1 << 62, 1024, 8, 1, F32), INVALID),    # overflow
    ((NUL, NUL, NUL, 0, 64, 8, 1, F32), OK),
])
def test_moe_route_validation(lib, args, code):
    assert lib.rf_moe_route(*args, NUL) == code
    if code != OK:
        assert "rf_moe_route" in _msg(lib)


# ---------------------------------------------------------------------------
# the analytic kernel choice (host only)
# ---------------------------------------------------------------------------

def _plan_counts_numpy(kinds, bits, Lq, Lk, d, causal):
    """Brute-force work counts: tiles per tile-kernel workgroup, and per row the
    batches of visible keys (16 at d = 128, 32 at d = 64) of the row kernel."""
    import numpy as np
    bm, kb = (128, 16) if d == 128 else (64, 32)
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    vis = np.ones((Lq, Lk), bool) if not causal else (j <= i + (Lk - Lq))
    kind = np.ones((Lq, Lk), np.uint8) if kinds is None else kinds[i // 64, j // 64]
    vis_k = vis & (kind != 0)
    if bits is not None:
        word = bits[i // 64, j // 64, i % 64]
        bit = ((word >> (j % 64).astype(np.uint64)) & np.uint64(1)) == 1
        vis_e = vis_k & ((kind == 1) | bit)
    else:
        vis_e = vis_k
    tiles = 0
    for q0 in range(0, Lq, bm):
        rows = slice(q0, min(Lq, q0 + bm))
        last = min(Lk - 1, (min(Lq, q0 + bm) - 1) + (Lk - Lq)) if causal else Lk - 1
        for J in range(0, last // 64 + 1 if last >= 0 else 0):
            if (kind[rows, J * 64:(J + 1) * 64] != 0).any():
                tiles += bm // 64
    batches = int(sum(-(-int(n) // kb) for n in vis_e.sum(axis=1)))
    return tiles, batches


@pytest.mark.parametrize("Lq,Lk,d,causal", [(300, 500, 128, True), (300, 500, 64, True), (130, 700, 128, False),
                                           (64, 2048, 64, True), (1, 200, 128, True)])
def test_plan_counts_match_brute_force(Lq, Lk, d, causal):
    import numpy as np
    r = np.random.default_rng(Lq + Lk + d)
    nI, nJ = -(-Lq // 64), -(-Lk // 64)
    kinds = r.choice([0, 1, 2, 5], size=(nI, nJ), p=[0.4, 0.2, 0.3, 0.1]).astype(np.uint8)
    bits = (r.integers(0, 2 ** 62, size=(nI, nJ, 64), dtype=np.uint64) & r.integers(0, 2 ** 62, size=(nI, nJ, 64),
                                                                                    dtype=np.uint64))
    p = rf.rf_attention_plan(kinds, bits, 2, 3, Lq, Lk, d, causal)
    assert (p["tile_work"], p["row_batches"]) == _plan_counts_numpy(kinds, bits, Lq, Lk, d, causal)
    p0 = rf.rf_attention_plan(None, None, 1, 1, Lq, Lk, d, causal)     # dense
    assert (p0["tile_work"], p0["row_batches"]) == _plan_counts_numpy(None, None, Lq, Lk, d, causal)


def test_plan_choices_at_the_extremes():
    import numpy as np
    # dense causal prefill: the tile kernel
    assert rf.rf_attention_plan(None, None, 4, 32, 4096, 4096, 128, True)["kernel"] == "tile"
    # a few scattered keys per row over long keys: the row kernel
    Lq, Lk = 256, 16384
    nI, nJ = Lq // 64, Lk // 64
    kinds = np.full((nI, nJ), 2, np.uint8)
    bits = np.zeros((nI, nJ, 64), np.uint64)
    r = np.random.default_rng(5)
    for I in range(nI):
        for rr in range(64):
            for J in r.choice(nJ, 4, replace=False):
                bits[I, J, rr] |= np.uint64(1) << np.uint64(r.integers(64))
    p = rf.rf_attention_plan(kinds, bits, 1, 8, Lq, Lk, 128, False)
    assert p["kernel"] == "row" and p["est_row_us"] < p["est_tile_us"]


@pytest.mark.parametrize("args,code", [
    ((NUL, NUL, 1, 1, 64, 64, 128, 1, NUL, NUL, NUL, NUL, NUL), INVALID),     # NULL kernel out
    ((NUL, FAKE, 1, 1, 64, 64, 128, 1, "k", NUL, NUL, NUL, NUL), INVALID),    # bits without kinds
    ((NUL, NUL, 1, 1, 64, 64, 96, 1, "k", NUL, NUL, NUL, NUL), UNSUP),
    ((NUL, NUL, -1, 1, 64, 64, 128, 1, "k", NUL, NUL, NUL, NUL), INVALID),
])
def test_plan_validation(lib, args, code):
    kern = ctypes.c_int(0)
    args = tuple(ctypes.byref(kern) if a == "k" else a for a in args)
    assert lib.rf_attention_plan(*args) == code


ROW = dict(ATT, kinds=NUL, bits=NUL)


def att_row(lib, **kw):
    a = dict(ROW, **kw)
    return lib.rf_attention_fwd_rowwise(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Lq"], a["Lk"],
                                        a["d"], a["scale"], a["causal"], a["kinds"], a["bits"], a["dtype"], NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=9), INVALID), (dict(B=-1), INVALID), (dict(d=0), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(dtype=F32), UNSUP), (dict(d=96), UNSUP), (dict(q=NUL), INVALID), (dict(k=NUL), INVALID),
    (dict(o=P(0x10008)), UNSUP), (dict(bits=FAKE), INVALID), (dict(bits=P(0x10004), kinds=FAKE), INVALID),
    (dict(B=0), OK), (dict(Lq=0), OK), (dict(Lk=1 << 23), UNSUP),   # 2^23 keys x 128 x 2 B = 2^31 per head
])
def test_rowwise_validation(lib, kw, code):
    assert att_row(lib, **kw) == code
    if code != OK:
        assert "rf_attention_fwd_rowwise" in _msg(lib)


# ---------------------------------------------------------------------------
# Binding checks on caller-supplied outputs: the C ABI sees only pointers, so
# the binding must refuse an output of the wrong shape or dtype before the
# call (CPU tensors: the checks run before the device check).
# ---------------------------------------------------------------------------

def _t(*shape, dtype="bf16"):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


@pytest.mark.parametrize("case", ["o_shape", "o_dtype", "lse_shape", "lse_dtype", "kv_dtype"])
def test_binding_decode_splitkv_checks_outputs(case):
    q, k, v = _t(2, 3, 1, 64), _t(2, 3, 100, 64), _t(2, 3, 100, 64)
    kw = {}
    if case == "o_shape":
        kw["out"] = _t(2, 3, 1, 32)
    elif case == "o_dtype":
        kw["out"] = _t(2, 3, 1, 64, dtype="f32")
    elif case == "lse_shape":
        kw["lse"] = _t(2, 2, dtype="f32")
    elif case == "lse_dtype":
        kw["lse"] = _t(2, 3)
    else:
        k = _t(2, 3, 100, 64, dtype="f32")
    with pytest.raises(ValueError):
        rf.rf_attention_decode_splitkv(q, k, v, num_splits=4, **kw)


@pytest.mark.parametrize("case", ["o_shape", "o_dtype", "lse_shape", "kv_dtype"])
def test_binding_decode_gqa_checks_outputs(case):
    q, k, v = _t(2, 8, 64), _t(2, 2, 100, 64), _t(2, 2, 100, 64)
    kw = {}
    if case == "o_shape":
        kw["out"] = _t(2, 4, 64)
    elif case == "o_dtype":
        kw["out"] = _t(2, 8, 64, dtype="f32")
    elif case == "lse_shape":
        kw["lse"] = _t(2, 2, dtype="f32")
    else:
        v = _t(2, 2, 100, 64, dtype="f32")
    with pytest.raises(ValueError):
        rf.rf_attention_decode_gqa(q, k, v, num_splits=2, **kw)


@pytest.mark.parametrize("case", ["o_shape", "o_dtype", "lse_shape", "lse_dtype"])
def test_binding_lse_merge_checks_outputs(case):
    op, lp = _t(5, 3, 64, dtype="f32"), _t(5, 3, dtype="f32")
    kw = {}
    if case == "o_shape":
        kw["out"] = _t(4, 64, dtype="f32")
    elif case == "o_dtype":
        kw.update(out=_t(5, 64, dtype="f32"), out_dtype=_t(1).dtype)
    elif case == "lse_shape":
        kw["lse"] = _t(3, dtype="f32")
    else:
        kw["lse"] = _t(5)
    with pytest.raises(ValueError):
        rf.rf_lse_merge(op, lp, **kw)


def test_binding_attention_mod_checks_lse():
    q = _t(1, 2, 70, 64)
    with pytest.raises(ValueError):
        rf.rf_attention_fwd_mod(q, q, q, window=16, lse=_t(1, 2, 69, dtype="f32"))
    with pytest.raises(ValueError):
        rf.rf_attention_fwd_mod(q, q, q, window=16, lse=_t(1, 2, 70))


@pytest.mark.parametrize("case", ["o_shape", "lse_shape", "kv_dtype"])
def test_binding_rowwise_checks_outputs(case):
    q = _t(1, 2, 70, 64)
    k = _t(1, 2, 70, 64)
    kw = {}
    if case == "o_shape":
        kw["out"] = _t(1, 2, 70, 32)
    elif case == "lse_shape":
        kw["lse"] = _t(1, 2, 71, dtype="f32")
    else:
        k = _t(1, 2, 70, 64, dtype="f32")
    with pytest.raises(ValueError):
        rf.rf_attention_fwd_rowwise(q, k, k, **kw)


def test_library_binds_to_torchs_hip_runtime():
    """Loading librf through the binding before anything touches torch still
    leaves ONE HIP runtime and one HSA runtime in the process (torch ships its
    own copies under the system's sonames; two runtimes in one process make
    librf's calls find no device)."""
    import subprocess
    import sys
    code = ("import online_softmax_attention_pass_amd as rf; rf.load(); import torch; "
            "maps = open('/proc/self/maps').read().split('\\n'); "
            "libs = {l.split()[-1] for l in maps if 'libamdhip64' in l or 'libhsa-runtime64' in l}; "
            "print(len([x for x in libs if 'amdhip64' in x]), len([x for x in libs if 'hsa-runtime64' in x]))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split()[-2:] == ["1", "1"], r.stdout
