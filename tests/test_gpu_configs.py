"""Parity at the five workload sizes, in the launch configuration the benchmark times.

Inputs are the seeded draws of ``workloads`` at full size. For the five
workloads the oracle computes EVERY output (one head or block of rows per
task, over the host's cores) and the kernels' outputs are compared with it
element by element. Gates: fp32 outputs 1e-5, bf16 outputs 1e-2, LSE 1e-3
(max abs over all outputs). For the bf16 workloads the seed's output-rounding
floor max|bf16(O) - O| over all outputs is computed before the GPU call,
checked against the stored one, and printed beside the error. The extension
workloads and the long-sequence cases check sampled heads and rows.
"""
import json
import math
import os

import numpy as np
import pytest

import full_oracle as F
import oracle as O
import workloads as W
from gpu_util import assert_close, dev_bf16, dev_f32, host_f64, max_abs_err, note

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _report(name, err_o, err_l, ref_o=None):
    floor = "" if ref_o is None else f" bf16 floor {max_abs_err(O.round_to_bf16(ref_o), ref_o):.3e}"
    print(f"\n[parity] {name}: max|dO| {err_o:.3e} max|dLSE| {err_l:.3e}{floor}", flush=True)


def _same_again(first, again, what):
    """The kernels have no atomics and no order-dependent reductions, so a second
    call on the same inputs must give the same bits; a difference means a race
    (for instance a shared-memory tile read before another wave's load landed)."""
    import torch
    for a, b in zip(first, again):
        assert torch.equal(a, b), f"{what}: two calls on the same inputs differ"


def _qkv_full(cfg):
    c = W.CONFIGS[cfg]
    return [W.normal_tensor(c["seed"], tid, c["B"], c["H"], L, c["d"], c["dtype"])
            for tid, L in ((W.TID_Q, c.get("Lq", 1)), (W.TID_K, c["Lk"]), (W.TID_V, c["Lk"]))]


def test_single_head_attention_f32(rf_gpu):
    c = W.CONFIGS["attn_f32"]
    q, k, v = _qkv_full("attn_f32")
    note("single-head fp32 attention, full")
    o, lse = rf_gpu.rf_attention_fwd(dev_f32(q), dev_f32(k), dev_f32(v), scale=c["scale"], causal=False)
    ref_o, ref_lse = O.attention(q, k, v, c["scale"])
    e_o = assert_close(host_f64(o), ref_o, 1e-5, "attn_f32 O")
    e_l = assert_close(host_f64(lse), ref_lse, 1e-3, "attn_f32 LSE")
    _report("attn_f32", e_o, e_l)


def test_config2_softmax_rows(rf_gpu):
    """Every row of the 4096 x 32768 softmax against the oracle (row blocks
    over the host's cores), element by element at 1e-5."""
    import torch
    c = W.CONFIGS["softmax"]
    x = W.softmax_rows_input(c["seed"], c["rows"], c["cols"])
    note("softmax rows, full")
    xd = dev_f32(x)
    y = rf_gpu.rf_softmax_rows(xd)
    _same_again((y,), (rf_gpu.rf_softmax_rows(xd),), "softmax")
    sums = y.double().sum(dim=1)
    assert float((sums - 1).abs().max()) < 1e-4                  # every row sums to 1
    got = y.cpu().numpy()
    del y, xd
    err = 0.0
    for r0, r1, ref in F.softmax_reference_blocks("softmax"):
        err = max(err, max_abs_err(got[r0:r1].astype(np.float64), ref))
    _report(f"softmax (all {c['rows']} rows)", err, 0.0)
    assert err <= 1e-5


def _stored_floor(cfg):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "output_floors.json")
    return json.load(open(path))[cfg]


def _full_parity(cfg, o, lse, ref_o, ref_l, floor):
    got_o, got_l = host_f64(o), host_f64(lse)
    r = F.check_bf16_gates(cfg, got_o, got_l, ref_o, ref_l)
    _report(f"{cfg} (every output: {ref_o.size} of O, {ref_l.size} of LSE)", r["max_err_o"], r["max_err_lse"])
    print(f"[parity] {cfg}: full-output bf16 floor {floor['floor']:.3e} (at {floor['floor_at']}, "
          f"O = {floor['o_at_floor']:.4f}); max|O| {floor['max_abs_o']:.3f}", flush=True)
    for line in r["unattainable"]:
        print(f"[parity] {cfg}: {line}", flush=True)
    print(f"[parity] {cfg}: max|dO| over the {r['gated_outputs']} outputs whose floor is within the gate "
          f"{r['max_err_o_gated']:.3e}", flush=True)


@pytest.mark.parametrize("cfg", ["prefill", "sparse"])
def test_config_attention_bf16(rf_gpu, cfg):
    """Causal prefill (B4 H32 L4096 d128) and block-sparse (B2 H16 L8192 d64):
    the oracle first computes every output on the host's cores, with the
    seed's bf16 output-rounding floor (checked against the stored one); then
    the kernel's O and LSE are compared with it everywhere."""
    import torch
    c = W.CONFIGS[cfg]
    note(f"{cfg}: oracle over every head on the host")
    ref_o, ref_l = F.full_reference(cfg)
    floor = F.floor_summary(cfg, ref_o)
    print(f"\n[parity] {cfg}: bf16 floor before the GPU call {floor['floor']:.3e}", flush=True)
    assert abs(floor["floor"] - _stored_floor(cfg)["floor"]) <= 1e-12
    q, k, v = _qkv_full(cfg)
    bm = W.config_block_mask(cfg)
    note(f"{cfg} full")
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    bmd = None if bm is None else torch.from_numpy(bm).cuda()
    o, lse = rf_gpu.rf_attention_fwd(qd, kd, vd, scale=c["scale"], causal=c["causal"], block_mask=bmd)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    _same_again((o, lse), rf_gpu.rf_attention_fwd(qd, kd, vd, scale=c["scale"], causal=c["causal"], block_mask=bmd),
                f"{cfg}")
    _full_parity(cfg, o, lse, ref_o, ref_l, floor)


def test_config4_decode(rf_gpu):
    """Split-KV decode (B64 H32 Lk32768 d128, 16 splits): every one of the 2048
    heads against the unsplit oracle, computed on the host's cores first."""
    import torch
    c = W.CONFIGS["decode"]
    B, H, Lk, d, S = c["B"], c["H"], c["Lk"], c["d"], c["num_splits"]
    note("split-KV decode: oracle over every head on the host")
    ref_o, ref_l = F.full_reference("decode")
    floor = F.floor_summary("decode", ref_o)
    print(f"\n[parity] decode: bf16 floor before the GPU call {floor['floor']:.3e}", flush=True)
    assert abs(floor["floor"] - _stored_floor("decode")["floor"]) <= 1e-12
    q = W.normal_tensor(c["seed"], W.TID_Q, B, H, 1, d, "bf16")
    note("split-KV decode: generating K/V (32 GiB)")
    k = W.normal_tensor(c["seed"], W.TID_K, B, H, Lk, d, "bf16")
    kd = dev_bf16(k)
    del k
    v = W.normal_tensor(c["seed"], W.TID_V, B, H, Lk, d, "bf16")
    vd = dev_bf16(v)
    del v
    note("split-KV decode, full")
    qd = dev_bf16(q)
    o, lse = rf_gpu.rf_attention_decode_splitkv(qd, kd, vd, scale=c["scale"], num_splits=S)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    _same_again((o, lse), rf_gpu.rf_attention_decode_splitkv(qd, kd, vd, scale=c["scale"], num_splits=S), "split-KV decode")
    del kd, vd
    _full_parity("decode", o, lse, ref_o, ref_l, floor)


# ---------------------------------------------------------------------------
# Long key sequences: large in-head offsets, many tiles and splits, ragged ends
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
def test_attention_bf16_long_keys(rf_gpu, d):
    """600,007 keys (ragged), 200 query rows, causal (bottom-right): every row
    sweeps ~9,400 key tiles; sampled rows at tile edges against the oracle."""
    B, H, Lq, Lk = 1, 1, 200, 600_007
    q = W.normal_tensor(120, W.TID_Q, B, H, Lq, d, "bf16")
    k = W.normal_tensor(120, W.TID_K, B, H, Lk, d, "bf16")
    v = W.normal_tensor(120, W.TID_V, B, H, Lk, d, "bf16")
    scale = 1 / math.sqrt(d)
    note(f"long keys d={d} Lk={Lk}")
    o, lse = rf_gpu.rf_attention_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=scale, causal=True)
    rows = [0, 31, 32, 63, 64, 127, 128, 199]
    ref_o, ref_lse = O.attention(*(O.bf16_bits_to_f64(a) for a in (q, k, v)), scale, True, q_rows=rows)
    got_o = host_f64(o)[:, :, rows]
    got_l = host_f64(lse)[:, :, rows]
    e_o = assert_close(got_o, ref_o, 1e-2, "long keys O")
    e_l = assert_close(got_l, ref_lse, 1e-3, "long keys LSE")
    _report(f"long keys d{d}", e_o, e_l, ref_o)


def test_attention_and_decode_at_the_size_limit(rf_gpu):
    """The largest key range the boundary accepts at d = 128 (Lk d 2 just below
    2^31 bytes per head, 8,388,607 keys): a causal 64-row prefill (one
    workgroup sweeps every key tile) and a 64-way split-KV decode over the same
    K and V. Sampled prefill rows and the whole decode against the oracle."""
    d = 128
    Lk = (1 << 31) // (d * 2) - 1
    assert Lk * d * 2 < (1 << 31)
    note(f"size limit d={d} Lk={Lk}")
    k = W.normal_tensor(122, W.TID_K, 1, 1, Lk, d, "bf16")
    v = W.normal_tensor(122, W.TID_V, 1, 1, Lk, d, "bf16")
    qa = W.normal_tensor(122, W.TID_Q, 1, 1, 64, d, "bf16")
    qd = W.normal_tensor(123, W.TID_Q, 1, 1, 1, d, "bf16")
    scale = 1 / math.sqrt(d)
    kd, vd = dev_bf16(k), dev_bf16(v)
    o, lse = rf_gpu.rf_attention_fwd(dev_bf16(qa), kd, vd, scale=scale, causal=True)
    od, lsed = rf_gpu.rf_attention_decode_splitkv(dev_bf16(qd), kd, vd, scale=scale, num_splits=64)
    del kd, vd
    k64, v64 = O.bf16_bits_to_f64(k), O.bf16_bits_to_f64(v)
    del k, v
    rows = [0, 31, 32, 63]
    ref_o, ref_lse = O.attention(O.bf16_bits_to_f64(qa), k64, v64, scale, True, q_rows=rows)
    e_o = assert_close(host_f64(o)[:, :, rows], ref_o, 1e-2, "size-limit prefill O")
    e_l = assert_close(host_f64(lse)[:, :, rows], ref_lse, 1e-3, "size-limit prefill LSE")
    _report("size limit prefill d128", e_o, e_l, ref_o)
    ref_o, ref_lse = O.attention(O.bf16_bits_to_f64(qd), k64, v64, scale)
    e_o = assert_close(host_f64(od), ref_o, 1e-2, "size-limit decode O")
    e_l = assert_close(host_f64(lsed), ref_lse[:, :, 0], 1e-3, "size-limit decode LSE")
    _report("size limit decode d128", e_o, e_l, ref_o)


def test_decode_long_keys(rf_gpu):
    """2,000,003 keys split 61 ways (ragged last split), checked whole."""
    B, H, Lk, d, S = 1, 1, 2_000_003, 128, 61
    q = W.normal_tensor(121, W.TID_Q, B, H, 1, d, "bf16")
    k = W.normal_tensor(121, W.TID_K, B, H, Lk, d, "bf16")
    v = W.normal_tensor(121, W.TID_V, B, H, Lk, d, "bf16")
    scale = 1 / math.sqrt(d)
    note(f"decode long keys Lk={Lk} S={S}")
    o, lse = rf_gpu.rf_attention_decode_splitkv(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=scale, num_splits=S)
    ref_o, ref_lse = O.attention(*(O.bf16_bits_to_f64(a) for a in (q, k, v)), scale)
    e_o = assert_close(host_f64(o), ref_o, 1e-2, "decode long O")
    e_l = assert_close(host_f64(lse), ref_lse[:, :, 0], 1e-3, "decode long LSE")
    _report("decode long keys", e_o, e_l, ref_o)


def test_extension_bitmap_full_size(rf_gpu):
    """Element bitmaps inside partial tiles at B2 H16 L8192 d64 (a 512-key
    element-level causal window plus random tiles): two heads, rows at tile and
    window edges, against the oracle."""
    import torch
    c = W.EXTENSION_CONFIGS["bitmap"]
    q, k, v = (W.normal_tensor(c["seed"], t, c["B"], c["H"], c["Lq"], c["d"], "bf16")
               for t in (W.TID_Q, W.TID_K, W.TID_V))
    kinds, bits = W.extension_bitmap_mask()
    note("extension bitmap full size")
    args = (dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.from_numpy(kinds).cuda(),
            torch.from_numpy(bits.view(np.int64)).cuda())
    o, lse = rf_gpu.rf_attention_fwd_bitmap(*args, scale=c["scale"], causal=c["causal"])
    _same_again((o, lse), rf_gpu.rf_attention_fwd_bitmap(*args, scale=c["scale"], causal=c["causal"]), "bitmap")
    got_o, got_l = host_f64(o), host_f64(lse)
    rows = [0, 1, 63, 64, 511, 512, 513, 4095, 4096, 8000, 8191]
    e_o = e_l = 0.0
    for b, h in ((0, 0), (1, 15)):
        ref_o, ref_lse = O.attention(*(O.bf16_bits_to_f64(a[b:b + 1, h:h + 1]) for a in (q, k, v)), c["scale"],
                                     c["causal"], kinds, q_rows=rows, tile_bits=bits)
        e_o = max(e_o, assert_close(got_o[b:b + 1, h:h + 1, rows], ref_o, 1e-2, "bitmap O"))
        e_l = max(e_l, assert_close(got_l[b:b + 1, h:h + 1, rows], ref_lse, 1e-3, "bitmap LSE"))
    assert np.all(np.isfinite(got_l))
    _report("extension bitmap", e_o, e_l)


def test_extension_bigbird_chunk_full_size(rf_gpu):
    """256 queries over 16384 keys under a BigBird-style element mask (64
    global keys, a 256-key causal window, 64 random keys per row), by the row
    kernel and by the tile kernel: sampled heads and rows against the oracle,
    and the two kernels against each other on every row."""
    import torch
    c = W.EXTENSION_CONFIGS["bigbird_chunk"]
    B, H, Lq, Lk, d = c["B"], c["H"], c["Lq"], c["Lk"], c["d"]
    q = W.normal_tensor(c["seed"], W.TID_Q, B, H, Lq, d, "bf16")
    k, v = (W.normal_tensor(c["seed"], t, B, H, Lk, d, "bf16") for t in (W.TID_K, W.TID_V))
    vis = W.bigbird_chunk_mask(c["seed"], Lq, Lk, c["n_global"], c["window"], c["n_random"])
    kinds, bits = W.element_mask_tiles(vis)
    assert rf_gpu.rf_attention_plan(kinds, bits, B, H, Lq, Lk, d, c["causal"])["kernel"] == "row"
    note("extension bigbird chunk full size")
    args = (dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.from_numpy(kinds).cuda(),
            torch.from_numpy(bits.view(np.int64)).cuda())
    o, lse = rf_gpu.rf_attention_fwd_rowwise(*args, scale=c["scale"], causal=c["causal"])
    _same_again((o, lse), rf_gpu.rf_attention_fwd_rowwise(*args, scale=c["scale"], causal=c["causal"]), "rowwise")
    ot, lt = rf_gpu.rf_attention_fwd_bitmap(*args, scale=c["scale"], causal=c["causal"])
    got_o, got_l = host_f64(o), host_f64(lse)
    rows = [0, 1, 63, 64, 127, 128, 200, 255]
    e_o = e_l = 0.0
    for h in (0, 17, 31):
        ref_o, ref_lse = O.attention(*(O.bf16_bits_to_f64(a[:, h:h + 1]) for a in (q, k, v)), c["scale"],
                                     c["causal"], kinds, q_rows=rows, tile_bits=bits)
        e_o = max(e_o, assert_close(got_o[:, h:h + 1, rows], ref_o, 1e-2, "bigbird O"))
        e_l = max(e_l, assert_close(got_l[:, h:h + 1, rows], ref_lse, 1e-3, "bigbird LSE"))
    assert np.all(np.isfinite(got_l))
    assert_close(got_o, host_f64(ot), 1e-2, "row vs tile O")
    assert_close(got_l, host_f64(lt), 1e-3, "row vs tile LSE")
    _report("extension bigbird chunk", e_o, e_l)


def test_extension_layernorm_full_size(rf_gpu):
    """Layer normalisation of fp32 4096 x 32768 (the softmax workload's shape):
    sampled rows against the oracle, every row's statistics cheaply."""
    import torch
    c = W.EXTENSION_CONFIGS["layernorm"]
    x = W.softmax_rows_input(c["seed"], c["rows"], c["cols"])
    g, b = W.layernorm_affine(c["seed"], c["cols"])
    note("extension layernorm full size")
    y, mean, rstd = rf_gpu.rf_layernorm_rows(dev_f32(x), torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda(),
                                             eps=c["eps"])
    rows = [0, 1, 2047, 4095]
    ry, rm, rr = O.layernorm_rows(x[rows].astype(np.float64), g, b, c["eps"])
    e = assert_close(host_f64(y)[rows], ry, 1e-5, "layernorm y")
    # all rows: the statistics against the oracle's
    _, rm_all, rr_all = O.layernorm_rows(x.astype(np.float64), None, None, c["eps"])
    assert np.all(np.abs(host_f64(mean) - rm_all) <= 1e-6 * np.abs(rm_all) + 1e-6)
    assert np.all(np.abs(host_f64(rstd) - rr_all) <= 1e-6 * np.abs(rr_all) + 1e-6)
    _report("extension layernorm", e, 0.0)


@pytest.mark.parametrize("name", ["gqa_decode", "mla_decode"])
def test_extension_gqa_full_size(rf_gpu, name):
    """Grouped-query decode at full size (Lk 32768, d 128): 8 query heads per
    key/value head, and 128 query heads on one cache; sampled query heads
    against the oracle."""
    import torch
    c = W.EXTENSION_CONFIGS[name]
    B, Hq, Hkv, Lk, d, S = c["B"], c["Hq"], c["Hkv"], c["Lk"], c["d"], c["num_splits"]
    G = Hq // Hkv
    note(f"extension {name}: generating inputs")
    q, k, v = W.gqa_inputs(c)
    kd, vd = dev_bf16(k), dev_bf16(v)
    note(f"extension {name} full")
    qd = dev_bf16(q)
    o, lse = rf_gpu.rf_attention_decode_gqa(qd, kd, vd, scale=c["scale"], num_splits=S)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    _same_again((o, lse), rf_gpu.rf_attention_decode_gqa(qd, kd, vd, scale=c["scale"], num_splits=S), name)
    picks = [(0, 0), (B - 1, Hq - 1), (17, G - 1), (40, G % Hq), (63, Hq // 2), (5, 3)]
    worst_o = worst_l = 0.0
    refs = []
    for b, hq in picks:
        j = hq // G
        ref_o, ref_lse = O.decode_gqa(O.bf16_bits_to_f64(q[b:b + 1, hq:hq + 1]), O.bf16_bits_to_f64(k[b:b + 1, j:j + 1]),
                                      O.bf16_bits_to_f64(v[b:b + 1, j:j + 1]), c["scale"])
        got = host_f64(o[b, hq])
        worst_o = max(worst_o, max_abs_err(got, ref_o[0, 0]))
        worst_l = max(worst_l, max_abs_err(host_f64(lse[b, hq:hq + 1]), ref_lse[0]))
        # Beyond the absolute gate: over 32768 keys the rounding of P to bf16
        # averages out, so each element is within one bf16 rounding of the exact
        # value plus 1e-4 (at |O| ~ 0.03 the absolute gate alone is loose).
        assert np.all(np.abs(got - ref_o[0, 0]) <= 2.0 ** -8 * np.abs(ref_o[0, 0]) + 1e-4), (name, b, hq)
        refs.append(ref_o[0, 0])
    _report(f"extension {name} ({len(picks)} query heads)", worst_o, worst_l, np.concatenate(refs))
    assert worst_o <= 1e-2 and worst_l <= 1e-3


def test_extension_moe_route_full_size(rf_gpu):
    """Routing of 131072 tokens over 256 experts (top 8, renormalised): every
    token's experts against the oracle, exactly, and every weight."""
    import torch
    c = W.EXTENSION_CONFIGS["moe"]
    x = W.moe_logits(c["seed"], c["T"], c["E"])
    note("extension moe full size")
    xd = dev_f32(x)
    idx, w = rf_gpu.rf_moe_route(xd, c["k"], c["renorm"])
    _same_again((idx, w), rf_gpu.rf_moe_route(xd, c["k"], c["renorm"]), "moe")
    ref_idx, ref_w = O.moe_route(x.astype(np.float64), c["k"], c["renorm"])
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    e = float(np.abs(w.cpu().numpy().astype(np.float64) - ref_w).max())
    assert e <= 1e-5
    _report("extension moe", e, 0.0)
