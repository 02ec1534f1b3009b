"""The split-KV decode entry point that allocates nothing.

rf_attention_decode_splitkv_noalloc keeps its partials in the library's own
device array instead of a caller workspace. It runs the same kernels as
rf_attention_decode_splitkv, so its outputs must equal that entry point's bit
for bit; two calls in a row, the second smaller, show that what the first
call left in the shared array does not leak into the second.
"""
import ctypes

import numpy as np
import pytest

import online_softmax_attention_pass_amd as rf
import oracle as O
import workloads as W
from gpu_util import dev_bf16, host_f64, max_abs_err, note


def test_noalloc_refuses_partials_beyond_its_scratch():
    """Checked before any HIP call: partials above the 32 MiB scratch are an
    RF_ERR_WORKSPACE error that names the limit."""
    lib = rf.load()
    fake = ctypes.c_void_p(0x10000)
    # 1024 * 64 heads * 16 splits * 129 floats = 541 MB of partials
    st = lib.rf_attention_decode_splitkv_noalloc(fake, fake, fake, fake, None, 1024, 64, 100, 128, 0.1, 16,
                                                 rf.RF_BF16, None)
    assert st == rf.RF_ERR_WORKSPACE
    assert b"scratch" in lib.rf_last_error_message()
    # the ordinary checks come first, as in the workspace entry point
    st = lib.rf_attention_decode_splitkv_noalloc(fake, fake, fake, fake, None, 2, 2, 100, 96, 0.1, 4, rf.RF_BF16, None)
    assert st == rf.RF_ERR_UNSUPPORTED
    st = lib.rf_attention_decode_splitkv_noalloc(fake, fake, fake, fake, None, 2, 2, 100, 128, 0.1, 0, rf.RF_BF16, None)
    assert st == rf.RF_ERR_INVALID_ARG


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point(rf_gpu):
    import torch
    # the decode workload's B, H, d and splits (16.1 MiB of partials, half the
    # scratch) over 2048 keys, then a smaller call of every size
    cases = [(64, 32, 2048, 128, 16), (3, 5, 1001, 64, 7)]
    for i, (B, H, Lk, d, S) in enumerate(cases):
        seed = 131 + i
        q = W.normal_tensor(seed, W.TID_Q, B, H, 1, d, "bf16")
        k = W.normal_tensor(seed, W.TID_K, B, H, Lk, d, "bf16")
        v = W.normal_tensor(seed, W.TID_V, B, H, Lk, d, "bf16")
        qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
        note(f"decode noalloc B={B} H={H} Lk={Lk} d={d} S={S}")
        ws = torch.full((rf_gpu.rf_attention_decode_splitkv_workspace_size(B, H, d, S) // 4,), float("nan"),
                        device="cuda")
        o_ws, l_ws = rf_gpu.rf_attention_decode_splitkv(qd, kd, vd, num_splits=S, workspace=ws)
        o_na, l_na = rf_gpu.rf_attention_decode_splitkv_noalloc(qd, kd, vd, num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na), (B, H, Lk, d, S)
        # and the gates against the oracle on a few heads
        for b, h in ((0, 0), (B - 1, H - 1)):
            ro, rl = O.attention(*(O.bf16_bits_to_f64(a[b:b + 1, h:h + 1]) for a in (q, k, v)), 1 / np.sqrt(d))
            assert max_abs_err(host_f64(o_na[b, h]), ro[0, 0]) <= 1e-2
            assert max_abs_err(host_f64(l_na[b, h:h + 1]), rl[0, 0]) <= 1e-3
