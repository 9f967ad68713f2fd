"""decode_attn_fwd_noalloc (the entry point that allocates nothing) through
the C ABI against decode_attn_fwd on the same inputs: two calls in a row on
the library's scratch array, the second with a smaller step, each bit-equal to
decode_attn_fwd's output and within the oracle's tolerance."""
import ctypes

import numpy as np
import pytest
import torch

import decode_attention_output_amd as da
import oracle
import workloads
from gpu_helpers import PoisonedWorkspace, assert_bf16_close, dev_bf16, dev_i32, host_words

pytestmark = pytest.mark.gpu

CASES = [
    # (batch, Hq, Hkv, seq_lens, max_seq_len, hidden): the large single-launch step (stream-K
    # attention and the MFMA projection's items in one grid), then a smaller step that runs as the
    # small single-launch step
    (6, 32, 8, [3000, 40, 2048, 999, 64, 2500], 3000, 4096),
    (1, 8, 2, [300], 300, 512),
]


def _noalloc(q, k, v, s, w, out):
    B, Hq, D = q.shape
    _, Hkv, Lmax, _ = k.shape
    shape = da.make_shape(B, Hq, Hkv, Lmax, w.shape[1], D)
    rc = da.load_library().decode_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), s.data_ptr(),
                                                   w.data_ptr(), out.data_ptr(), ctypes.byref(shape),
                                                   torch.cuda.current_stream().cuda_stream)
    assert rc == da.DA_OK, da.status_str(rc)


def test_noalloc_matches_decode_attn_fwd_twice(gpu):
    plans = [da.decode_attn_plan(da.make_shape(c[0], c[1], c[2], c[4], c[5])).fused for c in CASES]
    assert plans == [2, 1]
    for i, (B, Hq, Hkv, sl, Lmax, hidden) in enumerate(CASES):
        inp = workloads.custom_decode_inputs(B, Hq, Hkv, sl, max_seq_len=Lmax, hidden=hidden, seed=900 + i)
        q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
        s, w = dev_i32(inp["seq_lens"]), dev_bf16(inp["o_weight"])
        want = host_words(da.decode_attn_fwd(q, k, v, s, w, workspace=PoisonedWorkspace()))
        out = torch.full((B, hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
        _noalloc(q, k, v, s, w, out)
        torch.cuda.synchronize()
        assert da.decode_attn_step_status(None) == da.DA_OK
        got = host_words(out)
        np.testing.assert_array_equal(got, want)
        ref = oracle.decode_step(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["o_weight"])
        assert_bf16_close(got, ref["out_ref"], "noalloc call %d" % i)
