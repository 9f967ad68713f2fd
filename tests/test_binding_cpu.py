"""The torch wrappers refuse tensors that disagree with each other before any
call reaches the library: the C ABI sees only pointers and sizes taken from
q and the caches, so a mismatched weight, output or cache would otherwise make
the kernels read or write past an allocation. Runs on the CPU: the shape checks
come first, and the library is replaced by one that fails if it is reached."""
import pytest
import torch

import decode_attention_output_amd as da


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def refuse(*a, **k):
        raise AssertionError("the library was reached")
    monkeypatch.setattr(da, "load_library", refuse)


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _decode(B=2, Hq=8, Hkv=2, D=128, L=64, N=256):
    return dict(q=_t(B, Hq, D), k_cache=_t(B, Hkv, L, D), v_cache=_t(B, Hkv, L, D),
                seq_lens=_t(B, dtype=torch.int32), o_weight=_t(Hq * D, N))


BAD_DECODE = [
    ("v_cache", _t(2, 2, 65, 128), "v_cache must have shape"),
    ("k_cache", _t(3, 2, 64, 128), "does not match q"),
    ("k_cache", _t(2, 2, 64, 64), "does not match q"),
    ("seq_lens", _t(3, dtype=torch.int32), "seq_lens must have shape"),
    ("o_weight", _t(8 * 128 + 8, 256), "rows"),
    ("q", _t(2, 8), "dimensions"),
    ("out", _t(2, 255), "out must have shape"),
]


@pytest.mark.parametrize("name,bad,msg", BAD_DECODE, ids=[f"{b[0]}-{i}" for i, b in enumerate(BAD_DECODE)])
def test_decode_fwd_refuses_mismatched_tensors(name, bad, msg):
    args = _decode()
    args[name] = bad
    with pytest.raises(ValueError, match=msg):
        da.decode_attn_fwd(args["q"], args["k_cache"], args["v_cache"], args["seq_lens"], args["o_weight"],
                           out=args.get("out"))
    with pytest.raises(ValueError, match=msg):
        da.DecodeStep(args["q"], args["k_cache"], args["v_cache"], args["seq_lens"], args["o_weight"],
                      out=args.get("out"))


def test_decode_only_refuses_a_wrong_output_and_debug_buffers():
    a = _decode()
    with pytest.raises(ValueError, match="out must have shape"):
        da.decode_attn_only(a["q"], a["k_cache"], a["v_cache"], a["seq_lens"], out=_t(2, 256))
    with pytest.raises(ValueError, match="debug_scores must have shape"):
        da.decode_attn_only(a["q"], a["k_cache"], a["v_cache"], a["seq_lens"],
                            debug_scores=_t(2, 8, 63, dtype=torch.float32), debug_lse=_t(2, 8, dtype=torch.float32))
    with pytest.raises(ValueError, match="go together"):
        da.decode_attn_only(a["q"], a["k_cache"], a["v_cache"], a["seq_lens"],
                            debug_scores=_t(2, 8, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="out must have shape"):
        da.AttentionStep(a["q"], a["k_cache"], a["v_cache"], a["seq_lens"], out=_t(2, 8 * 128 + 1))


def test_consistent_cpu_tensors_are_refused_as_host_memory():
    a = _decode()
    with pytest.raises(ValueError, match="device tensor"):
        da.decode_attn_fwd(a["q"], a["k_cache"], a["v_cache"], a["seq_lens"], a["o_weight"])


def test_matmul_wrappers_refuse_mismatched_tensors():
    with pytest.raises(ValueError, match="rows"):
        da.oproj_fwd(_t(1, 512), _t(256, 512))
    with pytest.raises(ValueError, match="out must have shape"):
        da.oproj_fwd(_t(4, 512), _t(512, 256), out=_t(4, 128))
    with pytest.raises(ValueError, match="out must have shape"):
        da.OprojStep(_t(4, 512), _t(512, 256), out=_t(3, 256))
    with pytest.raises(ValueError, match="rows"):
        da.gemm_f16(_t(256, 1024, dtype=torch.float16), _t(512, 512, dtype=torch.float16))
    with pytest.raises(TypeError):
        da.gemm_f16(_t(256, 1024), _t(1024, 512))  # bf16 where fp16 is required


def test_prefill_refuses_mismatched_tensors():
    q, k, v, cl = _t(2, 17, 8, 128), _t(2, 2, 40, 128), _t(2, 2, 40, 128), _t(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="ctx_lens must have shape"):
        da.prefill_attn_fwd(q, k, v, _t(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="v_cache must have shape"):
        da.prefill_attn_fwd(q, k, _t(2, 2, 41, 128), cl)
    with pytest.raises(ValueError, match="out must have shape"):
        da.prefill_attn_fwd(q, k, v, cl, out=_t(2, 17, 8 * 128 - 8))
