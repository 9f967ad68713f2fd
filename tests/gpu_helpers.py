"""Shared helpers of the GPU parity tests: host<->device words and the
tolerances of the comparison."""
import numpy as np
import torch

# Tolerances of the comparison with the oracle's unrounded double results.
ABS_TOL = 1e-2           # bf16 outputs: max |gpu - ref|
REL_TOL = 2.0 ** -7      # bf16 outputs: max |gpu - ref| / |ref| where |ref| >= REL_FLOOR
REL_FLOOR = 1e-2
SCORE_TOL = 1e-4         # fp32 scores: |gpu - ref| <= SCORE_TOL * max(|ref|, 1)


COUNTER_BLOCK = 65536    # the first bytes of every workspace: arrival counters, zero between calls


class PoisonedWorkspace:
    """A workspace whose scratch data (every byte past the counter block) is
    refilled with 0xFF -- NaN as fp32 and as bf16 -- on the call's stream before
    every call, so that a read of a partial result that was never written shows
    up as NaN in the output instead of passing as a stale or zero value."""

    def __init__(self, device=None):
        import decode_attention_output_amd as da

        self._ws = da.Workspace(device)

    @property
    def buf(self):
        return self._ws.buf

    def get(self, nbytes: int, stream=None):
        buf = self._ws.get(nbytes, stream)
        if buf is not None and buf.numel() > COUNTER_BLOCK:
            s = stream if stream is not None else torch.cuda.current_stream()
            with torch.cuda.stream(s):
                buf[COUNTER_BLOCK:].fill_(0xFF)
        return buf


def dev_bf16(words: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).view(torch.bfloat16).to(device)


def dev_f16(words: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).view(torch.float16).to(device)


def dev_i32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def host_words(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_words_to_f64(w: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).view(torch.bfloat16).double().numpy()


def ulp_distance_bf16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between two arrays of finite bf16 words."""
    def ordered(w):
        w = w.astype(np.int32)
        return np.where(w & 0x8000, 0x8000 - (w & 0x7FFF), 0x8000 + (w & 0x7FFF))
    return np.abs(ordered(a) - ordered(b))


def assert_bf16_close(gpu_words: np.ndarray, ref: np.ndarray, what: str):
    g = bf16_words_to_f64(gpu_words)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), "%s: non-finite GPU output (%d entries)" % (what, np.sum(~np.isfinite(g)))
    err = np.abs(g - ref)
    max_abs = float(err.max()) if err.size else 0.0
    mask = np.abs(ref) >= REL_FLOOR
    max_rel = float((err[mask] / np.abs(ref[mask])).max()) if np.any(mask) else 0.0
    assert max_abs <= ABS_TOL and max_rel <= REL_TOL, (
        "%s: max abs %.3g (tol %.3g), max rel %.3g (tol %.3g) at %s" %
        (what, max_abs, ABS_TOL, max_rel, REL_TOL, np.unravel_index(np.argmax(err), err.shape)))
    return max_abs, max_rel


def assert_scores_close(gpu: np.ndarray, ref: np.ndarray, what: str):
    err = np.abs(gpu.astype(np.float64) - ref)
    bound = SCORE_TOL * np.maximum(np.abs(ref), 1.0)
    bad = err > bound
    assert not np.any(bad), "%s: %d scores off, worst %.3g" % (what, int(bad.sum()), float((err / bound).max()))


def assert_within_fp32_sum_bound(gpu_words: np.ndarray, ref: np.ndarray, x_words: np.ndarray, w_words: np.ndarray,
                                 what: str):
    """gpu = bf16(fp32 sum of x @ w) in any order: compare with the exact result
    under the classical bound n*u*sum|x_k w_kn| (u = 2^-24) plus one bf16 step."""
    x = np.abs(bf16_words_to_f64(x_words))
    w = np.abs(bf16_words_to_f64(w_words))
    K = x.shape[1]
    mag = x @ w
    g = bf16_words_to_f64(gpu_words)
    bound = K * 2.0 ** -24 * mag + 2.0 ** -8 * np.abs(ref) + 1e-30
    err = np.abs(g - ref)
    bad = err > bound
    assert not np.any(bad), "%s: %d entries beyond the fp32 summation bound (worst ratio %.3g)" % (
        what, int(bad.sum()), float((err / bound).max()))
