"""Helpers for GPU tests: storage conversion between numpy (bf16 as uint16
bits) and torch device tensors.  No arithmetic of the method lives here."""
import numpy as np
import pytest
import torch


# Attention log-sum-exp (natural log of the softmax normaliser of the scaled
# logits), checked per (row, query head): 2e-2 absolute, the output bound
# applied to the normaliser's logarithm (a factor of at most e^0.02 in the
# normaliser of every row).
LSE_TOL = 2e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import non_prefix_kv_token_amd as ct
    ct.lib()  # fails loudly if the HIP library is missing
    return ct


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    if a.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    if a.dtype == np.int32:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    raise TypeError(a.dtype)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def ulp_distance_bf16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| in units in the last place for bf16 bit patterns (same sign)."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)
    return np.abs(key(a) - key(b))


def assert_rotated_keys(got: np.ndarray, want: np.ndarray, ulp_fn=None) -> None:
    """Assembled (rotated) keys against the oracle's.  Both sides rotate in
    fp64 and round once; they differ only in the sine and cosine, a few fp64
    ulps apart, so an element may round the other way only when its exact
    value lies that close to a rounding boundary (about one in 10^9).  At
    most one element in a million may differ, by one ulp.  A rounding slip of
    the kind double rounding makes (one value in 2^16) fails this at the
    full workload sizes."""
    ulp = (ulp_fn or ulp_distance_bf16)(got, want)
    assert ulp.max() <= 1, f"max {ulp.max()} ulp"
    n_off = int((ulp != 0).sum())
    assert n_off <= max(1, ulp.size // 1_000_000), f"{n_off} of {ulp.size} keys differ by one ulp"


def ulp_distance_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def key(x):
        x = x.view(np.int32).astype(np.int64)
        return np.where(x < 0, -(x & 0x7FFFFFFF), x)
    return np.abs(key(a) - key(b))


def check_index_sets(sel_gpu, sel_orc, s_orc, k, band=1e-6):
    """Bit-exact index sets, except members of the symmetric difference whose
    oracle score is within `band` (relative) of the k-th ranked oracle score."""
    a, b = set(sel_gpu.tolist()), set(sel_orc.tolist())
    assert len(a) == len(b) == k
    diff = a ^ b
    if not diff:
        return 0
    kth = np.sort(s_orc)[::-1][k - 1]
    for i in diff:
        assert abs(s_orc[i] - kth) <= band * kth, (i, s_orc[i], kth)
    return len(diff)


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values around |x| (8 significant bits)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 0.5 * 2.0 ** (e - 7)
