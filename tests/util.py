"""Small helpers shared by the tests (no method arithmetic here)."""
import numpy as np
import torch


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> numpy uint16 bit patterns."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def band_check(gpu_idx, ref_idx, ref_scores, n, k, rel=1e-3):
    """Index-set parity: the GPU must return exactly min(k, n) distinct positions in
    [0, n), ascending, padded with -1; positions where the sets differ must all lie in
    the band |s_j - T| <= rel*|T| around the oracle's k-th largest score T.
    Returns (ok, message)."""
    kk = min(k, n)
    g = np.asarray(gpu_idx)
    head, tail = g[:kk], g[kk:]
    if np.any(tail != -1):
        return False, "padding after the first min(k,n) entries is not -1"
    if kk == 0:
        return True, ""
    if np.any(head < 0) or np.any(head >= n):
        return False, f"index out of range: min {head.min()} max {head.max()} n {n}"
    if np.any(np.diff(head) <= 0):
        return False, "indices not strictly ascending (duplicate or unsorted)"
    r = np.asarray(ref_idx)[:kk]
    s = np.asarray(ref_scores, dtype=np.float64)
    T = np.sort(s[r])[0]
    diff = np.setxor1d(head, r)
    if diff.size == 0:
        return True, ""
    bad = diff[np.abs(s[diff] - T) > rel * abs(T)]
    if bad.size:
        return False, f"{bad.size} differing positions outside the band (T={T}), e.g. {bad[:5]}"
    return True, f"{diff.size // 2} swaps inside the band"
