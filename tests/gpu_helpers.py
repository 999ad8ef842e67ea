"""Helpers for the GPU parity tests: run the oracle on the same inputs the HIP path
receives, and compare with the tolerances the tests state."""
import sys

import numpy as np
import torch

from oracle import jssa
from oracle.numerics import bf16_to_f32, fp8e4m3_to_f32
from tests.util import band_check, bits, from_bits

# Output tolerance of the step for bf16 inputs with fp32 accumulation, bf16 output.
OUT_TOL_BF16 = 2e-2
# fp32 output: logits carry ~1e-6 relative error and exp2 ~1 ulp, so weights are
# accurate to ~1e-5 relative; with |v| < 8 the output error stays well below this.
OUT_TOL_F32 = 2e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def kproj_oracle(K_bits: np.ndarray, M: np.ndarray, fmt: str = "bf16") -> np.ndarray:
    """Projected cache for every (b, h) from the oracle's key projection (bf16 bits,
    or FP8 E4M3 bytes with fmt="fp8")."""
    B, H, cap, _ = K_bits.shape
    out = np.empty((B, H, cap, M.shape[1]), dtype=np.uint8 if fmt == "fp8" else np.uint16)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, cap, 4096):
                out[b, h, r0:r0 + 4096] = jssa.project_keys(K_bits[b, h, r0:r0 + 4096], M[h], fmt)
    return out


def kproj_close(gpu_bits: np.ndarray, ref_bits: np.ndarray, K_bits: np.ndarray, M: np.ndarray):
    """Projected-cache parity: the GPU takes an fp32 dot over d and rounds it to bf16;
    the oracle rounds the (near-exact) fp64 dot once. Allowed gap per element: one
    bf16 ulp of the larger result plus the fp32 dot error bound
    d * 2^-24 * sum_c |M_ic k_c|. Returns (ok, fraction of bit-identical elements).
    Shapes: gpu/ref [..., rows, r], K [..., rows, d], M [r, d]."""
    g = bf16_to_f32(gpu_bits).astype(np.float64)
    r = bf16_to_f32(ref_bits).astype(np.float64)
    kf = np.abs(bf16_to_f32(K_bits).astype(np.float64))
    err = kf @ np.abs(M.astype(np.float64)).T * (M.shape[1] * 2.0 ** -24)
    mag = np.maximum(np.abs(g), np.abs(r))
    ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 2.0 ** -126))) - 7)
    ok = bool(np.all(np.abs(g - r) <= ulp + err))
    return ok, float(np.mean(gpu_bits == ref_bits))


def kproj_close_fp8(gpu_bytes: np.ndarray, ref_bytes: np.ndarray, K_bits: np.ndarray, M: np.ndarray):
    """FP8 projected-cache parity: the GPU rounds its fp32 dot to E4M3 (saturating),
    the oracle rounds the fp64 dot once. Allowed gap per element: one E4M3 quantum at
    the larger magnitude (2^(e-3) for normals, 2^-9 below 2^-6) plus the fp32 dot error
    bound. Returns (ok, fraction of identical bytes)."""
    g = fp8e4m3_to_f32(gpu_bytes).astype(np.float64)
    r = fp8e4m3_to_f32(ref_bytes).astype(np.float64)
    kf = np.abs(bf16_to_f32(K_bits).astype(np.float64))
    err = kf @ np.abs(M.astype(np.float64)).T * (M.shape[1] * 2.0 ** -24)
    mag = np.maximum(np.abs(g), np.abs(r))
    quantum = np.exp2(np.maximum(np.floor(np.log2(np.maximum(mag, 2.0 ** -9))), -6) - 3)
    ok = bool(np.all(np.abs(g - r) <= quantum + err))
    return ok, float(np.mean(gpu_bytes == ref_bytes))


def kproj_torch(K: torch.Tensor, M: torch.Tensor) -> torch.Tensor:
    """Projected cache built with plain torch ops on the GPU (fp32 products, bf16
    round to nearest even). Used only to prepare inputs at sizes where the oracle's
    projection would be slow; it is not the HIP path."""
    B, H, cap, d = K.shape
    out = torch.empty(B, H, cap, M.shape[1], dtype=torch.bfloat16, device=K.device)
    for b in range(B):
        for h in range(H):
            out[b, h] = (K[b, h].float() @ M[h].T).to(torch.bfloat16)
    return out


def ref_unit(q_bits, K_bits, V_bits, kproj_bits, M, b, h, G, n, k, scale, fmt="bf16"):
    """Oracle results for one unit: (out fp64 [G, d], idx, scores)."""
    return jssa.decode_unit(q_bits[b, h * G:(h + 1) * G], K_bits[b, h], V_bits[b, h], kproj_bits[b, h],
                            M[h], n, k, scale, fmt)


def check_unit(gpu_out, gpu_idx, q_bits, K_bits, V_bits, kproj_bits, M, b, h, G, n, k, scale, tol, tag="",
               fmt="bf16"):
    """Index-set parity (band rule) and output parity (oracle attention over the
    GPU's own index set; also over the oracle's set when the two sets agree)."""
    ref_out, ref_idx, s = ref_unit(q_bits, K_bits, V_bits, kproj_bits, M, b, h, G, n, k, scale, fmt)
    gi = np.asarray(gpu_idx)
    ok, msg = band_check(gi, ref_idx, s, n, k)
    assert ok, f"{tag} unit ({b},{h}): {msg}"
    mine = jssa.attend(q_bits[b, h * G:(h + 1) * G], K_bits[b, h][:n], V_bits[b, h][:n], gi, scale)
    err = np.max(np.abs(np.asarray(gpu_out, dtype=np.float64) - mine)) if mine.size else 0.0
    assert err <= tol, f"{tag} unit ({b},{h}): max |out - oracle(out over GPU idx)| = {err} > {tol}"
    if np.array_equal(gi[:min(k, n)], ref_idx[:min(k, n)]):
        err2 = np.max(np.abs(np.asarray(gpu_out, dtype=np.float64) - ref_out))
        assert err2 <= tol, f"{tag} unit ({b},{h}): max |out - oracle| = {err2}"
    return msg


__all__ = ["kproj_close", "kproj_close_fp8", "bits", "from_bits", "bf16_to_f32", "band_check", "kproj_oracle", "kproj_torch", "check_unit", "say",
           "OUT_TOL_BF16", "OUT_TOL_F32"]
