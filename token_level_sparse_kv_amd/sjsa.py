"""ctypes binding of libsjsa (the MI355X JSSA sparse-decode library).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, turned into pointers, and the work is enqueued on torch's current
stream. Every computation runs in the library's HIP kernels; there is no CPU or
PyTorch fallback, and a missing library raises at load time.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libsjsa.so")

SJSA_FLAG_OUT_F32 = 1
SJSA_FLAG_WRITE_SCORES = 2
SJSA_FLAG_KPROJ_FP8 = 4
KPROJ_FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)   # OCP E4M3 bytes
SJSA_MAX_K = 1 << 20


class SjsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"sjsa error {status}: {message}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("fused_wait_us", ctypes.c_int32),
    ]


_lib = None

_P = ctypes.c_void_p
_SIGS = {
    "sjsa_append_kv": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    "sjsa_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32]),
    "sjsa_decode_step": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                        ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]),
    "sjsa_decode_step_append": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                               ctypes.c_int32, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]),
    "sjsa_decode_step_append_noalloc": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P,
                                                       _P, ctypes.c_int32, ctypes.c_float, _P, _P, _P]),
    "sjsa_prep_append": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                        _P, ctypes.c_size_t, _P]),
    "sjsa_score": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, ctypes.c_int32, _P, ctypes.c_size_t,
                                  _P]),
    "sjsa_prep": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, ctypes.c_int32, _P, ctypes.c_size_t, _P]),
    "sjsa_scan": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, ctypes.c_size_t, _P]),
    "sjsa_prep_scan": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, _P, _P,
                                      ctypes.c_size_t, _P]),
    "sjsa_select": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]),
    "sjsa_attend": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, ctypes.c_int32, _P, ctypes.c_float,
                                   _P, _P, ctypes.c_size_t, _P]),
    "sjsa_topk": (ctypes.c_int, [ctypes.POINTER(Shape), _P, ctypes.c_int64, _P, ctypes.c_int32, _P, _P,
                                 ctypes.c_size_t, _P]),
    "sjsa_gated_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int32]),
    "sjsa_gated_decode_step": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, ctypes.c_int64, _P,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                              _P, _P, _P, ctypes.c_size_t, _P]),
    "sjsa_block_keys": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    "sjsa_block_append": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_int32, _P, _P, ctypes.c_int32, _P, _P, _P,
                                         _P, _P, _P, _P]),
    "sjsa_block_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int32]),
    "sjsa_block_decode_step": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, _P,
                                              _P, ctypes.c_size_t, _P]),
    "sjsa_calib_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int64]),
    "sjsa_calib_accumulate": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, ctypes.c_int64, _P, _P, _P,
                                             ctypes.c_size_t, _P]),
    "sjsa_calib_basis": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "sjsa_workspace_scores_offset": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "sjsa_workspace_score_stride": (ctypes.c_int64, [ctypes.POINTER(Shape)]),
    "sjsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}


def lib():
    """Load libsjsa.so once. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m token_level_sparse_kv_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int):
    if status != 0:
        raise SjsaError(status, lib().sjsa_status_string(status).decode())


def make_shape(batch, n_kv_heads, group, head_dim, rank, capacity, out_f32=False, write_scores=False,
               kproj_fp8=False, fused_wait_us=0) -> Shape:
    """fused_wait_us: how long a scan workgroup of the fused prep + scan launch waits for
    its unit's prep (0: the library default of 200 us; negative: no wait, so every unit
    takes the exact path)."""
    flags = ((SJSA_FLAG_OUT_F32 if out_f32 else 0) | (SJSA_FLAG_WRITE_SCORES if write_scores else 0)
             | (SJSA_FLAG_KPROJ_FP8 if kproj_fp8 else 0))
    return Shape(batch, n_kv_heads, group, head_dim, rank, flags, capacity, fused_wait_us)


def kproj_is_fp8(Kproj: torch.Tensor) -> bool:
    """The projected cache is bf16, or FP8 E4M3 given as uint8 / float8_e4m3fn bytes."""
    if Kproj.dtype == torch.bfloat16:
        return False
    if Kproj.dtype in KPROJ_FP8_DTYPES:
        return True
    raise TypeError(f"Kproj must be bfloat16, uint8 or float8_e4m3fn (got {Kproj.dtype})")


def _need_kproj(Kproj: torch.Tensor, shape=None, fp8=None):
    """Kproj checks; with fp8 given, its format must match the call's shape flags."""
    is8 = kproj_is_fp8(Kproj)
    if fp8 is not None and is8 != bool(fp8):
        raise TypeError("Kproj's dtype does not match the shape's SJSA_FLAG_KPROJ_FP8 flag")
    _need(Kproj, "Kproj", Kproj.dtype, shape)
    return is8


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def shape_of(q: torch.Tensor, K: torch.Tensor, M: torch.Tensor, out_f32=False, Kproj=None) -> Shape:
    B, Hkv, cap, d = K.shape
    Hq = q.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    fp8 = Kproj is not None and kproj_is_fp8(Kproj)
    return make_shape(B, Hkv, Hq // Hkv, d, M.shape[1], cap, out_f32, kproj_fp8=fp8)


def workspace_size(shape: Shape, k: int) -> int:
    n = lib().sjsa_decode_workspace_size(ctypes.byref(shape), int(k))
    if n == 0:
        raise SjsaError(-2, "invalid shape or k for the workspace query")
    return int(n)


def alloc_workspace(shape: Shape, k: int, device=None) -> torch.Tensor:
    return torch.empty(workspace_size(shape, k), dtype=torch.uint8, device=device or "cuda")


def scores_view(shape: Shape, workspace: torch.Tensor) -> torch.Tensor:
    """The fp32 score buffer inside a workspace, viewed as [B, H_kv, stride]; filled by a
    score() call made with write_scores=True."""
    off = lib().sjsa_workspace_scores_offset(ctypes.byref(shape))
    stride = lib().sjsa_workspace_score_stride(ctypes.byref(shape))
    n = shape.batch * shape.n_kv_heads * stride * 4
    return workspace[off:off + n].view(torch.float32).view(shape.batch, shape.n_kv_heads, stride)


def append_kv(k_new, v_new, M, pos, K, V, Kproj, stream=None):
    """Write n_new tokens per (b, h) at slots pos[b].. into K, V and Kproj (in place)."""
    B, Hkv, cap, d = K.shape
    r = M.shape[1]
    T = k_new.shape[2]
    _need(K, "K", torch.bfloat16)
    _need(V, "V", torch.bfloat16, K.shape)
    fp8 = _need_kproj(Kproj, (B, Hkv, cap, r))
    _need(k_new, "k_new", torch.bfloat16, (B, Hkv, T, d))
    _need(v_new, "v_new", torch.bfloat16, (B, Hkv, T, d))
    _need(M, "M", torch.float32, (Hkv, r, d))
    _need(pos, "pos", torch.int32, (B,))
    shape = make_shape(B, Hkv, 1, d, r, cap, kproj_fp8=fp8)
    _check(lib().sjsa_append_kv(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), T, _ptr(M), _ptr(pos),
                                _ptr(K), _ptr(V), _ptr(Kproj), _stream(stream)))


def _step_checks(q, K, V, Kproj, M, seq_len):
    B, Hkv, cap, d = K.shape
    r = M.shape[1]
    _need(q, "q", torch.bfloat16)
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != d:
        raise ValueError(f"q has shape {tuple(q.shape)}, expected [B={B}, H_q, d={d}]")
    _need(K, "K", torch.bfloat16)
    _need(V, "V", torch.bfloat16, K.shape)
    if Kproj is not None:
        _need_kproj(Kproj, (B, Hkv, cap, r))
    _need(M, "M", torch.float32, (Hkv, r, d))
    _need(seq_len, "seq_len", torch.int32, (B,))


def decode_step(q, K, V, Kproj, M, seq_len, k, sm_scale=0.0, out=None, idx=None, workspace=None,
                out_f32=False, stream=None):
    """One sparse decode step. Returns (out [B, H_q, d], idx [B, H_kv, k])."""
    _step_checks(q, K, V, Kproj, M, seq_len)
    shape = shape_of(q, K, M, out_f32, Kproj)
    B, Hkv = shape.batch, shape.n_kv_heads
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32 if out_f32 else torch.bfloat16, device=q.device)
    if idx is None:
        idx = torch.empty((B, Hkv, int(k)), dtype=torch.int32, device=q.device)
    _need(out, "out", torch.float32 if out_f32 else torch.bfloat16, q.shape)
    _need(idx, "idx", torch.int32, (B, Hkv, int(k)))
    if workspace is None:
        workspace = alloc_workspace(shape, k, q.device)
    _check(lib().sjsa_decode_step(ctypes.byref(shape), _ptr(q), _ptr(K), _ptr(V), _ptr(Kproj), _ptr(M),
                                  _ptr(seq_len), int(k), float(sm_scale), _ptr(out), _ptr(idx),
                                  _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, idx


def _append_one_checks(k_new, v_new, pos, K, M):
    B, Hkv, cap, d = K.shape
    _need(k_new, "k_new", torch.bfloat16, (B, Hkv, 1, d))
    _need(v_new, "v_new", torch.bfloat16, (B, Hkv, 1, d))
    _need(pos, "pos", torch.int32, (B,))


def decode_step_append(k_new, v_new, pos, q, K, V, Kproj, M, seq_len, k, sm_scale=0.0, out=None, idx=None,
                       workspace=None, out_f32=False, stream=None):
    """Append the step's new token (k_new, v_new [B, H_kv, 1, d] at slots pos[b]) to K, V
    and Kproj, then run one sparse decode step; the same results as append_kv followed
    by decode_step. Returns (out, idx)."""
    _step_checks(q, K, V, Kproj, M, seq_len)
    _append_one_checks(k_new, v_new, pos, K, M)
    shape = shape_of(q, K, M, out_f32, Kproj)
    B, Hkv = shape.batch, shape.n_kv_heads
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32 if out_f32 else torch.bfloat16, device=q.device)
    if idx is None:
        idx = torch.empty((B, Hkv, int(k)), dtype=torch.int32, device=q.device)
    _need(out, "out", torch.float32 if out_f32 else torch.bfloat16, q.shape)
    _need(idx, "idx", torch.int32, (B, Hkv, int(k)))
    if workspace is None:
        workspace = alloc_workspace(shape, k, q.device)
    _check(lib().sjsa_decode_step_append(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(q),
                                         _ptr(K), _ptr(V), _ptr(Kproj), _ptr(M), _ptr(seq_len), int(k),
                                         float(sm_scale), _ptr(out), _ptr(idx), _ptr(workspace),
                                         workspace.numel(), _stream(stream)))
    return out, idx


def decode_step_append_noalloc(k_new, v_new, pos, q, K, V, Kproj, M, seq_len, k, out, idx, sm_scale=0.0,
                               out_f32=False, stream=None):
    """decode_step_append with the library's static scratch array instead of a
    workspace: the call allocates nothing (out and idx must be given). Shapes whose
    workspace exceeds the array are rejected (SjsaError, SJSA_ERR_SCRATCH). Calls that
    overlap on one GPU race. Returns (out, idx)."""
    _step_checks(q, K, V, Kproj, M, seq_len)
    _append_one_checks(k_new, v_new, pos, K, M)
    shape = shape_of(q, K, M, out_f32, Kproj)
    _need(out, "out", torch.float32 if out_f32 else torch.bfloat16, q.shape)
    _need(idx, "idx", torch.int32, (shape.batch, shape.n_kv_heads, int(k)))
    _check(lib().sjsa_decode_step_append_noalloc(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(q),
                                                 _ptr(K), _ptr(V), _ptr(Kproj), _ptr(M), _ptr(seq_len), int(k),
                                                 float(sm_scale), _ptr(out), _ptr(idx), _stream(stream)))
    return out, idx


NOALLOC_SCRATCH_BYTES = 64 << 20


def score(q, Kproj, M, seq_len, k, workspace, write_scores=False, stream=None):
    """Scoring prep + score scan into the workspace (candidates for budget k). With
    write_scores the dense fp32 scores are stored too and returned as a
    [B, H_kv, stride] view; otherwise returns None."""
    B, Hkv, cap, r = Kproj.shape
    d = M.shape[2]
    shape = make_shape(B, Hkv, q.shape[1] // Hkv, d, r, cap, write_scores=write_scores,
                       kproj_fp8=kproj_is_fp8(Kproj))
    _need(q, "q", torch.bfloat16, (B, shape.group * Hkv, d))
    _need_kproj(Kproj)
    _need(M, "M", torch.float32, (Hkv, r, d))
    _need(seq_len, "seq_len", torch.int32, (B,))
    _check(lib().sjsa_score(ctypes.byref(shape), _ptr(q), _ptr(Kproj), _ptr(M), _ptr(seq_len), int(k),
                            _ptr(workspace), workspace.numel(), _stream(stream)))
    return scores_view(shape, workspace) if write_scores else None


def prep(shape: Shape, q, M, Kproj, seq_len, k, workspace, stream=None):
    """Scoring prep only (mean query, projection, candidate threshold for budget k)."""
    _need(q, "q", torch.bfloat16, (shape.batch, shape.n_kv_heads * shape.group, shape.head_dim))
    _need(M, "M", torch.float32, (shape.n_kv_heads, shape.rank, shape.head_dim))
    _need_kproj(Kproj, (shape.batch, shape.n_kv_heads, shape.capacity, shape.rank), bool(shape.flags & SJSA_FLAG_KPROJ_FP8))
    _need(seq_len, "seq_len", torch.int32, (shape.batch,))
    _check(lib().sjsa_prep(ctypes.byref(shape), _ptr(q), _ptr(M), _ptr(Kproj), _ptr(seq_len), int(k),
                           _ptr(workspace), workspace.numel(), _stream(stream)))


def prep_append(shape: Shape, k_new, v_new, pos, q, K, V, M, Kproj, seq_len, k, workspace, stream=None):
    """Scoring prep that first appends the step's new token (as decode_step_append)."""
    _need(q, "q", torch.bfloat16, (shape.batch, shape.n_kv_heads * shape.group, shape.head_dim))
    _need(M, "M", torch.float32, (shape.n_kv_heads, shape.rank, shape.head_dim))
    _need(K, "K", torch.bfloat16, (shape.batch, shape.n_kv_heads, shape.capacity, shape.head_dim))
    _need(V, "V", torch.bfloat16, K.shape)
    _need_kproj(Kproj, (shape.batch, shape.n_kv_heads, shape.capacity, shape.rank), bool(shape.flags & SJSA_FLAG_KPROJ_FP8))
    _need(seq_len, "seq_len", torch.int32, (shape.batch,))
    _append_one_checks(k_new, v_new, pos, K, M)
    _check(lib().sjsa_prep_append(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(q), _ptr(K),
                                  _ptr(V), _ptr(Kproj), _ptr(M), _ptr(seq_len), int(k), _ptr(workspace),
                                  workspace.numel(), _stream(stream)))


def scan(shape: Shape, Kproj, seq_len, workspace, stream=None):
    """Score scan only (after prep)."""
    _need_kproj(Kproj, (shape.batch, shape.n_kv_heads, shape.capacity, shape.rank), bool(shape.flags & SJSA_FLAG_KPROJ_FP8))
    _need(seq_len, "seq_len", torch.int32, (shape.batch,))
    _check(lib().sjsa_scan(ctypes.byref(shape), _ptr(Kproj), _ptr(seq_len), _ptr(workspace), workspace.numel(),
                           _stream(stream)))


def prep_scan(shape: Shape, q, M, Kproj, seq_len, k, workspace, k_new=None, v_new=None, pos=None, K=None, V=None,
              stream=None):
    """Prep and scan in one launch, as the decode steps run them; with k_new (and
    v_new, pos, K, V) the step's new token is appended first, as prep_append does.
    select() must follow on the same workspace before the next prep_scan()."""
    _need(q, "q", torch.bfloat16, (shape.batch, shape.n_kv_heads * shape.group, shape.head_dim))
    _need(M, "M", torch.float32, (shape.n_kv_heads, shape.rank, shape.head_dim))
    _need_kproj(Kproj, (shape.batch, shape.n_kv_heads, shape.capacity, shape.rank), bool(shape.flags & SJSA_FLAG_KPROJ_FP8))
    _need(seq_len, "seq_len", torch.int32, (shape.batch,))
    if k_new is not None:
        _need(K, "K", torch.bfloat16, (shape.batch, shape.n_kv_heads, shape.capacity, shape.head_dim))
        _need(V, "V", torch.bfloat16, K.shape)
        _append_one_checks(k_new, v_new, pos, K, M)
    _check(lib().sjsa_prep_scan(ctypes.byref(shape), _ptr(q), _ptr(M), _ptr(Kproj), _ptr(seq_len), int(k),
                                _ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(K), _ptr(V), _ptr(workspace),
                                workspace.numel(), _stream(stream)))


def select(shape: Shape, Kproj, seq_len, k, workspace, idx=None, stream=None):
    """Top-k from what score() left in the workspace."""
    if idx is None:
        idx = torch.empty((shape.batch, shape.n_kv_heads, int(k)), dtype=torch.int32, device=workspace.device)
    _need(idx, "idx", torch.int32, (shape.batch, shape.n_kv_heads, int(k)))
    _need_kproj(Kproj, (shape.batch, shape.n_kv_heads, shape.capacity, shape.rank), bool(shape.flags & SJSA_FLAG_KPROJ_FP8))
    _check(lib().sjsa_select(ctypes.byref(shape), _ptr(Kproj), _ptr(seq_len), int(k), _ptr(idx), _ptr(workspace),
                             workspace.numel(), _stream(stream)))
    return idx


def topk(scores, seq_len, k, workspace=None, idx=None, group=1, rank=16, stream=None):
    """Top-k of caller fp32 scores [B, H_kv, stride] (the first seq_len[b] entries valid)."""
    B, Hkv, stride = scores.shape
    _need(scores, "scores", torch.float32)
    _need(seq_len, "seq_len", torch.int32, (B,))
    shape = make_shape(B, Hkv, group, 128, rank, stride)
    if workspace is None:
        workspace = alloc_workspace(shape, k, scores.device)
    if idx is None:
        idx = torch.empty((B, Hkv, int(k)), dtype=torch.int32, device=scores.device)
    _check(lib().sjsa_topk(ctypes.byref(shape), _ptr(scores), stride, _ptr(seq_len), int(k), _ptr(idx),
                           _ptr(workspace), workspace.numel(), _stream(stream)))
    return idx


def attend(q, K, V, idx, seq_len, sm_scale=0.0, out=None, workspace=None, out_f32=False, rank=16,
           stream=None):
    """Gather-free attention of every query head over its KV head's idx [B, H_kv, k]."""
    B, Hkv, cap, d = K.shape
    _need(q, "q", torch.bfloat16)
    _need(K, "K", torch.bfloat16)
    _need(V, "V", torch.bfloat16, K.shape)
    _need(seq_len, "seq_len", torch.int32, (B,))
    k = idx.shape[2]
    _need(idx, "idx", torch.int32, (B, Hkv, k))
    shape = make_shape(B, Hkv, q.shape[1] // Hkv, d, rank, cap, out_f32)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32 if out_f32 else torch.bfloat16, device=q.device)
    _need(out, "out", torch.float32 if out_f32 else torch.bfloat16, q.shape)
    if workspace is None:
        workspace = alloc_workspace(shape, k, q.device)
    _check(lib().sjsa_attend(ctypes.byref(shape), _ptr(q), _ptr(K), _ptr(V), _ptr(idx), int(k), _ptr(seq_len),
                             float(sm_scale), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def default_sm_scale(head_dim: int = 128) -> float:
    return 1.0 / math.sqrt(head_dim)


def gated_shape(q: torch.Tensor, K: torch.Tensor, out_f32=False) -> Shape:
    B, Hkv, cap, d = K.shape
    Hq = q.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    return make_shape(B, Hkv, Hq // Hkv, d, 0, cap, out_f32)


def gated_workspace(shape: Shape, unit_size: int, k_units: int, device=None) -> torch.Tensor:
    n = lib().sjsa_gated_workspace_size(ctypes.byref(shape), int(unit_size), int(k_units))
    if n == 0:
        raise SjsaError(-2, "invalid shape, unit size or unit budget for the gated step")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def gated_decode_step(q, K, V, gate_scores, seq_len, unit_size, k_units, lam=1.0, sm_scale=0.0, out=None,
                      idx=None, workspace=None, out_f32=False, stream=None):
    """Gated-logit sparse decode step over context units of unit_size tokens: the
    current unit plus the k_units - 1 units with the largest gates, attention logits
    biased by lam * ln g. gate_scores [B, H_kv, >= ceil(cap/unit_size)] fp32 (the
    gates are their softmax over each sequence's units). Returns (out [B, H_q, d],
    idx [B, H_kv, k_units * unit_size])."""
    B, Hkv, cap, d = K.shape
    _need(q, "q", torch.bfloat16, (B, q.shape[1], d))
    _need(K, "K", torch.bfloat16, (B, Hkv, cap, d))
    _need(V, "V", torch.bfloat16, (B, Hkv, cap, d))
    _need(seq_len, "seq_len", torch.int32, (B,))
    if gate_scores.dim() != 3 or tuple(gate_scores.shape[:2]) != (B, Hkv):
        raise ValueError("gate_scores must be [B, H_kv, units]")
    _need(gate_scores, "gate_scores", torch.float32)
    shape = gated_shape(q, K, out_f32)
    ktok = int(unit_size) * int(k_units)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32 if out_f32 else torch.bfloat16, device=q.device)
    if idx is None:
        idx = torch.empty((B, Hkv, ktok), dtype=torch.int32, device=q.device)
    _need(out, "out", torch.float32 if out_f32 else torch.bfloat16, q.shape)
    _need(idx, "idx", torch.int32, (B, Hkv, ktok))
    if workspace is None:
        workspace = gated_workspace(shape, unit_size, k_units, q.device)
    _check(lib().sjsa_gated_decode_step(ctypes.byref(shape), _ptr(q), _ptr(K), _ptr(V), _ptr(gate_scores),
                                        int(gate_scores.shape[2]), _ptr(seq_len), int(unit_size), int(k_units),
                                        float(lam), float(sm_scale), _ptr(out), _ptr(idx), _ptr(workspace),
                                        workspace.numel(), _stream(stream)))
    return out, idx


def block_cache(K: torch.Tensor, block_size: int, int4: bool = False, bf16: bool = True):
    """Empty block-key caches for K [B, H_kv, cap, d]: (Kc bf16 or None, Kq uint8 or None,
    Ks fp16 or None), floor(cap / block_size) blocks per (b, h)."""
    B, Hkv, cap, d = K.shape
    nb = cap // int(block_size)
    Kc = torch.zeros(B, Hkv, nb, d, dtype=torch.bfloat16, device=K.device) if bf16 else None
    Kq = torch.zeros(B, Hkv, nb, d // 2, dtype=torch.uint8, device=K.device) if int4 else None
    Ks = torch.zeros(B, Hkv, nb, d // 64, dtype=torch.float16, device=K.device) if int4 else None
    return Kc, Kq, Ks


def _block_cache_checks(K, block_size, Kc, Kq, Ks):
    B, Hkv, cap, d = K.shape
    nb = cap // int(block_size)
    if Kc is None and (Kq is None or Ks is None):
        raise ValueError("give the bf16 block keys Kc, or the INT4 pair Kq and Ks")
    if (Kq is None) != (Ks is None):
        raise ValueError("Kq and Ks go together")
    if Kc is not None:
        _need(Kc, "Kc", torch.bfloat16, (B, Hkv, nb, d))
    if Kq is not None:
        _need(Kq, "Kq", torch.uint8, (B, Hkv, nb, d // 2))
        _need(Ks, "Ks", torch.float16, (B, Hkv, nb, d // 64))


def block_keys(K, seq_len, block_size, Kc=None, Kq=None, Ks=None, stream=None):
    """Keys of every complete block (mean of its keys, bf16; and/or the INT4 form)."""
    B, Hkv, cap, d = K.shape
    _need(K, "K", torch.bfloat16, (B, Hkv, cap, d))
    _need(seq_len, "seq_len", torch.int32, (B,))
    _block_cache_checks(K, block_size, Kc, Kq, Ks)
    shape = make_shape(B, Hkv, 1, d, 0, cap)
    _check(lib().sjsa_block_keys(ctypes.byref(shape), int(block_size), _ptr(K), _ptr(seq_len), _ptr(Kc), _ptr(Kq),
                                 _ptr(Ks), _stream(stream)))


def block_append(k_new, v_new, pos, K, V, block_size, Kc=None, Kq=None, Ks=None, stream=None):
    """Append T tokens per (b, h) at slots pos[b].. and write the keys of the blocks they complete."""
    B, Hkv, cap, d = K.shape
    T = k_new.shape[2]
    _need(K, "K", torch.bfloat16, (B, Hkv, cap, d))
    _need(V, "V", torch.bfloat16, (B, Hkv, cap, d))
    _need(k_new, "k_new", torch.bfloat16, (B, Hkv, T, d))
    _need(v_new, "v_new", torch.bfloat16, (B, Hkv, T, d))
    _need(pos, "pos", torch.int32, (B,))
    _block_cache_checks(K, block_size, Kc, Kq, Ks)
    shape = make_shape(B, Hkv, 1, d, 0, cap)
    _check(lib().sjsa_block_append(ctypes.byref(shape), int(block_size), _ptr(k_new), _ptr(v_new), int(T), _ptr(pos),
                                   _ptr(K), _ptr(V), _ptr(Kc), _ptr(Kq), _ptr(Ks), _stream(stream)))


def block_workspace(shape: Shape, block_size: int, k_blocks: int, device=None) -> torch.Tensor:
    n = lib().sjsa_block_workspace_size(ctypes.byref(shape), int(block_size), int(k_blocks))
    if n == 0:
        raise SjsaError(-2, "invalid shape, block size or block budget for the block-sparse step")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def block_decode_step(q, K, V, seq_len, block_size, k_blocks, Kc=None, Kq=None, Ks=None, n_init=1, n_local=2,
                      sm_scale=0.0, out=None, idx=None, workspace=None, out_f32=False, stream=None):
    """Block-sparse decode step: block scores from the bf16 keys Kc (or the INT4 keys
    Kq, Ks when Kc is None), forced first/local blocks plus the best others up to
    k_blocks, attention over their positions. Returns (out [B, H_q, d],
    idx [B, H_kv, k_blocks * block_size])."""
    B, Hkv, cap, d = K.shape
    _need(q, "q", torch.bfloat16, (B, q.shape[1], d))
    _need(K, "K", torch.bfloat16, (B, Hkv, cap, d))
    _need(V, "V", torch.bfloat16, (B, Hkv, cap, d))
    _need(seq_len, "seq_len", torch.int32, (B,))
    _block_cache_checks(K, block_size, Kc, Kq, Ks)
    shape = gated_shape(q, K, out_f32)
    ktok = int(block_size) * int(k_blocks)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32 if out_f32 else torch.bfloat16, device=q.device)
    if idx is None:
        idx = torch.empty((B, Hkv, ktok), dtype=torch.int32, device=q.device)
    _need(out, "out", torch.float32 if out_f32 else torch.bfloat16, q.shape)
    _need(idx, "idx", torch.int32, (B, Hkv, ktok))
    if workspace is None:
        workspace = block_workspace(shape, block_size, k_blocks, q.device)
    _check(lib().sjsa_block_decode_step(ctypes.byref(shape), int(block_size), _ptr(q), _ptr(K), _ptr(V), _ptr(Kc),
                                        _ptr(Kq), _ptr(Ks), _ptr(seq_len), int(k_blocks), int(n_init), int(n_local),
                                        float(sm_scale), _ptr(out), _ptr(idx), _ptr(workspace), workspace.numel(),
                                        _stream(stream)))
    return out, idx


def calib_workspace(q, k) -> torch.Tensor:
    """Workspace for calib_accumulate with these q [B, H_q, T, d] and k [B, H_kv, T, d]."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    shape = make_shape(B, Hkv, Hq // Hkv, d, 0, 1)
    n = lib().sjsa_calib_workspace_size(ctypes.byref(shape), int(T))
    if n == 0:
        raise SjsaError(-2, "invalid shape for the calibration accumulation")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def calib_accumulate(q, k, SQ, SK, workspace=None, stream=None):
    """Add one prefill's second-moment sums to the fp64 accumulators SQ, SK [H_kv, d, d]
    (device): q [B, H_q, T, d], k [B, H_kv, T, d] bf16."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    _need(q, "q", torch.bfloat16, (B, Hq, T, d))
    _need(k, "k", torch.bfloat16, (B, Hkv, T, d))
    _need(SQ, "SQ", torch.float64, (Hkv, d, d))
    _need(SK, "SK", torch.float64, (Hkv, d, d))
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    shape = make_shape(B, Hkv, Hq // Hkv, d, 0, 1)
    if workspace is None:
        workspace = calib_workspace(q, k)
    _check(lib().sjsa_calib_accumulate(ctypes.byref(shape), _ptr(q), _ptr(k), int(T), _ptr(SQ), _ptr(SK),
                                       _ptr(workspace), workspace.numel(), _stream(stream)))


def calib_basis(SQ, SK, r):
    """Host: the basis M [H_kv, r, d] fp32 and the eigenvalues [H_kv, d] (descending) of
    SQ/tr(SQ) + SK/tr(SK), from accumulated sums given as host arrays [H_kv, d, d]."""
    import numpy as np
    sq = np.ascontiguousarray(SQ.cpu().numpy() if isinstance(SQ, torch.Tensor) else SQ, dtype=np.float64)
    sk = np.ascontiguousarray(SK.cpu().numpy() if isinstance(SK, torch.Tensor) else SK, dtype=np.float64)
    H, d, _ = sq.shape
    M = np.empty((H, int(r), d), dtype=np.float32)
    w = np.empty((H, d), dtype=np.float64)
    _check(lib().sjsa_calib_basis(sq.ctypes.data, sk.ctypes.data, H, d, int(r), M.ctypes.data, w.ctypes.data))
    return M, w
