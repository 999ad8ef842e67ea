"""MI355X-native JSSA token-level sparse decode: hand-written HIP kernels for
gfx950 behind the C ABI in include/sjsa.h, with a thin ctypes binding."""
from .sjsa import (SjsaError, Shape, make_shape, shape_of, workspace_size, alloc_workspace,  # noqa: F401
                   scores_view, append_kv, decode_step, decode_step_append, decode_step_append_noalloc, score, prep, prep_append, scan, prep_scan,
                   select, topk, attend, gated_decode_step, gated_workspace, gated_shape,
                   block_cache, block_keys, block_append, block_workspace, block_decode_step,
                   calib_accumulate, calib_workspace, calib_basis, lib, LIB_PATH,
                   SJSA_FLAG_OUT_F32, SJSA_FLAG_KPROJ_FP8, SJSA_MAX_K, NOALLOC_SCRATCH_BYTES, kproj_is_fp8)
