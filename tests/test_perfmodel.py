"""The byte model against hand arithmetic for the 128K batch-16 step."""
from token_level_sparse_kv_amd.perfmodel import dense_kv_bytes, step_bytes


def test_long_batched_step_bytes():
    t = step_bytes(16, 8, 4, 128, 32, 131072, 4096)
    assert t["scan_kproj"] == 16 * 8 * 131072 * 64 == 1073741824
    assert t["attend_kv_rows"] == 16 * 8 * 4096 * 512 == 268435456
    assert t["select_idx"] == 2097152
    assert t["q"] == t["out"] == t["M"] == 131072
    assert t["append"] == 139264
    assert t["total"] == 1344806912
    assert dense_kv_bytes(16, 8, 128, 131072) == 8589934592
    # the FP8 score cache the pages deploy would be at most 6.25% of the bf16 KV cache at r=32
    assert (32 * 1) / (2 * 128 * 2) == 0.0625


def test_long_batched_step_bytes_fp8_cache():
    t = step_bytes(16, 8, 4, 128, 32, 131072, 4096, kb=1)
    assert t["scan_kproj"] == 16 * 8 * 131072 * 32 == 536870912
    assert t["append"] == 16 * 8 * (4 * 128 * 2 + 32) == 135168
    assert t["total"] == 1344806912 - 536870912 - 4096 == 807931904
