"""Host-side checks of the C ABI: every declared symbol is exported, the workspace
layout is consistent, and invalid arguments are rejected before any launch.
No call here reaches the GPU (every call fails validation first)."""
import ctypes
import os
import re

import pytest

import token_level_sparse_kv_amd as sj

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "sjsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sjsa_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert "sjsa_decode_step" in names and "sjsa_append_kv" in names
    lib = ctypes.CDLL(sj.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def _shape(**kw):
    base = dict(batch=2, n_kv_heads=8, group=4, head_dim=128, rank=32, capacity=1000, flags=0, fused_wait_us=0)
    base.update(kw)
    s = sj.make_shape(base["batch"], base["n_kv_heads"], base["group"], base["head_dim"], base["rank"],
                      base["capacity"], fused_wait_us=base["fused_wait_us"])
    s.flags = base["flags"]
    return s


def test_workspace_size_and_layout():
    L = sj.lib()
    s = _shape()
    ws = sj.workspace_size(s, 256)
    off = L.sjsa_workspace_scores_offset(ctypes.byref(s))
    stride = L.sjsa_workspace_score_stride(ctypes.byref(s))
    assert stride >= 1000 and stride % 64 == 0
    assert off % 256 == 0
    assert ws >= off + 2 * 8 * stride * 4
    assert ws % 256 == 0
    # bigger budgets never need less workspace
    assert sj.workspace_size(s, 4096) >= ws
    # invalid shapes or k give 0
    assert L.sjsa_decode_workspace_size(ctypes.byref(_shape(head_dim=64)), 256) == 0
    assert L.sjsa_decode_workspace_size(ctypes.byref(s), 0) == 0
    assert L.sjsa_decode_workspace_size(None, 16) == 0


@pytest.mark.parametrize("rank,cap", [(16, 1000), (32, 131072), (64, 150001)])
def test_workspace_layout_does_not_depend_on_the_cache_format(rank, cap):
    # stage calls that do not name the projected cache's format (attend) share the
    # workspace of those that do: the FP8 flag changes neither the size nor an offset
    L = sj.lib()
    a = _shape(rank=rank, capacity=cap)
    b = _shape(rank=rank, capacity=cap, flags=4)      # SJSA_FLAG_KPROJ_FP8
    for k in (256, 4096):
        assert sj.workspace_size(a, k) == sj.workspace_size(b, k) > 0
    assert L.sjsa_workspace_scores_offset(ctypes.byref(a)) == L.sjsa_workspace_scores_offset(ctypes.byref(b))


FAKE = 1 << 20          # aligned, never dereferenced: every call below fails validation


def _step(shape, k=16, ws_bytes=1 << 30, ptrs=None, sm_scale=0.0):
    L = sj.lib()
    p = [ctypes.c_void_p(FAKE)] * 9 if ptrs is None else ptrs
    return L.sjsa_decode_step(ctypes.byref(shape), p[0], p[1], p[2], p[3], p[4], p[5], k, sm_scale, p[6], p[7],
                              p[8], ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), -3), (dict(rank=24), -3), (dict(group=3), -3), (dict(group=16), -3),
    (dict(flags=8), -3),
    (dict(batch=0), -2), (dict(capacity=0), -2), (dict(capacity=(1 << 30) + 1), -2),
    (dict(batch=1000, n_kv_heads=100), -2), (dict(fused_wait_us=1000001), -2),
])
def test_bad_shapes(kw, status):
    assert _step(_shape(**kw)) == status


def test_bad_k_null_workspace_alignment():
    s = _shape()
    assert _step(s, k=0) == -4
    assert _step(s, k=(1 << 20) + 1) == -4
    ptrs = [ctypes.c_void_p(FAKE)] * 9
    ptrs[3] = None
    assert _step(s, ptrs=ptrs) == -1
    assert _step(s, ws_bytes=1024) == -5
    ptrs = [ctypes.c_void_p(FAKE)] * 9
    ptrs[0] = ctypes.c_void_p(FAKE + 2)
    assert _step(s, ptrs=ptrs) == -7
    ptrs = [ctypes.c_void_p(FAKE)] * 9
    ptrs[8] = ctypes.c_void_p(FAKE + 64)            # workspace needs 256-byte alignment
    assert _step(s, ptrs=ptrs) == -7
    assert _step(s, sm_scale=float("nan")) == -2
    L = sj.lib()
    assert L.sjsa_decode_step(None, *([None] * 6), 16, 0.0, None, None, None, 0, None) == -1


def test_stage_validation():
    L = sj.lib()
    s = _shape()
    f = ctypes.c_void_p(FAKE)
    assert L.sjsa_score(ctypes.byref(s), f, f, f, f, 16, f, 16, None) == -5
    assert L.sjsa_score(ctypes.byref(s), f, f, f, f, 0, f, 1 << 30, None) == -4
    assert L.sjsa_prep(ctypes.byref(s), f, f, None, f, 16, f, 1 << 30, None) == -1
    assert L.sjsa_scan(ctypes.byref(s), f, f, f, 16, None) == -5
    assert L.sjsa_select(ctypes.byref(s), f, f, 0, f, f, 1 << 30, None) == -4
    assert L.sjsa_select(ctypes.byref(s), None, f, 8, f, f, 1 << 30, None) == -1
    assert L.sjsa_topk(ctypes.byref(s), f, 999, f, 8, f, f, 1 << 30, None) == -2      # stride < cap
    assert L.sjsa_topk(ctypes.byref(s), f, 1002, f, 8, f, f, 1 << 30, None) == -2     # stride % 4
    assert L.sjsa_attend(ctypes.byref(s), f, f, f, f, 8, f, 0.0, f, f, 100, None) == -5
    assert L.sjsa_append_kv(ctypes.byref(s), f, f, 0, f, f, f, f, f, None) == -2
    assert L.sjsa_append_kv(ctypes.byref(s), f, None, 1, f, f, f, f, f, None) == -1
    for st in (0, -1, -2, -3, -4, -5, -6, -7, 5):
        assert isinstance(L.sjsa_status_string(st), bytes)


def test_fused_append_validation():
    L = sj.lib()
    s = _shape()
    f = ctypes.c_void_p(FAKE)
    args = [f] * 9                              # k_new, v_new, pos, q, K, V, Kproj, M, seq_len
    bad = list(args)
    bad[0] = None
    assert L.sjsa_decode_step_append(ctypes.byref(s), *bad, 16, 0.0, f, f, f, 1 << 30, None) == -1
    bad = list(args)
    bad[2] = ctypes.c_void_p(FAKE + 2)          # pos needs 4-byte alignment
    assert L.sjsa_decode_step_append(ctypes.byref(s), *bad, 16, 0.0, f, f, f, 1 << 30, None) == -7
    assert L.sjsa_decode_step_append(ctypes.byref(s), *args, 0, 0.0, f, f, f, 1 << 30, None) == -4
    assert L.sjsa_decode_step_append(ctypes.byref(s), *args, 16, 0.0, f, f, f, 1024, None) == -5
    assert L.sjsa_prep_append(ctypes.byref(s), *args, 16, f, 1024, None) == -5
    bad = list(args)
    bad[4] = None
    assert L.sjsa_prep_append(ctypes.byref(s), *bad, 16, f, 1 << 30, None) == -1


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 128, dtype=torch.bfloat16)
    K = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16)
    M = torch.zeros(1, 16, 128)
    with pytest.raises(ValueError):
        sj.decode_step(q, K, K, torch.zeros(1, 1, 64, 16, dtype=torch.bfloat16), M,
                       torch.zeros(1, dtype=torch.int32), 8)


def test_gated_validation():
    L = sj.lib()
    s = _shape(rank=0)                  # the gated step reads no scoring cache: rank is ignored
    f = ctypes.c_void_p(FAKE)

    def call(shape=s, unit=64, k_units=32, stride=16, lam=1.0, sm=0.0, ws=1 << 30, gates=f, out=f):
        return L.sjsa_gated_decode_step(ctypes.byref(shape), f, f, f, gates, stride, f, unit, k_units, lam, sm,
                                        out, f, f, ws, None)

    assert L.sjsa_gated_workspace_size(ctypes.byref(s), 64, 32) > 0
    assert L.sjsa_gated_workspace_size(ctypes.byref(s), 64, 0) == 0
    assert L.sjsa_gated_workspace_size(ctypes.byref(_shape(head_dim=64)), 64, 32) == 0
    assert call(k_units=0) == -2
    assert call(k_units=4097) == -2                       # above SJSA_MAX_SELECT_UNITS
    assert call(unit=0) == -2
    assert call(unit=1 << 12, k_units=512) == -4          # more than SJSA_MAX_K positions
    assert call(stride=15) == -2                          # ceil(1000 / 64) = 16 units per row
    assert call(lam=float("inf")) == -2
    assert call(sm=float("nan")) == -2
    assert call(ws=1024) == -5
    assert call(gates=None) == -1
    assert call(out=ctypes.c_void_p(FAKE + 4)) == -7
    assert call(shape=_shape(group=3)) == -3


def test_block_validation():
    L = sj.lib()
    s = _shape(rank=0)
    f = ctypes.c_void_p(FAKE)

    def step(shape=s, bs=64, kb=16, n_init=1, n_local=2, sm=0.0, ws=1 << 30, Kc=f, Kq=None, Ks=None, out=f):
        return L.sjsa_block_decode_step(ctypes.byref(shape), bs, f, f, f, Kc, Kq, Ks, f, kb, n_init, n_local, sm, out,
                                        f, f, ws, None)

    assert L.sjsa_block_workspace_size(ctypes.byref(s), 64, 16) > 0
    assert L.sjsa_block_workspace_size(ctypes.byref(s), 0, 16) == 0
    assert L.sjsa_block_workspace_size(ctypes.byref(s), 64, 0) == 0
    assert step(bs=0) == -2 and step(bs=4097) == -2
    assert step(kb=0) == -2 and step(kb=4097) == -2
    assert step(bs=4096, kb=257) == -4                   # more than SJSA_MAX_K positions
    assert step(n_init=-1) == -2 and step(n_local=-1) == -2
    assert step(kb=4, n_init=2, n_local=3) == -2         # forced blocks beyond the budget
    assert step(Kc=None) == -1                           # neither bf16 keys nor the INT4 pair
    assert step(Kc=None, Kq=f) == -1
    assert step(Kc=None, Kq=f, Ks=ctypes.c_void_p(FAKE + 1)) == -7
    assert step(sm=float("inf")) == -2
    assert step(ws=1024) == -5
    assert step(out=ctypes.c_void_p(FAKE + 8)) == -7
    assert step(shape=_shape(head_dim=96)) == -3
    assert L.sjsa_block_keys(ctypes.byref(s), 64, f, f, None, f, None, None) == -1     # Kq without Ks
    assert L.sjsa_block_keys(ctypes.byref(s), 64, f, None, f, None, None, None) == -1  # no seq_len
    assert L.sjsa_block_append(ctypes.byref(s), 64, f, f, 0, f, f, f, f, None, None, None) == -2
    assert L.sjsa_block_append(ctypes.byref(s), 64, f, f, 1, None, f, f, f, None, None, None) == -1


def test_shape_struct_layout_matches_the_header(tmp_path):
    # the binding's ctypes struct has the C layout of sjsa_shape (size and every field
    # offset), as a C compiler lays it out from include/sjsa.h
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f for f, _ in sj.Shape._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"sjsa.h\"\nint main(void) {\n"
                   + f'  printf("%zu\\n", sizeof(sjsa_shape));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(sjsa_shape, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(sj.Shape)
    assert got[1:] == [getattr(sj.Shape, f).offset for f in fields]


def test_noalloc_rejects_shapes_beyond_its_scratch():
    # the allocation-free step checks the shape's workspace against its static scratch
    # array before touching the device: 16 x 8 units at 131072 slots need ~136 MiB
    big = sj.make_shape(16, 8, 4, 128, 32, 131072)
    assert sj.workspace_size(big, 4096) > sj.NOALLOC_SCRATCH_BYTES
    L = sj.lib()
    p = [ctypes.c_void_p(FAKE)] * 12
    st = L.sjsa_decode_step_append_noalloc(ctypes.byref(big), *p[:9], 4096, 0.0, p[9], p[10], None)
    assert st == -8
    assert "static array" in L.sjsa_status_string(-8).decode()
    # invalid shapes and budgets are reported as for the workspace form
    assert L.sjsa_decode_step_append_noalloc(ctypes.byref(_shape(rank=24)), *p[:9], 16, 0.0, p[9], p[10],
                                             None) == -3
    assert L.sjsa_decode_step_append_noalloc(ctypes.byref(_shape()), *p[:9], 0, 0.0, p[9], p[10], None) == -4


def test_noalloc_capacity_stated_in_the_header():
    # include/sjsa.h states the allocation-free step's reach: up to 58 (sequence, KV
    # head) pairs at 131072 slots, r = 32, k = 4096, and about 2.8 MiB for one sequence
    # of 32768 tokens with 8 KV heads at k = 2048
    cap = sj.NOALLOC_SCRATCH_BYTES
    assert sj.workspace_size(sj.make_shape(58, 1, 4, 128, 32, 131072), 4096) <= cap
    assert sj.workspace_size(sj.make_shape(59, 1, 4, 128, 32, 131072), 4096) > cap
    assert sj.workspace_size(sj.make_shape(2, 29, 4, 128, 32, 131072), 4096) <= cap
    small = sj.workspace_size(sj.make_shape(1, 8, 4, 128, 32, 32768), 2048) / 2**20
    assert 2.75 <= small <= 2.85, small
