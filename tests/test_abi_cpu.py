"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol the header declares, sizes the superarbol, and rejects bad
arguments before touching a device."""
import ctypes
import os
import re

import pytest

from conditional_draft_tree_depth_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dtree.h")).read()
    return set(re.findall(r"\b(dtree_[a-z_]+)\s*\(", src))


def test_header_and_binding_agree():
    assert _declared() == set(_lib.EXPORTS)


def test_library_exports_every_symbol():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), name


def test_superarbol_sizes():
    lib = _lib.load()
    f = lambda *a: lib.dtree_superarbol_nodes(ctypes.byref(_lib.params(*a)))
    assert f(4, 8, 2, 4, 16, -0.1) == 23
    assert f(16, 32, 4, 8, 64, -0.05) == 469
    assert f(16, 64, 8, 32, 256, -0.02) == 3657
    assert f(16, 32, 4, 16, 128, -0.05) == 917
    assert f(16, 128, 8, 64, 512, 0.0) == 7241
    assert f(0, 8, 2, 4, 16, -0.1) == -1


def test_create_rejects_bad_arguments_before_device():
    lib = _lib.load()
    ctx = ctypes.c_void_p()
    caps = _lib.dtree_caps(1, 4, 8, 2, 4, 16)
    w = _lib.dtree_weights(64, 512, 32, 32, 16, 7, *([ctypes.c_void_p(16)] * 9))
    assert lib.dtree_create(ctypes.byref(w), ctypes.byref(caps), 0, ctypes.byref(ctx)) == 3
    w.wtype = 1   # bf16 with d % 128 != 0
    assert lib.dtree_create(ctypes.byref(w), ctypes.byref(caps), 0, ctypes.byref(ctx)) == 2
    assert b"128" in lib.dtree_last_error(None)
    w.wtype = 0
    bad = _lib.dtree_caps(1, 40, 8, 2, 4, 16)     # depth cap too large
    assert lib.dtree_create(ctypes.byref(w), ctypes.byref(bad), 0, ctypes.byref(ctx)) == 2
    bad = _lib.dtree_caps(1, 4, 256, 2, 4, 16)    # M cap too large
    assert lib.dtree_create(ctypes.byref(w), ctypes.byref(bad), 0, ctypes.byref(ctx)) == 2
    assert lib.dtree_create(None, ctypes.byref(caps), 0, ctypes.byref(ctx)) == 1
    assert lib.dtree_destroy(None) == 0
    assert lib.dtree_build_round(None, None, 1, *([None] * 9)) == 1
    assert lib.dtree_set_scoring(None, 0) == 1


def test_binding_refuses_missing_library(tmp_path):
    saved = _lib._lib
    try:
        _lib._lib = None
        with pytest.raises(RuntimeError):
            _lib.load(str(tmp_path / "nope.so"))
    finally:
        _lib._lib = saved


def test_static_round_refuses_oversized_workspace_before_device():
    """The allocation-free round sizes its workspace on the host and refuses
    one beyond its fixed device array before touching a device."""
    lib = _lib.load()
    w = _lib.dtree_weights(4096, 151936, 4096, 1024, 256, 1, *([ctypes.c_void_p(256)] * 9))
    p = _lib.params(16, 32, 4, 16, 128, -0.05)
    ptrs = [ctypes.c_void_p(256)] * 8
    code = lib.dtree_build_round_static(ctypes.byref(w), ctypes.byref(p), 8, *ptrs, None)
    assert code == 2   # DTREE_E_SHAPE
    assert b"static scratch" in lib.dtree_last_error(None)
    assert lib.dtree_build_round_static(None, ctypes.byref(p), 1, *ptrs, None) == 1
    p.beta = 0.5
    assert lib.dtree_build_round_static(ctypes.byref(w), ctypes.byref(p), 1, *ptrs, None) == 1


def _attn(**over):
    a = dict(batch=1, n_max=65, Hq=32, Hkv=8, dh=128, L_cap=4161, Q=256, K=256, V=256,
             prefix_len=256, n_nodes=256, mask=256, scale=0.088, O=256, splits=0, workspace=None,
             workspace_bytes=0)
    a.update(over)
    return _lib.dtree_attn_args(*[a[f] for f, _ in _lib.dtree_attn_args._fields_])


def test_attention_workspace_sizes():
    """Split choice and workspace size are host arithmetic.  Qwen3-4B (65
    nodes x 4 heads: three blocks of 128 query rows per KV head, 66 key
    tiles) takes 11 splits, 8 requests of 129 tree tokens (5 blocks per KV
    head) take 3, and one split needs no workspace."""
    ws = _lib.dtree_tree_attention_workspace
    size = lambda rows: ((rows * 128 * 4 + 255) // 256) * 256 + rows * 8
    assert ws(_attn()) == size(8 * 11 * 384)
    assert ws(_attn(splits=1)) == 0
    assert ws(_attn(batch=8, n_max=129, L_cap=4225)) == size(8 * 8 * 3 * 640)
    assert ws(_attn(splits=3)) == size(8 * 3 * 384)


@pytest.mark.parametrize("over,code", [
    (dict(dh=96), 2), (dict(Hq=30), 2), (dict(Hkv=0), 2), (dict(L_cap=10), 2),
    (dict(scale=0.0), 1), (dict(scale=float("nan")), 1), (dict(splits=-1), 1),
    (dict(batch=0), 1), (dict(n_max=5000, L_cap=9000), 2), (dict(Hq=8 * 65), 2),
    (dict(Q=None), 1), (dict(O=None), 1), (dict(mask=None), 1), (dict(K=264), 1),
    (dict(splits=4), 1),                       # needs a workspace
    (dict(splits=4, workspace=256, workspace_bytes=16), 1),
])
def test_attention_rejects_bad_arguments_before_device(over, code):
    lib = _lib.load()
    a = _attn(**over)
    assert lib.dtree_tree_attention(ctypes.byref(a), None) == code
    assert lib.dtree_last_error(None)


def test_heap_node_bound_and_builder_rejections():
    lib = _lib.load()
    p = _lib.params(16, 32, 4, 8, 64, -0.05)
    assert lib.dtree_heap_nodes(ctypes.byref(p)) == 4 * 65 + 1
    p.B = 0
    assert lib.dtree_heap_nodes(ctypes.byref(p)) == -1
    assert lib.dtree_set_builder(None, 1) == 1   # null context
