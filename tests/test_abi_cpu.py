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
