"""Host-side checks of the C ABI (no GPU needed): every symbol declared in
include/eagle.h is exported by libeagle.so, and argument errors are reported
before any launch."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

import eagle_feature_level_amd as E
from eagle_feature_level_amd import _abi


def _declared():
    with open(os.path.join(ROOT, "include", "eagle.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(eagle_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = _abi.load()
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_abi.EXPORTED)


def test_strerror():
    lib = _abi.load()
    assert lib.eagle_strerror(0) == b"ok"
    assert b"workspace" in lib.eagle_strerror(-3)


def test_argument_errors_need_no_device():
    lib = _abi.load()
    # null shape
    assert lib.eagle_workspace_bytes(None, 1, 1, 1) == 0
    shape = E.make_shape(4096, 32, 32, 128, 11008, 32000)
    assert lib.eagle_workspace_bytes(ctypes.byref(shape), 0, 1, 1) == 0
    assert lib.eagle_workspace_bytes(ctypes.byref(shape), 5, 1, 1024) > 0
    bad = E.make_shape(4096, 30, 4, 128, 11008, 32000)  # heads not a multiple of kv heads
    assert lib.eagle_workspace_bytes(ctypes.byref(bad), 5, 1, 1024) == 0
    # blocked weight copies: columns a multiple of 128, rows padded to 16
    assert lib.eagle_blocked_weight_bytes(40, 384) == 48 * 384 * 2
    assert lib.eagle_blocked_weight_bytes(32000, 4096) == 32000 * 4096 * 2
    assert lib.eagle_blocked_weight_bytes(16, 100) == 0 and lib.eagle_blocked_weight_bytes(0, 128) == 0
    assert lib.eagle_block_weight(None, 16, 128, None, None) == _abi.EAGLE_EINVAL
    # draft step with null pointers
    w = E.eagle_weights()
    rows = E.make_rows(3, 1, 3, None, None, None)
    out = E.make_out(None, None, None, 4, None, None)
    rc = lib.eagle_draft_step(ctypes.byref(shape), ctypes.byref(w), 0, ctypes.byref(rows), None, None,
                              ctypes.byref(out), None, 0, None)
    assert rc == _abi.EAGLE_EINVAL
    # verify: bad sizes and flags
    assert lib.eagle_verify(-1, 5, 10, *([None] * 5), 0, 0, 0, *([None] * 5), 0, None) == _abi.EAGLE_EINVAL
    assert lib.eagle_verify(1, 0, 10, *([None] * 5), 0, 0, 0, *([None] * 5), 0, None) == _abi.EAGLE_EINVAL
    assert lib.eagle_verify(0, 5, 10, *([None] * 5), 0, 0, 0, *([None] * 5), 0, None) == _abi.EAGLE_OK  # empty batch
    # a workspace below eagle_verify_workspace_bytes is refused before anything runs
    need = lib.eagle_verify_workspace_bytes(2, 26)
    assert need >= 2 * 26 * 12 and lib.eagle_verify_workspace_bytes(1, 0) == 0
    assert lib.eagle_verify(2, 26, 10, *([1] * 5), 0, 0, 0, *([1] * 4), 1, need - 1, None) == _abi.EAGLE_EWORKSPACE
    # top-k larger than supported / than the vocabulary
    assert lib.eagle_softmax_topk(1, 8, 1, 9, 1, 1, 1, 1, 1 << 20, None) == _abi.EAGLE_EINVAL
    assert lib.eagle_softmax_topk(1, 64, 1, 17, 1, 1, 1, 1, 1 << 20, None) == _abi.EAGLE_EUNSUPPORTED
    assert lib.eagle_softmax_topk(0, 64, None, 4, None, None, None, None, 0, None) == _abi.EAGLE_OK
    # tree calls
    pool = E.eagle_pool()
    assert lib.eagle_tree_init(1, ctypes.byref(pool), None, 0, None) == _abi.EAGLE_EINVAL
    assert lib.eagle_tree_finalize(1, 60, 65, ctypes.byref(pool), *([None] * 13), None) == _abi.EAGLE_EINVAL
    # a finalize whose kept nodes cannot fit (m + 1 > n_nodes, or the whole pool with m = 0) is refused
    pool = E.eagle_pool(200, *([1] * 9))
    assert lib.eagle_tree_finalize(1, 60, 40, ctypes.byref(pool), *([1] * 13), None) == _abi.EAGLE_EINVAL
    assert lib.eagle_tree_finalize(1, 0, 61, ctypes.byref(pool), *([1] * 13), None) == _abi.EAGLE_EINVAL
    # HEAD_ONLY and FEATURES_ONLY together are refused
    rows = E.make_rows(3, 1, 3, 1, 1, 1, 1, 1, 1)
    out = E.make_out(1, None, None, 1, None, None)
    rc = lib.eagle_draft_step(ctypes.byref(shape), ctypes.byref(w), _abi.EAGLE_HEAD_ONLY | _abi.EAGLE_FEATURES_ONLY,
                              ctypes.byref(rows), 1, None, ctypes.byref(out), 1, 1 << 30, None)
    assert rc == _abi.EAGLE_EINVAL
    # catch-up rows: null outputs, too many rows per sequence
    assert lib.eagle_catchup_rows(1, 5, 4, *([None] * 5), 0, *([None] * 8), None) == _abi.EAGLE_EINVAL
    assert lib.eagle_catchup_rows(1, 5, 64, *([1] * 5), 0, *([1] * 8), None) == _abi.EAGLE_EUNSUPPORTED
    assert lib.eagle_catchup_rows(0, 5, 4, *([None] * 5), 0, *([None] * 8), None) == _abi.EAGLE_OK
    # catch-up commit: the root-feature gather needs all three of feat, last_row and root_feat
    assert lib.eagle_commit_catchup(ctypes.byref(shape), 1, *([1] * 8), 1, None, None, 1, None) == _abi.EAGLE_EINVAL
    assert lib.eagle_commit_catchup(ctypes.byref(shape), 1, *([None] * 8), None, None, None, None, None) == \
        _abi.EAGLE_EINVAL


def test_python_binding_raises_on_error():
    shape = E.make_shape(4096, 32, 32, 128, 11008, 32000)

    class _FakeWs:
        def numel(self):
            return 0

        def element_size(self):
            return 1

        def data_ptr(self):
            return 0
    with pytest.raises(E.EagleError):
        E.eagle_draft_step(shape, E.eagle_weights(), 0, E.make_rows(2, 1, 2, None, None, None), None, None,
                           E.make_out(None, None, None, 4, None, None), _FakeWs(), stream=0)
