"""MI355X (gfx950) EAGLE draft-and-verify hot path: Python binding.

The functions below carry the C ABI's names (include/eagle.h) and only marshal
arguments: torch tensors give device pointers, torch's current stream gives the
HIP stream.  Every step of the path runs in libeagle.so's HIP kernels; if the
library is not built (python -m eagle_feature_level_amd.build) or the device
is not a gfx950, the calls raise.
"""
from __future__ import annotations

import ctypes

from . import _abi
from ._abi import (EAGLE_ACT_BF16, EAGLE_BF16, EAGLE_COMMIT_BAD_PATH, EAGLE_COMMIT_OVERFLOW, EAGLE_F32,
                   EAGLE_F_BADTREE, EAGLE_F_NAN, EAGLE_F_QEMPTY, EAGLE_F_QZERO, EAGLE_F_ZRES, EAGLE_FEATURES_ONLY,
                   EAGLE_HEAD_ONLY, EAGLE_MAX_SLOTS, EAGLE_MAX_TOPK, EAGLE_SAMPLE_CHILDREN, EAGLE_VERIFY_GREEDY,
                   EAGLE_VERIFY_IID, EAGLE_VERIFY_NOALLOC_MAX_NODES, EagleError, eagle_draft_out, eagle_kv, eagle_pool, eagle_rows, eagle_shape,
                   eagle_weights)

__all__ = ["eagle_blocked_weight_bytes", "eagle_block_weight", "eagle_workspace_bytes", "eagle_draft_step", "eagle_softmax_topk", "eagle_tree_init", "eagle_tree_expand",
           "eagle_tree_finalize", "eagle_verify", "eagle_verify_workspace_bytes", "make_shape", "make_weights",
           "make_rows", "make_kv", "make_out",
           "make_pool", "EagleError", "EAGLE_HEAD_ONLY", "EAGLE_ACT_BF16", "EAGLE_SAMPLE_CHILDREN",
           "eagle_sample_topk", "eagle_fuse_features", "eagle_fuse_workspace_bytes", "eagle_commit",
           "EAGLE_COMMIT_OVERFLOW", "EAGLE_COMMIT_BAD_PATH", "EAGLE_VERIFY_GREEDY", "EAGLE_VERIFY_IID", "EAGLE_BF16",
           "EAGLE_F32", "EAGLE_MAX_SLOTS", "EAGLE_MAX_TOPK", "eagle_profile_enable", "eagle_profile_reset",
           "eagle_profile_disable", "eagle_profile_read", "eagle_catchup_rows", "eagle_commit_catchup",
           "EAGLE_FEATURES_ONLY", "eagle_verify_noalloc", "EAGLE_VERIFY_NOALLOC_MAX_NODES", "EAGLE_F_ZRES", "EAGLE_F_QZERO", "EAGLE_F_QEMPTY", "EAGLE_F_NAN", "EAGLE_F_BADTREE"]

WEIGHT_NAMES = [f[0] for f in eagle_weights._fields_]


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _keep(struct, *tensors):
    """The structs hold raw device pointers; keep the tensors they point into
    alive for as long as the struct lives."""
    struct._keep = tuple(t for t in tensors if t is not None and not isinstance(t, int))
    return struct


def make_shape(d, n_heads, n_kv_heads, head_dim, ffn, vocab, rms_eps=1e-5, rope_theta=1e4, dtype="bf16"):
    return eagle_shape(d, n_heads, n_kv_heads, head_dim, ffn, vocab, rms_eps, rope_theta,
                       EAGLE_BF16 if dtype == "bf16" else EAGLE_F32)


def make_weights(tensors: dict):
    """Weight tensors by name; the blocked copies (names ending in _b) are optional."""
    return _keep(eagle_weights(*[_ptr(tensors.get(n)) for n in WEIGHT_NAMES]), *[tensors.get(n) for n in WEIGHT_NAMES])


def eagle_blocked_weight_bytes(rows, cols) -> int:
    return int(_abi.load().eagle_blocked_weight_bytes(rows, cols))


def eagle_block_weight(w, rows, cols, out, stream=None):
    lib = _abi.load()
    _abi.check("eagle_block_weight", lib.eagle_block_weight(_ptr(w), rows, cols, _ptr(out), _stream(stream)))


def make_rows(n_rows, batch, max_rows_per_seq, row_start, token, parent, pos=None, slot=None, mask=None):
    return _keep(eagle_rows(n_rows, batch, max_rows_per_seq, _ptr(row_start), _ptr(token), _ptr(parent), _ptr(pos),
                            _ptr(slot), _ptr(mask)), row_start, token, parent, pos, slot, mask)


def make_kv(prefix_k, prefix_v, prefix_off, prefix_len, max_prefix_len, tree_k, tree_v, prefix_cap=None,
            prefix_len_sum=0):
    return _keep(eagle_kv(_ptr(prefix_k), _ptr(prefix_v), _ptr(prefix_off), _ptr(prefix_len), max_prefix_len,
                          _ptr(tree_k), _ptr(tree_v), _ptr(prefix_cap), int(prefix_len_sum)), prefix_k, prefix_v,
                 prefix_off, prefix_len, tree_k, tree_v, prefix_cap)


def make_out(feat, logits, lse, topk, topk_idx, topk_logq, seed=0, round_=0, row_base=0):
    return _keep(eagle_draft_out(_ptr(feat), _ptr(logits), _ptr(lse), topk, _ptr(topk_idx), _ptr(topk_logq), seed,
                                 round_, row_base), feat, logits, lse, topk_idx, topk_logq)


def make_pool(cap, parent, token, depth, logv, feat_row, slot, mask, count, frontier):
    ts = (parent, token, depth, logv, feat_row, slot, mask, count, frontier)
    return _keep(eagle_pool(cap, *[_ptr(t) for t in ts]), *ts)


def eagle_workspace_bytes(shape, max_rows, max_batch, max_prefix_len) -> int:
    lib = _abi.load()
    return int(lib.eagle_workspace_bytes(ctypes.byref(shape), max_rows, max_batch, max_prefix_len))


def eagle_draft_step(shape, weights, flags, rows, feat_in, kv, out, workspace, stream=None):
    lib = _abi.load()
    rc = lib.eagle_draft_step(ctypes.byref(shape), ctypes.byref(weights), flags, ctypes.byref(rows), _ptr(feat_in),
                              ctypes.byref(kv) if kv is not None else None, ctypes.byref(out), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _abi.check("eagle_draft_step", rc)


def eagle_softmax_topk(n_rows, vocab, logits, topk, lse, topk_idx, topk_logq, workspace, stream=None):
    lib = _abi.load()
    rc = lib.eagle_softmax_topk(n_rows, vocab, _ptr(logits), topk, _ptr(lse), _ptr(topk_idx), _ptr(topk_logq),
                                _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _abi.check("eagle_softmax_topk", rc)


def eagle_commit(shape, batch, n_nodes, path, accept_len, node_slot, tree_k, tree_v, prefix_k, prefix_v, prefix_off,
                 prefix_len, prefix_cap, out_flags, stream=None):
    lib = _abi.load()
    rc = lib.eagle_commit(ctypes.byref(shape), batch, n_nodes, _ptr(path), _ptr(accept_len), _ptr(node_slot),
                          _ptr(tree_k), _ptr(tree_v), _ptr(prefix_k), _ptr(prefix_v), _ptr(prefix_off),
                          _ptr(prefix_len), _ptr(prefix_cap), _ptr(out_flags), _stream(stream))
    _abi.check("eagle_commit", rc)


def eagle_catchup_rows(batch, n_nodes, max_depth, tree_token, path, accept_len, next_token, prefix_len, feat_row0,
                       row_token, row_parent, row_pos, row_slot, row_mask, row_start, last_row, count, stream=None):
    lib = _abi.load()
    rc = lib.eagle_catchup_rows(batch, n_nodes, max_depth, _ptr(tree_token), _ptr(path), _ptr(accept_len),
                                _ptr(next_token), _ptr(prefix_len), feat_row0, _ptr(row_token), _ptr(row_parent),
                                _ptr(row_pos), _ptr(row_slot), _ptr(row_mask), _ptr(row_start), _ptr(last_row),
                                _ptr(count), _stream(stream))
    _abi.check("eagle_catchup_rows", rc)


def eagle_commit_catchup(shape, batch, count, tree_k, tree_v, prefix_k, prefix_v, prefix_off, prefix_len, prefix_cap,
                         feat, last_row, root_feat, out_flags, stream=None):
    lib = _abi.load()
    rc = lib.eagle_commit_catchup(ctypes.byref(shape), batch, _ptr(count), _ptr(tree_k), _ptr(tree_v), _ptr(prefix_k),
                                  _ptr(prefix_v), _ptr(prefix_off), _ptr(prefix_len), _ptr(prefix_cap), _ptr(feat),
                                  _ptr(last_row), _ptr(root_feat), _ptr(out_flags), _stream(stream))
    _abi.check("eagle_commit_catchup", rc)


def eagle_fuse_workspace_bytes(shape, max_rows):
    return _abi.load().eagle_fuse_workspace_bytes(ctypes.byref(shape), max_rows)


def eagle_fuse_features(shape, w_fuse, b_fuse, n_rows, low, mid, high, g, workspace, stream=None):
    lib = _abi.load()
    rc = lib.eagle_fuse_features(ctypes.byref(shape), _ptr(w_fuse), _ptr(b_fuse), n_rows, _ptr(low), _ptr(mid),
                                 _ptr(high), _ptr(g), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream))
    _abi.check("eagle_fuse_features", rc)


def eagle_sample_topk(n_rows, vocab, logits, topk, seed, round_, row_base, lse, topk_idx, topk_logq, workspace,
                      stream=None):
    lib = _abi.load()
    rc = lib.eagle_sample_topk(n_rows, vocab, _ptr(logits), topk, seed, round_, row_base, _ptr(lse), _ptr(topk_idx),
                               _ptr(topk_logq), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream))
    _abi.check("eagle_sample_topk", rc)


def eagle_tree_init(batch, pool, root_token, root_feat_row0, stream=None):
    lib = _abi.load()
    _abi.check("eagle_tree_init", lib.eagle_tree_init(batch, ctypes.byref(pool), _ptr(root_token), root_feat_row0,
                                                      _stream(stream)))


def eagle_tree_expand(batch, k, step, static_nchild, pool, n_prev, topk, topk_idx, topk_logq, n_next, feat_row0,
                      prefix_len, next_token, next_parent, next_pos, next_slot, next_mask, next_row_start,
                      stream=None):
    lib = _abi.load()
    rc = lib.eagle_tree_expand(batch, k, step, _ptr(static_nchild), ctypes.byref(pool), n_prev, topk, _ptr(topk_idx),
                               _ptr(topk_logq), n_next, feat_row0, _ptr(prefix_len), _ptr(next_token),
                               _ptr(next_parent), _ptr(next_pos), _ptr(next_slot), _ptr(next_mask),
                               _ptr(next_row_start), _stream(stream))
    _abi.check("eagle_tree_expand", rc)


def eagle_tree_finalize(batch, m, n_nodes, pool, prefix_len, tree_parent, tree_token, tree_depth, tree_pool,
                        tree_mask, tree_qrow, row_token, row_parent, row_pos, row_slot, row_mask, row_start,
                        stream=None):
    lib = _abi.load()
    rc = lib.eagle_tree_finalize(batch, m, n_nodes, ctypes.byref(pool), _ptr(prefix_len), _ptr(tree_parent),
                                 _ptr(tree_token), _ptr(tree_depth), _ptr(tree_pool), _ptr(tree_mask),
                                 _ptr(tree_qrow), _ptr(row_token), _ptr(row_parent), _ptr(row_pos), _ptr(row_slot),
                                 _ptr(row_mask), _ptr(row_start), _stream(stream))
    _abi.check("eagle_tree_finalize", rc)


def eagle_verify(batch, n_nodes, vocab, tree_parent, tree_token, target_logits, draft_logits, draft_row, seed, round_,
                 flags, out_path, out_accept_len, out_next_token, out_flags, workspace=None, stream=None):
    """workspace: None, or a device tensor of at least eagle_verify_workspace_bytes(batch, n_nodes) bytes."""
    lib = _abi.load()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.eagle_verify(batch, n_nodes, vocab, _ptr(tree_parent), _ptr(tree_token), _ptr(target_logits),
                          _ptr(draft_logits), _ptr(draft_row), seed, round_, flags, _ptr(out_path),
                          _ptr(out_accept_len), _ptr(out_next_token), _ptr(out_flags), _ptr(workspace), nbytes,
                          _stream(stream))
    _abi.check("eagle_verify", rc)


def eagle_verify_noalloc(batch, n_nodes, vocab, tree_parent, tree_token, target_logits, draft_logits, draft_row, seed,
                         round_, flags, out_path, out_accept_len, out_next_token, out_flags, stream=None):
    """eagle_verify with the library's own per-device scratch (no workspace, nothing allocated)."""
    lib = _abi.load()
    rc = lib.eagle_verify_noalloc(batch, n_nodes, vocab, _ptr(tree_parent), _ptr(tree_token), _ptr(target_logits),
                                  _ptr(draft_logits), _ptr(draft_row), seed, round_, flags, _ptr(out_path),
                                  _ptr(out_accept_len), _ptr(out_next_token), _ptr(out_flags), _stream(stream))
    _abi.check("eagle_verify_noalloc", rc)


def eagle_verify_workspace_bytes(batch, n_nodes):
    return int(_abi.load().eagle_verify_workspace_bytes(batch, n_nodes))


def eagle_profile_enable(max_launches: int):
    _abi.check("eagle_profile_enable", _abi.load().eagle_profile_enable(max_launches))


def eagle_profile_reset():
    _abi.check("eagle_profile_reset", _abi.load().eagle_profile_reset())


def eagle_profile_disable():
    _abi.check("eagle_profile_disable", _abi.load().eagle_profile_disable())


def eagle_profile_read(role) -> dict:
    """Launch count, summed duration (ms), algorithmic bytes and flops of one
    kernel role ('lm_head', 'gate_up', ... or its index) since the last reset."""
    if isinstance(role, str):
        role = _abi.ROLES.index(role)
    n = ctypes.c_int32()
    ms, by, fl = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _abi.check("eagle_profile_read", _abi.load().eagle_profile_read(role, ctypes.byref(n), ctypes.byref(ms),
                                                                      ctypes.byref(by), ctypes.byref(fl)))
    return dict(launches=n.value, ms=ms.value, bytes=by.value, flops=fl.value)
