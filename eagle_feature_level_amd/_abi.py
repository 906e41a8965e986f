"""ctypes view of include/eagle.h: struct layouts, argument types, loader.

Argument marshalling only; every computation runs in the HIP library.  The
library is loaded from this package directory; if it is missing or the device
is not a gfx950, calls raise instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libeagle.so")

c_i32, c_u64, c_f32, c_vp, c_size = ctypes.c_int32, ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

EAGLE_OK, EAGLE_EINVAL, EAGLE_EUNSUPPORTED, EAGLE_EWORKSPACE, EAGLE_EHIP = 0, -1, -2, -3, -4
EAGLE_F32, EAGLE_BF16 = 0, 1
EAGLE_HEAD_ONLY, EAGLE_ACT_BF16, EAGLE_SAMPLE_CHILDREN, EAGLE_FEATURES_ONLY = 1, 2, 4, 8
EAGLE_VERIFY_GREEDY, EAGLE_VERIFY_IID = 1, 2
EAGLE_MAX_SLOTS, EAGLE_MAX_TOPK = 64, 16
EAGLE_VERIFY_NOALLOC_MAX_NODES = 8192
EAGLE_COMMIT_OVERFLOW, EAGLE_COMMIT_BAD_PATH = 1, 2
EAGLE_F_ZRES, EAGLE_F_QZERO, EAGLE_F_QEMPTY, EAGLE_F_NAN, EAGLE_F_BADTREE = 1, 2, 4, 8, 16
ROLES = ("fc", "qkv", "rope", "attn", "o", "gate_up", "down", "lm_head", "topk", "rows")


class eagle_shape(ctypes.Structure):
    _fields_ = [("d", c_i32), ("n_heads", c_i32), ("n_kv_heads", c_i32), ("head_dim", c_i32), ("ffn", c_i32),
                ("vocab", c_i32), ("rms_eps", c_f32), ("rope_theta", c_f32), ("dtype", c_i32)]


class eagle_weights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in ("embed", "fc_w", "fc_b", "norm1", "norm2", "wq", "wk", "wv", "wo", "w_gate",
                                    "w_up", "w_down", "lm_head", "fc_w_b", "wq_b", "wk_b", "wv_b", "wo_b",
                                    "w_gate_b", "w_up_b", "w_down_b", "lm_head_b")]


class eagle_rows(ctypes.Structure):
    _fields_ = [("n_rows", c_i32), ("batch", c_i32), ("max_rows_per_seq", c_i32), ("row_start", c_vp),
                ("token", c_vp), ("parent", c_vp), ("pos", c_vp), ("slot", c_vp), ("mask", c_vp)]


class eagle_kv(ctypes.Structure):
    _fields_ = [("prefix_k", c_vp), ("prefix_v", c_vp), ("prefix_off", c_vp), ("prefix_len", c_vp),
                ("max_prefix_len", c_i32), ("tree_k", c_vp), ("tree_v", c_vp), ("prefix_cap", c_vp),
                ("prefix_len_sum", ctypes.c_int64)]


class eagle_draft_out(ctypes.Structure):
    _fields_ = [("feat", c_vp), ("logits", c_vp), ("lse", c_vp), ("topk", c_i32), ("topk_idx", c_vp),
                ("topk_logq", c_vp), ("seed", c_u64), ("round", c_u64), ("row_base", c_i32)]


class eagle_pool(ctypes.Structure):
    _fields_ = [("cap", c_i32), ("parent", c_vp), ("token", c_vp), ("depth", c_vp), ("logv", c_vp),
                ("feat_row", c_vp), ("slot", c_vp), ("mask", c_vp), ("count", c_vp), ("frontier", c_vp)]


P = ctypes.POINTER
_SIGS = {
    "eagle_workspace_bytes": (c_size, [P(eagle_shape), c_i32, c_i32, c_i32]),
    "eagle_draft_step": (c_i32, [P(eagle_shape), P(eagle_weights), c_i32, P(eagle_rows), c_vp, P(eagle_kv),
                                 P(eagle_draft_out), c_vp, c_size, c_vp]),
    "eagle_softmax_topk": (c_i32, [c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "eagle_fuse_workspace_bytes": (c_size, [P(eagle_shape), c_i32]),
    "eagle_fuse_features": (c_i32, [P(eagle_shape), c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "eagle_commit": (c_i32, [P(eagle_shape), c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                             c_vp, c_vp, c_vp]),
    "eagle_catchup_rows": (c_i32, [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp,
                                   c_vp, c_vp, c_vp, c_vp, c_vp]),
    "eagle_commit_catchup": (c_i32, [P(eagle_shape), c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                     c_vp, c_vp, c_vp, c_vp]),
    "eagle_sample_topk": (c_i32, [c_i32, c_i32, c_vp, c_i32, c_u64, c_u64, c_i32, c_vp, c_vp, c_vp, c_vp, c_size,
                                  c_vp]),
    "eagle_tree_init": (c_i32, [c_i32, P(eagle_pool), c_vp, c_i32, c_vp]),
    "eagle_tree_expand": (c_i32, [c_i32, c_i32, c_i32, c_vp, P(eagle_pool), c_i32, c_i32, c_vp, c_vp, c_i32, c_i32,
                                  c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "eagle_tree_finalize": (c_i32, [c_i32, c_i32, c_i32, P(eagle_pool), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                    c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "eagle_verify": (c_i32, [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_u64, c_u64, c_i32, c_vp, c_vp,
                             c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "eagle_verify_workspace_bytes": (ctypes.c_size_t, [c_i32, c_i32]),
    "eagle_verify_noalloc": (c_i32, [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_u64, c_u64, c_i32, c_vp,
                                     c_vp, c_vp, c_vp, c_vp]),
    "eagle_blocked_weight_bytes": (ctypes.c_size_t, [c_i32, c_i32]),
    "eagle_block_weight": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp]),
    "eagle_profile_enable": (c_i32, [c_i32]),
    "eagle_profile_reset": (c_i32, []),
    "eagle_profile_disable": (c_i32, []),
    "eagle_profile_read": (c_i32, [c_i32, P(c_i32), P(ctypes.c_double), P(ctypes.c_double), P(ctypes.c_double)]),
    "eagle_strerror": (ctypes.c_char_p, [c_i32]),
    "eagle_last_hip_error": (c_i32, []),
}
EXPORTED = tuple(_SIGS)

_lib = None


class EagleError(RuntimeError):
    def __init__(self, fn: str, code: int, hip: int = 0):
        self.code = code
        msg = _lib.eagle_strerror(code).decode() if _lib is not None else str(code)
        super().__init__(f"{fn} failed: {msg} (code {code}{', hipError ' + str(hip) if code == EAGLE_EHIP else ''})")


def load(path: str = LIB_PATH):
    """Load libeagle.so (no GPU needed to load).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run python -m eagle_feature_level_amd.build")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, code: int):
    if code != EAGLE_OK:
        raise EagleError(fn, code, _lib.eagle_last_hip_error() if _lib is not None else 0)
