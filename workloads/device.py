"""Upload seeded workloads to the GPU as torch tensors (data movement only)."""
from __future__ import annotations

import numpy as np
import torch

from . import Config, Shape, Weights, to_bf16_bits


def tensor(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """fp32 numpy array -> device tensor of dtype 'bf16' (bit-exact RNE) or 'f32'."""
    if dtype == "bf16":
        bits = to_bf16_bits(np.ascontiguousarray(arr, dtype=np.float32))
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def weights(w: Weights, dtype: str, device="cuda") -> dict:
    return {name: tensor(a, dtype, device) for name, a in w.items()}


def shape_dict(s: Shape) -> dict:
    return dict(d=s.d, n_heads=s.n_heads, n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, ffn=s.ffn, vocab=s.vocab,
                rms_eps=s.rms_eps, rope_theta=s.rope_theta, dtype=s.dtype)


def prefix(ks, vs, lens, dtype: str, device="cuda") -> dict:
    """Pack per-sequence [Hkv, L, hd] K and V contiguously; offsets in elements."""
    offs, o = [], 0
    for k in ks:
        offs.append(o)
        o += k.size
    flat_k = np.concatenate([k.reshape(-1) for k in ks]) if o else np.zeros(8, np.float32)
    flat_v = np.concatenate([v.reshape(-1) for v in vs]) if o else np.zeros(8, np.float32)
    return dict(k=tensor(flat_k, dtype, device), v=tensor(flat_v, dtype, device),
                off=torch.tensor(offs, dtype=torch.int64, device=device),
                len=torch.tensor(np.asarray(lens, dtype=np.int32), device=device), max_len=int(max(lens)) if len(lens) else 0)


def ints(a, device="cuda", dtype=torch.int32) -> torch.Tensor:
    return torch.tensor(np.asarray(a), dtype=dtype, device=device)


def masks(a, device="cuda") -> torch.Tensor:
    """uint64 bitmasks carried in an int64 tensor (same bits)."""
    return torch.from_numpy(np.asarray(a, dtype=np.uint64).view(np.int64)).to(device)
