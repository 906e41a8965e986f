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


def prefix(ks, vs, lens, dtype: str, device="cuda", extra: int = 0) -> dict:
    """Per-sequence [Hkv, L, hd] K and V in one buffer, offsets in elements.
    extra = 0: packed [Hkv][L][hd].  extra > 0: each kv head gets room for
    `extra` more positions, [Hkv][L + extra][hd] (zero-filled), and the dict
    carries the capacities ("cap") and max_len = the largest capacity."""
    offs, o, parts_k, parts_v = [], 0, [], []
    for k, v in zip(ks, vs):
        H, L, hd = k.shape
        offs.append(o)
        pk = np.zeros((H, L + extra, hd), np.float32)
        pv = np.zeros((H, L + extra, hd), np.float32)
        pk[:, :L], pv[:, :L] = k, v
        parts_k.append(pk.reshape(-1))
        parts_v.append(pv.reshape(-1))
        o += pk.size
    flat_k = np.concatenate(parts_k) if o else np.zeros(8, np.float32)
    flat_v = np.concatenate(parts_v) if o else np.zeros(8, np.float32)
    lens = np.asarray(lens, dtype=np.int32)
    out = dict(k=tensor(flat_k, dtype, device), v=tensor(flat_v, dtype, device),
               off=torch.tensor(offs, dtype=torch.int64, device=device),
               len=torch.tensor(lens, device=device), max_len=int(lens.max() + extra) if len(lens) else 0)
    if extra:
        out["cap"] = torch.tensor(lens + extra, dtype=torch.int32, device=device)
    return out


def ints(a, device="cuda", dtype=torch.int32) -> torch.Tensor:
    return torch.tensor(np.asarray(a), dtype=dtype, device=device)


def masks(a, device="cuda") -> torch.Tensor:
    """uint64 bitmasks carried in an int64 tensor (same bits)."""
    return torch.from_numpy(np.asarray(a, dtype=np.uint64).view(np.int64)).to(device)
