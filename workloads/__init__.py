"""Seeded synthetic inputs for the EAGLE draft/verify hot path.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic: no GEMM, no softmax, no tree logic.  Both the fp64 CPU
oracle tests and the HIP path's tests/bench take their inputs from here, so the
two sides see identical bits.

Every stream is numpy ``PCG64(SeedSequence([config_id, stream_id]))``.  Values
that the GPU stores in bf16 are rounded to bf16 (round-to-nearest-even) here,
once, so that the fp32 arrays handed to the oracle are exactly the bf16 values
handed to the GPU.

Workload shapes follow the draft heads the EAGLE pages describe: a frozen
target embedding and LM head, an FC layer 2d->d with bias, and one LLaMA-style
decoder layer (EAGLE study note, sections 4.1 and 4.3; "eagle feature-level
speculative decoding", section on what the draft head contains).
"""
from __future__ import annotations

import dataclasses
import numpy as np

# stream ids: one independent PCG64 stream per kind of input
S_WEIGHTS, S_EMBED, S_LMHEAD, S_FEAT, S_PREFIX, S_TOKENS, S_LENS, S_NOISE, S_FEATNOISE, S_MISC, S_TRUEFEAT = range(11)


def rng(config_id: int, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config_id, stream, sub])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest even.  NaN is kept quiet."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    r = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_values(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value, returned as fp32."""
    return from_bf16_bits(to_bf16_bits(x))


@dataclasses.dataclass(frozen=True)
class Shape:
    d: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 1e4
    dtype: str = "bf16"  # "bf16" or "f32"


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    shape: Shape
    batch: int
    prefix: tuple  # ("fixed", L) or ("uniform", lo, hi)
    tree: str  # "chain5", "static26", "dynamic"
    topk: int
    depth: int  # deepest drafted node depth
    rerank_m: int  # drafted nodes kept (dynamic trees); 0 = whole template
    feat_noise: bool = False


# The five workloads.  Shapes: LLaMA2-7B / 13B / 70B-shaped draft heads (the
# pages' target models, EAGLE study note section 4.3) and one tiny head.
CONFIGS = {
    1: Config(1, "tiny-chain5-f32", Shape(64, 4, 4, 16, 172, 512, dtype="f32"), 1, ("fixed", 32),
              "chain5", 1, 4, 0),
    2: Config(2, "7b-static26-bf16", Shape(4096, 32, 32, 128, 11008, 32000), 1, ("fixed", 1024),
              "static26", 4, 5, 0),
    3: Config(3, "7b-eagle2-bf16", Shape(4096, 32, 32, 128, 11008, 32000), 1, ("fixed", 2048),
              "dynamic", 10, 6, 60),
    4: Config(4, "13b-eagle2-b8-bf16", Shape(5120, 40, 40, 128, 13824, 32000), 8, ("uniform", 512, 4096),
              "dynamic", 10, 6, 60),
    5: Config(5, "70b-gqa-eagle2-b16-bf16", Shape(8192, 64, 8, 128, 28672, 32000), 16, ("fixed", 4096),
              "dynamic", 10, 6, 60, feat_noise=True),
}

# Static tree templates, BFS order, node 0 = root, siblings contiguous in rank
# order.  chain5: root + 4 drafted nodes.  static26: depth 5, branching 4/3/2/1
# by depth favouring rank-0 children (a node at depth t with sibling rank r gets
# max(0, b_t - r) children, b = 4,3,2,1), then one extra rank-0 child under the
# two depth-4 nodes with the lowest path rank-sum.
TEMPLATES = {
    "chain5": [-1, 0, 1, 2, 3],
    "static26": [-1, 0, 0, 0, 0, 1, 1, 1, 2, 2, 3, 5, 5, 6, 8, 8, 9, 10, 10, 11, 13, 14, 16, 17, 19, 20],
}


def template_child_counts(parents) -> np.ndarray:
    n = len(parents)
    c = np.zeros(n, dtype=np.int32)
    for p in parents[1:]:
        c[p] += 1
    return c


def normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


@dataclasses.dataclass
class Weights:
    """Draft-head weights, row-major [out, in] (y = x W^T); fp32 arrays whose
    values are bf16-representable when the shape's dtype is bf16."""
    embed: np.ndarray  # [V, d]
    fc_w: np.ndarray  # [d, 2d]
    fc_b: np.ndarray  # [d]
    norm1: np.ndarray  # [d]
    norm2: np.ndarray  # [d]
    wq: np.ndarray  # [Hq*hd, d]
    wk: np.ndarray  # [Hkv*hd, d]
    wv: np.ndarray  # [Hkv*hd, d]
    wo: np.ndarray  # [d, Hq*hd]
    w_gate: np.ndarray  # [F, d]
    w_up: np.ndarray  # [F, d]
    w_down: np.ndarray  # [d, F]
    lm_head: np.ndarray  # [V, d]

    def items(self):
        return [(f.name, getattr(self, f.name)) for f in dataclasses.fields(self)]


def make_weights(cfg: Config, std: float = 0.02) -> Weights:
    """Matrices, FC bias, embedding and LM head ~ N(0, std^2); RMSNorm gains
    1 + N(0, std^2) so that a kernel ignoring the gain is visible."""
    s = cfg.shape
    hq, hkv = s.n_heads * s.head_dim, s.n_kv_heads * s.head_dim
    shapes = [("fc_w", (s.d, 2 * s.d)), ("fc_b", (s.d,)), ("norm1", (s.d,)), ("norm2", (s.d,)),
              ("wq", (hq, s.d)), ("wk", (hkv, s.d)), ("wv", (hkv, s.d)), ("wo", (s.d, hq)),
              ("w_gate", (s.ffn, s.d)), ("w_up", (s.ffn, s.d)), ("w_down", (s.d, s.ffn))]
    out = {}
    for i, (name, shp) in enumerate(shapes):
        g = rng(cfg.cid, S_WEIGHTS, i)
        a = normal(g, shp, std)
        if name.startswith("norm"):
            a = (a + np.float32(1.0)).astype(np.float32)
        out[name] = a
    out["embed"] = normal(rng(cfg.cid, S_EMBED), (s.vocab, s.d), std)
    out["lm_head"] = normal(rng(cfg.cid, S_LMHEAD), (s.vocab, s.d), std)
    if s.dtype == "bf16":
        for k in out:
            out[k] = bf16_values(out[k])
    return Weights(**out)


def make_prefix_lens(cfg: Config) -> np.ndarray:
    if cfg.prefix[0] == "fixed":
        return np.full(cfg.batch, cfg.prefix[1], dtype=np.int32)
    lo, hi = cfg.prefix[1], cfg.prefix[2]
    return rng(cfg.cid, S_LENS).integers(lo, hi + 1, size=cfg.batch, dtype=np.int64).astype(np.int32)


def make_prefix_kv(cfg: Config, lens: np.ndarray):
    """Prefix K (already rotated) and V of the draft layer, ~N(0,1), one array
    [Hkv, L_b, hd] per sequence."""
    s = cfg.shape
    ks, vs = [], []
    for b, L in enumerate(lens):
        gk = rng(cfg.cid, S_PREFIX, 2 * b)
        gv = rng(cfg.cid, S_PREFIX, 2 * b + 1)
        k = normal(gk, (s.n_kv_heads, int(L), s.head_dim), 1.0)
        v = normal(gv, (s.n_kv_heads, int(L), s.head_dim), 1.0)
        if s.dtype == "bf16":
            k, v = bf16_values(k), bf16_values(v)
        ks.append(k)
        vs.append(v)
    return ks, vs


def make_root_features(cfg: Config) -> np.ndarray:
    """True target features at each sequence's last committed position, ~N(0,1)
    (plus U(-0.1,0.1) noise for the 70B workload).  Rounded to bf16 values for
    bf16 workloads so the GPU's bf16 GEMM operand is exact."""
    s = cfg.shape
    f = normal(rng(cfg.cid, S_FEAT), (cfg.batch, s.d), 1.0)
    if cfg.feat_noise:
        f = (f + rng(cfg.cid, S_FEATNOISE).uniform(-0.1, 0.1, size=f.shape).astype(np.float32)).astype(np.float32)
    if s.dtype == "bf16":
        f = bf16_values(f)
    return f


def make_root_tokens(cfg: Config) -> np.ndarray:
    return rng(cfg.cid, S_TOKENS).integers(0, cfg.shape.vocab, size=cfg.batch, dtype=np.int64).astype(np.int32)


def make_true_features(cfg: Config, rnd: int, n_rows: int) -> np.ndarray:
    """Stand-in for the target's features at the tree nodes of round `rnd`
    (the target's tree forward is not part of this path): ~N(0, 1), plus
    U(-0.1, 0.1) noise for the 70B workload, bf16 values for bf16 workloads;
    one row per (sequence, tree node).  The first round's root rows are the
    true root features (make_root_features); the caller puts them there."""
    s = cfg.shape
    f = normal(rng(cfg.cid, S_TRUEFEAT, 2 * rnd), (n_rows, s.d), 1.0)
    if cfg.feat_noise:
        f = (f + rng(cfg.cid, S_TRUEFEAT, 2 * rnd + 1).uniform(-0.1, 0.1, size=f.shape).astype(np.float32)).astype(
            np.float32)
    if s.dtype == "bf16":
        f = bf16_values(f)
    return f


def make_target_noise(cfg: Config, n_rows: int, sub: int = 0, std: float = 0.5) -> np.ndarray:
    """N(0, std^2) noise added to draft logits to synthesise target logits."""
    return normal(rng(cfg.cid, S_NOISE, sub), (n_rows, cfg.shape.vocab), std)


def uniform_ints(cid: int, sub: int, shape, lo: int, hi: int) -> np.ndarray:
    return rng(cid, S_MISC, sub).integers(lo, hi, size=shape, dtype=np.int64)


def normal_array(cid: int, sub: int, shape, std: float = 1.0) -> np.ndarray:
    return normal(rng(cid, S_MISC, sub), shape, std)
