"""How exact must the activation operand of the weight products be?  The draft
step's weight products (FC, QKV, O, gate/up, down, LM head) are emulated in
fp64 under three operand schemes and compared with the exact fp64 draft step
(the oracle), against the 2e-2 bar on features and logits:

  split  - hi = x with its low 16 bits dropped, lo = bf16(x - hi), x W ~ hi W + lo W
           (the kernels' default: two bf16 MFMAs per product);
  bf16   - one rounding, bf16(x) W (EAGLE_ACT_BF16: one MFMA);
  fp8lo  - hi W in bf16 plus the correction term in OCP FP8 E4M3 with a
           power-of-two scale per row and 32-wide K block (what the scaled fp8
           MFMA of gfx950 would take at twice the bf16 rate): hi W + q8(lo) q8(W).

The weights are the draft-head workloads' N(0, 0.02) matrices; the KV cache is
bf16 in every scheme.  At the 7B shape the fp8 correction meets the bar and
one bf16 rounding does not; at the 70B shape (EAGLE_SLOW_TESTS=1: ~2 minutes,
~20 GB of host memory) only the split operand does, so the fp8 correction is
no replacement for the second bf16 MFMA there.  Draft head and operand
contract: "eagle feature-level speculative decoding", the draft-head section
("草稿头到底包含什么") and the correctness section ("正确性与状态边界").
"""
import dataclasses
import os

import numpy as np
import pytest

from oracle import draft as OD
from oracle.numerics import round_bf16
from workloads import CONFIGS, bf16_values, make_prefix_kv, make_weights, normal_array

BAR = 2e-2


def trunc_bf16(x):
    b = np.asarray(x, np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return b.view(np.float32).astype(np.float64)


def q_e4m3(x):
    """Round to OCP FP8 E4M3: 3 mantissa bits, normals from 2^-6, subnormal step
    2^-9, largest finite 448 (saturating), ties to even."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6.0)
    q = np.exp2(e - 3)
    return np.clip(np.round(x / q) * q, -448.0, 448.0)


def q_e4m3_blocks(x, blk=32):
    """E4M3 after a power-of-two scale per row and blk-wide block of the last
    axis that brings the block's largest magnitude into (224, 448]."""
    x = np.asarray(x, np.float64)
    R, K = x.shape
    xb = x.reshape(R, K // blk, blk)
    m = np.max(np.abs(xb), axis=2, keepdims=True)
    s = np.exp2(np.floor(np.log2(448.0 / np.where(m > 0, m, 1.0))))
    return (q_e4m3(xb * s) / s).reshape(R, K)


def _matmul(scheme, cache):
    def mm(x, w):
        x = np.asarray(x, np.float64)
        w64 = np.asarray(w, np.float64)
        if scheme == "bf16":
            return round_bf16(x) @ w64.T
        hi = trunc_bf16(x)
        if scheme == "split":
            return hi @ w64.T + round_bf16(x - hi) @ w64.T
        if id(w) not in cache:
            cache[id(w)] = q_e4m3_blocks(w64)
        return hi @ w64.T + q_e4m3_blocks(x - hi) @ cache[id(w)].T
    return mm


def _deviations(monkeypatch, cfg_id, M, seed=21, lens=(300, 77)):
    shape = CONFIGS[cfg_id].shape
    cfg = dataclasses.replace(CONFIGS[2], cid=100 + seed, shape=shape, batch=len(lens))
    w = make_weights(cfg, std=0.02)
    ks, vs = make_prefix_kv(cfg, np.asarray(lens))
    n_feat = 9
    feat = bf16_values(normal_array(200 + seed, 0, (n_feat, shape.d)))
    g = np.random.default_rng(1000 + seed)
    B = len(lens)
    rows = {k: [] for k in ("seq", "token", "parent", "pos", "slot", "mask")}
    for r in range(M):
        b = r % B
        rows["seq"].append(b)
        rows["token"].append(int(g.integers(0, shape.vocab)))
        rows["parent"].append(int(g.integers(0, n_feat)))
        rows["pos"].append(lens[b] + 1)
        rows["slot"].append(8 + r)
        rows["mask"].append((1 << (8 + r)) | 1)
    hkv, hd = shape.n_kv_heads, shape.head_dim
    tk0 = bf16_values(normal_array(300 + seed, 0, (B, 64, hkv, hd)))
    tv0 = bf16_values(normal_array(300 + seed, 1, (B, 64, hkv, hd)))

    def step():
        return OD.draft_step(shape, w, rows, feat, ks, vs, np.asarray(lens), tk0.astype(np.float64).copy(),
                             tv0.astype(np.float64).copy(), mirror=True)

    exact = step()
    dev = {}
    cache = {}
    for scheme in ("split", "bf16", "fp8lo"):
        monkeypatch.setattr(OD, "matmul_t", _matmul(scheme, cache))
        o = step()
        dev[scheme] = (float(np.max(np.abs(o["feat"] - exact["feat"]))),
                       float(np.max(np.abs(o["logits"] - exact["logits"]))))
        print(f"shape {cfg_id} {scheme:6s}: feature max-abs {dev[scheme][0]:.3e}, logit max-abs {dev[scheme][1]:.3e}")
    return dev


def test_e4m3_rounding():
    # representable values stay, ties go to the even mantissa, subnormals step by 2^-9, 448 saturates
    vals = np.array([1.0, 1.125, 1.0625, 1.1875, 448.0, 500.0, -3.25, 2.0**-9, 2.0**-10, 3 * 2.0**-10, 0.0])
    want = np.array([1.0, 1.125, 1.0, 1.25, 448.0, 448.0, -3.25, 2.0**-9, 0.0, 2.0**-8, 0.0])
    assert np.array_equal(q_e4m3(vals), want)
    # the block scale keeps a block's largest magnitude in (224, 448] before rounding
    x = np.array([[3e-3] + [1e-4] * 31])
    assert abs(q_e4m3_blocks(x)[0, 0] - 3e-3) <= 3e-3 * 2.0**-4


def test_operand_schemes_7b(monkeypatch):
    dev = _deviations(monkeypatch, 2, M=6)
    assert max(dev["split"]) < 1e-3
    assert max(dev["fp8lo"]) < BAR
    assert max(dev["bf16"]) > BAR


@pytest.mark.skipif(not os.environ.get("EAGLE_SLOW_TESTS"), reason="70B-shape fp64 draft step: set EAGLE_SLOW_TESTS=1")
def test_operand_schemes_70b(monkeypatch):
    dev = _deviations(monkeypatch, 5, M=4)
    assert max(dev["split"]) < BAR
    assert max(dev["fp8lo"]) > BAR
    assert max(dev["bf16"]) > BAR
