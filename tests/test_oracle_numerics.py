"""Pins for the oracle's building blocks, Philox and shapes (CPU only)."""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import numerics as N
from oracle.philox import philox4x64_10, philox4x64_10_np, uniform, uniforms_np
from oracle.shapes import trainable_params
from workloads import to_bf16_bits, from_bf16_bits

from conftest import GOLDEN


def test_philox_matches_numpy_generator():
    # numpy's Philox bit generator is Philox4x64-10; it increments the counter
    # before each block, so block i uses counter (i+1, 0, 0, 0).
    for key in [(1, 2), (0, 0), (0xDEADBEEFCAFEF00D, 7), (2**64 - 1, 2**63)]:
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.zeros(4, dtype=np.uint64))
        ref = bg.random_raw(4 * 6)
        mine = []
        for i in range(6):
            mine.extend(philox4x64_10((i + 1, 0, 0, 0), key))
        assert [int(x) for x in ref] == mine
        v = philox4x64_10_np(np.arange(1, 7), 0, 0, 0, key)
        got = np.stack(v, axis=1).reshape(-1)
        assert [int(x) for x in got] == mine


def test_philox_high_counter_words_match_numpy():
    # numpy carries into the higher counter words; start just below a carry.
    key = (3, 5)
    c = np.array([2**64 - 2, 9, 0, 0], dtype=np.uint64)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=c)
    ref = [int(x) for x in bg.random_raw(8)]
    mine = list(philox4x64_10((2**64 - 1, 9, 0, 0), key)) + list(philox4x64_10((0, 10, 0, 0), key))
    assert ref == mine


def test_uniform_grid_and_vectorised_agree():
    u = uniforms_np(0, 3, np.arange(50) % 5, np.arange(50) // 5, 64)
    for i in range(50):
        assert u[i] == uniform(0, 3, i % 5, i // 5, 64)
    assert np.all(u >= 0) and np.all(u < 1)
    assert np.all(u * 2**24 == np.floor(u * 2**24))


def test_round_bf16_matches_torch_rne():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(20000) * s for s in (1e-3, 1.0, 37.0)]).astype(np.float32)
    # exact halfway cases: bf16 value + half an ulp
    base = from_bf16_bits(to_bf16_bits(x[:1000]))
    ulp_half = np.abs(base) * 2.0**-8
    x = np.concatenate([x, (base + ulp_half).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(N.round_bf16(x).astype(np.float32), ref)
    assert np.array_equal(from_bf16_bits(to_bf16_bits(x)), ref)


def test_rmsnorm_closed_form():
    x = np.array([[3.0, 4.0]])
    # mean square = 12.5
    out = N.rmsnorm(x, np.array([1.0, 2.0]), 0.0)
    assert np.allclose(out, [[3 / np.sqrt(12.5), 8 / np.sqrt(12.5)]], rtol=0, atol=1e-15)


def test_rope_is_rotation_with_relative_phase():
    g = np.random.default_rng(1)
    q, k = g.standard_normal(128), g.standard_normal(128)
    for pos in (0, 1, 17, 4000):
        assert np.isclose(np.linalg.norm(N.rope_rotate_half(q, pos, 1e4)), np.linalg.norm(q), rtol=1e-13)
    assert np.allclose(N.rope_rotate_half(q, 0, 1e4), q)
    # scores depend only on the position difference
    a = N.rope_rotate_half(q, 1000, 1e4) @ N.rope_rotate_half(k, 990, 1e4)
    b = N.rope_rotate_half(q, 35, 1e4) @ N.rope_rotate_half(k, 25, 1e4)
    assert np.isclose(a, b, rtol=1e-9, atol=1e-9)
    # position 1, first pair rotates by exactly 1 radian
    e = np.zeros(128)
    e[0] = 1.0
    r = N.rope_rotate_half(e, 1, 1e4)
    assert np.isclose(r[0], np.cos(1.0)) and np.isclose(r[64], np.sin(1.0))


def test_softmax_and_lse_against_scipy():
    g = np.random.default_rng(2)
    v = g.standard_normal(32000) * 3
    assert np.isclose(N.logsumexp(v), scipy.special.logsumexp(v), rtol=0, atol=1e-12)
    assert np.allclose(N.softmax(v), scipy.special.softmax(v), rtol=1e-12, atol=0)


def test_silu_closed_form():
    assert N.silu(np.array([0.0]))[0] == 0.0
    assert np.isclose(N.silu(np.array([1.0]))[0], 1.0 / (1.0 + np.exp(-1.0)))


def test_param_counts_match_page_table():
    with open(os.path.join(GOLDEN, "param_table.json")) as f:
        table = json.load(f)
    for row in table["rows"]:
        n = trainable_params(**row["shape"])
        assert round(n / 1e9, 2) == row["billions"], (row["target"], n)
