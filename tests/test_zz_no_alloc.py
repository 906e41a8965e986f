"""eagle_verify_noalloc, the verification entry point that allocates nothing
(its per-node results live in the library's own per-device array), called
through the C ABI and checked against eagle_verify with a caller workspace:
identical paths, accepted lengths, next tokens and flags, on two calls in a
row, the second over a smaller input (the array keeps the first call's
contents, which the second must not see).  Sizes beyond the array are refused."""
import ctypes

import numpy as np
import pytest
import torch

import eagle_feature_level_amd as E
from eagle_feature_level_amd import _abi
from workloads import TEMPLATES
from workloads import device as dev

pytestmark = pytest.mark.gpu


def _case(seed, parent_list, B, V, noise):
    g = np.random.default_rng(seed)
    N = len(parent_list)
    draft = g.standard_normal((B, N, V), dtype=np.float32) * np.float32(1.7)
    target = draft + g.standard_normal((B, N, V), dtype=np.float32) * np.float32(noise)
    target[:, 0] = draft[:, 0]
    tokens = np.zeros((B, N), np.int32)
    for b in range(B):
        for u in range(N):
            kids = [i for i in range(N) if parent_list[i] == u]
            order = np.lexsort((np.arange(V), -draft[b, u]))
            for r, c in enumerate(kids):
                tokens[b, c] = order[r]
    return draft.reshape(B * N, V), target.reshape(B * N, V), tokens


def _outputs(B, N, fill):
    i32 = dict(dtype=torch.int32, device="cuda")
    return (torch.full((B * N,), fill, **i32), torch.full((B,), fill, **i32), torch.full((B,), fill, **i32),
            torch.full((B,), fill, **i32))


def _both(parent_list, B, V, seed, rnd, flags, noise):
    N = len(parent_list)
    draft, target, tokens = _case(seed, parent_list, B, V, noise)
    par = dev.ints(np.tile(np.asarray(parent_list, np.int32), B))
    tok = dev.ints(tokens.reshape(-1))
    tg, dr = torch.from_numpy(target).cuda(), torch.from_numpy(draft).cuda()
    rows = dev.ints(np.arange(B * N, dtype=np.int32))
    ref = _outputs(B, N, -5)
    ws = torch.empty(E.eagle_verify_workspace_bytes(B, N), dtype=torch.uint8, device="cuda")
    E.eagle_verify(B, N, V, par, tok, tg, dr, rows, 0, rnd, flags, *ref, workspace=ws)
    got = _outputs(B, N, -7)
    lib = _abi.load()
    rc = lib.eagle_verify_noalloc(B, N, V, par.data_ptr(), tok.data_ptr(), tg.data_ptr(), dr.data_ptr(),
                                  rows.data_ptr(), 0, rnd, flags, *[t.data_ptr() for t in got],
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == _abi.EAGLE_OK, lib.eagle_strerror(rc)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    return [t.cpu().numpy() for t in got]


def test_noalloc_verify_matches_workspace_verify_on_two_calls():
    # first call: 300 static-26 trees (7800 nodes, near the array's limit), vocabulary 4096
    first = _both(TEMPLATES["static26"], 300, 4096, seed=1, rnd=0, flags=0, noise=1.0)
    assert (first[1] >= 2).all()  # the root's first child is always accepted (q == p at the root)
    # second call: fewer, smaller trees, greedy mode, another vocabulary
    second = _both(TEMPLATES["chain5"], 3, 512, seed=2, rnd=5, flags=E.EAGLE_VERIFY_GREEDY, noise=0.5)
    assert second[0].shape == (15,)


def test_noalloc_verify_refuses_sizes_beyond_its_array():
    lib = _abi.load()
    big = (_abi.EAGLE_VERIFY_NOALLOC_MAX_NODES // 61) + 1
    rc = lib.eagle_verify_noalloc(big, 61, 32000, *([1] * 5), 0, 0, 0, *([1] * 4), None)
    assert rc == _abi.EAGLE_EUNSUPPORTED
    assert lib.eagle_verify_noalloc(0, 61, 32000, *([None] * 5), 0, 0, 0, *([None] * 4), None) == _abi.EAGLE_OK
