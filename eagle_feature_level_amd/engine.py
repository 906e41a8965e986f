"""Device buffers and call sequence of one EAGLE draft-and-verify round.

Only sequences C-ABI calls; all arithmetic is in the HIP kernels.  The order
follows the pages' draft loop ("EAGLE 推测解码为什么比 Medusa 快" section 6.1;
"EAGLE 完全拆解", four-step pipeline): the root distribution from the root
feature, then per depth an expansion step and one draft step over the new
frontier, then rerank/flatten, an optional draft step over every drafted node
of the flattened tree, and verification.  Between rounds, catch_up() rebuilds
the drafter's rows over the committed tokens from the target's true features
and commits them ("eagle feature-level speculative decoding", KV commit
section: the drafter continues from the committed path A-B-X); the next round
then starts from the root rows it leaves behind (next_round_inputs()).

Feature rows and logit rows share one index space: rows [0, B) are the root
rows (true features, root logits); each depth step appends B * n rows.
"""
from __future__ import annotations

import dataclasses

import torch

from . import (EAGLE_ACT_BF16, EAGLE_FEATURES_ONLY, EAGLE_HEAD_ONLY, EAGLE_SAMPLE_CHILDREN, eagle_block_weight,
               eagle_blocked_weight_bytes, eagle_catchup_rows, eagle_commit_catchup, eagle_draft_step,
               eagle_tree_expand, eagle_tree_finalize, eagle_tree_init, eagle_verify, eagle_verify_workspace_bytes,
               eagle_workspace_bytes, make_kv, make_out, make_pool, make_rows, make_shape, make_weights)


@dataclasses.dataclass
class Step:
    n_prev: int
    n_next: int
    feat_row0: int
    token: torch.Tensor
    parent: torch.Tensor
    pos: torch.Tensor
    slot: torch.Tensor
    mask: torch.Tensor
    row_start: torch.Tensor


class EagleRound:
    def __init__(self, shape: dict, weights: dict, batch: int, kind: str, k: int, depth: int, m: int = 0,
                 template=None, prefix=None, device="cuda", act_bf16=False, blocked=True):
        """shape: d, n_heads, n_kv_heads, head_dim, ffn, vocab, rms_eps, rope_theta, dtype.
        weights: name -> device tensor.  prefix: dict(k, v, off, len, max_len[, cap]) device tensors (cap:
        per-sequence capacity of each kv head's positions, needed by catch_up(); max_len must cover it).
        act_bf16: False (default: split-bf16 operands, within 2e-2 of the fp64
        oracle at every workload), True (EAGLE_ACT_BF16 on every draft step of a
        bf16 workload), or "auto" (EAGLE_ACT_BF16 on steps over more than
        ACT_BF16_MIN_ROWS rows, where one MFMA per product instead of two matters).
        Rounding the activations to bf16 measured 0.03-0.18 max-abs off the fp64
        logits at the 7B-70B shapes, so it is opt-in.
        blocked (bf16 workloads): also keep the weight matrices in the blocked
        layout (eagle_block_weight) for the draft steps' weight-streaming GEMMs;
        the same results, one more copy of the weights in device memory."""
        self.act_bf16 = act_bf16
        self.shape_d = shape
        self.shape = make_shape(**shape)
        self.weights_t = dict(weights)
        if blocked and shape["dtype"] == "bf16":
            for n in ("fc_w", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "lm_head"):
                t = weights[n]
                rows, cols = t.shape[0], t.numel() // t.shape[0]
                out = torch.empty(eagle_blocked_weight_bytes(rows, cols), dtype=torch.uint8, device=device)
                eagle_block_weight(t, rows, cols, out)
                self.weights_t[n + "_b"] = out
        self.weights = make_weights(self.weights_t)
        self.B, self.kind, self.k, self.depth, self.m = batch, kind, k, depth, m
        self.dev = device
        d, V = shape["d"], shape["vocab"]
        hkv, hd = shape["n_kv_heads"], shape["head_dim"]
        kvdt = torch.bfloat16 if shape["dtype"] == "bf16" else torch.float32
        i32 = dict(dtype=torch.int32, device=device)
        B = batch
        if kind == "dynamic":
            self.cap = 1 + k + (depth - 1) * k * k
            self.nchild = None
            self.topk = k
            ns = [k] * (depth - 1)
            self.n_nodes = m + 1
        else:
            tmpl = list(template)
            self.cap = len(tmpl)
            nch = [0] * len(tmpl)
            dep = [0] * len(tmpl)
            for i in range(1, len(tmpl)):
                nch[tmpl[i]] += 1
                dep[i] = dep[tmpl[i]] + 1
            self.nchild = torch.tensor(nch, **i32)
            self.topk = max(1, max(nch))
            ns = [sum(1 for i in range(len(tmpl)) if dep[i] == s + 1 and nch[i] > 0) for s in range(depth - 1)]
            self.n_nodes = len(tmpl)
        self.ns = ns
        total = B + sum(B * n for n in ns)
        self.total_rows = total
        self.feat = torch.zeros(total, d, dtype=torch.float32, device=device)
        self.logits = torch.zeros(total, V, dtype=torch.float32, device=device)
        self.lse = torch.zeros(total, dtype=torch.float32, device=device)
        self.topk_idx = torch.zeros(total, self.topk, **i32)
        self.topk_logq = torch.zeros(total, self.topk, dtype=torch.float32, device=device)
        self.root_rows = torch.arange(B, **i32)
        self.root_start = torch.arange(B + 1, **i32)
        # pool
        cap = self.cap
        self.pool_t = dict(parent=torch.zeros(B * cap, **i32), token=torch.zeros(B * cap, **i32),
                           depth=torch.zeros(B * cap, **i32),
                           logv=torch.zeros(B * cap, dtype=torch.float32, device=device),
                           feat_row=torch.zeros(B * cap, **i32), slot=torch.zeros(B * cap, **i32),
                           mask=torch.zeros(B * cap, dtype=torch.int64, device=device),
                           count=torch.zeros(B, **i32), frontier=torch.zeros(B * 64, **i32))
        self.pool = make_pool(cap, **self.pool_t)
        # per-step rows
        self.steps = []
        row0 = B
        n_prev = 1
        for n in ns:
            self.steps.append(Step(n_prev, n, row0, torch.zeros(B * n, **i32), torch.zeros(B * n, **i32),
                                   torch.zeros(B * n, **i32), torch.zeros(B * n, **i32),
                                   torch.zeros(B * n, dtype=torch.int64, device=device), torch.zeros(B + 1, **i32)))
            row0 += B * n
            n_prev = n
        self.last_n = n_prev
        # final tree and tree-wide rows
        N = self.n_nodes
        self.tree = dict(parent=torch.zeros(B * N, **i32), token=torch.zeros(B * N, **i32),
                         depth=torch.zeros(B * N, **i32), pool=torch.zeros(B * N, **i32),
                         mask=torch.zeros(B * N, dtype=torch.int64, device=device), qrow=torch.zeros(B * N, **i32))
        nw = B * (N - 1)
        self.tw = dict(token=torch.zeros(nw, **i32), parent=torch.zeros(nw, **i32), pos=torch.zeros(nw, **i32),
                       slot=torch.zeros(nw, **i32), mask=torch.zeros(nw, dtype=torch.int64, device=device),
                       row_start=torch.zeros(B + 1, **i32))
        self.tw_feat = torch.zeros(max(nw, 1), d, dtype=torch.float32, device=device)
        self.tw_logits = torch.zeros(max(nw, 1), V, dtype=torch.float32, device=device)
        self.tw_lse = torch.zeros(max(nw, 1), dtype=torch.float32, device=device)
        self.tw_idx = torch.zeros(max(nw, 1), 1, **i32)
        self.tw_logq = torch.zeros(max(nw, 1), 1, dtype=torch.float32, device=device)
        # KV
        self.tree_k = torch.zeros(B, 64, hkv, hd, dtype=kvdt, device=device)
        self.tree_v = torch.zeros(B, 64, hkv, hd, dtype=kvdt, device=device)
        self.tw_tree_k = torch.zeros_like(self.tree_k)
        self.tw_tree_v = torch.zeros_like(self.tree_v)
        self.prefix = prefix
        # the prefix lengths' sum at construction, for the measurement hook's byte count only
        len_sum = int(prefix["len"].sum().item()) if prefix.get("len") is not None else 0
        self.kv = make_kv(prefix["k"], prefix["v"], prefix["off"], prefix["len"], prefix["max_len"], self.tree_k,
                          self.tree_v, prefix.get("cap"), len_sum)
        self.tw_kv = make_kv(prefix["k"], prefix["v"], prefix["off"], prefix["len"], prefix["max_len"],
                             self.tw_tree_k, self.tw_tree_v, prefix.get("cap"), len_sum)
        self.c_flags = torch.zeros(B, dtype=torch.int32, device=device)
        # catch-up rows between rounds: R = depth + 1 rows per sequence (the root and every accepted drafted
        # node, each joined with the token after it), their f^, which of them starts the next round, and
        # how many slots each sequence commits
        R = depth + 1
        self.cu_R = R
        self.cu = dict(token=torch.zeros(B * R, **i32), parent=torch.zeros(B * R, **i32),
                       pos=torch.zeros(B * R, **i32), slot=torch.zeros(B * R, **i32),
                       mask=torch.zeros(B * R, dtype=torch.int64, device=device), row_start=torch.zeros(B + 1, **i32),
                       last_row=torch.zeros(B, **i32), count=torch.zeros(B, **i32))
        self.cu_feat = torch.zeros(B * R, d, dtype=torch.float32, device=device)
        max_rows = max([B] + [B * n for n in ns] + [nw, B * R])
        ws = max(eagle_workspace_bytes(self.shape, max_rows, B, prefix["max_len"]),
                 eagle_verify_workspace_bytes(B, self.n_nodes))
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        # verify outputs
        self.v_path = torch.zeros(B * N, **i32)
        self.v_len = torch.zeros(B, **i32)
        self.v_next = torch.zeros(B, **i32)
        self.v_flags = torch.zeros(B, **i32)

    # ------------------------------------------------------------------ calls
    ACT_BF16_MIN_ROWS = 16

    def act_flag(self, n_rows: int) -> int:
        """EAGLE_ACT_BF16 or 0 for a draft step over n_rows rows."""
        if self.shape_d["dtype"] != "bf16":
            return 0
        on = self.act_bf16 if self.act_bf16 != "auto" else n_rows > self.ACT_BF16_MIN_ROWS
        return EAGLE_ACT_BF16 if on else 0

    def _sample_flag(self, sample):
        return EAGLE_SAMPLE_CHILDREN if sample is not None else 0

    def root_features(self) -> torch.Tensor:
        """The engine's own root-feature rows [B, d] (fp32): a caller that writes
        the target's last features here before a round saves the round's copy."""
        return self.feat[:self.B]

    def root_head(self, root_feat: torch.Tensor, sample=None):
        B = self.B
        if root_feat.data_ptr() != self.feat.data_ptr():  # already in place: no copy
            self.feat[:B].copy_(root_feat)
        rows = make_rows(B, B, 1, self.root_start, None, self.root_rows)
        seed, rnd = sample if sample is not None else (0, 0)
        out = make_out(None, self.logits, self.lse, self.topk, self.topk_idx, self.topk_logq, seed, rnd, 0)
        eagle_draft_step(self.shape, self.weights, EAGLE_HEAD_ONLY | self.act_flag(B) | self._sample_flag(sample),
                         rows, self.feat, None, out, self.workspace)

    def draft_phase(self, root_feat: torch.Tensor, root_token: torch.Tensor, sample=None):
        """Root head, then expand + draft step per depth, then rerank/flatten.
        sample = (seed, round): every expanded node's children are drawn
        without replacement from its draft distribution (EAGLE_SAMPLE_CHILDREN,
        row ids = the round's feature rows) instead of taken as its top-k."""
        B, k = self.B, self.k
        self.root_head(root_feat, sample)
        eagle_tree_init(B, self.pool, root_token, 0)
        prev_row0, n_prev = 0, 1
        for s in range(self.depth):
            last = s == self.depth - 1
            if last:
                # final expansion: create the deepest children; no further draft step
                st = self._scratch_step()
                n_next = 0
            else:
                st = self.steps[s]
                n_next = st.n_next
            eagle_tree_expand(B, k, s, self.nchild, self.pool, n_prev, self.topk, self.topk_idx[prev_row0:],
                              self.topk_logq[prev_row0:], n_next, st.feat_row0, self.prefix["len"], st.token,
                              st.parent, st.pos, st.slot, st.mask, st.row_start)
            if last:
                break
            n = B * st.n_next
            rows = make_rows(n, B, st.n_next, st.row_start, st.token, st.parent, st.pos, st.slot, st.mask)
            seed, rnd = sample if sample is not None else (0, 0)
            out = make_out(self.feat[st.feat_row0:], self.logits[st.feat_row0:], self.lse[st.feat_row0:], self.topk,
                           self.topk_idx[st.feat_row0:], self.topk_logq[st.feat_row0:], seed, rnd, st.feat_row0)
            eagle_draft_step(self.shape, self.weights, self.act_flag(n) | self._sample_flag(sample), rows, self.feat,
                             self.kv, out, self.workspace)
            prev_row0, n_prev = st.feat_row0, st.n_next
        t = self.tree
        eagle_tree_finalize(B, self.m, self.n_nodes, self.pool, self.prefix["len"], t["parent"], t["token"],
                            t["depth"], t["pool"], t["mask"], t["qrow"], self.tw["token"], self.tw["parent"],
                            self.tw["pos"], self.tw["slot"], self.tw["mask"], self.tw["row_start"])

    def _scratch_step(self):
        if not hasattr(self, "_scratch"):
            B, k = self.B, max(self.k, 1)
            i32 = dict(dtype=torch.int32, device=self.dev)
            self._scratch = Step(0, k, self.total_rows, torch.zeros(B * k, **i32), torch.zeros(B * k, **i32),
                                 torch.zeros(B * k, **i32), torch.zeros(B * k, **i32),
                                 torch.zeros(B * k, dtype=torch.int64, device=self.dev), torch.zeros(B + 1, **i32))
        return self._scratch

    def tree_wide(self):
        """One draft step over every drafted node of the flattened tree."""
        nw = self.B * (self.n_nodes - 1)
        rows = make_rows(nw, self.B, self.n_nodes - 1, self.tw["row_start"], self.tw["token"], self.tw["parent"],
                         self.tw["pos"], self.tw["slot"], self.tw["mask"])
        out = make_out(self.tw_feat, self.tw_logits, self.tw_lse, 1, self.tw_idx, self.tw_logq)
        eagle_draft_step(self.shape, self.weights, self.act_flag(nw), rows, self.feat, self.tw_kv, out,
                         self.workspace)

    def verify(self, target_logits: torch.Tensor, seed: int, round_: int, flags: int = 0):
        t = self.tree
        eagle_verify(self.B, self.n_nodes, self.shape_d["vocab"], t["parent"], t["token"], target_logits,
                     self.logits, t["qrow"], seed, round_, flags, self.v_path, self.v_len, self.v_next, self.v_flags,
                     workspace=self.workspace)

    def catch_up(self, true_feat: torch.Tensor):
        """After verify: the drafter's rows over each sequence's committed
        tokens (the root and the accepted drafted nodes, each joined with the
        token after it, the verifier's next token last), computed from the
        target's true features true_feat [B * n_nodes, d] fp32 (row b*N + node:
        the target's feature at every tree node of this round, root included),
        committed to the prefix KV cache (eagle_catchup_rows, one draft step
        with EAGLE_FEATURES_ONLY, eagle_commit_catchup).  The next round's root
        features land in the engine's root rows and its root tokens are this
        round's next tokens (next_round_inputs()).  Needs prefix capacity;
        per-sequence commit status in c_flags."""
        B, N, R = self.B, self.n_nodes, self.cu_R
        c, p = self.cu, self.prefix
        eagle_catchup_rows(B, N, R - 1, self.tree["token"], self.v_path, self.v_len, self.v_next, p["len"], 0,
                           c["token"], c["parent"], c["pos"], c["slot"], c["mask"], c["row_start"], c["last_row"],
                           c["count"])
        rows = make_rows(B * R, B, R, c["row_start"], c["token"], c["parent"], c["pos"], c["slot"], c["mask"])
        out = make_out(self.cu_feat, None, None, 1, None, None)
        eagle_draft_step(self.shape, self.weights, EAGLE_FEATURES_ONLY | self.act_flag(B * R), rows, true_feat,
                         self.kv, out, self.workspace)
        eagle_commit_catchup(self.shape, B, c["count"], self.tree_k, self.tree_v, p["k"], p["v"], p["off"], p["len"],
                             p.get("cap"), self.cu_feat, c["last_row"], self.feat[:B], self.c_flags)

    def next_round_inputs(self):
        """(root features, root tokens) of the round after catch_up(): the
        engine's own root rows and this round's next tokens; pass them to
        draft_phase (no copy is made)."""
        return self.feat[:self.B], self.v_next

    # ------------------------------------------------------------ HIP graph
    def capture_round(self, root_feat: torch.Tensor, root_token: torch.Tensor, target_logits: torch.Tensor,
                      seed: int, round_: int, flags: int = 0):
        """Record one whole round (draft phase + verify) as a HIP graph over
        this engine's buffers; replay_round() re-runs every kernel of it.  The
        inputs are read from the given tensors at replay time (write new root
        features, tokens or target logits into them in place); seed, round and
        flags are fixed at capture.  Nothing in a round allocates or clears
        memory with a memset, so the whole round is capturable."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # one eager round on the capture stream's side first
            self.draft_phase(root_feat, root_token)
            self.verify(target_logits, seed, round_, flags)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.draft_phase(root_feat, root_token)
            self.verify(target_logits, seed, round_, flags)
        self._graph = g
        return g

    def replay_round(self):
        self._graph.replay()
