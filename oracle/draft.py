"""One draft step of the EAGLE feature-level draft head, fp64 (test infrastructure only).

Follows the pages' description of the draft head:

* the advanced (shifted) token's embedding comes from the frozen target
  embedding and is concatenated after the parent feature, [f ; e(t)] in R^{2d}
  ("EAGLE 推测解码为什么比 Medusa 快" section 4.1; "eagle feature-level
  speculative decoding", section "Advanced Token" and the fusion-layer section,
  h = W z + b);
* an FC layer compresses 2d -> d, then one decoder layer predicts the next
  feature f^ (same sections; the decoder is LLaMA-style: pre-norm RMSNorm,
  rotary attention, SwiGLU MLP, residuals);
* attention sees the prefix plus only the node's tree ancestors and itself
  ("eagle feature-level speculative decoding", section "Tree Attention 如何一次
  验证多条路径", the mask M_uv and the visibility table);
* the frozen shared LM head maps f^ to vocabulary logits (study note section
  4.2; q = softmax(LM_Head(f^))).

The first draft distribution of a round comes straight from the true feature
(``head_only``): q = softmax(LM_Head(f_j)), which is the target's own p
(study note sections 6.1 and 7.1).

Precision reading for bf16 workloads: weights, embedding, LM head and the KV
cache are bf16 values; activations are carried at full precision.  So with
``mirror=True`` the only rounding is of the rotated k and of v when they are
stored into the bf16 tree slots (the cache format); everything else is fp64.

``act_bf16=True`` is the other bf16 contract a draft step can be run under
(bf16 matrix-unit operands on both sides): the activation operand of each of
the six weight products -- [f ; e], RMSNorm(x)*g1, the attention output,
RMSNorm(h)*g2, the SwiGLU activation and f^ entering the LM head -- is rounded
to the nearest bf16 value before the product; the products, norms, softmax and
residual stream stay fp64.
"""
from __future__ import annotations

import numpy as np

from .numerics import matmul_t, rmsnorm, rope_rotate_half, round_bf16, silu, softmax

N_SLOTS = 64


def _r(x, on):
    return round_bf16(x) if on else np.asarray(x, dtype=np.float64)


def new_tree_kv(shape, batch: int):
    """Tree K/V slots [B, 64, Hkv, hd], NaN until written so that reading an
    unwritten slot poisons the result."""
    k = np.full((batch, N_SLOTS, shape.n_kv_heads, shape.head_dim), np.nan)
    return k, k.copy()


def head_logits(shape, w, feats: np.ndarray, mirror: bool = True, act_bf16: bool = False) -> np.ndarray:
    """Root distribution logits from true features: LM_Head(f) (no final norm,
    no bias: f is exactly the LM head's input)."""
    return matmul_t(_r(feats, act_bf16 and shape.dtype == "bf16"), w.lm_head)


def tree_attention_row(q_heads, seq_prefix_k, seq_prefix_v, L, tree_k_seq, tree_v_seq, mask, n_heads,
                       n_kv_heads):
    """Attention of one query row.  q_heads [Hq, hd] (already rotated).  Keys:
    prefix positions 0..L-1 plus every tree slot whose bit is set in mask.
    Explicit loop over heads and over the visible key list."""
    hd = q_heads.shape[-1]
    group = n_heads // n_kv_heads
    slots = [s for s in range(N_SLOTS) if (int(mask) >> s) & 1]
    out = np.zeros((n_heads, hd))
    for h in range(n_heads):
        g = h // group
        # visible keys: prefix positions 0..L-1, then the visible tree slots
        keys = np.concatenate([seq_prefix_k[g, :L], tree_k_seq[slots, g]]).astype(np.float64).reshape(-1, hd)
        vals = np.concatenate([seq_prefix_v[g, :L], tree_v_seq[slots, g]]).astype(np.float64).reshape(-1, hd)
        scores = keys @ q_heads[h] / np.sqrt(hd)
        p = softmax(scores)
        out[h] = p @ vals
    return out


def draft_step(shape, w, rows: dict, feat_buf: np.ndarray, prefix_k, prefix_v, prefix_len,
               tree_k: np.ndarray, tree_v: np.ndarray, mirror: bool = True, want_logits: bool = True,
               act_bf16: bool = False):
    """One draft step over a set of tree rows.

    rows: dict of equal-length arrays
      seq    - sequence index b
      token  - the node's advanced token t (its own token)
      parent - row of feat_buf holding the parent feature (true f_j or a
               predicted f^)
      pos    - rotary position of the row (prefix length + depth - 1)
      slot   - tree slot that receives this row's k, v
      mask   - uint64 bitmask of visible tree slots (ancestors and self)
    prefix_k/v: per sequence [Hkv, L_b, hd] (K already rotated).
    tree_k/v:   [B, 64, Hkv, hd], updated in place with this step's k, v.

    Returns dict with f^ ('feat'), 'logits' and intermediates.
    """
    on = mirror and shape.dtype == "bf16"
    ra = act_bf16 and shape.dtype == "bf16"  # bf16 operand of each weight product
    d, hq, hkv, hd = shape.d, shape.n_heads, shape.n_kv_heads, shape.head_dim
    seq = np.asarray(rows["seq"])
    M = len(seq)
    tok = np.asarray(rows["token"])
    par = np.asarray(rows["parent"])
    pos = np.asarray(rows["pos"])
    slot = np.asarray(rows["slot"])
    mask = np.asarray(rows["mask"], dtype=np.uint64)

    # a1, a2: [f_parent ; e(t)] -> FC 2d->d with bias
    a = np.concatenate([np.asarray(feat_buf, np.float64)[par], np.asarray(w.embed, np.float64)[tok]], axis=1)
    x = matmul_t(_r(a, ra), w.fc_w) + np.asarray(w.fc_b, np.float64)

    # a3: RMSNorm -> q, k, v
    n1 = _r(rmsnorm(x, w.norm1, shape.rms_eps), ra)
    q = matmul_t(n1, w.wq).reshape(M, hq, hd)
    k = matmul_t(n1, w.wk).reshape(M, hkv, hd)
    v = matmul_t(n1, w.wv).reshape(M, hkv, hd)

    # a4: rotary embedding at the row's position; k, v into the row's tree slot
    for r in range(M):
        for h in range(hq):
            q[r, h] = rope_rotate_half(q[r, h], int(pos[r]), shape.rope_theta)
        for h in range(hkv):
            k[r, h] = rope_rotate_half(k[r, h], int(pos[r]), shape.rope_theta)
    k, v = _r(k, on), _r(v, on)  # the KV cache stores bf16
    for r in range(M):
        tree_k[seq[r], slot[r]] = k[r]
        tree_v[seq[r], slot[r]] = v[r]

    # a5: tree attention over prefix + visible tree slots
    attn = np.zeros((M, hq, hd))
    pkv = {}
    for r in range(M):
        b = int(seq[r])
        if b not in pkv:
            pkv[b] = (np.asarray(prefix_k[b], np.float64), np.asarray(prefix_v[b], np.float64))
        attn[r] = tree_attention_row(q[r], pkv[b][0], pkv[b][1], int(prefix_len[b]), tree_k[b], tree_v[b], mask[r],
                                     hq, hkv)
    attn = attn.reshape(M, hq * hd)

    # a6: O projection + residual
    h_res = x + matmul_t(_r(attn, ra), w.wo)

    # a7: RMSNorm -> SwiGLU MLP + residual
    n2 = _r(rmsnorm(h_res, w.norm2, shape.rms_eps), ra)
    act = silu(matmul_t(n2, w.w_gate)) * matmul_t(n2, w.w_up)
    feat = h_res + matmul_t(_r(act, ra), w.w_down)

    out = {"x": x, "q": q, "k": k, "v": v, "attn": attn, "h": h_res, "feat": feat}
    # a8: frozen shared LM head
    if want_logits:
        out["logits"] = matmul_t(_r(feat, ra), w.lm_head)
    return out


def fuse_features(shape, w_fuse, b_fuse, low, mid, high) -> np.ndarray:
    """EAGLE-3 input fusion ("EAGLE 完全拆解", EAGLE-3 part): the target's low-,
    mid- and high-layer features of a position, each d wide, concatenated to 3d
    and compressed back to d by an FC layer, g = FC([l; m; h]) = [l; m; h] W^T
    (+ b).  g then stands where the feature f stands in [f ; e(t)]."""
    cat = np.concatenate([np.asarray(low, np.float64), np.asarray(mid, np.float64), np.asarray(high, np.float64)],
                         axis=1)
    g = matmul_t(cat, w_fuse)
    if b_fuse is not None:
        g = g + np.asarray(b_fuse, np.float64)
    return g
