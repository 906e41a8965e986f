"""Draft-head parameter count (test infrastructure only).

The trainable part of the EAGLE draft head is the FC fusion layer (2d -> d,
with bias) and one decoder layer; the embedding and LM head are the target's
own, frozen, and not counted ("EAGLE 推测解码为什么比 Medusa 快" section 4.1 and
the trainable-parameter table of section 4.3).
"""


def trainable_params(d: int, n_heads: int, n_kv_heads: int, head_dim: int, ffn: int) -> int:
    fc = 2 * d * d + d
    attn = d * n_heads * head_dim + 2 * d * n_kv_heads * head_dim + n_heads * head_dim * d
    mlp = 3 * d * ffn
    norms = 2 * d
    return fc + attn + mlp + norms
