"""Plain, slow fp64 CPU oracle for the EAGLE draft-and-verify hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (``eagle_feature_level_amd``) and imports nothing from it.

What each module follows (page titles as they appear in the sources):

* ``numerics``  - bf16 rounding of GEMM operands, RMSNorm, RoPE, SiLU, softmax.
* ``draft``     - one draft step of the feature-level draft head: gather the
  frozen embedding of the advanced token, concatenate with the parent feature
  [f ; e(t)], FC 2d->d (+bias), one LLaMA-style decoder layer whose attention
  sees the prefix plus the node's tree ancestors only, and the frozen shared LM
  head ("EAGLE 推测解码为什么比 Medusa 快" section 4.1 and section 6.1;
  "eagle feature-level speculative decoding", sections "草稿头到底包含什么" and
  "Tree Attention 如何一次验证多条路径").
* ``topk``      - softmax log-normaliser and per-row top-k (ties -> lower index).
* ``tree``      - EAGLE-2 expand / rerank (study note section 10.3, value =
  product of confidences along the path) and static templates.
* ``philox``    - Philox4x64-10 counter-based generator (Salmon et al., SC'11).
* ``verify``    - tree-structured recursive rejection sampling (study note
  section 6.2; "eagle feature-level speculative decoding", section
  "随机采样验证"; "EAGLE 完全拆解", section on why plain draft models fall short),
  greedy verification, textbook one-token speculative sampling, and an exact
  enumerator of the verifier's output law for tiny vocabularies.
* ``shapes``    - trainable-parameter count of FC + one decoder layer.
"""
