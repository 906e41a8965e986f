/*
 * eagle.h - C ABI of the MI355X (gfx950) EAGLE draft-and-verify hot path.
 *
 * One round of EAGLE feature-level speculative decoding, as the pages describe
 * it, is: a draft head (frozen target embedding, FC 2d->d over [f ; e(t)], one
 * decoder layer, frozen shared LM head) grows a token tree from the last true
 * target feature; EAGLE-2 chooses which nodes to expand and which to keep by
 * the product of draft confidences along each path; the target's distributions
 * over the tree are then checked by recursive rejection sampling, which keeps
 * the output distribution equal to the target's.
 *   - "EAGLE 推测解码为什么比 Medusa 快" (zzszmyf.github.io), sections 4.1, 6.1,
 *     6.2, 7.1 and 10.3;
 *   - "eagle feature-level speculative decoding" (charlestar.github.io),
 *     sections on the draft head, tree attention, greedy and sampling
 *     verification;
 *   - "EAGLE 完全拆解" (pinghaoyang.com.cn), sections on the draft head and on
 *     EAGLE-2.
 *
 * Conventions (all entry points):
 *   - Every pointer argument is DEVICE memory owned by the caller, unless the
 *     argument is a pointer to one of the small structs below, which are host
 *     structs passed by pointer and read during the call only.  The library
 *     never allocates or frees device memory in a call; scratch space comes in
 *     through `workspace` (size from eagle_workspace_bytes).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Nothing synchronises with the host.  Calls on different streams
 *     must not share a workspace.
 *   - Return value: EAGLE_OK (0) or a negative EAGLE_E* code.  Argument errors
 *     are detected on the host before any launch, so a failing call launches
 *     nothing.  eagle_last_hip_error() gives the hipError_t behind EAGLE_EHIP.
 *   - Matrices are row-major.  Weights are [out, in]: y = x W^T.
 *   - Outputs are a pure function of the inputs (and of seed/round for
 *     eagle_verify): reduction orders are fixed, no atomics decide values.
 */
#ifndef EAGLE_H
#define EAGLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *eagle_stream_t; /* hipStream_t */

enum {
  EAGLE_OK = 0,
  EAGLE_EINVAL = -1,       /* null pointer, bad size, inconsistent shape   */
  EAGLE_EUNSUPPORTED = -2, /* dtype, top-k > 16, > 64 tree nodes, not gfx950 */
  EAGLE_EWORKSPACE = -3,   /* workspace smaller than eagle_workspace_bytes */
  EAGLE_EHIP = -4          /* a HIP launch or query failed                 */
};

enum { EAGLE_F32 = 0, EAGLE_BF16 = 1 };

/* Largest tree per sequence: node masks are 64-bit. */
#define EAGLE_MAX_SLOTS 64
/* Largest per-row top-k. */
#define EAGLE_MAX_TOPK 16

/* Draft-head shape.  d = hidden size (the feature width), n_heads query
 * heads and n_kv_heads key/value heads of head_dim each (n_heads a multiple
 * of n_kv_heads), ffn = SwiGLU width, vocab = shared vocabulary size.
 * dtype EAGLE_BF16: weights, embedding, LM head and K/V are bf16, GEMMs run on
 * bf16 matrix cores with fp32 accumulation (activations as split bf16 pairs);
 * EAGLE_F32: everything fp32. */
typedef struct {
  int32_t d, n_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps;    /* RMSNorm epsilon, e.g. 1e-5                    */
  float rope_theta; /* rotary base, e.g. 1e4                         */
  int32_t dtype;    /* EAGLE_BF16 or EAGLE_F32                       */
} eagle_shape;

/* Draft-head weights (element type = shape.dtype), device pointers.
 * embed/lm_head are the target's frozen embedding and LM head [vocab, d];
 * fc_w [d, 2d] and fc_b [d] fuse [f ; e(t)]; the decoder layer is pre-norm
 * (norm1/norm2 gains [d]), wq [Hq*hd, d], wk/wv [Hkv*hd, d], wo [d, Hq*hd],
 * w_gate/w_up [ffn, d], w_down [d, ffn]. */
typedef struct {
  const void *embed, *fc_w, *fc_b, *norm1, *norm2, *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down, *lm_head;
  /* Optional, bf16 workloads (NULL: not given): copies of the nine weight
   * matrices above in the blocked layout written by eagle_block_weight.
   * Where all of a product's matrices have one (wq, wk and wv together;
   * w_gate and w_up together), the draft step's GEMMs read the copies, whose
   * every 4 KB block is one 128-column step of 16 rows, instead of the
   * row-major matrices, which remain required; results are identical. */
  const void *fc_w_b, *wq_b, *wk_b, *wv_b, *wo_b, *w_gate_b, *w_up_b, *w_down_b, *lm_head_b;
} eagle_weights;

/* Rows of one draft step (device arrays of n_rows entries unless stated).
 * A row is one expanded tree node: its input is the parent's feature and the
 * node's own (advanced) token.  Rows of one sequence are contiguous:
 * sequence b owns rows [row_start[b], row_start[b+1]). */
typedef struct {
  int32_t n_rows;           /* host: number of rows                            */
  int32_t batch;            /* host: number of sequences                       */
  int32_t max_rows_per_seq; /* host: max over b of row_start[b+1]-row_start[b] */
  const int32_t *row_start; /* [batch+1]                                       */
  const int32_t *token;     /* advanced token of the row, 0 <= t < vocab       */
  const int32_t *parent;    /* row of feat_in holding the parent feature       */
  const int32_t *pos;       /* rotary position (prefix_len + depth - 1)        */
  const int32_t *slot;      /* tree slot (0..63) receiving this row's k, v     */
  const uint64_t *mask;     /* tree slots visible to the row: ancestors + self */
} eagle_rows;

/* Draft-layer KV.  Prefix K (already rotated) and V are stored per sequence
 * as [Hkv][C_b][hd] starting at element prefix_off[b], positions 0..L_b-1 of
 * each kv head used; C_b = prefix_cap[b] (room for eagle_commit to append), or
 * C_b = L_b when prefix_cap is NULL (packed).  Tree slots hold the k, v of
 * drafted nodes: [batch][64][Hkv][hd].  Element type = shape.dtype. */
typedef struct {
  const void *prefix_k, *prefix_v;
  const int64_t *prefix_off; /* [batch] element offsets                        */
  const int32_t *prefix_len; /* [batch] L_b >= 0                               */
  int32_t max_prefix_len;    /* host: max over b of L_b (an upper bound is fine) */
  void *tree_k, *tree_v;     /* written: the rows' slots                        */
  const int32_t *prefix_cap; /* [batch] C_b >= L_b, or NULL (C_b = L_b)         */
  int64_t prefix_len_sum;    /* host: sum over b of L_b if known, else 0; used
                                only by the measurement hook's byte count
                                (0: max_prefix_len per sequence)                */
} eagle_kv;

/* Outputs of a draft step. */
typedef struct {
  float *feat;       /* [n_rows, d] predicted feature f^ (unused with HEAD_ONLY) */
  float *logits;     /* [n_rows, vocab] LM-head logits                          */
  float *lse;        /* [n_rows] log-sum-exp of each logits row                 */
  int32_t topk;      /* 1..16                                                   */
  int32_t *topk_idx; /* [n_rows, topk] ranked tokens, ties -> lower index        */
  float *topk_logq;  /* [n_rows, topk] logit - lse of those tokens               */
  /* EAGLE_SAMPLE_CHILDREN only: Philox key (seed, round) and the id of the
   * call's first row (row r draws with counter row_base + r; give every row
   * of a round a distinct id). */
  uint64_t seed, round;
  int32_t row_base;
} eagle_draft_out;

/* Flags of eagle_draft_step.
 * EAGLE_HEAD_ONLY: the root distribution only (see below).
 * EAGLE_ACT_BF16 (bf16 workloads only, else EAGLE_EINVAL): the activation
 *   operand of each of the six weight GEMMs (FC, QKV, O, gate/up, down, LM
 *   head) is rounded once to bf16, round to nearest even, and enters the
 *   matrix units as one bf16 value: one MFMA per product instead of two.  The
 *   rounded values are [f ; e], RMSNorm(x) * norm1, the attention output,
 *   RMSNorm(h) * norm2 (rounded after the row scale), the SwiGLU activation
 *   and f^ (for the LM head).  Everything else is unchanged (fp32 activations,
 *   fp32 accumulation, attention on split operands).  For steps over many rows
 *   (the matrix units are the bound above a few hundred rows) this halves the
 *   matrix work.  It is outside the 2e-2 logit tolerance at the 7B-70B draft
 *   head shapes: measured against an fp64 evaluation that rounds the same
 *   operands, the logits differ by up to ~0.03 (7B), ~0.05 (13B) and ~0.18
 *   (70B), because fp32-vs-fp64 differences upstream flip later roundings;
 *   without the flag (split operands) every workload stays within 2e-4. */
/* EAGLE_SAMPLE_CHILDREN: topk_idx holds `topk` tokens drawn without
 *   replacement from each row's softmax, in draw order (Gumbel-top-k, as in
 *   eagle_sample_topk below) instead of the `topk` most probable ones; lse and
 *   topk_logq are unchanged in meaning.  Children proposed this way are the
 *   without-replacement draw that eagle_verify's default rule is exact for
 *   ("eagle feature-level speculative decoding", sampled verification: the
 *   siblings' sampling scheme must match the verifier's). */
/* EAGLE_FEATURES_ONLY: the step stops after f^ (and the rows' k, v in their
 *   tree slots): no LM head, no softmax or top-k; out->logits, lse, topk_idx
 *   and topk_logq may be NULL.  The catch-up step between rounds uses it (see
 *   eagle_catchup_rows).  Not combinable with EAGLE_HEAD_ONLY. */
enum { EAGLE_HEAD_ONLY = 1, EAGLE_ACT_BF16 = 2, EAGLE_SAMPLE_CHILDREN = 4, EAGLE_FEATURES_ONLY = 8 };

/* Blocked copy of a bf16 weight matrix W [rows, cols] (row-major, cols a
 * multiple of 128): 16-row by 128-column blocks of 4 KB, the blocks of each
 * 16-row band in column order, inside a block the four 32-column quarters in
 * turn, each 16 rows of 32 values:
 *   out[(t * cols/128 + s) * 2048 + ((c / 32) * 16 + r) * 32 + c % 32]
 *     = W[16 t + r][128 s + c]
 * (rows past the end are 0), so that a GEMM streaming 16-row bands reads each
 * band as one contiguous run, its lanes' reads adjacent.  The layout only serves the kernels' memory
 * access; the pages' method is unchanged.  eagle_blocked_weight_bytes gives
 * the size of out (0 for an invalid shape); w and out are 16-byte aligned
 * device buffers, written on `stream`. */
size_t eagle_blocked_weight_bytes(int32_t rows, int32_t cols);
int eagle_block_weight(const void *w, int32_t rows, int32_t cols, void *out, eagle_stream_t stream);

/* Bytes of workspace needed by eagle_draft_step / eagle_softmax_topk for up
 * to max_rows rows, max_batch sequences and prefixes up to max_prefix_len.
 * Returns 0 for an invalid shape. */
size_t eagle_workspace_bytes(const eagle_shape *shape, int32_t max_rows, int32_t max_batch, int32_t max_prefix_len);

/* One draft step over a set of tree rows ("EAGLE 推测解码为什么比 Medusa 快",
 * sections 4.1-4.2 (draft head: frozen embedding of the advanced token, FC over
 * [f ; e], one decoder layer, frozen shared LM head) and 6.1 (the draft loop:
 * the first distribution from the true feature, later ones from predicted
 * features); "eagle feature-level speculative decoding", sections on the draft
 * head and on tree attention (each node sees the prefix, its ancestors and
 * itself)).
 *
 * Without flags, per row r (sequence b):
 *   a   = [f ; e] with f = feat_in[parent[r]] and e = embed[token[r]]      (2d)
 *   x   = a fc_w^T + fc_b
 *   q,k,v = RMSNorm(x) * norm1 times wq, wk, wv; q and k rotated (RoPE,
 *         rotate-half pairing i <-> i+hd/2, frequency theta^(-2i/hd)) at
 *         pos[r]; k, v written to tree slot slot[r] of sequence b
 *   att = per query head h (kv head h / (Hq/Hkv)): softmax over the prefix
 *         keys 0..L_b-1 and the tree slots set in mask[r], scale 1/sqrt(hd)
 *   h   = x + att wo^T
 *   f^  = h + (silu(n2 w_gate^T) * (n2 w_up^T)) w_down^T, n2 = RMSNorm(h)*norm2
 *   logits = f^ lm_head^T; lse; top-k of the row.
 * With EAGLE_HEAD_ONLY: logits = feat_in[parent[r]] lm_head^T (the root
 * distribution from the true feature; the decoder is skipped and kv, feat may
 * be NULL).
 *
 * Precision (bf16 workloads): weights, embedding, LM head and the KV cache are
 * bf16; activations (features, residuals, q, attention output, SwiGLU
 * activation) are fp32 and enter the matrix units as a pair of bf16 values
 * (hi, lo = x - hi) with fp32 accumulation, so the only activation rounding to
 * bf16 is the store of k and v into the tree slots; with EAGLE_ACT_BF16 the
 * GEMM activation operands are rounded to bf16 as described above.  feat_in is
 * fp32 [*, d].
 * Rows that attend to each other's slots may share one call: every row's
 * k, v is written before any row's attention runs. */
int eagle_draft_step(const eagle_shape *shape, const eagle_weights *w, int32_t flags, const eagle_rows *rows,
                     const float *feat_in, const eagle_kv *kv, const eagle_draft_out *out, void *workspace,
                     size_t workspace_bytes, eagle_stream_t stream);

/* Softmax normaliser and top-k of n_rows fp32 rows of `vocab` logits:
 * lse[r] = log sum exp(logits[r]); topk_idx[r] = the `topk` largest entries
 * by (value desc, index asc), -0.0 equal to +0.0; topk_logq = value - lse.
 * Uses the workspace sized by eagle_workspace_bytes. */
int eagle_softmax_topk(int32_t n_rows, int32_t vocab, const float *logits, int32_t topk, float *lse,
                       int32_t *topk_idx, float *topk_logq, void *workspace, size_t workspace_bytes,
                       eagle_stream_t stream);

/* Sampled proposals: like eagle_softmax_topk, but the ranking key of token v
 * in row r is logit + g with g = -log(-log(u)), u from word v % 4 of
 * Philox4x64-10 (Salmon et al., SC'11) counter (row_base + r, v / 4, 0, 1) under
 * key (seed, round), u = ((w >> 41) + 0.5) * 2^-23 (fp32 throughout).  The
 * `topk` tokens are then `topk` draws without replacement from softmax(row),
 * in draw order (Gumbel-top-k); lse and topk_logq (= logit - lse) are those of
 * the plain logits.  vocab <= 524288 (else EAGLE_EUNSUPPORTED).  Uses the
 * workspace sized by eagle_workspace_bytes. */
int eagle_sample_topk(int32_t n_rows, int32_t vocab, const float *logits, int32_t topk, uint64_t seed, uint64_t round,
                      int32_t row_base, float *lse, int32_t *topk_idx, float *topk_logq, void *workspace,
                      size_t workspace_bytes, eagle_stream_t stream);

/* EAGLE-3 three-feature fusion: g = [l ; m ; h] w_fuse^T (+ b_fuse), the
 * target's low-, mid- and high-layer features of one position concatenated
 * (3d) and compressed back to d by an FC layer ("EAGLE 完全拆解", EAGLE-3
 * part: g = FC([l; m; h]), then [g ; e(t)] enters the draft layer as the
 * feature does in EAGLE-1/2).  w_fuse [d, 3d] and b_fuse [d] (NULL: no bias)
 * in shape.dtype; low, mid, high, g fp32 [n_rows, d] device arrays.  The GEMM
 * runs like the draft step's (split-bf16 operands for bf16 weights).
 * Workspace: eagle_fuse_workspace_bytes(shape, max_rows). */
size_t eagle_fuse_workspace_bytes(const eagle_shape *shape, int32_t max_rows);
int eagle_fuse_features(const eagle_shape *shape, const void *w_fuse, const void *b_fuse, int32_t n_rows,
                        const float *low, const float *mid, const float *high, float *g, void *workspace,
                        size_t workspace_bytes, eagle_stream_t stream);

/* Candidate pool of the tree builder: per sequence b, entries
 * [b*cap, (b+1)*cap) of each array; node 0 is the root. */
typedef struct {
  int32_t cap;          /* host: pool entries per sequence            */
  int32_t *parent;      /* pool id of the parent (-1 for the root)    */
  int32_t *token;       /* node token                                 */
  int32_t *depth;       /* 0 for the root                             */
  float *logv;          /* log value: fp32 sum of logq along the path */
  int32_t *feat_row;    /* row of the node's feature once expanded    */
  int32_t *slot;        /* tree slot of its decoder row               */
  uint64_t *mask;       /* visible slots of its decoder row           */
  int32_t *count;       /* [batch] pool size                          */
  int32_t *frontier;    /* [batch*EAGLE_MAX_SLOTS] current frontier   */
} eagle_pool;

/* Reset each sequence's pool to its root: token root_token[b], feature row
 * root_feat_row0 + b, log value 0, frontier = {root}. */
int eagle_tree_init(int32_t batch, const eagle_pool *pool, const int32_t *root_token, int32_t root_feat_row0,
                    eagle_stream_t stream);

/* One expansion step ("EAGLE 推测解码为什么比 Medusa 快" section 10.3 and
 * exercise 5: a node's value is the product of the draft confidences on its
 * path, and the k most valuable nodes of the newest layer are expanded; the
 * static templates are the fixed tree shapes of EAGLE-1).
 * The previous draft step ran n_prev rows per sequence
 * (row b*n_prev + f = frontier position f of sequence b) and produced
 * topk_idx/topk_logq [batch*n_prev, topk].
 *   EAGLE-2 (static_nchild == NULL): every frontier node gets its top `k`
 *     tokens as children, logv(child) = fl32(logv(parent) + logq); the next
 *     frontier is the k children of largest logv (ties -> earlier creation;
 *     creation order = (frontier position, rank)).  n_next must equal k, or
 *     0 for the last expansion (children created, no next frontier or rows).
 *   Static template (static_nchild = child count per template node, indexed
 *     by pool id, which equals the template's BFS index): node u gets its
 *     top static_nchild[u] tokens; the next frontier is every new child with
 *     children of its own, in creation order.  n_next = their number.
 * The next draft step's rows are written to next_rows (batch*n_next rows,
 * row_start[b] = b*n_next): token, parent = the parent's feature row,
 * pos = prefix_len[b] + depth - 1, slot = (EAGLE-2) step*k + f or (static)
 * the pool id, mask = parent's mask | (1 << slot).  The frontier node at
 * position f gets feature row feat_row0 + b*n_next + f.
 * Limits: k <= topk <= 16, n_prev * k <= 256, slots < 64.  static_nchild must
 * hold pool->cap entries.  A sequence whose expansion cannot be carried out
 * has its pool->count set to -1 and nothing added (its finalize then yields
 * the root only): the pool would exceed pool->cap, a new child's log value is
 * NaN (a NaN logit row makes its lse and every log q NaN), or (templates) a
 * node asks for more children than topk, or the children with children of
 * their own are not exactly n_next. */
int eagle_tree_expand(int32_t batch, int32_t k, int32_t step, const int32_t *static_nchild, const eagle_pool *pool,
                      int32_t n_prev, int32_t topk, const int32_t *topk_idx, const float *topk_logq, int32_t n_next,
                      int32_t feat_row0, const int32_t *prefix_len, int32_t *next_token, int32_t *next_parent,
                      int32_t *next_pos, int32_t *next_slot, uint64_t *next_mask, int32_t *next_row_start,
                      eagle_stream_t stream);

/* Rerank and flatten ("EAGLE 推测解码为什么比 Medusa 快" section 10.3: keep the
 * m most valuable nodes of the whole tree, ties to the shallower node, which
 * is a connected tree; "eagle feature-level speculative decoding", tree
 * attention section: a node's mask holds its ancestors and itself).
 * Keeps the m pool nodes (root excluded) of largest logv,
 * ties -> shallower, then earlier creation (m = 0: keep all), which is a
 * connected tree; orders the root first and the rest by (depth, creation), so
 * siblings stay in rank order.  Writes n_nodes = m+1 (or the pool size) nodes
 * per sequence at [b*n_nodes, ...): tree_parent (tree index, -1 root),
 * tree_token, tree_depth, tree_pool, tree_mask (bit t for node t and each
 * non-root ancestor), tree_qrow (feature/logit row where the node was
 * expanded, -1 if never).  Also writes the rows of a "tree-wide" draft step
 * over the n_nodes-1 drafted nodes (row b*(n_nodes-1) + t-1 for node t):
 * token, parent feature row, pos = prefix_len[b] + depth - 1, slot = t,
 * mask = tree_mask. n_nodes <= 64, and every kept node must fit: n_nodes >=
 * m + 1 (m > 0) or >= pool->cap (m = 0), else EAGLE_EINVAL.  When a sequence
 * keeps fewer nodes than n_nodes - 1 (a pool smaller than m + 1, or an invalid
 * pool: the root alone), entries past its last node are padding: tree_parent
 * -2, token 0, depth 0, tree_pool -1, qrow -1, mask = own bit; its tree-wide
 * rows there are token 0 at the root's feature row and position L_b. */
int eagle_tree_finalize(int32_t batch, int32_t m, int32_t n_nodes, const eagle_pool *pool, const int32_t *prefix_len,
                        int32_t *tree_parent, int32_t *tree_token, int32_t *tree_depth, int32_t *tree_pool,
                        uint64_t *tree_mask, int32_t *tree_qrow, int32_t *row_token, int32_t *row_parent,
                        int32_t *row_pos, int32_t *row_slot, uint64_t *row_mask, int32_t *row_start,
                        eagle_stream_t stream);

/* Flags of eagle_verify. */
enum { EAGLE_VERIFY_GREEDY = 1, EAGLE_VERIFY_IID = 2 };
/* Per-sequence status bits written to out_flags: ZRES a residual had mass 0
 * (current p kept), QZERO a candidate had q(x) = 0, QEMPTY q ran out of mass
 * (remaining siblings skipped), NAN a NaN logit, BADTREE a node with children
 * but no draft row (draft_row < 0: the correction is drawn from its p). */
enum { EAGLE_F_ZRES = 1, EAGLE_F_QZERO = 2, EAGLE_F_QEMPTY = 4, EAGLE_F_NAN = 8, EAGLE_F_BADTREE = 16 };

/* Tree-structured recursive rejection sampling, one walk per sequence
 * ("EAGLE 推测解码为什么比 Medusa 快" section 6.2: accept with probability
 * min(1, p/q), else resample from norm(max(0, p - q)), node by node along the
 * tree; "eagle feature-level speculative decoding", sections "Greedy 验证" and
 * "随机采样验证"; "EAGLE 完全拆解", EAGLE-2 part: siblings tried as successive
 * rounds).
 * Tree: n_nodes nodes per sequence (node 0 = root, tree_parent < own index,
 * siblings in rank order).  target_logits [batch*n_nodes, vocab]: row
 * b*n_nodes+i is the target's logits after node i.  q at node i is
 * softmax(draft_logits[draft_row[b*n_nodes+i]]) (only read for nodes with
 * children).  At node u with children c_1..c_m: p = softmax(target row u)
 * (greedy: onehot of its argmax, ties -> lower index).  Child c_i is
 * accepted iff u_i < p(x)/q(x) (x = its token; q(x) = 0: iff p(x) > 0),
 * u_i = Philox4x64-10 uniform of counter (b, u, i, 0) and key (seed, round),
 * (w0 >> 40) * 2^-24.  On rejection p <- norm(max(0, p - q)) (kept if that
 * mass is 0) and, unless EAGLE_VERIFY_IID, q <- norm(q without x).  If all
 * children are rejected the correction is drawn from p by inverse CDF in
 * token order with uniform event 64; at an accepted leaf the bonus is drawn
 * from that leaf's p the same way.
 * Outputs: out_path[b*n_nodes + j] = j-th accepted node (-1 padded),
 * out_accept_len[b] = accepted nodes + 1, out_next_token[b], out_flags[b].
 * workspace: device memory of at least eagle_verify_workspace_bytes(batch,
 * n_nodes) bytes, owned by the caller and overwritten, or NULL.  What happens
 * at a node depends only on the node (its rows, its children, its uniforms),
 * so with a workspace every node of every tree is processed at once, one
 * workgroup each, and a second launch walks the trees through the per-node
 * results; without it, one workgroup per sequence processes the nodes on its
 * path.  Both run the same per-node arithmetic, so the outputs are identical.
 * A non-NULL workspace below the size returns EAGLE_EWORKSPACE.
 * vocab <= 32768, n_nodes <= 64. */
int eagle_verify(int32_t batch, int32_t n_nodes, int32_t vocab, const int32_t *tree_parent, const int32_t *tree_token,
                 const float *target_logits, const float *draft_logits, const int32_t *draft_row, uint64_t seed,
                 uint64_t round, int32_t flags, int32_t *out_path, int32_t *out_accept_len, int32_t *out_next_token,
                 int32_t *out_flags, void *workspace, size_t workspace_bytes, eagle_stream_t stream);

/* Accepted-path commit of the draft layer's KV cache ("eagle feature-level
 * speculative decoding", KV commit as a transaction: only the accepted path
 * enters the cache, rejected branches are dropped).  For each sequence b with
 * A = accept_len[b] - 1 accepted drafted nodes (out_path / out_accept_len of
 * eagle_verify): node path[b*n_nodes + j], j < A, has its k, v in tree slot
 * node_slot[b*n_nodes + node] (node_slot NULL: slot = node, the tree-wide
 * step's layout) of tree_k/tree_v [batch][64][Hkv][hd]; it is copied to
 * prefix position prefix_len[b] + j of every kv head (layout of eagle_kv with
 * capacity prefix_cap[b]; NULL = no room), then prefix_len[b] += A.
 * out_flags[b] (written): 0, EAGLE_COMMIT_OVERFLOW (L_b + A > capacity: nothing
 * copied, length unchanged) or EAGLE_COMMIT_BAD_PATH (a node or slot index out
 * of range: nothing done).  Element type = shape->dtype.  Device arrays,
 * caller-owned; asynchronous on `stream`.  A later draft step must be given a
 * max_prefix_len that covers the grown lengths (e.g. the capacities).
 * The slots hold whatever k, v the caller's draft step wrote there.  The
 * drafter must continue from rows built on the target's TRUE features (the
 * KV-commit section: after A-B-D was drafted and A-B-X committed, no state
 * predicted along D, nor the draft's own predicted features of A-B, carries
 * over; study note section 6.2: the accepted path's true features start the
 * next round).  The tree-wide step's slots satisfy that for depth-1 nodes
 * only (their parent is the true root feature); eagle_catchup_rows +
 * eagle_commit_catchup below build and commit the right rows. */
enum { EAGLE_COMMIT_OVERFLOW = 1, EAGLE_COMMIT_BAD_PATH = 2 };
int eagle_commit(const eagle_shape *shape, int32_t batch, int32_t n_nodes, const int32_t *path,
                 const int32_t *accept_len, const int32_t *node_slot, const void *tree_k, const void *tree_v,
                 void *prefix_k, void *prefix_v, const int64_t *prefix_off, int32_t *prefix_len,
                 const int32_t *prefix_cap, int32_t *out_flags, eagle_stream_t stream);

/* Catch-up rows of the drafter between rounds ("eagle feature-level
 * speculative decoding", KV commit section: the drafter continues from the
 * committed path A-B-X; "EAGLE 推测解码为什么比 Medusa 快" section 6.2 and
 * implementation note 3: the true features of the accepted path, which the
 * target's verification forward computed, start the next round).
 * Input: a verified tree (tree_token [batch, n_nodes], node 0 = the root at
 * sequence position L_b = prefix_len[b]) and eagle_verify's out_path,
 * out_accept_len and out_next_token.  With A = accept_len[b] - 1 accepted
 * drafted nodes x_1..x_A and the next token X, the drafter's row at sequence
 * position L_b + i (i = 0..A) joins the true feature there with the embedding
 * of the token after it:
 *   row i = [f_true(node at path position i) ; e(x_{i+1})], x_{A+1} = X,
 * rotary position L_b + i, tree slot i, visible slots 0..i (a chain).  The
 * true feature of tree node n is feature row feat_row0 + b*n_nodes + n (the
 * caller's buffer of the target's features at every tree node; the root is
 * node 0).  Writes R = max_depth + 1 rows per sequence (rows [b*R, (b+1)*R),
 * row_start[b] = b*R): rows past A repeat row A in their own slot (same
 * token, parent and position, visible slots 0..A-1 and its own), so the call
 * has a fixed shape.  last_row[b] = b*R + A (the row of X: its f^ is the next
 * round's root feature), count[b] = A + 1 (slots to commit), or -1 for a
 * malformed verification result (accept_len outside 1..min(max_depth,
 * n_nodes-1)+1 or a path node outside 1..n_nodes-1: its rows are those of
 * A = 0 and nothing is committed).  Run eagle_draft_step with
 * EAGLE_FEATURES_ONLY over these rows (feat_in = the true features), then
 * eagle_commit_catchup.  n_nodes <= 64, max_depth + 1 <= 64, max_depth >= the
 * deepest accepted path.  Device arrays, caller-owned; asynchronous. */
int eagle_catchup_rows(int32_t batch, int32_t n_nodes, int32_t max_depth, const int32_t *tree_token,
                       const int32_t *path, const int32_t *accept_len, const int32_t *next_token,
                       const int32_t *prefix_len, int32_t feat_row0, int32_t *row_token, int32_t *row_parent,
                       int32_t *row_pos, int32_t *row_slot, uint64_t *row_mask, int32_t *row_start, int32_t *last_row,
                       int32_t *count, eagle_stream_t stream);

/* The catch-up commit: tree slots 0..count[b]-1 of sequence b (the catch-up
 * step's k, v in tree_k/tree_v [batch][64][Hkv][hd]) are appended to its
 * prefix at positions L_b.. of every kv head and prefix_len[b] grows by
 * count[b]; out_flags[b] = 0, EAGLE_COMMIT_OVERFLOW (no room: nothing copied,
 * length unchanged) or EAGLE_COMMIT_BAD_PATH (count outside 0..64: nothing
 * done).  If feat is not NULL, root_feat[b] = feat[last_row[b]] (d fp32
 * values: the catch-up step's f^ of X, the next round's root feature); feat,
 * last_row and root_feat are all given or all NULL.  Element type of the
 * caches = shape->dtype.  Device arrays, caller-owned; asynchronous. */
int eagle_commit_catchup(const eagle_shape *shape, int32_t batch, const int32_t *count, const void *tree_k,
                         const void *tree_v, void *prefix_k, void *prefix_v, const int64_t *prefix_off,
                         int32_t *prefix_len, const int32_t *prefix_cap, const float *feat, const int32_t *last_row,
                         float *root_feat, int32_t *out_flags, eagle_stream_t stream);

/* eagle_verify for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, results and per-node kernels as eagle_verify with a
 * workspace, but the per-node results live in the library's own file-scope
 * device array (one per GPU, 8192 * 12 + 1024 bytes, held until the process
 * ends), so the call allocates nothing and takes no workspace.  batch *
 * n_nodes <= EAGLE_VERIFY_NOALLOC_MAX_NODES, else EAGLE_EUNSUPPORTED.  Calls
 * that overlap on one GPU (different streams or host threads) share the array
 * and race; calls ordered on one stream do not. */
#define EAGLE_VERIFY_NOALLOC_MAX_NODES 8192
int eagle_verify_noalloc(int32_t batch, int32_t n_nodes, int32_t vocab, const int32_t *tree_parent,
                         const int32_t *tree_token, const float *target_logits, const float *draft_logits,
                         const int32_t *draft_row, uint64_t seed, uint64_t round, int32_t flags, int32_t *out_path,
                         int32_t *out_accept_len, int32_t *out_next_token, int32_t *out_flags, eagle_stream_t stream);

/* Bytes of workspace eagle_verify uses for batch x n_nodes trees (12 per node
 * plus alignment); 0 for an invalid size. */
size_t eagle_verify_workspace_bytes(int32_t batch, int32_t n_nodes);

/* Measurement hook.  While enabled, each kernel launch of eagle_draft_step is
 * timed by a pair of HIP events: a bf16 GEMM over at most 16 rows (one kernel)
 * records its own execution start and stop (hipExtLaunchKernel events, no
 * dispatch gap); every other launch is bracketed by events recorded on the
 * call's stream.  Each pair is tagged
 * with its role and with the algorithmic bytes it must move (weights once,
 * activations in and out) and flops.  The events are created by
 * eagle_profile_enable (not during a call); recording stops silently once
 * max_launches pairs are used.  eagle_profile_read synchronises on the
 * recorded events and returns, for one role, the number of launches, their
 * summed duration in ms, bytes and flops; eagle_profile_reset rewinds the
 * recording without destroying the events.  Not thread-safe: one measuring
 * thread per process. */
enum {
  EAGLE_ROLE_FC = 0, EAGLE_ROLE_QKV, EAGLE_ROLE_ROPE, EAGLE_ROLE_ATTN, EAGLE_ROLE_O, EAGLE_ROLE_GATE_UP,
  EAGLE_ROLE_DOWN, EAGLE_ROLE_LM_HEAD, EAGLE_ROLE_TOPK, EAGLE_ROLE_ROWS, EAGLE_ROLE_COUNT
};  /* EAGLE_ROLE_ROWS: per-row set-up (sequence index, [f ; e] concatenation).
     * With bf16 weights and at most 8 rows, RoPE and the tree-slot write run in
     * the QKV launch's epilogue: that call records no EAGLE_ROLE_ROPE launch, and
     * its QKV bytes count rotated q out (fp32) and k, v out (cache type). */
int eagle_profile_enable(int32_t max_launches);
int eagle_profile_reset(void);
int eagle_profile_disable(void);
int eagle_profile_read(int32_t role, int32_t *launches, double *total_ms, double *bytes, double *flops);

/* Message for an EAGLE_E* code. */
const char *eagle_strerror(int code);
/* hipError_t of the last EAGLE_EHIP on this thread. */
int eagle_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE_H */
