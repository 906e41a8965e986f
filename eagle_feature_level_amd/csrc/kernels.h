// Internal launch interface between the C ABI (capi.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

struct RopeArgs {
  const float* qkv;  // [n_rows, (hq + 2 hkv) hd] fp32
  const int32_t* pos;
  const int32_t* slot;
  const int32_t* row_start;  // [batch + 1]: rows of sequence b are [row_start[b], row_start[b+1])
  int batch;
  float* q_out;  // [n_rows, hq hd] rotated q
  void* tree_k;
  void* tree_v;
  int n_rows, hq, hkv, hd;
  float theta;
};

struct AttnArgs {
  const float* q;  // rotated q [n_rows, hq hd]
  const uint64_t* mask;
  const int32_t* row_start;
  const void* prefix_k;
  const void* prefix_v;
  const int64_t* prefix_off;
  const int32_t* prefix_len;
  const int32_t* prefix_cap;  // per-head stride in positions, or nullptr: L_b
  const void* tree_k;
  const void* tree_v;
  float* part;  // [n_splits, n_rows, hq, hd + 2]
  float* out;   // [n_rows, hq hd]
  // or, when set (bf16 K/V), the output as the split bf16 operand of the next
  // GEMM instead of out: hi [n_rows, hq hd], then lo [n_rows, hq hd]
  uint16_t* outb;
  int n_rows, batch, hq, hkv, split_len, n_splits;
};

// Row set-up: xin[m] = [feat[parent[m]] ; embed[token[m]]] (fp32, 2d).
struct RowSetupArgs {
  int n_rows;
  const int32_t* parent;
  const int32_t* token;
  const float* feat;  // [*, d] fp32
  const void* embed;  // [vocab, d] bf16 or fp32
  int d;
  float* xin;  // [n_rows, 2d]
};
hipError_t launch_row_setup(const RowSetupArgs& a, bool bf16, hipStream_t s);
// out[m] = [low[m] ; mid[m] ; high[m]], fp32 rows of d values each
hipError_t launch_concat3(const float* low, const float* mid, const float* high, int n_rows, int d, float* out,
                          hipStream_t s);
hipError_t launch_rope_kv(const RopeArgs& a, bool bf16, hipStream_t s);
// Key splits of one attention call: split s covers prefix keys [s*split_len,
// (s+1)*split_len).  bf16: the tree slots go with the last split; fp32: they
// are one more split of their own.  max_queries = most rows of one sequence
// times query heads per kv head.
struct AttnPlan {
  int split_len, n_splits;
};
AttnPlan attn_plan(bool bf16, int max_prefix, int batch, int hkv, int max_queries);
hipError_t launch_attention(const AttnArgs& a, bool bf16, int hd, int max_queries, hipStream_t s);

// softmax + top-k.  With `smp`, the ranking key of token v in row r is
// logit + g, g = -log(-log(u)) from Philox counter (smp->row_base + r, v / 4,
// 0, 1) under key (seed, round), word v % 4, u = ((w >> 41) + 0.5) 2^-23: the k
// tokens then are k draws without replacement from the row's softmax, in draw
// order (Gumbel-top-k); lse and logq stay those of the plain logits.
struct TopkSample {
  uint64_t seed, round;
  int row_base;
};
constexpr int TOPK_SAMPLE_MAX_VOCAB = 64 * 32 * 256;  // the chunked pass only
size_t topk_workspace_bytes(int n_rows, int vocab);
hipError_t launch_softmax_topk(int n_rows, int vocab, const float* logits, int k, float* lse, int32_t* idx,
                               float* logq, void* ws, hipStream_t s, const TopkSample* smp = nullptr);

// tree builder
struct PoolArgs {
  int cap;
  int32_t* parent;
  int32_t* token;
  int32_t* depth;
  float* logv;
  int32_t* feat_row;
  int32_t* slot;
  uint64_t* mask;
  int32_t* count;
  int32_t* frontier;
};
hipError_t launch_tree_init(int batch, const PoolArgs& p, const int32_t* root_token, int root_feat_row0,
                            hipStream_t s);
struct ExpandArgs {
  PoolArgs pool;
  int k, step, n_prev, topk, n_next, feat_row0;
  const int32_t* nchild;  // NULL = EAGLE-2
  const int32_t* topk_idx;
  const float* topk_logq;
  const int32_t* prefix_len;
  int32_t *next_token, *next_parent, *next_pos, *next_slot, *next_row_start;
  uint64_t* next_mask;
  int batch;
};
hipError_t launch_tree_expand(const ExpandArgs& a, hipStream_t s);
struct FinalizeArgs {
  PoolArgs pool;
  int m, n_nodes, batch;
  const int32_t* prefix_len;
  int32_t *tree_parent, *tree_token, *tree_depth, *tree_pool, *tree_qrow;
  uint64_t* tree_mask;
  int32_t *row_token, *row_parent, *row_pos, *row_slot, *row_start;
  uint64_t* row_mask;
};
hipError_t launch_tree_finalize(const FinalizeArgs& a, hipStream_t s);

// verification
struct VerifyArgs {
  int batch, n_nodes, vocab;
  const int32_t* parent;
  const int32_t* token;
  const float* target;
  const float* draft;
  const int32_t* draft_row;
  uint64_t seed, round;
  int flags;
  int32_t *path, *accept_len, *next_token, *out_flags;
  // per-node results, [batch*n_nodes] each (workspace)
  int32_t* node_next;   // accepted child, -1 if none
  int32_t* node_tok;    // correction / bonus token when node_next < 0
  int32_t* node_flags;  // status bits raised at the node
};
size_t verify_workspace_bytes(int batch, int n_nodes);
hipError_t launch_verify(VerifyArgs a, void* ws, hipStream_t s);
// Device address (current device) of the library's own verify scratch, which
// holds the per-node results of up to VERIFY_NOALLOC_MAX_NODES nodes.
constexpr int VERIFY_NOALLOC_MAX_NODES = 8192;
hipError_t verify_scratch_address(void** ptr);

// accepted-path commit of the draft KV cache
constexpr int kCommitOverflow = 1, kCommitBadPath = 2;  // = EAGLE_COMMIT_OVERFLOW / _BAD_PATH
struct CommitArgs {
  int batch, n_nodes, hkv, hd;
  const int32_t* path;        // [batch, n_nodes]: accepted drafted nodes, -1 padded; nullptr: slot mode
  const int32_t* accept_len;  // [batch]: accepted nodes + 1 (slot mode: slots 0..n-1 to append)
  const int32_t* node_slot;   // [batch, n_nodes] tree slot of each node, or nullptr: slot = node
  const void* tree_k;
  const void* tree_v;
  void* prefix_k;
  void* prefix_v;
  const int64_t* prefix_off;
  int32_t* prefix_len;
  const int32_t* prefix_cap;  // or nullptr: capacity = length (no room)
  int32_t* out_flags;
};
hipError_t launch_commit(const CommitArgs& a, bool bf16, hipStream_t s);

// catch-up rows of the drafter over each sequence's committed tokens
struct CatchupArgs {
  int batch, n_nodes, max_depth, feat_row0;
  const int32_t* tree_token;  // [batch, n_nodes]
  const int32_t* path;        // [batch, n_nodes] verified path
  const int32_t* accept_len;  // [batch]
  const int32_t* next_token;  // [batch]
  const int32_t* prefix_len;  // [batch]
  int32_t *row_token, *row_parent, *row_pos, *row_slot, *row_start, *last_row, *count;
  uint64_t* row_mask;
};
hipError_t launch_catchup_rows(const CatchupArgs& a, hipStream_t s);
hipError_t launch_gather_rows(const float* feat, const int32_t* rows, int batch, int d, float* out, hipStream_t s);
