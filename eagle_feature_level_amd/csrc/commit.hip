// Accepted-path commit of the draft layer's KV cache.
//
// Verification accepts a path of drafted nodes; only their k, v may enter the
// cache, the rejected branches' entries are dropped, and the cache is then
// advanced by the accepted length ("eagle feature-level speculative
// decoding", section on committing the KV cache as a transaction).  The
// accepted node at path position j sits at rotary position L_b + j (its depth
// is j + 1), so the j-th accepted node's tree slot is copied to prefix
// position L_b + j of every kv head, then L_b grows by the accepted count.
// Two launches: the copy (one workgroup per (sequence, kv head), all heads
// read the old L_b) and the length update (one thread per sequence).
//
// The drafter's own state after a round ("eagle feature-level speculative
// decoding", KV commit section: if the tree held A-B-D and the target
// accepted A-B and then X, the drafter continues from A-B-X, not from D's
// predicted state; study note section 6.2: the accepted path's true features
// start the next round): its rows over the committed tokens are recomputed
// from the target's true features.  catchup_rows_kernel lays them out for one
// draft step (row i of sequence b joins the true feature of the token at path
// position i with the embedding of the token after it, at position L_b + i,
// tree slot i, seeing slots 0..i); the slot commit then appends slots
// 0..A_b to the prefix and the row of the verifier's next token hands its
// predicted feature to the next round's root.
#include "common.h"
#include "kernels.h"

namespace {

// Accepted drafted nodes of sequence b, or -1 if the path is malformed (a
// node or slot index out of range); also the prefix capacity.  Slot mode
// (no path): accept_len holds the number of slots 0.. to append.
__device__ __forceinline__ int accepted_count(const CommitArgs& a, int b, int* cap) {
  const int L = a.prefix_len[b];
  *cap = a.prefix_cap ? a.prefix_cap[b] : L;
  if (!a.path) {
    const int n = a.accept_len[b];
    return (n < 0 || n > 64) ? -1 : n;
  }
  int A = a.accept_len[b] - 1;
  if (A < 0) A = 0;
  if (A > a.n_nodes - 1) return -1;
  for (int j = 0; j < A; ++j) {
    const int node = a.path[(size_t)b * a.n_nodes + j];
    if (node < 1 || node >= a.n_nodes) return -1;
    const int slot = a.node_slot ? a.node_slot[(size_t)b * a.n_nodes + node] : node;
    if (slot < 0 || slot >= 64) return -1;
  }
  return A;
}

template <typename T>
__global__ void __launch_bounds__(64) commit_copy_kernel(CommitArgs a) {
  const int b = blockIdx.x, h = blockIdx.y;
  int C;
  const int A = accepted_count(a, b, &C);
  const int L = a.prefix_len[b];
  if (A <= 0 || L + A > C) return;
  for (int j = 0; j < A; ++j) {
    int slot = j;
    if (a.path) {
      const int node = a.path[(size_t)b * a.n_nodes + j];
      slot = a.node_slot ? a.node_slot[(size_t)b * a.n_nodes + node] : node;
    }
    const size_t src = (((size_t)b * 64 + slot) * a.hkv + h) * a.hd;
    const size_t dst = (size_t)a.prefix_off[b] + ((size_t)h * C + L + j) * a.hd;
    for (int i = threadIdx.x; i < a.hd; i += 64) {
      ((T*)a.prefix_k)[dst + i] = ((const T*)a.tree_k)[src + i];
      ((T*)a.prefix_v)[dst + i] = ((const T*)a.tree_v)[src + i];
    }
  }
}

__global__ void commit_len_kernel(CommitArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.batch) return;
  int C;
  const int A = accepted_count(a, b, &C);
  const int L = a.prefix_len[b];
  int flags = 0;
  if (A < 0)
    flags = kCommitBadPath;
  else if (L + A > C)
    flags = kCommitOverflow;
  else
    a.prefix_len[b] = L + A;
  a.out_flags[b] = flags;
}

// One thread per catch-up row (b, i), i = 0..R-1, R = max_depth + 1.
__global__ void catchup_rows_kernel(CatchupArgs a) {
  const int R = a.max_depth + 1;
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= a.batch * R) return;
  const int b = gid / R, i = gid % R;
  const size_t nb = (size_t)b * a.n_nodes;
  int A = a.accept_len[b] - 1;
  bool ok = A >= 0 && A <= a.max_depth && A <= a.n_nodes - 1;
  for (int j = 0; ok && j < A; ++j) {
    const int node = a.path[nb + j];
    ok = node >= 1 && node < a.n_nodes;
  }
  if (!ok) A = 0;  // malformed verification result: rows of A = 0, nothing committed
  const int r = min(i, A);  // rows past A repeat row A in their own slot
  const int node = r == 0 ? 0 : a.path[nb + r - 1];
  const int tok = r < A ? a.tree_token[nb + a.path[nb + r]] : a.next_token[b];
  const uint64_t below = (1ull << r) - 1ull;  // slots 0..r-1 (r < 64)
  a.row_token[gid] = tok;
  a.row_parent[gid] = a.feat_row0 + (int)nb + node;
  a.row_pos[gid] = a.prefix_len[b] + r;
  a.row_slot[gid] = i;
  a.row_mask[gid] = below | (1ull << i);
  if (i == 0) {
    a.row_start[b] = b * R;
    if (b == a.batch - 1) a.row_start[a.batch] = a.batch * R;
    a.last_row[b] = b * R + A;
    a.count[b] = ok ? A + 1 : -1;
  }
}

// root_feat[b] = feat[last_row[b]] (d fp32 values), one workgroup per sequence.
__global__ void __launch_bounds__(256) gather_rows_kernel(const float* feat, const int32_t* rows, int d,
                                                          float* out) {
  const int b = blockIdx.x;
  const float* src = feat + (size_t)rows[b] * d;
  for (int i = threadIdx.x; i < d; i += 256) out[(size_t)b * d + i] = src[i];
}

}  // namespace

hipError_t launch_catchup_rows(const CatchupArgs& a, hipStream_t s) {
  const int n = a.batch * (a.max_depth + 1);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(catchup_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const float* feat, const int32_t* rows, int batch, int d, float* out, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(batch), dim3(256), 0, s, feat, rows, d, out);
  return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs& a, bool bf16, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  const dim3 g(a.batch, a.hkv);
  if (bf16)
    hipLaunchKernelGGL(commit_copy_kernel<bf16_t>, g, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(commit_copy_kernel<float>, g, dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(commit_len_kernel, dim3((a.batch + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}
