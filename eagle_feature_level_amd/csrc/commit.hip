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
#include "common.h"
#include "kernels.h"

namespace {

// Accepted drafted nodes of sequence b, or -1 if the path is malformed (a
// node or slot index out of range); also the prefix capacity.
__device__ __forceinline__ int accepted_count(const CommitArgs& a, int b, int* cap) {
  const int L = a.prefix_len[b];
  *cap = a.prefix_cap ? a.prefix_cap[b] : L;
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
    const int node = a.path[(size_t)b * a.n_nodes + j];
    const int slot = a.node_slot ? a.node_slot[(size_t)b * a.n_nodes + node] : node;
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

}  // namespace

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
