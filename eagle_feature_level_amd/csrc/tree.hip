// Draft-tree builder: EAGLE-2 expand and rerank, static templates.
//
// value(node) = product of draft confidences along the root-to-node path
// ("EAGLE 推测解码为什么比 Medusa 快" section 10.3), kept as a log-value
// logv(child) = fl32(logv(parent) + logq).  Expand: each frontier node gets its
// top-k tokens as children; the next frontier is the k children of largest
// value.  Rerank: keep the m most valuable nodes; since value never grows along
// a path and ties go to the shallower node, the kept set is a connected tree.
// Every selection is a rank computed by counting how many candidates beat a
// candidate under a strict total order, so results are exact and need no
// sort.  One workgroup per sequence: the pools are tiny (< 1000 nodes).
#include "common.h"
#include "kernels.h"

namespace {

__global__ void tree_init_kernel(PoolArgs p, const int32_t* root_token, int root_feat_row0, int batch) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const size_t base = (size_t)b * p.cap;
  p.parent[base] = -1;
  p.token[base] = root_token[b];
  p.depth[base] = 0;
  p.logv[base] = 0.f;
  p.feat_row[base] = root_feat_row0 + b;
  p.slot[base] = -1;
  p.mask[base] = 0ull;
  p.count[b] = 1;
  p.frontier[(size_t)b * 64] = 0;
}

constexpr int EX_MAX_CHILD = 256;  // 16 x 16

// Every global read the kernel needs is issued in its first phase (the
// frontier, then the frontier nodes' own fields and the sequence's counters),
// and in the second (the children's top-k entries); the rest works from LDS.
// Nothing is written to the pool before the expansion is known to be valid:
// a NaN log-value among the children (a NaN logit row gives every log q of
// that row NaN), a template asking a node for more children than its row
// ranks, or a template whose qualifying children differ in number from n_next
// mark the pool invalid (count = -1, the same as an overflow), so that every
// rank slot of the next frontier is filled whenever anything is written.
__global__ void __launch_bounds__(256) tree_expand_kernel(ExpandArgs a) {
  __shared__ int off[65];
  __shared__ int fr[64], fcnt[64], fdep[64], ffrow[64];
  __shared__ float flogv[64];
  __shared__ uint64_t fmask[64];
  __shared__ float clogv[EX_MAX_CHILD];
  __shared__ int cqual[EX_MAX_CHILD], cf[EX_MAX_CHILD], ctok[EX_MAX_CHILD];
  __shared__ int nf[64];
  __shared__ int s_total, s_cnt, s_plen, s_bad;
  const int b = blockIdx.x, t = threadIdx.x;
  const PoolArgs& p = a.pool;
  const size_t base = (size_t)b * p.cap;
  if (t < 64) nf[t] = -1;
  if (t < a.n_prev) {
    const int u = p.frontier[(size_t)b * 64 + t];
    fr[t] = u;
    fcnt[t] = a.nchild ? a.nchild[u] : a.k;
    flogv[t] = p.logv[base + u];
    fdep[t] = p.depth[base + u];
    fmask[t] = p.mask[base + u];
    ffrow[t] = p.feat_row[base + u];
  }
  if (t == 255) {
    s_cnt = p.count[b];
    s_plen = a.prefix_len[b];
  }
  __syncthreads();
  if (t == 0) {
    int acc = 0, bad = 0;
    for (int f = 0; f < a.n_prev; ++f) {
      off[f] = acc;
      acc += fcnt[f];
      bad |= (fcnt[f] < 0) | (fcnt[f] > a.topk);
    }
    off[a.n_prev] = acc;
    s_total = acc;
    s_bad = bad;
  }
  __syncthreads();
  const int total = s_total, cnt = s_cnt;
  if (s_bad || cnt < 0 || cnt + total > p.cap || total > EX_MAX_CHILD) {
    if (t == 0) p.count[b] = -1;  // overflow or invalid request: pool left unchanged, marked invalid
    return;
  }
  bool nan_child = false;
  int qual = 0;
  if (t < total) {
    int f = 0;
    while (off[f + 1] <= t) ++f;
    const int r = t - off[f];
    const int row = b * a.n_prev + f;
    const float lv = __fadd_rn(flogv[f], a.topk_logq[(size_t)row * a.topk + r]);
    clogv[t] = lv;
    cf[t] = f;
    ctok[t] = a.topk_idx[(size_t)row * a.topk + r];
    qual = a.nchild ? (a.nchild[cnt + t] > 0) : 1;
    cqual[t] = qual;
    nan_child = lv != lv;
  }
  const int n_nan = __syncthreads_count(nan_child);
  const int n_qual = __syncthreads_count(qual);
  if (n_nan || (a.nchild && n_qual != a.n_next)) {
    if (t == 0) p.count[b] = -1;
    return;
  }
  if (t < total) {
    const int f = cf[t];
    const int id = cnt + t;
    p.parent[base + id] = fr[f];
    p.token[base + id] = ctok[t];
    p.depth[base + id] = fdep[f] + 1;
    p.logv[base + id] = clogv[t];
    p.feat_row[base + id] = -1;
    p.slot[base + id] = -1;
    p.mask[base + id] = 0ull;
    int rank = 0;
    if (a.nchild) {
#pragma unroll 8
      for (int j = 0; j < t; ++j) rank += cqual[j];
      if (cqual[t] && rank < a.n_next) nf[rank] = t;
    } else {
      const float v = clogv[t];
#pragma unroll 8
      for (int j = 0; j < total; ++j) {
        const float w = clogv[j];
        rank += (int)(w > v) | ((int)(w == v) & (int)(j < t));
      }
      if (rank < a.n_next) nf[rank] = t;
    }
  }
  __syncthreads();
  if (t < a.n_next) {
    const int c = nf[t];  // the candidate (child index) of rank t; filled, as checked above
    const int node = cnt + c, f = cf[c];
    const int slot = a.nchild ? node : a.step * a.k + t;
    const uint64_t mask = fmask[f] | (1ull << slot);
    const int frow = a.feat_row0 + b * a.n_next + t;
    p.feat_row[base + node] = frow;
    p.slot[base + node] = slot;
    p.mask[base + node] = mask;
    p.frontier[(size_t)b * 64 + t] = node;
    const int r = b * a.n_next + t;
    a.next_token[r] = ctok[c];
    a.next_parent[r] = ffrow[f];
    a.next_pos[r] = s_plen + fdep[f];  // prefix length + depth(node) - 1
    a.next_slot[r] = slot;
    a.next_mask[r] = mask;
  }
  if (t == 0) {
    p.count[b] = cnt + total;
    a.next_row_start[b] = b * a.n_next;
    if (b == a.batch - 1) a.next_row_start[a.batch] = a.batch * a.n_next;
  }
}

constexpr int FIN_MAX_POOL = 2048;

__global__ void __launch_bounds__(512) tree_finalize_kernel(FinalizeArgs a) {
  __shared__ float lv[FIN_MAX_POOL];
  __shared__ int dp[FIN_MAX_POOL];
  __shared__ int where[FIN_MAX_POOL];
  __shared__ int kept[FIN_MAX_POOL];
  __shared__ int ppar[FIN_MAX_POOL], ptok[FIN_MAX_POOL], pfrow[FIN_MAX_POOL];
  __shared__ int s_plen;
  __shared__ int tpool[64];
  __shared__ int tpar[64];
  __shared__ uint64_t tmask[64];
  const int b = blockIdx.x, t = threadIdx.x;
  const PoolArgs& p = a.pool;
  const size_t base = (size_t)b * p.cap;
  int cnt = p.count[b];
  if (cnt < 1 || cnt > FIN_MAX_POOL) cnt = 1;  // invalid pool: root only
  // every pool field the kernel reads, in one parallel pass (the later phases use LDS)
  for (int i = t; i < cnt; i += 512) {
    lv[i] = p.logv[base + i];
    dp[i] = p.depth[base + i];
    ppar[i] = p.parent[base + i];
    ptok[i] = p.token[base + i];
    pfrow[i] = p.feat_row[base + i];
    where[i] = -1;
  }
  if (t == 511) s_plen = a.prefix_len[b];
  __syncthreads();
  // selection: rank among candidates 1..cnt-1 by (logv desc, depth asc, id asc)
  const int ncand = cnt - 1;
  const int nkeep = (a.m > 0 && a.m < ncand) ? a.m : ncand;
  for (int i = 1 + t; i < cnt; i += 512) {
    int keep = 1;
    if (a.m > 0 && a.m < ncand) {
      const float v = lv[i];
      const int d = dp[i];
      int rank = 0;
#pragma unroll 8
      for (int j = 1; j < cnt; ++j) {  // branch-free: both fields read, the test in bit operations
        const float w = lv[j];
        const int dj = dp[j];
        rank += (int)(w > v) | ((int)(w == v) & ((int)(dj < d) | ((int)(dj == d) & (int)(j < i))));
      }
      keep = rank < a.m;
    }
    kept[i] = keep;
  }
  __syncthreads();
  // flatten: root first, kept nodes by (depth, id)
  for (int i = 1 + t; i < cnt; i += 512) {
    if (!kept[i]) continue;
    const int d = dp[i];
    int pos = 1;
#pragma unroll 8
    for (int j = 1; j < cnt; ++j) {
      const int dj = dp[j];
      pos += kept[j] & ((int)(dj < d) | ((int)(dj == d) & (int)(j < i)));
    }
    where[i] = pos;
    if (pos < 64) tpool[pos] = i;
  }
  if (t == 0) {
    where[0] = 0;
    tpool[0] = 0;
  }
  __syncthreads();
  const int n = a.n_nodes;
  const int nreal = min(nkeep + 1, n);
  if (t < n) {
    const size_t o = (size_t)b * n + t;
    if (t < nreal) {
      const int i = tpool[t];
      const int pp = (t == 0) ? -1 : where[ppar[i]];
      tpar[t] = pp;
      a.tree_parent[o] = pp;
      a.tree_token[o] = ptok[i];
      a.tree_depth[o] = dp[i];
      a.tree_pool[o] = i;
      a.tree_qrow[o] = pfrow[i];
    } else {
      tpar[t] = -2;
      a.tree_parent[o] = -2;
      a.tree_token[o] = 0;
      a.tree_depth[o] = 0;
      a.tree_pool[o] = -1;
      a.tree_qrow[o] = -1;
    }
  }
  __syncthreads();
  // mask of node u: its own bit and its ancestors' up to (not including) the
  // root, each thread walking its own chain (parents precede children)
  if (t < n) {
    uint64_t m = 0ull;
    if (t >= 1) {
      m = 1ull << t;
      if (t < nreal)
        for (int v = tpar[t], hop = 0; v > 0 && hop < 64; v = tpar[v], ++hop) m |= 1ull << v;
    }
    tmask[t] = m;
  }
  __syncthreads();
  if (t < n) {
    a.tree_mask[(size_t)b * n + t] = tmask[t];
    if (t >= 1) {
      const int r = b * (n - 1) + (t - 1);
      if (t < nreal) {
        const int i = tpool[t];
        a.row_token[r] = ptok[i];
        a.row_parent[r] = pfrow[ppar[i]];
        a.row_pos[r] = s_plen + dp[i] - 1;
      } else {
        a.row_token[r] = 0;
        a.row_parent[r] = pfrow[0];
        a.row_pos[r] = s_plen;
      }
      a.row_slot[r] = t;
      a.row_mask[r] = tmask[t];
    }
  }
  if (t == 0) {
    a.row_start[b] = b * (n - 1);
    if (b == a.batch - 1) a.row_start[a.batch] = a.batch * (n - 1);
  }
}

}  // namespace

hipError_t launch_tree_init(int batch, const PoolArgs& p, const int32_t* root_token, int root_feat_row0,
                            hipStream_t s) {
  hipLaunchKernelGGL(tree_init_kernel, dim3((batch + 63) / 64), dim3(64), 0, s, p, root_token, root_feat_row0, batch);
  return hipGetLastError();
}

hipError_t launch_tree_expand(const ExpandArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(tree_expand_kernel, dim3(a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tree_finalize(const FinalizeArgs& a, hipStream_t s) {
  if (a.pool.cap > FIN_MAX_POOL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_finalize_kernel, dim3(a.batch), dim3(512), 0, s, a);
  return hipGetLastError();
}
