// Tree-structured recursive rejection sampling.
//
// Rule for one draft token x ~ q against the target p: accept with probability
// min(1, p(x)/q(x)); else draw from norm(max(0, p - q)) ("EAGLE 推测解码为什么比
// Medusa 快" section 6.2; "eagle feature-level speculative decoding", section
// "随机采样验证").  On a tree it is applied from the root: a node's children are
// tried in rank order; after a rejection p becomes the residual and (default)
// the rejected token is removed from q, which is renormalised.  All children
// rejected -> correction draw from the residual; accepted leaf -> bonus draw
// from the leaf's p.  Greedy mode replaces p by the onehot of the argmax.
//
// Uniforms: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11), counter
// (sequence, node, event, 0), key (seed, round), u = (word0 >> 40) * 2^-24;
// event i = test of the i-th child, event 64 = correction / bonus draw.
//
// What happens at a node does not depend on the path that reached it: p and q
// come from the node's own rows, the uniforms from (sequence, node, event).
// So with a workspace every node of every tree is processed at once, one
// 1024-thread workgroup each (which child it accepts, else the correction or
// bonus token, and the status bits it raises), and a second launch walks the
// trees through those results, one thread per sequence.  Without a
// workspace, one workgroup per sequence processes the nodes along its path.
// Thread t holds EPT tokens, in runs of up to 4 consecutive ones laid out so
// that each load instruction of a wave reads one contiguous span of the row
// (coalesced); p lives in registers, q in the thread's own LDS column, a node
// needs block reductions only, and the inverse-CDF draw is one token-order
// scan.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int VT = 1024;
constexpr int NW = VT / WAVE;

__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t round, uint64_t c0, uint64_t c1, uint64_t c2) {
  uint64_t w[4];
  philox4x64_10(seed, round, c0, c1, c2, 0, w);
  return (float)(w[0] >> 40) * 5.9604644775390625e-08f;  // 2^-24
}

__device__ __forceinline__ float bsum(float v, float* red) { return block_sum<VT>(v, red); }
__device__ __forceinline__ float bmax(float v, float* red) { return block_max<VT>(v, red); }

__device__ __forceinline__ int bmin_int(int v, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, WAVE));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = min(r, red[i]);
  return r;
}

// Token layout: thread t (wave w, lane l) holds its EPT tokens in chunks of
// CW = min(EPT, 4) consecutive ones; chunk j sits at w*EPT*64 + j*64*CW + l*CW,
// so a wave's load of chunk j is 64*CW consecutive floats.  Element e = j*CW + c.
template <int EPT>
struct Lay {
  static constexpr int CW = EPT < 4 ? EPT : 4, J = EPT / CW, SPAN = EPT * WAVE;
};
template <int EPT>
__device__ __forceinline__ int tok_of(int t, int e) {
  using L = Lay<EPT>;
  return (t / WAVE) * L::SPAN + (e / L::CW) * (WAVE * L::CW) + (t % WAVE) * L::CW + e % L::CW;
}
// the thread and element holding token y
template <int EPT>
__device__ __forceinline__ void owner_of(int y, int* t, int* e) {
  using L = Lay<EPT>;
  const int w = y / L::SPAN, r = y % L::SPAN;
  const int j = r / (WAVE * L::CW), r2 = r % (WAVE * L::CW);
  *t = w * WAVE + r2 / L::CW;
  *e = j * L::CW + r2 % L::CW;
}

// Inverse CDF in token order: smallest y with cum(y) > u * sum(w).  The
// running sum before a token is (waves before) + (chunks before, in this wave)
// + (lanes before, in this chunk) + (this run's earlier tokens).
template <int EPT>
__device__ int draw_token(const float (&w)[EPT], int vocab, float u, float* fred, int* ired) {
  using L = Lay<EPT>;
  const int lane = threadIdx.x & (WAVE - 1), wv = threadIdx.x / WAVE;
  float lex[L::J], coff[L::J];
  float off = 0.f;
#pragma unroll
  for (int j = 0; j < L::J; ++j) {
    float sj = 0.f;
#pragma unroll
    for (int c = 0; c < L::CW; ++c) sj += w[j * L::CW + c];
    float inc = sj;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
      const float tv = __shfl_up(inc, o, WAVE);
      if (lane >= o) inc += tv;
    }
    lex[j] = inc - sj;
    coff[j] = off;
    off += __shfl(inc, WAVE - 1, WAVE);
  }
  __syncthreads();
  if (lane == 0) fred[wv] = off;
  __syncthreads();
  float before = 0.f, total = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i < wv) before += fred[i];
    total += fred[i];
  }
  const float T = u * total;
  int cand = 0x7fffffff, last = -1;
#pragma unroll
  for (int j = 0; j < L::J; ++j) {
    float c = before + coff[j] + lex[j];
#pragma unroll
    for (int cc = 0; cc < L::CW; ++cc) {
      const int e = j * L::CW + cc;
      const int y = tok_of<EPT>(threadIdx.x, e);
      if (y < vocab) {
        c += w[e];
        if (w[e] > 0.f) last = y;
        if (c > T && cand == 0x7fffffff && w[e] > 0.f) cand = y;
      }
    }
  }
  const int y = bmin_int(cand, ired);
  if (y != 0x7fffffff) return y;
  return -bmin_int(-last, ired);  // rounding left no boundary above T: last positive token
}

// Thread t's EPT entries of a row in the layout above; -inf beyond the vocabulary.
// With V a multiple of 4 and an aligned row, every chunk is one 16-byte load
// per lane (from an address clamped into the row; lanes past the end discard
// it); otherwise element loads.  The choice is uniform over the launch.
template <int EPT>
__device__ __forceinline__ bool load_row(const float* row, int V, float (&v)[EPT]) {
  using L = Lay<EPT>;
  bool bad = false;
  if (L::CW == 4 && V % 4 == 0 && ((uintptr_t)row & 15) == 0) {
#pragma unroll
    for (int j = 0; j < L::J; ++j) {
      const int y0 = tok_of<EPT>(threadIdx.x, j * L::CW);
      const float4 f = *(const float4*)(row + min(y0, V - 4));
      const bool in = y0 < V;
      v[j * L::CW] = in ? f.x : -INFINITY;
      v[j * L::CW + 1] = in ? f.y : -INFINITY;
      v[j * L::CW + 2] = in ? f.z : -INFINITY;
      v[j * L::CW + 3] = in ? f.w : -INFINITY;
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int y = tok_of<EPT>(threadIdx.x, e);
      v[e] = y < V ? row[y] : -INFINITY;
    }
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) bad |= (v[e] != v[e]);
  return bad;
}

// Shared state of one node's processing.
template <int EPT>
struct NodeShared {
  float fred[NW];
  int ired[NW];
  // one-barrier reductions: partials alternate between two buffers, and a
  // buffer is written again only after every thread has passed the barrier
  // of the reduction that followed its last use
  float rv[2][2][NW];
  int rany[2][NW];
  float2 pq[2];  // (p(x), raw q(x)) of the child under test, same buffer as its reduction
  int kids[64], ktok[64];
  // exp(draft logit - max) of the node, element e of thread t at ql[e * VT +
  // t] (lanes on consecutive banks); removed tokens are set to 0
  float ql[EPT * VT];
};

// Sum (SUM) or max of two values per thread over the block, with one barrier;
// also ORs `flag` over the block into *any when any is set.
template <bool SUM, int EPT>
__device__ __forceinline__ float2 red2(float x, float y, NodeShared<EPT>& sh, int& buf, bool flag = false,
                                       bool* any = nullptr) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  x = SUM ? wave_sum(x) : wave_max(x);
  y = SUM ? wave_sum(y) : wave_max(y);
  const bool wf = __ballot(flag) != 0ull;
  if (l == 0) {
    sh.rv[buf][0][w] = x;
    sh.rv[buf][1][w] = y;
    sh.rany[buf][w] = wf;
  }
  __syncthreads();
  float sx = SUM ? 0.f : -INFINITY, sy = sx;
  int f = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    sx = SUM ? sx + sh.rv[buf][0][i] : fmaxf(sx, sh.rv[buf][0][i]);
    sy = SUM ? sy + sh.rv[buf][1][i] : fmaxf(sy, sh.rv[buf][1][i]);
    f |= sh.rany[buf][i];
  }
  if (any) *any = f != 0;
  buf ^= 1;
  return make_float2(sx, sy);
}

// Node u of sequence b: returns (accepted child, 0) or (-1, correction or
// bonus token); ORs the status bits it raises into *flags (uniform).  buf is
// the reduction buffer parity, carried across calls.
template <int EPT>
__device__ __forceinline__ int2 node_step(const VerifyArgs& a, NodeShared<EPT>& sh, int b, int u, int* flags,
                                          int& buf) {
  const int t = threadIdx.x;
  const int N = a.n_nodes, V = a.vocab;
  const size_t nb = (size_t)b * N;
  const bool greedy = a.flags & 1, iid = a.flags & 2;
  float* fred = sh.fred;
  int* ired = sh.ired;
#define Q(e) sh.ql[(e) * VT + t]
  // children of u in index order (n_nodes <= 64): every wave takes the same
  // ballot over the parent array, so the count needs no barrier; wave 0
  // publishes the list (visible after the first reduction's barrier)
  const int lane = t & (WAVE - 1);
  const int drow_idx = a.draft_row[nb + u];
  const int par = lane < N ? a.parent[nb + lane] : -2;
  float p[EPT];  // current target distribution (normalised)
  const bool bad = load_row<EPT>(a.target + (nb + u) * V, V, p);
  const bool kid = lane > u && lane < N && par == u;
  const uint64_t km = __ballot(kid);
  const int nk = __popcll(km);
  if (t < WAVE && kid) {
    const int rk = __popcll(km & ((1ull << lane) - 1ull));
    sh.kids[rk] = lane;
    sh.ktok[rk] = a.token[nb + lane];
  }
  // the draft row, only for a node with children: raw logits into q's columns
  // (only thread t touches its column)
  const bool have_q = nk > 0 && drow_idx >= 0;
  float dmx = -INFINITY;
  if (have_q) {
    float dv[EPT];
    load_row<EPT>(a.draft + (size_t)drow_idx * V, V, dv);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      dmx = fmaxf(dmx, dv[e]);
      Q(e) = dv[e];
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < EPT; ++e) mx = fmaxf(mx, p[e]);
  bool any_nan;
  const float2 mm = red2<false>(mx, dmx, sh, buf, bad, &any_nan);  // also publishes the children
  if (any_nan) *flags |= 8;
  mx = mm.x;
  dmx = mm.y;
  float ls = 0.f, ds = 0.f;
  if (greedy) {
    int cand = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (p[e] == mx) cand = min(cand, tok_of<EPT>(t, e));
    const int am = bmin_int(cand, ired);
#pragma unroll
    for (int e = 0; e < EPT; ++e) p[e] = (tok_of<EPT>(t, e) == am) ? 1.f : 0.f;
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      p[e] = (p[e] == -INFINITY) ? 0.f : __expf(p[e] - mx);
      ls += p[e];
    }
  }
  if (have_q) {
    // q(y) = exp(d_y - dmx) / S over the tokens not removed, the exponentials taken once
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      Q(e) = (Q(e) == -INFINITY) ? 0.f : __expf(Q(e) - dmx);
      ds += Q(e);
    }
  }
  float S = 0.f;
  if (!greedy || have_q) {
    const float2 sums = red2<true>(ls, ds, sh, buf);
    if (!greedy) {
      const float inv = 1.f / sums.x;
#pragma unroll
      for (int e = 0; e < EPT; ++e) p[e] *= inv;
    }
    S = sums.y;
  }
  if (nk == 0) return make_int2(-1, draw_token<EPT>(p, V, philox_uniform(a.seed, a.round, b, u, 64), fred, ired));
  if (drow_idx < 0) {  // no draft row for a node with children: a malformed tree
    *flags |= 16;
    return make_int2(-1, draw_token<EPT>(p, V, philox_uniform(a.seed, a.round, b, u, 64), fred, ired));
  }
  for (int i = 0; i < nk; ++i) {
    if (!(S > 0.f)) {
      *flags |= 4;
      break;
    }
    const int c = sh.kids[i];
    const int x = sh.ktok[i];
    const float r = philox_uniform(a.seed, a.round, b, u, i);
    const bool x_ok = x >= 0 && x < V;
    int ot = -1, oe = 0;
    if (x_ok) owner_of<EPT>(x, &ot, &oe);
    const bool owner = t == ot;
    // residual mass norm(max(0, p - q)) taken before the test (needed only on a
    // rejection; a zero mass leaves p untouched), one reduction with p(x), q(x)
    const float invS = 1.f / S;
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) rs += fmaxf(0.f, p[e] - Q(e) * invS);
    const int pb = buf;
    if (owner) {
      float px = 0.f;
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if (e == oe) px = p[e];
      sh.pq[pb] = make_float2(px, Q(oe));
    }
    const float Z = red2<true>(rs, 0.f, sh, buf).x;
    const float px = x_ok ? sh.pq[pb].x : 0.f;
    const float qx = x_ok ? sh.pq[pb].y / S : 0.f;
    bool ok;
    if (qx > 0.f) {
      ok = r < px / qx;
    } else {
      *flags |= 2;
      ok = px > 0.f;
    }
    if (ok) return make_int2(c, 0);
    // residual update; without iid the rejected token leaves q (its column
    // zeroed) and the remaining mass is summed in the same pass over q
    const int xe = (!iid && owner) ? oe : -1;
    float qs = 0.f;
    if (Z > 0.f) {
      const float inv = 1.f / Z;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const float qe = Q(e);
        p[e] = fmaxf(0.f, p[e] - qe * invS) * inv;
        qs += (e == xe) ? 0.f : qe;
      }
    } else {
      *flags |= 1;  // zero residual mass (reachable only through rounding): keep p
#pragma unroll
      for (int e = 0; e < EPT; ++e) qs += (e == xe) ? 0.f : Q(e);
    }
    if (xe >= 0) Q(xe) = 0.f;
    if (!iid) S = red2<true>(qs, 0.f, sh, buf).x;  // renormalise q
  }
#undef Q
  // every child rejected: correction from the residual
  return make_int2(-1, draw_token<EPT>(p, V, philox_uniform(a.seed, a.round, b, u, 64), fred, ired));
}

// One workgroup per sequence, along its path.
template <int EPT>
__global__ void __launch_bounds__(VT) verify_kernel(VerifyArgs a) {
  __shared__ NodeShared<EPT> sh;
  const int b = blockIdx.x, N = a.n_nodes;
  int flags = 0, u = 0, nacc = 0, next_tok = 0, buf = 0;
  for (int level = 0; level <= N; ++level) {
    const int2 r = node_step<EPT>(a, sh, b, u, &flags, buf);
    if (r.x < 0) {
      next_tok = r.y;
      break;
    }
    if (threadIdx.x == 0) a.path[(size_t)b * N + nacc] = r.x;
    ++nacc;
    u = r.x;
  }
  if (threadIdx.x == 0) {
    for (int j = nacc; j < N; ++j) a.path[(size_t)b * N + j] = -1;
    a.accept_len[b] = nacc + 1;
    a.next_token[b] = next_tok;
    a.out_flags[b] = flags;
  }
}

// One workgroup per node of every tree: its result into the workspace.
template <int EPT>
__global__ void __launch_bounds__(VT) verify_node_kernel(VerifyArgs a) {
  __shared__ NodeShared<EPT> sh;
  const int N = a.n_nodes;
  const int b = blockIdx.x / N, u = blockIdx.x % N;
  int flags = 0, buf = 0;
  const int2 r = node_step<EPT>(a, sh, b, u, &flags, buf);
  if (threadIdx.x == 0) {
    a.node_next[blockIdx.x] = r.x;
    a.node_tok[blockIdx.x] = r.y;
    a.node_flags[blockIdx.x] = flags;
  }
}

// One wave per sequence: lane u holds node u's result (n_nodes <= 64), and
// the walk through them moves by lane shuffles, with no dependent global reads.
__global__ void __launch_bounds__(64) verify_walk_kernel(VerifyArgs a) {
  const int b = blockIdx.x, l = threadIdx.x;
  const int N = a.n_nodes;
  const size_t base = (size_t)b * N;
  int nx = -1, tk = 0, fl = 0;
  if (l < N) {
    nx = a.node_next[base + l];
    tk = a.node_tok[base + l];
    fl = a.node_flags[base + l];
  }
  int flags = 0, u = 0, nacc = 0, next_tok = 0, mine = -1;
  for (int level = 0; level <= N; ++level) {
    flags |= __shfl(fl, u, WAVE);
    const int c = __shfl(nx, u, WAVE);
    if (c < 0) {
      next_tok = __shfl(tk, u, WAVE);
      break;
    }
    if (l == nacc) mine = c;
    ++nacc;
    u = c;
  }
  if (l < N) a.path[base + l] = l < nacc ? mine : -1;
  if (l == 0) {
    a.accept_len[b] = nacc + 1;
    a.next_token[b] = next_tok;
    a.out_flags[b] = flags;
  }
}

}  // namespace

size_t verify_workspace_bytes(int batch, int n_nodes) { return (size_t)batch * n_nodes * 12 + 1024; }

hipError_t launch_verify(VerifyArgs a, void* ws, hipStream_t s) {
  if (a.vocab > 32 * VT) return hipErrorInvalidValue;
  const int EPT = a.vocab <= VT ? 1 : a.vocab <= 4 * VT ? 4 : 32;
  if (!ws) {
    if (EPT == 1) hipLaunchKernelGGL(verify_kernel<1>, dim3(a.batch), dim3(VT), 0, s, a);
    else if (EPT == 4) hipLaunchKernelGGL(verify_kernel<4>, dim3(a.batch), dim3(VT), 0, s, a);
    else hipLaunchKernelGGL(verify_kernel<32>, dim3(a.batch), dim3(VT), 0, s, a);
    return hipGetLastError();
  }
  const size_t n = (size_t)a.batch * a.n_nodes;
  const size_t step = (n * 4 + 255) / 256 * 256;
  char* w = (char*)ws;
  a.node_next = (int32_t*)w;
  a.node_tok = (int32_t*)(w + step);
  a.node_flags = (int32_t*)(w + 2 * step);
  const dim3 g((unsigned)n);
  if (EPT == 1) hipLaunchKernelGGL(verify_node_kernel<1>, g, dim3(VT), 0, s, a);
  else if (EPT == 4) hipLaunchKernelGGL(verify_node_kernel<4>, g, dim3(VT), 0, s, a);
  else hipLaunchKernelGGL(verify_node_kernel<32>, g, dim3(VT), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_walk_kernel, dim3(a.batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

// The per-node results of eagle_verify_noalloc live in this file-scope device
// array instead of a caller workspace: room for VERIFY_NOALLOC_MAX_NODES nodes
// (the workspace layout above, 12 bytes per node plus alignment).  Each GPU
// holds its own copy for the life of the process.  Nothing in it needs
// clearing: the node kernel writes every node's three entries before the walk
// reads them.  Calls that overlap on one GPU share it and race.
static __device__ __align__(256) unsigned char scratch[(size_t)VERIFY_NOALLOC_MAX_NODES * 12 + 1024];
static_assert(sizeof(scratch) >= (size_t)VERIFY_NOALLOC_MAX_NODES * 12 + 1024, "scratch holds the largest call");

hipError_t verify_scratch_address(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {  // first call on this device, with it current: its copy's device address
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}
