// Softmax normaliser + per-row top-k over the vocabulary.
//
// EAGLE-2 ranks a node's children by the draft confidence (the softmax
// probability) and multiplies confidences along paths ("EAGLE 推测解码为什么比
// Medusa 快" section 10.3); this kernel gives, per logits row, lse and the top-k
// tokens with logq = logit - lse.  Ranking key: (value desc, index asc), one
// 64-bit integer per entry so every comparison is exact.
//
// Two launches.  Pass 1: a row is cut into at most 64 chunks, one wave each;
// a lane holds its share of the chunk in registers, computes (max, sum of exp)
// branch-free and keeps its 4 best entries sorted; the wave pops its k best by
// k rounds of a DPP wave maximum (a lane whose 4 are used up refills from its
// registers, below the last popped key).  Pass 2: one wave per row pops the k
// best of the chunks' lists (lane c holds chunk c's) the same way and merges
// (max, sum) in a fixed order.  One CU streams a 128 KB row at only ~6 GB/s with these per-entry
// costs, so a row is spread over many CUs.  Vocabularies above 524288 use the
// generic pair (per-thread K-deep lists, any number of chunks).
#include "common.h"
#include "kernels.h"

namespace {

__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = (m == -INFINITY ? 0.f : s * __expf(m - M)) + (m2 == -INFINITY ? 0.f : s2 * __expf(m2 - M));
  m = M;
}

template <int K>
__device__ __forceinline__ void list_insert(uint64_t (&lst)[K], uint64_t key) {
  if (key > lst[K - 1]) {
    lst[K - 1] = key;
#pragma unroll
    for (int i = K - 1; i > 0; --i) {
      if (lst[i] > lst[i - 1]) {
        const uint64_t t = lst[i];
        lst[i] = lst[i - 1];
        lst[i - 1] = t;
      }
    }
  }
}

// Pops the wave-wide largest head `k` times; result r-th in out[r] (uniform).
template <int K>
__device__ __forceinline__ void wave_topk(uint64_t (&lst)[K], int k, uint64_t* out) {
  for (int r = 0; r < k; ++r) {
    const uint64_t head = lst[0];
    const uint64_t best = wave_max_u64(head);
    if (head == best && best != 0ull) {
#pragma unroll
      for (int i = 0; i < K - 1; ++i) lst[i] = lst[i + 1];
      lst[K - 1] = 0ull;
    }
    out[r] = best;
  }
}

template <int K>
__global__ void __launch_bounds__(256) topk_partial(const float* __restrict__ logits, int vocab, int chunk, int k,
                                                    float2* __restrict__ ms_out, uint64_t* __restrict__ keys_out) {
  __shared__ uint64_t wkeys[4][K];
  __shared__ float2 wms[4];
  const int row = blockIdx.y, c = blockIdx.x, nchunks = gridDim.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float* x = logits + (size_t)row * vocab;
  const int c0 = c * chunk, c1 = min(vocab, c0 + chunk);
  float m = -INFINITY, s = 0.f;
  uint64_t lst[K];
#pragma unroll
  for (int i = 0; i < K; ++i) lst[i] = 0ull;
  for (int i = c0 + threadIdx.x * 4; i < c1; i += 256 * 4) {
    const float4 v = *(const float4*)(x + i);
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float t = e[j];
      if (t > m) {
        s = (m == -INFINITY ? 0.f : s * __expf(m - t)) + 1.f;
        m = t;
      } else if (t != -INFINITY) {
        s += __expf(t - m);
      } else if (t != t) {
        s = t;  // NaN propagates into lse
      }
      list_insert<K>(lst, topk_key(t, (uint32_t)(i + j)));
    }
  }
  // wave merge of (m, s) with a fixed butterfly order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, WAVE), s2 = __shfl_xor(s, o, WAVE);
    ms_merge(m, s, m2, s2);
  }
  uint64_t best[K];
  wave_topk<K>(lst, k, best);
  if (lane == 0) {
    for (int r = 0; r < k; ++r) wkeys[wv][r] = best[r];
    wms[wv] = make_float2(m, s);
  }
  __syncthreads();
  if (wv == 0) {
    // each lane holds at most one candidate: lanes r*4 + w
    uint64_t cand[1] = {0ull};
    if (lane < 4 * k) cand[0] = wkeys[lane % 4][lane / 4];
    uint64_t outk[K];
    // single-entry lists: pop k times
    for (int r = 0; r < k; ++r) {
      const uint64_t b = wave_max_u64(cand[0]);
      if (cand[0] == b) cand[0] = 0ull;
      outk[r] = b;
    }
    if (lane == 0) {
      float mm = wms[0].x, ss = wms[0].y;
      for (int w = 1; w < 4; ++w) ms_merge(mm, ss, wms[w].x, wms[w].y);
      const size_t o = (size_t)row * nchunks + c;
      ms_out[o] = make_float2(mm, ss);
      for (int r = 0; r < k; ++r) keys_out[o * K + r] = outk[r];
    }
  }
}

template <int K>
__global__ void __launch_bounds__(64) topk_merge(const float2* __restrict__ ms_in, const uint64_t* __restrict__ keys_in,
                                                 int nchunks, int k, float* lse, int32_t* idx, float* logq) {
  const int row = blockIdx.x, lane = threadIdx.x;
  float m = -INFINITY, s = 0.f;
  uint64_t lst[K];
#pragma unroll
  for (int i = 0; i < K; ++i) lst[i] = 0ull;
  if (lane < nchunks) {
    const size_t o = (size_t)row * nchunks + lane;
    const float2 v = ms_in[o];
    m = v.x;
    s = v.y;
#pragma unroll
    for (int i = 0; i < K; ++i) lst[i] = (i < k) ? keys_in[o * K + i] : 0ull;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, WAVE), s2 = __shfl_xor(s, o, WAVE);
    ms_merge(m, s, m2, s2);
  }
  const float l = m + __logf(s);
  uint64_t best[K];
  wave_topk<K>(lst, k, best);
  if (lane == 0) lse[row] = l;
  if (lane < k) {
    uint64_t b = best[0];
#pragma unroll
    for (int r = 1; r < K; ++r)
      if (lane == r) b = best[r];
    idx[(size_t)row * k + lane] = (int32_t)key_index(b);
    logq[(size_t)row * k + lane] = key_value(b) - l;
  }
}

// ---------------------------------------------------------------------------
// Chunked pass with DPP pops.
// ---------------------------------------------------------------------------
constexpr int TK_L = 4;        // entries a lane keeps sorted
constexpr int TK_KMAX = 16;    // largest k
constexpr int TK_CHUNKS = 64;  // most chunks per row: one per lane of the merge

// Wave-wide maximum of a 64-bit key by DPP (quad swaps, half-row and row
// mirrors, row broadcasts 15 and 31: the total lands in lane 63), returned
// wave-uniform.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const uint32_t wlo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xf, false);
  const uint32_t whi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xf, false);
  const uint64_t w = ((uint64_t)whi << 32) | wlo;
  return w > v ? w : v;
}
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  v = dpp_max_step<0xb1, 0xf>(v);   // quad_perm 1,0,3,2
  v = dpp_max_step<0x4e, 0xf>(v);   // quad_perm 2,3,0,1
  v = dpp_max_step<0x141, 0xf>(v);  // row_half_mirror
  v = dpp_max_step<0x140, 0xf>(v);  // row_mirror
  v = dpp_max_step<0x142, 0xa>(v);  // row_bcast:15
  v = dpp_max_step<0x143, 0xc>(v);  // row_bcast:31
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Sorted list of a lane's best entries as (float key, index); entries are
// offered in increasing index order, so a strict > keeps the lower index
// first among equal values.
struct LaneList {
  uint32_t f[TK_L];
  int i[TK_L];
  int n;
  __device__ __forceinline__ void clear() {
    n = 0;
#pragma unroll
    for (int j = 0; j < TK_L; ++j) {
      f[j] = 0u;
      i[j] = -1;
    }
  }
  // Empty slots hold (0, -1); once the new entry has found its place, every
  // later slot takes the entry displaced from the slot before (an empty
  // marker carried into an empty slot changes nothing).
  __device__ __forceinline__ void offer(uint32_t fk, int ix) {
    if (n == TK_L && fk <= f[TK_L - 1]) return;
    uint32_t cf = fk;
    int ci = ix;
    bool shifting = false;
#pragma unroll
    for (int j = 0; j < TK_L; ++j) {
      if (shifting || i[j] < 0 || cf > f[j]) {
        const uint32_t tf = f[j];
        const int ti = i[j];
        f[j] = cf;
        i[j] = ci;
        cf = tf;
        ci = ti;
        shifting = true;
      }
    }
    if (n < TK_L) ++n;
  }
  __device__ __forceinline__ uint64_t head() const {
    return i[0] < 0 ? 0ull : (((uint64_t)f[0] << 32) | (uint64_t)(0xffffffffu - (uint32_t)i[0]));
  }
  __device__ __forceinline__ void pop() {
#pragma unroll
    for (int j = 0; j < TK_L - 1; ++j) {
      f[j] = f[j + 1];
      i[j] = i[j + 1];
    }
    f[TK_L - 1] = 0u;
    i[TK_L - 1] = -1;
    --n;
  }
};

// Gumbel perturbation of the ranking keys (sampled proposals): g(v) =
// -log(-log(u)), u from word v % 4 of Philox counter (row id, v / 4, 0, 1),
// u = ((w >> 41) + 0.5) 2^-23, exactly representable and inside (0, 1).  Adding
// independent Gumbel noise to the logits and keeping the k largest gives k
// draws without replacement from softmax(logits), in draw order (the
// Gumbel-top-k construction).
__device__ __forceinline__ float4 gumbel4(const TopkSample& sm, int row, int v0) {
  uint64_t w[4];
  philox4x64_10(sm.seed, sm.round, (uint64_t)(uint32_t)(sm.row_base + row), (uint64_t)(v0 >> 2), 0, 1, w);
  float g[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float u = ((float)(w[c] >> 41) + 0.5f) * 1.1920928955078125e-07f;  // 2^-23
    g[c] = -logf(-logf(u));
  }
  return make_float4(g[0], g[1], g[2], g[3]);
}

// Entry j*256 + lane*4 + c of a chunk (c < 4): consecutive lanes hold
// consecutive float4s.  Only entries ranking below `below` are offered.
template <int NE>
__device__ __forceinline__ void fill_list(LaneList& L, const float4 (&v)[NE], int base, int end, uint64_t below) {
  L.clear();
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    const int i0 = base + j * 256 + (int)(threadIdx.x & 63) * 4;
    const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (i0 + c < end) {
        const uint32_t fk = float_key(e[c]);
        const uint64_t key = ((uint64_t)fk << 32) | (uint64_t)(0xffffffffu - (uint32_t)(i0 + c));
        if (key < below) L.offer(fk, i0 + c);
      }
    }
  }
}

// grid (chunks, rows), one wave; chunk c covers [c * NE * 256, +NE * 256).
// SAMPLE: the chunk's k best by Gumbel-perturbed logits (lse from the plain ones).
template <int NE, bool SAMPLE>
__global__ void __launch_bounds__(64) topk_chunk_part(const float* __restrict__ logits, int vocab, int k,
                                                     float2* __restrict__ ms_out, uint64_t* __restrict__ keys_out,
                                                     TopkSample sm) {
  const int row = blockIdx.y, c = blockIdx.x, nch = gridDim.x, lane = threadIdx.x;
  const float* x = logits + (size_t)row * vocab;
  const int base = c * NE * 256, end = min(vocab, base + NE * 256);
  float4 v[NE];
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    const int i0 = base + j * 256 + lane * 4;
    v[j] = (i0 < end) ? *(const float4*)(x + i0) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  }
  // (max, sum of exp): padding entries are -inf, which add nothing unless the
  // lane holds nothing else (then its max is -inf and the merge drops it); NaN
  // propagates through the sum; an entry equal to the max counts 1, so +inf
  // gives lse = +inf and a row of -inf gives -inf
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NE; ++j) m = fmaxf(fmaxf(fmaxf(m, v[j].x), v[j].y), fmaxf(v[j].z, v[j].w));
  float s = 0.f;
  auto ex = [&](float t) { return t == m ? 1.f : __expf(t - m); };
#pragma unroll
  for (int j = 0; j < NE; ++j) s += (ex(v[j].x) + ex(v[j].y)) + (ex(v[j].z) + ex(v[j].w));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, WAVE), s2 = __shfl_xor(s, o, WAVE);
    ms_merge(m, s, m2, s2);
  }
  if constexpr (SAMPLE) {  // ranking keys: the perturbed logits (-inf padding stays -inf)
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const int i0 = base + j * 256 + lane * 4;
      const float4 g = gumbel4(sm, row, i0);
      v[j].x += g.x;
      v[j].y += g.y;
      v[j].z += g.z;
      v[j].w += g.w;
    }
  }
  LaneList L;
  fill_list<NE>(L, v, base, end, ~0ull);
  uint64_t mine = 0ull;  // lane r: the chunk's r-th best
  for (int r = 0; r < k; ++r) {
    const uint64_t head = L.head();
    const uint64_t best = wave_max_key(head);
    if (lane == r) mine = best;
    if (head == best && best != 0ull) {
      L.pop();
      if (L.n == 0 && r + 1 < k) fill_list<NE>(L, v, base, end, best);  // used up: refill below `best`
    }
  }
  const size_t o = (size_t)row * nch + c;
  if (lane < k) keys_out[o * TK_KMAX + lane] = mine;
  if (lane == 0) ms_out[o] = make_float2(m, s);
}

// One wave per row: lane c holds chunk c's sorted list.  With sampled keys
// (logits != nullptr) logq is taken from the plain logit of each chosen token.
__global__ void __launch_bounds__(64) topk_chunk_merge(const float2* __restrict__ ms_in,
                                                      const uint64_t* __restrict__ keys_in, int nch, int k, float* lse,
                                                      int32_t* idx, float* logq, const float* __restrict__ logits,
                                                      int vocab) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const size_t o = (size_t)row * nch + lane;
  uint64_t cand[TK_KMAX];
#pragma unroll
  for (int r = 0; r < TK_KMAX; ++r) cand[r] = (lane < nch && r < k) ? keys_in[o * TK_KMAX + r] : 0ull;
  // (max, sum) over chunks in a fixed butterfly order; lanes >= nch hold (-inf, 0)
  float m = -INFINITY, s = 0.f;
  if (lane < nch) {
    const float2 v = ms_in[o];
    m = v.x;
    s = v.y;
  }
#pragma unroll
  for (int w = 32; w > 0; w >>= 1) {
    const float m2 = __shfl_xor(m, w, WAVE), s2 = __shfl_xor(s, w, WAVE);
    ms_merge(m, s, m2, s2);
  }
  uint64_t fin = 0ull;
  for (int r = 0; r < k; ++r) {
    const uint64_t best = wave_max_key(cand[0]);
    if (lane == r) fin = best;
    if (cand[0] == best && best != 0ull) {
#pragma unroll
      for (int j = 0; j < TK_KMAX - 1; ++j) cand[j] = cand[j + 1];
      cand[TK_KMAX - 1] = 0ull;
    }
  }
  const float l = __shfl(m, 0, WAVE) + __logf(__shfl(s, 0, WAVE));
  if (lane == 0) lse[row] = l;
  if (lane < k) {
    const uint32_t t = key_index(fin);
    idx[(size_t)row * k + lane] = (int32_t)t;
    const bool raw = logits != nullptr && t < (uint32_t)vocab;  // an empty key (0) names no token
    logq[(size_t)row * k + lane] = (raw ? logits[(size_t)row * vocab + t] : key_value(fin)) - l;
  }
}

// float4s per lane: as few as keep a row within max(16, 4096 / rows) chunks
// (64 at most), so a launch has a few thousand waves; 0 when a row does not
// fit in 64 chunks of 32 float4s per lane.
int topk_ne(int n_rows, int vocab) {
  int target = 4096 / (n_rows > 0 ? n_rows : 1);
  target = target < 16 ? 16 : target > TK_CHUNKS ? TK_CHUNKS : target;
  for (int ne = 1; ne <= 32; ne *= 2)
    if ((vocab + ne * 256 - 1) / (ne * 256) <= target) return ne;
  for (int ne = 1; ne <= 32; ne *= 2)
    if ((vocab + ne * 256 - 1) / (ne * 256) <= TK_CHUNKS) return ne;
  return 0;
}

int topk_chunk(int n_rows, int vocab) {
  int target = (4096 + n_rows - 1) / n_rows;
  if (target > 64) target = 64;
  if (target < 1) target = 1;
  int chunk = (vocab + target - 1) / target;
  chunk = (chunk + 1023) / 1024 * 1024;
  return chunk;
}

}  // namespace

size_t topk_workspace_bytes(int n_rows, int vocab) {
  const int chunk = topk_chunk(n_rows, vocab);
  const int nchunks = (vocab + chunk - 1) / chunk;
  const size_t generic = (size_t)n_rows * nchunks * (sizeof(float2) + 16 * sizeof(uint64_t)) + 256;
  const size_t chunked = (size_t)n_rows * TK_CHUNKS * (sizeof(float2) + TK_KMAX * sizeof(uint64_t)) + 512;
  return generic > chunked ? generic : chunked;
}

template <bool SAMPLE>
void launch_chunk_part(int ne, dim3 g, dim3 b, hipStream_t s, const float* logits, int vocab, int k, float2* cms,
                       uint64_t* ckeys, const TopkSample& sm) {
  switch (ne) {
    case 1: hipLaunchKernelGGL((topk_chunk_part<1, SAMPLE>), g, b, 0, s, logits, vocab, k, cms, ckeys, sm); break;
    case 2: hipLaunchKernelGGL((topk_chunk_part<2, SAMPLE>), g, b, 0, s, logits, vocab, k, cms, ckeys, sm); break;
    case 4: hipLaunchKernelGGL((topk_chunk_part<4, SAMPLE>), g, b, 0, s, logits, vocab, k, cms, ckeys, sm); break;
    case 8: hipLaunchKernelGGL((topk_chunk_part<8, SAMPLE>), g, b, 0, s, logits, vocab, k, cms, ckeys, sm); break;
    case 16: hipLaunchKernelGGL((topk_chunk_part<16, SAMPLE>), g, b, 0, s, logits, vocab, k, cms, ckeys, sm); break;
    default: hipLaunchKernelGGL((topk_chunk_part<32, SAMPLE>), g, b, 0, s, logits, vocab, k, cms, ckeys, sm); break;
  }
}

hipError_t launch_softmax_topk(int n_rows, int vocab, const float* logits, int k, float* lse, int32_t* idx,
                               float* logq, void* ws, hipStream_t s, const TopkSample* smp) {
  if (n_rows == 0) return hipSuccess;
  const int ne = topk_ne(n_rows, vocab);
  if (smp && ne == 0) return hipErrorInvalidValue;  // sampled keys: chunked pass only
  if (ne > 0) {
    const int nch = (vocab + ne * 256 - 1) / (ne * 256);
    float2* cms = (float2*)ws;
    uint64_t* ckeys = (uint64_t*)((char*)ws + (((size_t)n_rows * TK_CHUNKS * sizeof(float2) + 255) / 256) * 256);
    const dim3 g(nch, n_rows), b(64);
    if (smp)
      launch_chunk_part<true>(ne, g, b, s, logits, vocab, k, cms, ckeys, *smp);
    else
      launch_chunk_part<false>(ne, g, b, s, logits, vocab, k, cms, ckeys, TopkSample{0, 0, 0});
    hipLaunchKernelGGL(topk_chunk_merge, dim3(n_rows), b, 0, s, cms, ckeys, nch, k, lse, idx, logq,
                       smp ? logits : (const float*)nullptr, vocab);
    return hipGetLastError();
  }
  const int chunk = topk_chunk(n_rows, vocab);
  const int nchunks = (vocab + chunk - 1) / chunk;
  float2* ms = (float2*)ws;
  uint64_t* keys = (uint64_t*)((char*)ws + (((size_t)n_rows * nchunks * sizeof(float2) + 255) / 256) * 256);
  dim3 g1(nchunks, n_rows);
  if (k <= 4) {
    hipLaunchKernelGGL(topk_partial<4>, g1, dim3(256), 0, s, logits, vocab, chunk, k, ms, keys);
    hipLaunchKernelGGL(topk_merge<4>, dim3(n_rows), dim3(64), 0, s, ms, keys, nchunks, k, lse, idx, logq);
  } else {
    hipLaunchKernelGGL(topk_partial<16>, g1, dim3(256), 0, s, logits, vocab, chunk, k, ms, keys);
    hipLaunchKernelGGL(topk_merge<16>, dim3(n_rows), dim3(64), 0, s, ms, keys, nchunks, k, lse, idx, logq);
  }
  return hipGetLastError();
}
