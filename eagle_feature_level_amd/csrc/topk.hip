// Softmax normaliser + per-row top-k over the vocabulary.
//
// EAGLE-2 ranks a node's children by the draft confidence (the softmax
// probability) and multiplies confidences along paths ("EAGLE 推测解码为什么比
// Medusa 快" section 10.3); this kernel gives, per logits row, lse and the top-k
// tokens with logq = logit - lse.  Ranking key: (value desc, index asc), one
// 64-bit integer per entry so every comparison is exact.
//
// Pass 1 (grid chunks x rows): each thread streams float4s of its chunk,
// keeping an online (max, sum of exp) and a sorted top-K list in registers;
// the workgroup merges lists by K rounds of a wave-wide 64-bit max.
// Pass 2 (one wave per row): merges the chunks in a fixed order.
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
  return (size_t)n_rows * nchunks * (sizeof(float2) + 16 * sizeof(uint64_t)) + 256;
}

hipError_t launch_softmax_topk(int n_rows, int vocab, const float* logits, int k, float* lse, int32_t* idx,
                               float* logq, void* ws, hipStream_t s) {
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
