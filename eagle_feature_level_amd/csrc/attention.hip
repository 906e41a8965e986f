// Rotary embedding + tree-slot write, and tree attention for the draft layer.
//
// Tree attention: a drafted node attends to the prefix KV and to its own tree
// ancestors and itself only ("eagle feature-level speculative decoding",
// tree-attention section: M_uv = 0 iff v is an ancestor of u or v = u).  The
// visible tree slots of a row are a 64-bit mask.
//
// Layout of the work: one workgroup per (key split, kv head, sequence).  All
// query rows of that sequence and all query heads sharing the kv head read the
// same K/V tiles, so each prefix K/V tile is fetched from HBM once per call and
// staged in LDS (64 keys per tile).  The last split handles the 64 tree slots
// as one masked tile.  Each split writes (max, sum, unnormalised output)
// per query; attn_combine merges the splits with the usual log-sum-exp rule.
// Inside a workgroup, lane j of each wave owns key j of the tile for the
// scores; a wave owns a quarter of the query chunk, so the softmax statistics
// are plain wave reductions.
#include "common.h"
#include "kernels.h"

namespace {

template <typename T>
__device__ __forceinline__ float ld1(const T* p);
template <>
__device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld1<bf16_t>(const bf16_t* p) { return bf2f(*p); }

// eight consecutive elements (16-byte aligned for bf16, 32-byte for fp32) as fp32
template <typename T>
__device__ __forceinline__ void ld8(const T* p, float* f);
template <>
__device__ __forceinline__ void ld8<bf16_t>(const bf16_t* p, float* f) {
  const u32x4 v = *(const u32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void ld8<float>(const float* p, float* f) {
  const float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

template <typename T>
__device__ __forceinline__ void st1(T* p, float v);
template <>
__device__ __forceinline__ void st1<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void st1<bf16_t>(bf16_t* p, float v) { *p = f2bf(v); }

// qkv fp32 [M, (Hq + 2 Hkv) hd] -> rotated q (fp32) [M, Hq hd]; rotated k and v
// into tree slots in the KV cache's element type T.
template <typename T>
__global__ void __launch_bounds__(256) rope_kv_kernel(RopeArgs a) {
  const int r = blockIdx.x;
  const int hd = a.hd, half = hd / 2;
  const int nqkv = (a.hq + 2 * a.hkv) * hd;
  const float* src = a.qkv + (size_t)r * nqkv;
  const int pos = a.pos[r];
  const int b = a.seq_of_row ? a.seq_of_row[r] : 0;
  const int slot = a.slot[r];
  T* tk = (T*)a.tree_k + (((size_t)b * 64 + slot) * a.hkv) * hd;
  T* tv = (T*)a.tree_v + (((size_t)b * 64 + slot) * a.hkv) * hd;
  float* qo = a.q_out + (size_t)r * a.hq * hd;
  const int npairs = (a.hq + a.hkv) * half;
  for (int i = threadIdx.x; i < npairs; i += blockDim.x) {
    const int h = i / half, e = i % half;
    const double inv = exp2(-2.0 * (double)e / (double)hd * log2((double)a.theta));
    double sd, cd;
    sincos((double)pos * inv, &sd, &cd);
    const float c = (float)cd, s = (float)sd;
    const float* v = src + h * hd;
    const float x0 = v[e], x1 = v[e + half];
    const float y0 = x0 * c - x1 * s, y1 = x1 * c + x0 * s;
    if (h < a.hq) {
      qo[h * hd + e] = y0;
      qo[h * hd + e + half] = y1;
    } else {
      const int g = h - a.hq;
      st1<T>(tk + g * hd + e, y0);
      st1<T>(tk + g * hd + e + half, y1);
    }
  }
  const float* vs = src + (a.hq + a.hkv) * hd;
  for (int i = threadIdx.x; i < a.hkv * hd; i += blockDim.x) st1<T>(tv + i, vs[i]);
}

constexpr int KT = 64;  // keys per tile
constexpr int QC = 16;  // queries per chunk (4 per wave)
constexpr int QPW = QC / 4;

template <typename T, int HD>
__global__ void __launch_bounds__(256) attn_partial_kernel(AttnArgs a) {
  constexpr int KPAD = (sizeof(T) == 2) ? 8 : 4;
  constexpr int LW = HD + KPAD;  // padded LDS row, elements
  __shared__ __attribute__((aligned(16))) T ks[KT][LW];
  __shared__ __attribute__((aligned(16))) T vsm[KT][LW];
  __shared__ __attribute__((aligned(16))) float qs[QC][HD];
  __shared__ __attribute__((aligned(16))) float ps[QC][KT];
  __shared__ uint64_t qmask[QC];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int G = a.hq / a.hkv;
  const int r0 = a.row_start[b], nr = a.row_start[b + 1] - r0;
  const int nq = nr * G;
  const int L = a.prefix_len[b];
  // splits 0 .. n_splits-2 cover the prefix; the last split is the tree block
  const bool do_tree = (s == a.n_splits - 1);
  const int kbeg = do_tree ? 0 : s * a.split_len;
  const int kend = do_tree ? 0 : min(L, kbeg + a.split_len);
  const T* pk = (const T*)a.prefix_k + a.prefix_off[b] + (size_t)g * L * HD;
  const T* pv = (const T*)a.prefix_v + a.prefix_off[b] + (size_t)g * L * HD;
  const T* tk = (const T*)a.tree_k + ((size_t)b * 64 * a.hkv + g) * HD;  // slot stride hkv*HD
  const T* tv = (const T*)a.tree_v + ((size_t)b * 64 * a.hkv + g) * HD;
  const float scale = rsqrtf((float)HD);
  constexpr int DPL = HD / 64 > 0 ? HD / 64 : 1;  // output dims per lane
  const bool lane_dims = lane * DPL < HD;

  for (int qc0 = 0; qc0 < nq; qc0 += QC) {
    // queries of this chunk: q index qi -> row r0 + qi / G, head g*G + qi % G
    __syncthreads();
    for (int i = threadIdx.x; i < QC * HD; i += 256) {
      const int qq = i / HD, dd = i % HD;
      const int qi = qc0 + qq;
      float v = 0.f;
      if (qi < nq) {
        const int row = r0 + qi / G, h = g * G + qi % G;
        v = a.q[((size_t)row * a.hq + h) * HD + dd] * scale;
      }
      qs[qq][dd] = v;
    }
    if (threadIdx.x < QC) {
      const int qi = qc0 + threadIdx.x;
      qmask[threadIdx.x] = (qi < nq) ? a.mask[r0 + qi / G] : 0ull;
    }
    __syncthreads();
    uint64_t umask = 0;
#pragma unroll
    for (int i = 0; i < QC; ++i) umask |= qmask[i];

    float m_run[QPW], l_run[QPW], o[QPW][DPL];
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      m_run[i] = -INFINITY;
      l_run[i] = 0.f;
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) o[i][dd] = 0.f;
    }

    const int n_prefix_tiles = (kend > kbeg) ? (kend - kbeg + KT - 1) / KT : 0;
    const int n_tiles = n_prefix_tiles + (do_tree ? 1 : 0);
    for (int t = 0; t < n_tiles; ++t) {
      const bool tree_tile = (t == n_prefix_tiles);
      const int k0 = kbeg + t * KT;
      const int tlen = tree_tile ? KT : min(KT, kend - k0);
      __syncthreads();
      // stage K and V of the tile (zeros where no key)
      constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
      for (int i = threadIdx.x; i < KT * (HD / EPV); i += 256) {
        const int j = i / (HD / EPV), dd = (i % (HD / EPV)) * EPV;
        u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
        if (tree_tile) {
          if ((umask >> j) & 1ull) {
            kv = *(const u32x4*)(tk + (size_t)j * a.hkv * HD + dd);
            vv = *(const u32x4*)(tv + (size_t)j * a.hkv * HD + dd);
          }
        } else if (j < tlen) {
          kv = *(const u32x4*)(pk + (size_t)(k0 + j) * HD + dd);
          vv = *(const u32x4*)(pv + (size_t)(k0 + j) * HD + dd);
        }
        *(u32x4*)&ks[j][dd] = kv;
        *(u32x4*)&vsm[j][dd] = vv;
      }
      __syncthreads();
      // scores: lane j = key, this wave's queries wv, wv+4, ...
      float sc[QPW];
#pragma unroll
      for (int i = 0; i < QPW; ++i) sc[i] = 0.f;
      for (int d0 = 0; d0 < HD; d0 += 8) {
        float kd[8];
        ld8<T>(&ks[lane][d0], kd);
#pragma unroll
        for (int i = 0; i < QPW; ++i) {
          float qd[8];
          ld8<float>(&qs[wv + 4 * i][d0], qd);
#pragma unroll
          for (int e = 0; e < 8; ++e) sc[i] += qd[e] * kd[e];
        }
      }
#pragma unroll
      for (int i = 0; i < QPW; ++i) {
        const int qq = wv + 4 * i;
        bool valid = tree_tile ? ((qmask[qq] >> lane) & 1ull) : (lane < tlen);
        if (qc0 + qq >= nq) valid = false;
        const float sv = valid ? sc[i] : -INFINITY;
        const float tmax = wave_max(sv);
        const float mnew = fmaxf(m_run[i], tmax);
        const float p = (valid && mnew > -INFINITY) ? __expf(sv - mnew) : 0.f;
        const float alpha = (m_run[i] > -INFINITY) ? __expf(m_run[i] - mnew) : 0.f;
        l_run[i] = l_run[i] * alpha + wave_sum(p);
        m_run[i] = mnew;
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) o[i][dd] *= alpha;
        ps[qq][lane] = p;
      }
      __syncthreads();
      if (lane_dims) {
        for (int j0 = 0; j0 < KT; j0 += 4) {
          float vj[4][DPL];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int dd = 0; dd < DPL; ++dd) vj[jj][dd] = ld1<T>(&vsm[j0 + jj][lane * DPL + dd]);
#pragma unroll
          for (int i = 0; i < QPW; ++i) {
            const float4 p4 = *(const float4*)&ps[wv + 4 * i][j0];
#pragma unroll
            for (int dd = 0; dd < DPL; ++dd)
              o[i][dd] += p4.x * vj[0][dd] + p4.y * vj[1][dd] + p4.z * vj[2][dd] + p4.w * vj[3][dd];
          }
        }
      }
    }
    // write this split's partial results
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int qi = qc0 + wv + 4 * i;
      if (qi >= nq) continue;
      const int row = r0 + qi / G, h = g * G + qi % G;
      float* dst = a.part + (((size_t)s * a.n_rows + row) * a.hq + h) * (HD + 2);
      if (lane_dims) {
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) dst[2 + lane * DPL + dd] = o[i][dd];
      }
      if (lane == 0) {
        dst[0] = m_run[i];
        dst[1] = l_run[i];
      }
    }
  }
}

// Merge split partials: out[row, h*hd + d] (fp32) = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
// One workgroup per (row, head); the split weights are computed once in LDS.
__global__ void __launch_bounds__(128) attn_combine_kernel(AttnArgs a, int hd) {
  __shared__ float wsplit[1024];
  __shared__ float s_inv;
  const int row = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const size_t stride = (size_t)a.n_rows * a.hq * (hd + 2);
  const float* base = a.part + ((size_t)row * a.hq + h) * (hd + 2);
  if (t < WAVE) {
    float M = -INFINITY;
    for (int s = t; s < a.n_splits; s += WAVE) M = fmaxf(M, base[s * stride]);
    M = wave_max(M);
    float L = 0.f;
    for (int s = t; s < a.n_splits; s += WAVE) {
      const float m = base[s * stride];
      const float w = (m == -INFINITY) ? 0.f : __expf(m - M);
      wsplit[s] = w;
      L += w * base[s * stride + 1];
    }
    L = wave_sum(L);
    if (t == 0) s_inv = 1.f / L;
  }
  __syncthreads();
  for (int dd = t; dd < hd; dd += 128) {
    float acc = 0.f;
    for (int s = 0; s < a.n_splits; ++s) acc += wsplit[s] * base[s * stride + 2 + dd];
    a.out[((size_t)row * a.hq + h) * hd + dd] = acc * s_inv;
  }
}

}  // namespace

hipError_t launch_rope_kv(const RopeArgs& a, bool bf16, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(rope_kv_kernel<bf16_t>, dim3(a.n_rows), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(rope_kv_kernel<float>, dim3(a.n_rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

int attn_split_len(int max_prefix, int batch, int hkv) {
  // aim for ~2048 workgroups; splits are multiples of the 64-key tile
  const long want = 2048;
  long per = (long)batch * hkv;
  int split_len = KT;
  while ((long)((max_prefix + split_len - 1) / split_len) * per > want && split_len < (1 << 20)) split_len *= 2;
  return split_len;
}

// prefix splits plus one split for the tree block
int attn_n_splits(int max_prefix, int split_len) { return (max_prefix + split_len - 1) / split_len + 1; }

hipError_t launch_attention(const AttnArgs& a, bool bf16, int hd, hipStream_t s) {
  if (a.n_splits > 1024) return hipErrorInvalidValue;  // combine keeps one weight per split in LDS
  dim3 grid(a.n_splits, a.hkv, a.batch), blk(256);
  if (bf16) {
    if (hd != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_partial_kernel<bf16_t, 128>), grid, blk, 0, s, a);
  } else {
    if (hd == 16)
      hipLaunchKernelGGL((attn_partial_kernel<float, 16>), grid, blk, 0, s, a);
    else if (hd == 64)
      hipLaunchKernelGGL((attn_partial_kernel<float, 64>), grid, blk, 0, s, a);
    else if (hd == 128)
      hipLaunchKernelGGL((attn_partial_kernel<float, 128>), grid, blk, 0, s, a);
    else
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.n_rows, a.hq), dim3(128), 0, s, a, hd);
  return hipGetLastError();
}
