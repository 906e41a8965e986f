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
// into tree slots in the KV cache's element type T.  grid (rows, ceil((Hq +
// 2 Hkv) / 4)): a block takes four heads of one row from the list [q heads, k
// heads, v heads].  The rotation angles pos * theta^(-2e/hd) depend only on
// the row's position and the pair index e: computed once per block (fp64, so a
// position in the thousands keeps its phase exact to fp32), then shared.
constexpr int ROPE_HPB = 4;

template <typename T>
__global__ void __launch_bounds__(256) rope_kv_kernel(RopeArgs a) {
  __shared__ float cs[64], sn[64];
  __shared__ int s_b;
  const int r = blockIdx.x;
  const int hd = a.hd, half = hd / 2;
  const int nheads = a.hq + 2 * a.hkv;
  const int h0 = blockIdx.y * ROPE_HPB;
  const float* src = a.qkv + (size_t)r * nheads * hd;
  // the row's sequence: the one b with row_start[b] <= r < row_start[b+1]
  if (threadIdx.x == 0) s_b = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < a.batch; i += blockDim.x)
    if (a.row_start[i] <= r && r < a.row_start[i + 1]) s_b = i;
  __syncthreads();
  const int b = s_b;
  const int slot = a.slot[r];
  T* tk = (T*)a.tree_k + (((size_t)b * 64 + slot) * a.hkv) * hd;
  T* tv = (T*)a.tree_v + (((size_t)b * 64 + slot) * a.hkv) * hd;
  float* qo = a.q_out + (size_t)r * a.hq * hd;
  if (h0 < a.hq + a.hkv) {  // this block rotates something
    const int pos = a.pos[r];
    for (int e = threadIdx.x; e < half; e += blockDim.x) {
      const double inv = exp2(-2.0 * (double)e / (double)hd * log2((double)a.theta));
      double sd, cd;
      sincos((double)pos * inv, &sd, &cd);
      cs[e] = (float)cd;
      sn[e] = (float)sd;
    }
    __syncthreads();
  }
  const int hend = min(h0 + ROPE_HPB, nheads);
  for (int i = threadIdx.x; i < (hend - h0) * half; i += blockDim.x) {
    const int h = h0 + i / half, e = i % half;
    const float* v = src + (size_t)h * hd;
    if (h < a.hq + a.hkv) {
      const float c = cs[e], sv = sn[e];
      const float x0 = v[e], x1 = v[e + half];
      const float y0 = x0 * c - x1 * sv, y1 = x1 * c + x0 * sv;
      if (h < a.hq) {
        qo[h * hd + e] = y0;
        qo[h * hd + e + half] = y1;
      } else {
        const int g = h - a.hq;
        st1<T>(tk + g * hd + e, y0);
        st1<T>(tk + g * hd + e + half, y1);
      }
    } else {
      const int g = h - a.hq - a.hkv;
      st1<T>(tv + g * hd + e, v[e]);
      st1<T>(tv + g * hd + e + half, v[e + half]);
    }
  }
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
  const int C = a.prefix_cap ? a.prefix_cap[b] : L;  // per-head stride
  const T* pk = (const T*)a.prefix_k + a.prefix_off[b] + (size_t)g * C * HD;
  const T* pv = (const T*)a.prefix_v + a.prefix_off[b] + (size_t)g * C * HD;
  const T* tk = (const T*)a.tree_k + ((size_t)b * 64 * a.hkv + g) * HD;  // slot stride hkv*HD
  const T* tv = (const T*)a.tree_v + ((size_t)b * 64 * a.hkv + g) * HD;
  const float scale = rsqrtf((float)HD);
  constexpr int DPL = HD / 64 > 0 ? HD / 64 : 1;  // output dims per lane
  const bool lane_dims = lane * DPL < HD;

  // K/V tile staging: every load of a tile is issued before any LDS store, and
  // the next tile's loads are in flight while the current tile is used.
  constexpr int EPV = 16 / sizeof(T);            // elements per 16-byte vector
  constexpr int KVI = KT * (HD / EPV) / 256;     // vectors per thread per tile
  constexpr int QE = QC * HD / 256;              // query elements per thread
  static_assert(KVI >= 1 && QE >= 1, "tile shapes");
  u32x4 kr[KVI], vr[KVI];

  for (int qc0 = 0; qc0 < nq; qc0 += QC) {
    // queries of this chunk: q index qi -> row r0 + qi / G, head g*G + qi % G
    __syncthreads();
    {
      float qv[QE];
#pragma unroll
      for (int j = 0; j < QE; ++j) {
        const int i = threadIdx.x + j * 256;
        const int qq = i / HD, dd = i % HD;
        const int qi = qc0 + qq;
        qv[j] = 0.f;
        if (qi < nq) {
          const int row = r0 + qi / G, h = g * G + qi % G;
          qv[j] = a.q[((size_t)row * a.hq + h) * HD + dd] * scale;
        }
      }
#pragma unroll
      for (int j = 0; j < QE; ++j) {
        const int i = threadIdx.x + j * 256;
        qs[i / HD][i % HD] = qv[j];
      }
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
    // K and V of tile t into registers (zeros where no key)
    auto load_tile = [&](int t) {
      const bool tree_tile = (t == n_prefix_tiles);
      const int k0 = kbeg + t * KT;
      const int tlen = tree_tile ? KT : min(KT, kend - k0);
#pragma unroll
      for (int u = 0; u < KVI; ++u) {
        const int i = threadIdx.x + u * 256;
        const int j = i / (HD / EPV), dd = (i % (HD / EPV)) * EPV;
        kr[u] = u32x4{0, 0, 0, 0};
        vr[u] = u32x4{0, 0, 0, 0};
        if (tree_tile) {
          if ((umask >> j) & 1ull) {
            kr[u] = *(const u32x4*)(tk + (size_t)j * a.hkv * HD + dd);
            vr[u] = *(const u32x4*)(tv + (size_t)j * a.hkv * HD + dd);
          }
        } else if (j < tlen) {
          kr[u] = *(const u32x4*)(pk + (size_t)(k0 + j) * HD + dd);
          vr[u] = *(const u32x4*)(pv + (size_t)(k0 + j) * HD + dd);
        }
      }
    };
    if (n_tiles > 0) load_tile(0);
    for (int t = 0; t < n_tiles; ++t) {
      const bool tree_tile = (t == n_prefix_tiles);
      const int k0 = kbeg + t * KT;
      const int tlen = tree_tile ? KT : min(KT, kend - k0);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < KVI; ++u) {
        const int i = threadIdx.x + u * 256;
        const int j = i / (HD / EPV), dd = (i % (HD / EPV)) * EPV;
        *(u32x4*)&ks[j][dd] = kr[u];
        *(u32x4*)&vsm[j][dd] = vr[u];
      }
      __syncthreads();
      if (t + 1 < n_tiles) load_tile(t + 1);
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
// Up to CMB_PRE splits, a thread loads its output element's partial from every
// split at the start, beside the statistics (one round of independent loads
// instead of the statistics and then the values); the sum runs in split order
// either way.
constexpr int CMB_PRE = 16;

__global__ void __launch_bounds__(128) attn_combine_kernel(AttnArgs a, int hd) {
  __shared__ float wsplit[1024];
  __shared__ float s_inv;
  const int row = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const size_t stride = (size_t)a.n_rows * a.hq * (hd + 2);
  const float* base = a.part + ((size_t)row * a.hq + h) * (hd + 2);
  const bool pre = a.n_splits <= CMB_PRE && hd <= 128;  // uniform
  float v[CMB_PRE];
  if (pre) {
#pragma unroll
    for (int s = 0; s < CMB_PRE; ++s) v[s] = (s < a.n_splits && t < hd) ? base[s * stride + 2 + t] : 0.f;
  }
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
  if (pre) {
    if (t < hd) {
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < CMB_PRE; ++s)
        if (s < a.n_splits) acc += wsplit[s] * v[s];
      const size_t o = ((size_t)row * a.hq + h) * hd + t;
      if (a.outb)
        put_split1((bf16_t*)a.outb + o, (size_t)a.n_rows * a.hq * hd, acc * s_inv);
      else
        a.out[o] = acc * s_inv;
    }
    return;
  }
  for (int dd = t; dd < hd; dd += 128) {
    float acc = 0.f;
    for (int s = 0; s < a.n_splits; ++s) acc += wsplit[s] * base[s * stride + 2 + dd];
    const size_t o = ((size_t)row * a.hq + h) * hd + dd;
    if (a.outb)
      put_split1((bf16_t*)a.outb + o, (size_t)a.n_rows * a.hq * hd, acc * s_inv);
    else
      a.out[o] = acc * s_inv;
  }
}


// ---------------------------------------------------------------------------
// Tree attention on the matrix units: bf16 K/V cache, head_dim 128.
//
// One workgroup = (key split, kv head and query block, sequence); 4 waves x 16
// queries.  Per 64-key tile:
//   S^T = K Q^T   (v_mfma_f32_16x16x32_bf16; A = K rows from LDS, B = the
//                  wave's queries, held in registers as bf16 hi/lo pairs)
//   online softmax per query over the tile (fp32, exp of s - running max)
//   O^T += V^T P^T  (A = V^T from a transposed LDS tile, B = P^T straight from
//                  the S^T accumulators: the MFMA sums over keys, so the keys of
//                  a lane's accumulator block may stand in any order as long as
//                  the V^T rows use the same order)
// The next tile's K and V are loaded into registers while the current one is
// used.  The 64 tree slots ride with the last split as one more tile, masked
// per query by its row's ancestor bitmask (a split of their own when few
// groups share the chip).  With one split the normalised output is written
// directly; otherwise (max, sum, unnormalised output) per split goes to
// attn_combine_kernel.  (Merging the splits in the last workgroup to finish
// needs a device-scope release and acquire per workgroup; on this chip those
// write back and invalidate the whole L2 of the XCD and cost several times
// the separate launch.)
// ---------------------------------------------------------------------------
constexpr int AQ = 64;          // queries per workgroup
constexpr int AKROW = 128 + 8;  // K tile row (bf16): 272 B, rows land 4 banks apart
constexpr int AVROW = KT + 8;   // transposed V tile row (bf16): 144 B, 16-byte aligned

// Transposed V tile, row d = one dim.  Keys are stored in the order the PV
// MFMA consumes them: lane group gq of 32-key chunk kc takes keys
// kc*32 + 4gq + {0..3} and kc*32 + 16 + 4gq + {0..3}, so 4-key group k' (keys
// 4k'..4k'+3) sits at slot (k'/8)*8 + (k'%4)*2 + (k'/4)%2 (4 keys per slot)
// and a lane's 8 keys are one 16-byte read.
__device__ __forceinline__ int vt_col(int key4) { return ((key4 >> 3) * 8 + (key4 & 3) * 2 + ((key4 >> 2) & 1)) << 2; }

__device__ __forceinline__ floatx4 mfma16a(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Two fp32 values as packed bf16 (a in the low half): hi = cut to bf16 (exact
// remainder), lo = remainder rounded, ties away from zero.
__device__ __forceinline__ uint32_t asplit2(float a, float b, uint32_t* lo) {
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  const float ra = a - __uint_as_float(ua & 0xffff0000u), rb = b - __uint_as_float(ub & 0xffff0000u);
  *lo = __builtin_amdgcn_perm(__float_as_uint(rb) + 0x8000u, __float_as_uint(ra) + 0x8000u, 0x07060302u);
  return __builtin_amdgcn_perm(ub, ua, 0x07060302u);
}

template <bool KSPLIT>
__global__ void __launch_bounds__(256, KSPLIT ? 3 : 2) attn_mfma_kernel(AttnArgs a) {
  // K tile and transposed V tile; with KSPLIT the space then holds the four
  // waves' partial results for the merge
  constexpr int KS_BYTES = KT * AKROW * 2, VT_BYTES = 128 * AVROW * 2;
  static_assert(KS_BYTES + VT_BYTES >= 4 * 16 * (128 + 2) * 4, "merge space");
  __shared__ __attribute__((aligned(16))) unsigned char smem[KS_BYTES + VT_BYTES];
  bf16_t(*ks)[AKROW] = reinterpret_cast<bf16_t(*)[AKROW]>(smem);
  bf16_t(*vt)[AVROW] = reinterpret_cast<bf16_t(*)[AVROW]>(smem + KS_BYTES);
  __shared__ unsigned long long umask_s;
  // KSPLIT: the B operand of S^T (the same 16 queries in every wave), one copy
  __shared__ __attribute__((aligned(16))) u32x4 qf[KSPLIT ? 4 : 1][2][64];
  constexpr int QPB = KSPLIT ? 16 : AQ;  // queries per workgroup
  const int s = blockIdx.x;
  const int g = blockIdx.y % a.hkv, qb = blockIdx.y / a.hkv;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = lane & 15, gq = lane >> 4;
  const int G = a.hq / a.hkv;
  const int r0 = a.row_start[b], nr = a.row_start[b + 1] - r0;
  const int nq = nr * G;
  if (qb * QPB >= nq) return;  // whole workgroup: no queries in this block
  const int L = a.prefix_len[b];
  const int kbeg = s * a.split_len;
  const int kend = min(L, kbeg + a.split_len);
  const bool with_tree = (s == a.n_splits - 1);
  const int n_prefix_tiles = (kend > kbeg) ? (kend - kbeg + KT - 1) / KT : 0;
  const int n_tiles = n_prefix_tiles + (with_tree ? 1 : 0);
  const int C = a.prefix_cap ? a.prefix_cap[b] : L;  // per-head stride
  const bf16_t* pk = (const bf16_t*)a.prefix_k + a.prefix_off[b] + (size_t)g * C * 128;
  const bf16_t* pv = (const bf16_t*)a.prefix_v + a.prefix_off[b] + (size_t)g * C * 128;
  const bf16_t* tk = (const bf16_t*)a.tree_k + ((size_t)b * 64 * a.hkv + g) * 128;  // slot stride hkv*128
  const bf16_t* tv = (const bf16_t*)a.tree_v + ((size_t)b * 64 * a.hkv + g) * 128;

  // tile staging: thread t holds keys skey..skey+3, dims sdim..sdim+7 of K (16
  // lanes cover a key row) and keys vkey..vkey+3, dims vdim..vdim+7 of V (16
  // lanes cover one dim of 64 keys, so each transposed V row is written as one
  // contiguous 128-byte span)
  const int skey = (threadIdx.x >> 4) * 4, sdim = (threadIdx.x & 15) * 8;
  const int vkey = (threadIdx.x & 15) * 4, vdim = (threadIdx.x >> 4) * 8;
  u32x4 kr[4], vr[4];
  const bf16_t* pk0 = pk + (size_t)(kbeg + skey) * 128 + sdim;  // this thread's first key row
  const bf16_t* pv0 = pv + (size_t)(kbeg + vkey) * 128 + vdim;
  auto load_prefix_tile = [&](int t) {
    const int tlen = min(KT, kend - (kbeg + t * KT));
    const bf16_t* k1 = pk0 + (size_t)t * KT * 128;
    const bf16_t* v1 = pv0 + (size_t)t * KT * 128;
    if (tlen == KT) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kr[u] = *(const u32x4*)(k1 + u * 128);
        vr[u] = *(const u32x4*)(v1 + u * 128);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kr[u] = (skey + u < tlen) ? *(const u32x4*)(k1 + u * 128) : u32x4{0, 0, 0, 0};
        vr[u] = (vkey + u < tlen) ? *(const u32x4*)(v1 + u * 128) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto load_tree_tile = [&](uint64_t um) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = skey + u, jv = vkey + u;
      kr[u] = ((um >> j) & 1ull) ? *(const u32x4*)(tk + (size_t)j * a.hkv * 128 + sdim) : u32x4{0, 0, 0, 0};
      vr[u] = ((um >> jv) & 1ull) ? *(const u32x4*)(tv + (size_t)jv * a.hkv * 128 + vdim) : u32x4{0, 0, 0, 0};
    }
  };
  // the first prefix tile does not depend on anything below: start it now
  if (n_prefix_tiles > 0) load_prefix_tile(0);

  // tree slots any row of this sequence may see (only those are loaded)
  if (threadIdx.x == 0) umask_s = 0ull;
  __syncthreads();
  if (with_tree)
    for (int t = threadIdx.x; t < nr; t += 256) atomicOr(&umask_s, (unsigned long long)a.mask[r0 + t]);

  // this lane's query: q = qb*64 + wv*16 + c (KSPLIT: qb*16 + c, the same in
  // every wave) -> row r0 + q/G, head g*G + q%G
  const int qi = KSPLIT ? qb * 16 + c : qb * AQ + wv * 16 + c;
  const bool qv = qi < nq;
  const int row = r0 + (qv ? qi / G : 0);
  const int h = g * G + (qv ? qi % G : 0);
  const uint64_t qmask = qv ? a.mask[row] : 0ull;
  u32x4 qh[4], ql[4];  // B operand: lane (query c, group gq) holds dims dc*32 + gq*8 + i
  {
    const float* qp = a.q + ((size_t)row * a.hq + h) * 128;
    // scores come out in log2 units: softmax weights are then plain 2^x
    const float sc = rsqrtf(128.f) * 1.4426950408889634f;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
      if (qv) {
        v0 = *(const float4*)(qp + dc * 32 + gq * 8);
        v1 = *(const float4*)(qp + dc * 32 + gq * 8 + 4);
      }
      uint32_t l;
      qh[dc][0] = asplit2(v0.x * sc, v0.y * sc, &l); ql[dc][0] = l;
      qh[dc][1] = asplit2(v0.z * sc, v0.w * sc, &l); ql[dc][1] = l;
      qh[dc][2] = asplit2(v1.x * sc, v1.y * sc, &l); ql[dc][2] = l;
      qh[dc][3] = asplit2(v1.z * sc, v1.w * sc, &l); ql[dc][3] = l;
    }
    if constexpr (KSPLIT) {
      if (wv == 0) {
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
          qf[dc][0][lane] = qh[dc];
          qf[dc][1][lane] = ql[dc];
        }
      }
    }
  }
  __syncthreads();  // umask_s complete (and the shared q fragments)
  const uint64_t umask = umask_s;


  float m_run = -INFINITY, l_run = 0.f;
  floatx4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (n_prefix_tiles == 0 && n_tiles > 0) load_tree_tile(umask);
  for (int t = 0; t < n_tiles; ++t) {
    const bool tree_tile = (t == n_prefix_tiles);
    const int tlen = tree_tile ? KT : min(KT, kend - (kbeg + t * KT));
    __syncthreads();  // previous tile fully used
    // K rows as loaded; V transposed in registers: dim vdim+d gets keys vkey..vkey+3
#pragma unroll
    for (int u = 0; u < 4; ++u) *(u32x4*)&ks[skey + u][sdim] = kr[u];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // even dim 2e: low halves; odd dim 2e+1: high halves
      const uint32_t lo01 = __builtin_amdgcn_perm(vr[1][e], vr[0][e], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(vr[3][e], vr[2][e], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(vr[1][e], vr[0][e], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(vr[3][e], vr[2][e], 0x07060302u);
      const int col = vt_col(vkey >> 2);
      *(uint2*)&vt[vdim + 2 * e][col] = make_uint2(lo01, lo23);
      *(uint2*)&vt[vdim + 2 * e + 1][col] = make_uint2(hi01, hi23);
    }
    __syncthreads();
    if (t + 1 < n_prefix_tiles) load_prefix_tile(t + 1);
    else if (t + 1 == n_prefix_tiles && with_tree) load_tree_tile(umask);

    // S^T: lane (query c, gq) gets keys kb*16 + 4*gq + v, v < 4, for the
    // wave's key blocks: all four, or (KSPLIT) block wv alone
    constexpr int NKB = KSPLIT ? 1 : 4;
    floatx4 sacc[NKB];
#pragma unroll
    for (int i = 0; i < NKB; ++i) {
      const int kb = KSPLIT ? wv : i;
      sacc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < 4; ++dc) {
        const u32x4 A = *(const u32x4*)&ks[kb * 16 + c][dc * 32 + gq * 8];
        if constexpr (KSPLIT) {
          sacc[i] = mfma16a(A, qf[dc][0][lane], sacc[i]);
          sacc[i] = mfma16a(A, qf[dc][1][lane], sacc[i]);
        } else {
          sacc[i] = mfma16a(A, qh[dc], sacc[i]);
          sacc[i] = mfma16a(A, ql[dc], sacc[i]);
        }
      }
    }
    float sv[NKB][4];
#pragma unroll
    for (int i = 0; i < NKB; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) sv[i][v] = sacc[i][v];
    if (tree_tile || tlen < KT) {  // uniform: only the tree tile and a ragged last tile mask keys
#pragma unroll
      for (int i = 0; i < NKB; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int kk = (KSPLIT ? wv : i) * 16 + gq * 4 + v;
          const bool ok = tree_tile ? ((qmask >> kk) & 1ull) != 0 : kk < tlen;
          if (!ok) sv[i][v] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NKB; ++i) mx = fmaxf(fmaxf(mx, fmaxf(sv[i][0], sv[i][1])), fmaxf(sv[i][2], sv[i][3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
    const float mnew = fmaxf(m_run, mx);
    // rows whose keys so far are all masked keep mnew = -inf: their weights are 0
    const float mref = (mnew > -INFINITY) ? mnew : 0.f;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < NKB; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = __builtin_amdgcn_exp2f(sv[i][v] - mref);  // 2^-inf = 0
        sv[i][v] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 16, WAVE);
    ps += __shfl_xor(ps, 32, WAVE);
    if (mnew != m_run) {
      // rescale only when a running max moved (exact: otherwise the factor is 1)
      const float alpha = __builtin_amdgcn_exp2f(m_run - mref);  // m_run = -inf -> 0
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        oacc[db][0] *= alpha; oacc[db][1] *= alpha; oacc[db][2] *= alpha; oacc[db][3] *= alpha;
      }
    }
    l_run += ps;
    m_run = mnew;
    // O^T += V^T P^T over 32-key chunks: chunk kc uses key blocks 2kc, 2kc+1
    // (KSPLIT: the chunk holding block wv, the other block's weights zero)
    if constexpr (KSPLIT) {
      const int kc = wv >> 1;
      u32x4 Bh = u32x4{0u, 0u, 0u, 0u}, Bl = Bh;
      uint32_t l0, l1;
      const uint32_t h0 = asplit2(sv[0][0], sv[0][1], &l0), h1 = asplit2(sv[0][2], sv[0][3], &l1);
      if (wv & 1) {
        Bh[2] = h0; Bl[2] = l0; Bh[3] = h1; Bl[3] = l1;
      } else {
        Bh[0] = h0; Bl[0] = l0; Bh[1] = h1; Bl[1] = l1;
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int d = db * 16 + c;
        const u32x4 A = *(const u32x4*)&vt[d][(kc * 8 + gq * 2) * 4];
        oacc[db] = mfma16a(A, Bh, oacc[db]);
        oacc[db] = mfma16a(A, Bl, oacc[db]);
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        u32x4 Bh, Bl;
        uint32_t l;
        Bh[0] = asplit2(sv[2 * kc][0], sv[2 * kc][1], &l); Bl[0] = l;
        Bh[1] = asplit2(sv[2 * kc][2], sv[2 * kc][3], &l); Bl[1] = l;
        Bh[2] = asplit2(sv[2 * kc + 1][0], sv[2 * kc + 1][1], &l); Bl[2] = l;
        Bh[3] = asplit2(sv[2 * kc + 1][2], sv[2 * kc + 1][3], &l); Bl[3] = l;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int d = db * 16 + c;
          const u32x4 A = *(const u32x4*)&vt[d][(kc * 8 + gq * 2) * 4];
          oacc[db] = mfma16a(A, Bh, oacc[db]);
          oacc[db] = mfma16a(A, Bl, oacc[db]);
        }
      }
    }
  }

  if constexpr (KSPLIT) {
    // merge the four waves (disjoint key blocks of every tile, same queries)
    // through LDS: wave w's (max, sum) and unnormalised output per query
    __syncthreads();  // every wave done with the K and V tiles
    float* mst = reinterpret_cast<float*>(smem);  // [4][16][2] running (max, sum)
    float* mo = mst + 4 * 16 * 2;                  // [4][16][128] outputs
    if (gq == 0) {
      mst[(wv * 16 + c) * 2] = m_run;
      mst[(wv * 16 + c) * 2 + 1] = l_run;
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) *(floatx4*)&mo[(wv * 16 + c) * 128 + db * 16 + gq * 4] = oacc[db];
    __syncthreads();
    // thread t: query t / 16, dims (t % 16) * 8 .. + 8
    const int cq = threadIdx.x >> 4, d0 = (threadIdx.x & 15) * 8;
    const int qq = qb * 16 + cq;
    if (qq >= nq) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mst[(w * 16 + cq) * 2]);
    const float mref = (M > -INFINITY) ? M : 0.f;
    float wt[4], Ls = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wt[w] = __builtin_amdgcn_exp2f(mst[(w * 16 + cq) * 2] - mref);  // -inf -> 0
      Ls += wt[w] * mst[(w * 16 + cq) * 2 + 1];
    }
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += wt[w] * mo[(w * 16 + cq) * 128 + d0 + e];
      o[e] = acc;
    }
    const int qrow = r0 + qq / G, qh_ = g * G + qq % G;
    if (a.n_splits == 1) {
      const float inv = (Ls > 0.f) ? 1.f / Ls : 0.f;
      const size_t off = ((size_t)qrow * a.hq + qh_) * 128 + d0;
      const float4 v0 = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
      const float4 v1 = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
      if (a.outb) {
        put_split8((bf16_t*)a.outb + off, (size_t)a.n_rows * a.hq * 128, v0, v1);
      } else {
        *(float4*)(a.out + off) = v0;
        *(float4*)(a.out + off + 4) = v1;
      }
    } else {
      float* dst = a.part + (size_t)s * a.n_rows * a.hq * (128 + 2) + ((size_t)qrow * a.hq + qh_) * (128 + 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[2 + d0 + e] = o[e];
      if (d0 == 0) {
        dst[0] = M * 0.6931471805599453f;  // natural-log units for the combine
        dst[1] = Ls;
      }
    }
    return;
  }

  // lane (query c, gq) holds dims db*16 + 4*gq + v
  if (a.n_splits == 1) {
    if (!qv) return;
    const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
    const size_t off = ((size_t)row * a.hq + h) * 128;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const float4 v = make_float4(oacc[db][0] * inv, oacc[db][1] * inv, oacc[db][2] * inv, oacc[db][3] * inv);
      if (a.outb)
        put_split4((bf16_t*)a.outb + off + db * 16 + gq * 4, (size_t)a.n_rows * a.hq * 128, v);
      else
        *(float4*)(a.out + off + db * 16 + gq * 4) = v;
    }
    return;
  }
  const size_t sstride = (size_t)a.n_rows * a.hq * (128 + 2);  // between splits
  if (qv) {
    float* dst = a.part + s * sstride + ((size_t)row * a.hq + h) * (128 + 2);
#pragma unroll
    for (int db = 0; db < 8; ++db) {  // rows of hd + 2 floats: 8-byte aligned
      float* d4 = dst + 2 + db * 16 + gq * 4;
      d4[0] = oacc[db][0]; d4[1] = oacc[db][1]; d4[2] = oacc[db][2]; d4[3] = oacc[db][3];
    }
    if (gq == 0) {
      dst[0] = m_run * 0.6931471805599453f;  // back to natural-log units for the combine
      dst[1] = l_run;
    }
  }
}

}  // namespace

hipError_t launch_rope_kv(const RopeArgs& a, bool bf16, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  if (a.hd > 128 || a.hd % 2) return hipErrorInvalidValue;  // angle table holds 64 pairs
  const dim3 grid(a.n_rows, (a.hq + 2 * a.hkv + ROPE_HPB - 1) / ROPE_HPB);
  if (bf16)
    hipLaunchKernelGGL(rope_kv_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(rope_kv_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// fp32 scalar kernel: prefix splits of a multiple of the 64-key tile aiming at
// ~2048 workgroups, plus one split for the tree block.
static AttnPlan plan_scalar(int max_prefix, int batch, int hkv) {
  const long want = 2048;
  const long per = (long)batch * hkv;
  int split_len = KT;
  while ((long)((max_prefix + split_len - 1) / split_len) * per > want && split_len < (1 << 20)) split_len *= 2;
  return AttnPlan{split_len, (max_prefix + split_len - 1) / split_len + 1};
}

// bf16 matrix-core kernel: splits of whole tiles.  Fewer than 256 (sequence,
// kv head, query block) units -- single-sequence drafting -- are
// latency-bound: the tree slots get a split of their own and the prefix
// splits hold as few tiles as keep ~512 workgroups (two per compute unit), so
// no workgroup walks prefix tiles and the tree one after the other.  (With the
// key-split variant three fit per compute unit, but one-tile splits at 7B,
// 544 workgroups, measured 16.8 -> 19.5 us against two-tile splits.)  (Measured on the 7B shapes, 32 units: ~256 workgroups of 2-4 tiles
// beat 1024 of one tile by 10-43 %: each workgroup pays its set-up and the
// partials must be combined.)  From 256 units (13B / 70B batched): ~1024
// workgroups, the tree tile with the last split, within a few % of the best
// plan measured.
static AttnPlan plan_mfma(int max_prefix, int batch, int hkv, int max_queries) {
  const long qblocks = (max_queries + AQ - 1) / AQ;
  const long per = (long)batch * hkv * (qblocks > 0 ? qblocks : 1);
  const int tiles = (max_prefix + KT - 1) / KT;
  if (tiles <= 1) return AttnPlan{KT, 1};
  if (per < 256) {
    int tp = 1;
    while (tp < tiles && per * ((tiles + tp - 1) / tp + 1) > 512) ++tp;
    const int split_len = tp * KT;
    return AttnPlan{split_len, (max_prefix + split_len - 1) / split_len + 1};
  }
  const long target = 1024;
  int splits = (int)((target + per - 1) / per);
  if (splits > tiles) splits = tiles;
  if (splits < 1) splits = 1;
  const int tiles_per = (tiles + splits - 1) / splits;
  const int split_len = (tiles_per > 0 ? tiles_per : 1) * KT;
  const int n = (max_prefix + split_len - 1) / split_len;
  return AttnPlan{split_len, n > 0 ? n : 1};
}

AttnPlan attn_plan(bool bf16, int max_prefix, int batch, int hkv, int max_queries) {
  return bf16 ? plan_mfma(max_prefix, batch, hkv, max_queries) : plan_scalar(max_prefix, batch, hkv);
}

hipError_t launch_attention(const AttnArgs& a, bool bf16, int hd, int max_queries, hipStream_t s) {
  if (a.n_splits > 1024 || a.n_splits < 1) return hipErrorInvalidValue;  // combine keeps a weight per split in LDS
  if (a.outb && !bf16) return hipErrorInvalidValue;
  if (bf16) {
    if (hd != 128) return hipErrorInvalidValue;
    const int qblocks = (max_queries + AQ - 1) / AQ;
    if (qblocks < 1) return hipSuccess;
    if ((long)qblocks * a.hkv > 65535) return hipErrorInvalidValue;
    if (max_queries <= 16)  // every query of a kv head in one wave: the waves split the keys
      hipLaunchKernelGGL(attn_mfma_kernel<true>, dim3(a.n_splits, a.hkv, a.batch), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(attn_mfma_kernel<false>, dim3(a.n_splits, a.hkv * qblocks, a.batch), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_splits == 1) return e;
  } else {
    dim3 grid(a.n_splits, a.hkv, a.batch), blk(256);
    if (hd == 16)
      hipLaunchKernelGGL((attn_partial_kernel<float, 16>), grid, blk, 0, s, a);
    else if (hd == 64)
      hipLaunchKernelGGL((attn_partial_kernel<float, 64>), grid, blk, 0, s, a);
    else if (hd == 128)
      hipLaunchKernelGGL((attn_partial_kernel<float, 128>), grid, blk, 0, s, a);
    else
      return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.n_rows, a.hq), dim3(128), 0, s, a, hd);
  return hipGetLastError();
}
