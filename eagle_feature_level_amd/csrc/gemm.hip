// Draft-head GEMMs on gfx950: y[M, N] = x[M, K] W[N, K]^T.
//
// The draft step's GEMMs stream the whole draft head and the LM head once per
// call; with M <= 160 rows they are bound by HBM, not by the matrix units
// (arithmetic intensity ~M flop/byte against a ridge of ~315).  So:
//  * W (bf16) is the MFMA "A" operand and goes straight from HBM to VGPRs, each
//    lane pulling 32-64 contiguous bytes of a row per step; W is never staged
//    through LDS because every W element is used by exactly one wave.
//  * x is the MFMA "B" operand (M padded to 16).  The skinny kernel (M <= 16)
//    reads it straight from L2; the tiled kernel stages it through LDS so the
//    waves of a workgroup share it.
//  * Activations are fp32 and enter the matrix units as a pair of bf16 values,
//    hi = bf16(x) and lo = bf16(x - hi), two MFMAs into one fp32 accumulator:
//    the product then carries ~16 significant bits of x instead of 8, which
//    keeps a whole draft step within ~1e-3 of an fp64 evaluation.  Weights are
//    exact bf16.  In the HBM-bound regime the second MFMA costs nothing, so
//    both MFMAs always run: no MFMA sits under a data-dependent branch (the
//    compiler may drop the execz skip around a short block, and an MFMA does
//    not honour an all-zero EXEC).
//  * Since the MFMA sums over k, any permutation of k is fine as long as A and
//    B agree: a lane's 8-element group for MFMA j is taken from a contiguous
//    run of 32 (skinny) or 16 (tiled) elements, so the weight loads are wide.
//  * The skinny kernel splits K across the 8 waves of a workgroup and reduces
//    through LDS in a fixed order, then runs the fused epilogue: results are
//    deterministic and need no global atomics.
// MFMA v_mfma_f32_16x16x32_bf16 lane layout (lane l, r = l%16, g = l/16):
// A[r][g*8+i], B[g*8+i][r], D[g*4+v][r].
#include "common.h"
#include "gemm.h"

namespace {

constexpr int SK_NW = 8;       // waves per skinny workgroup
constexpr int SK_KSTEP = 128;  // K covered by one wave iteration (4 lane groups x 32)
constexpr int TL_BK = 64;      // K per tiled-kernel stage

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <typename T>
__device__ __forceinline__ const T* wrow(const GemmArgs& a, int n) {
  if (n < a.n_seg0) return (const T*)a.w0 + (size_t)n * a.K;
  n -= a.n_seg0;
  if (n < a.n_seg1) return (const T*)a.w1 + (size_t)n * a.K;
  n -= a.n_seg1;
  return (const T*)a.w2 + (size_t)n * a.K;
}

// Row scale of RMSNorm from per-tile sums of squares (fixed summation order).
__device__ __forceinline__ float row_scale(const GemmArgs& a, int m) {
  float s = 0.f;
  for (int t = 0; t < a.n_part_in; ++t) s += a.sumsq_in[(size_t)t * a.M + m];
  return 1.0f / sqrtf(s / (float)a.K + a.eps);
}

// RMSNorm scales of rows m_base .. m_base+BM-1 into LDS, all threads of the
// workgroup cooperating: 32 lanes per row, each summing every 32nd partial,
// then a fixed butterfly across the 32 lanes.  Ends with a barrier.
template <int NT>
__device__ __forceinline__ void row_scales_lds(const GemmArgs& a, int m_base, int BM, float* scale) {
  constexpr int ROWS = NT / 32;
  const int t = threadIdx.x, c = t & 31;
  for (int m0 = 0; m0 < BM; m0 += ROWS) {
    const int mm = m0 + t / 32, m = m_base + mm;
    float s = 0.f;
    if (mm < BM && m < a.M)
      for (int p = c; p < a.n_part_in; p += 32) s += a.sumsq_in[(size_t)p * a.M + m];
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, WAVE);
    if (c == 0 && mm < BM) scale[mm] = (m < a.M) ? 1.0f / sqrtf(s / (float)a.K + a.eps) : 1.f;
  }
  __syncthreads();
}

// Eight bf16 operand values as (hi, lo) pairs.
struct B8 {
  u32x4 hi, lo;
};

__device__ __forceinline__ uint32_t split2(float a, float b, uint32_t* lo) {
  const bf16_t ha = f2bf(a), hb = f2bf(b);
  *lo = pack_bf16x2(a - bf2f(ha), b - bf2f(hb));
  return (uint32_t)ha | ((uint32_t)hb << 16);
}

__device__ __forceinline__ B8 split8(float4 v0, float4 v1) {
  B8 r;
  uint32_t l;
  r.hi[0] = split2(v0.x, v0.y, &l); r.lo[0] = l;
  r.hi[1] = split2(v0.z, v0.w, &l); r.lo[1] = l;
  r.hi[2] = split2(v1.x, v1.y, &l); r.lo[2] = l;
  r.hi[3] = split2(v1.z, v1.w, &l); r.lo[3] = l;
  return r;
}

// Eight operand values of row m at columns k..k+7 (k % 8 == 0) as (hi, lo).
template <int LOAD>
__device__ __forceinline__ B8 load_b8(const GemmArgs& a, int m, int k, float rs) {
  const int row = a.xrows ? a.xrows[m] : m;
  const float4* p = (const float4*)((const float*)a.x + (size_t)row * a.ldx + k);
  float4 v0 = p[0], v1 = p[1];
  if constexpr (LOAD == LOAD_F32_NORM) {
    u32x4 gv = *(const u32x4*)((const bf16_t*)a.gain + k);
    float gs[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gs[2 * i] = __uint_as_float(gv[i] << 16);
      gs[2 * i + 1] = __uint_as_float(gv[i] & 0xffff0000u);
    }
    v0.x *= rs * gs[0]; v0.y *= rs * gs[1]; v0.z *= rs * gs[2]; v0.w *= rs * gs[3];
    v1.x *= rs * gs[4]; v1.y *= rs * gs[5]; v1.z *= rs * gs[6]; v1.w *= rs * gs[7];
  }
  return split8(v0, v1);
}

__device__ __forceinline__ floatx4 mfma16(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Logical weight row of A-tile `at` of workgroup tile `tile`.
template <int AT, int EPI>
__device__ __forceinline__ int tile_row(const GemmArgs& a, int tile, int at, int r, bool* ok) {
  if constexpr (EPI == EPI_SWIGLU) {
    constexpr int H = AT / 2;
    const int j = tile * 16 * H + (at % H) * 16 + r;
    *ok = j < a.ffn;
    return (at < H ? 0 : a.ffn) + (*ok ? j : 0);
  } else {
    const int n = tile * 16 * AT + at * 16 + r;
    *ok = n < a.N;
    return *ok ? n : 0;
  }
}

// ---------------------------------------------------------------------------
// Skinny kernel: M <= 16*MT, one workgroup = 16*AT weight rows, NW waves split K.
// Vector-memory loads complete in issue order, so the activations of a k-step
// are loaded in the same register stage as its weights: waiting for a stage
// never waits for a later prefetch.  Three stages, two in flight.
// ---------------------------------------------------------------------------
template <int AT, int MT, int LOAD>
struct SkStage {
  u32x4 A[AT][4];    // weight fragments
  u32x4 X[MT][8];    // raw fp32 activation bits
};

__device__ __forceinline__ float4 as_f4(u32x4 v) {
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

template <int AT, int MT, int NW, int LOAD, int EPI>
__global__ void __launch_bounds__(NW * 64) gemm_skinny(GemmArgs a) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x;

  const bf16_t* ap[AT];
#pragma unroll
  for (int at = 0; at < AT; ++at) {
    bool ok;
    const int n = tile_row<AT, EPI>(a, tile, at, r, &ok);
    ap[at] = wrow<bf16_t>(a, n) + g * 32;
  }
  // per-lane activation rows (rows >= M clamped to a valid row, zeroed at use)
  const float* xp[MT];
  bool mv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + r;
    mv[mt] = m < a.M;
    const int mm = mv[mt] ? m : 0;
    const int row = a.xrows ? a.xrows[mm] : mm;
    xp[mt] = (const float*)a.x + (size_t)row * a.ldx + g * 32;
  }
  const int nks = a.K / SK_KSTEP;
  SkStage<AT, MT, LOAD> S0, S1, S2;
  auto issue = [&](SkStage<AT, MT, LOAD>& st, int ks) {
#pragma unroll
    for (int at = 0; at < AT; ++at)
#pragma unroll
      for (int j = 0; j < 4; ++j) st.A[at][j] = *(const u32x4*)(ap[at] + (size_t)ks * SK_KSTEP + j * 8);
    const int k0 = ks * SK_KSTEP;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 8; ++q) st.X[mt][q] = *(const u32x4*)(xp[mt] + k0 + q * 4);
  };
  if (wv < nks) issue(S0, wv);
  if (wv + NW < nks) issue(S1, wv + NW);

  // RMSNorm row scales and gains (LDS), summed while the first stages are in flight
  __shared__ float scale[16 * MT];
  __shared__ float gain_s[LOAD == LOAD_F32_NORM ? 8192 : 1];
  float rs[MT];
  if constexpr (LOAD == LOAD_F32_NORM) {
    for (int k = threadIdx.x; k < a.K; k += NW * 64) gain_s[k] = bf2f(((const bf16_t*)a.gain)[k]);
    row_scales_lds<NW * 64>(a, 0, 16 * MT, scale);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) rs[mt] = (LOAD == LOAD_F32_NORM) ? scale[mt * 16 + r] : 1.f;

  floatx4 acc[AT][MT];
#pragma unroll
  for (int at = 0; at < AT; ++at)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[at][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](const SkStage<AT, MT, LOAD>& st, int ks) {
    const int k0 = ks * SK_KSTEP;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      B8 B[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float4 v0 = as_f4(st.X[mt][2 * j]), v1 = as_f4(st.X[mt][2 * j + 1]);
        if constexpr (LOAD == LOAD_F32_NORM) {
          const float* gs = &gain_s[k0 + g * 32 + j * 8];
          const float s0 = rs[mt];
          v0.x *= s0 * gs[0]; v0.y *= s0 * gs[1]; v0.z *= s0 * gs[2]; v0.w *= s0 * gs[3];
          v1.x *= s0 * gs[4]; v1.y *= s0 * gs[5]; v1.z *= s0 * gs[6]; v1.w *= s0 * gs[7];
        }
        B[mt] = split8(v0, v1);
        if (!mv[mt]) {
          B[mt].hi = u32x4{0, 0, 0, 0};
          B[mt].lo = u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int at = 0; at < AT; ++at)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[at][mt] = mfma16(st.A[at][j], B[mt].hi, acc[at][mt]);
          acc[at][mt] = mfma16(st.A[at][j], B[mt].lo, acc[at][mt]);
        }
    }
  };

  for (int ks = wv; ks < nks; ks += 3 * NW) {
    if (ks + 2 * NW < nks) issue(S2, ks + 2 * NW);
    step(S0, ks);
    if (ks + NW >= nks) break;
    if (ks + 3 * NW < nks) issue(S0, ks + 3 * NW);
    step(S1, ks + NW);
    if (ks + 2 * NW >= nks) break;
    if (ks + 4 * NW < nks) issue(S1, ks + 4 * NW);
    step(S2, ks + 2 * NW);
  }

  // Cross-wave reduction in a fixed order.
  constexpr int BN = 16 * AT;
  constexpr int BM = 16 * MT;
  __shared__ float red[NW][BM][BN + 4];
#pragma unroll
  for (int at = 0; at < AT; ++at)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wv][mt * 16 + r][at * 16 + g * 4 + v] = acc[at][mt][v];
  __syncthreads();

  if constexpr (EPI == EPI_SWIGLU) {
    constexpr int H = BN / 2;
    for (int e = threadIdx.x; e < BM * H; e += NW * 64) {
      const int m = e / H, jl = e % H;
      const int j = tile * H + jl;
      if (m < a.M && j < a.ffn) {
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          gs += red[w][m][jl];
          us += red[w][m][jl + H];
        }
        ((float*)a.yb)[(size_t)m * a.ldyb + j] = silu_f(gs) * us;
      }
    }
  } else {
    constexpr int ELEMS = BM * BN;
    for (int e0 = 0; e0 < ELEMS; e0 += NW * 64) {
      const int e = e0 + threadIdx.x;
      const bool act = e < ELEMS;
      const int m = act ? e / BN : 0, nl = act ? e % BN : 0;
      const int n = tile * BN + nl;
      const bool live = act && m < a.M && n < a.N;
      float y = 0.f;
      if (live) {
#pragma unroll
        for (int w = 0; w < NW; ++w) y += red[w][m][nl];
        if constexpr (EPI == EPI_BIAS_SUMSQ) y += bf2f(((const bf16_t*)a.bias)[n]);
        if constexpr (EPI == EPI_RESID || EPI == EPI_RESID_SUMSQ) y += a.resid[(size_t)m * a.ldr + n];
        a.y[(size_t)m * a.ldy + n] = y;
      }
      if constexpr (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
        float s = live ? y * y : 0.f;
#pragma unroll
        for (int o = BN / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, WAVE);
        if (act && nl == 0 && m < a.M) a.sumsq_out[(size_t)tile * a.M + m] = s;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel: 4 waves, each 16*AT weight rows x all 16*MT rows of x staged in
// LDS; split-K over gridDim.y, M blocks over gridDim.z.  Writes fp32 partials;
// gemm_reduce applies the epilogue.
// ---------------------------------------------------------------------------
template <int AT, int MT, int LOAD>
__global__ void __launch_bounds__(256) gemm_tiled(GemmArgs a, int logical_swiglu) {
  constexpr int BM = 16 * MT;
  constexpr int LDSW = TL_BK + 8;  // padded row (bf16 elements)
  __shared__ bf16_t xs[2][BM][LDSW];  // hi halves
  __shared__ bf16_t xl[2][BM][LDSW];  // lo halves
  __shared__ float scale[BM];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int m_base = blockIdx.z * BM;
  const int n_base = blockIdx.x * (64 * AT) + wv * 16 * AT;
  const int kper = a.K / a.splits;  // multiple of TL_BK
  const int k_begin = blockIdx.y * kper;
  const int nkb = kper / TL_BK;

  if constexpr (LOAD == LOAD_F32_NORM) row_scales_lds<256>(a, m_base, BM, scale);

  const bf16_t* ap[AT];
#pragma unroll
  for (int at = 0; at < AT; ++at) {
    const int n = n_base + at * 16 + r;
    ap[at] = wrow<bf16_t>(a, n < a.N ? n : 0) + k_begin + g * 16;
  }

  constexpr int GROUPS = BM * (TL_BK / 8);  // 8-element groups per x tile
  constexpr int GPT = (GROUPS + 255) / 256;
  B8 xr[GPT];
  auto load_x = [&](int kb) {
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int idx = threadIdx.x + i * 256;
      const int mm = idx / (TL_BK / 8), kg = idx % (TL_BK / 8);
      const int m = m_base + mm;
      xr[i].hi = u32x4{0, 0, 0, 0};
      xr[i].lo = u32x4{0, 0, 0, 0};
      if (idx < GROUPS && m < a.M) {
        const float rs = (LOAD == LOAD_F32_NORM) ? scale[mm] : 1.f;
        xr[i] = load_b8<LOAD>(a, m, k_begin + kb * TL_BK + kg * 8, rs);
      }
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int idx = threadIdx.x + i * 256;
      if (idx < GROUPS) {
        const int mm = idx / (TL_BK / 8), kg = idx % (TL_BK / 8);
        *(u32x4*)&xs[buf][mm][kg * 8] = xr[i].hi;
        *(u32x4*)&xl[buf][mm][kg * 8] = xr[i].lo;
      }
    }
  };

  floatx4 acc[AT][MT];
#pragma unroll
  for (int at = 0; at < AT; ++at)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[at][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  u32x4 A0[AT][2], A1[AT][2];
  auto loadA = [&](u32x4 (&dst)[AT][2], int kb) {
#pragma unroll
    for (int at = 0; at < AT; ++at)
#pragma unroll
      for (int j = 0; j < 2; ++j) dst[at][j] = *(const u32x4*)(ap[at] + (size_t)kb * TL_BK + j * 8);
  };
  auto compute = [&](const u32x4 (&A)[AT][2], int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 B[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) B[mt] = *(const u32x4*)&xs[buf][mt * 16 + r][g * 16 + j * 8];
#pragma unroll
      for (int at = 0; at < AT; ++at)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[at][mt] = mfma16(A[at][j], B[mt], acc[at][mt]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) B[mt] = *(const u32x4*)&xl[buf][mt * 16 + r][g * 16 + j * 8];
#pragma unroll
      for (int at = 0; at < AT; ++at)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[at][mt] = mfma16(A[at][j], B[mt], acc[at][mt]);
    }
  };

  load_x(0);
  store_x(0);
  loadA(A0, 0);
  __syncthreads();
  for (int kb = 0; kb < nkb; kb += 2) {
    if (kb + 1 < nkb) {
      loadA(A1, kb + 1);
      load_x(kb + 1);
    }
    compute(A0, 0);
    if (kb + 1 < nkb) store_x(1);
    __syncthreads();
    if (kb + 1 >= nkb) break;
    if (kb + 2 < nkb) {
      loadA(A0, kb + 2);
      load_x(kb + 2);
    }
    compute(A1, 1);
    if (kb + 2 < nkb) store_x(0);
    __syncthreads();
  }

  float* P = a.part + (size_t)blockIdx.y * a.M * a.N;
#pragma unroll
  for (int at = 0; at < AT; ++at) {
    const int n = n_base + at * 16 + g * 4;
    if (n >= a.N) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m_base + mt * 16 + r;
      if (m < a.M) *(floatx4*)(P + (size_t)m * a.N + n) = acc[at][mt];
    }
  }
}

// Sum split-K partials and apply the epilogue.  grid (ceil(Nout/1024), M).
template <int EPI>
__global__ void __launch_bounds__(256) gemm_reduce(GemmArgs a) {
  __shared__ float red[4];
  const int m = blockIdx.y;
  const int n = blockIdx.x * 1024 + threadIdx.x * 4;
  const int nout = (EPI == EPI_SWIGLU) ? a.ffn : a.N;
  const size_t stride = (size_t)a.M * a.N;
  float ss = 0.f;
  if (n < nout) {
    float4 s = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < a.splits; ++sp) {
      const float4 v = *(const float4*)(a.part + sp * stride + (size_t)m * a.N + n);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    if constexpr (EPI == EPI_SWIGLU) {
      float4 u = {0.f, 0.f, 0.f, 0.f};
      for (int sp = 0; sp < a.splits; ++sp) {
        const float4 v = *(const float4*)(a.part + sp * stride + (size_t)m * a.N + a.ffn + n);
        u.x += v.x; u.y += v.y; u.z += v.z; u.w += v.w;
      }
      const float4 o = {silu_f(s.x) * u.x, silu_f(s.y) * u.y, silu_f(s.z) * u.z, silu_f(s.w) * u.w};
      *(float4*)((float*)a.yb + (size_t)m * a.ldyb + n) = o;
    } else {
      if constexpr (EPI == EPI_BIAS_SUMSQ) {
        const bf16_t* b = (const bf16_t*)a.bias + n;
        s.x += bf2f(b[0]); s.y += bf2f(b[1]); s.z += bf2f(b[2]); s.w += bf2f(b[3]);
      }
      if constexpr (EPI == EPI_RESID || EPI == EPI_RESID_SUMSQ) {
        const float4 rr = *(const float4*)(a.resid + (size_t)m * a.ldr + n);
        s.x += rr.x; s.y += rr.y; s.z += rr.z; s.w += rr.w;
      }
      *(float4*)(a.y + (size_t)m * a.ldy + n) = s;
      ss = s.x * s.x + s.y * s.y + s.z * s.z + s.w * s.w;
    }
  }
  if constexpr (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
    const float t = block_sum<256>(ss, red);
    if (threadIdx.x == 0) a.sumsq_out[(size_t)blockIdx.x * a.M + m] = t;
  }
}

// ---------------------------------------------------------------------------
// fp32 path (tiny fp32 workloads): one thread per output, 64 outputs per block.
// ---------------------------------------------------------------------------
template <int LOAD>
__device__ __forceinline__ float load_x1(const GemmArgs& a, int m, int k, float rs) {
  const int row = (LOAD == LOAD_F32 && a.xrows) ? a.xrows[m] : m;
  float v = ((const float*)a.x)[(size_t)row * a.ldx + k];
  if constexpr (LOAD == LOAD_F32_NORM) v *= rs * ((const float*)a.gain)[k];
  return v;
}

template <int LOAD, int EPI>
__global__ void __launch_bounds__(64) gemm_f32(GemmArgs a) {
  const int m = blockIdx.y;
  const int n = blockIdx.x * 64 + threadIdx.x;
  const int nout = (EPI == EPI_SWIGLU) ? a.ffn : a.N;
  float rs = 1.f;
  if constexpr (LOAD == LOAD_F32_NORM) rs = row_scale(a, m);
  float y = 0.f;
  const bool live = n < nout;
  if (live) {
    if constexpr (EPI == EPI_SWIGLU) {
      const float* wg = wrow<float>(a, n);
      const float* wu = wrow<float>(a, a.ffn + n);
      float gs = 0.f, us = 0.f;
      for (int k = 0; k < a.K; ++k) {
        const float xv = load_x1<LOAD>(a, m, k, rs);
        gs += wg[k] * xv;
        us += wu[k] * xv;
      }
      ((float*)a.yb)[(size_t)m * a.ldyb + n] = silu_f(gs) * us;
    } else {
      const float* w = wrow<float>(a, n);
      for (int k = 0; k < a.K; ++k) y += w[k] * load_x1<LOAD>(a, m, k, rs);
      if constexpr (EPI == EPI_BIAS_SUMSQ) y += ((const float*)a.bias)[n];
      if constexpr (EPI == EPI_RESID || EPI == EPI_RESID_SUMSQ) y += a.resid[(size_t)m * a.ldr + n];
      a.y[(size_t)m * a.ldy + n] = y;
    }
  }
  if constexpr (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
    const float s = wave_sum(live ? y * y : 0.f);
    if (threadIdx.x == 0) a.sumsq_out[(size_t)blockIdx.x * a.M + m] = s;
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <int AT, int MT, int NW, int LOAD>
hipError_t skinny_epi(const GemmArgs& a, int epi, int* n_part, hipStream_t s) {
  const int BN = 16 * AT;
  dim3 blk(NW * 64);
  const dim3 grid((a.N + BN - 1) / BN);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_skinny<AT, MT, NW, LOAD, EPI_STORE>), grid, blk, 0, s, a); break;
    case EPI_BIAS_SUMSQ:
      hipLaunchKernelGGL((gemm_skinny<AT, MT, NW, LOAD, EPI_BIAS_SUMSQ>), grid, blk, 0, s, a);
      *n_part = grid.x;
      break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_skinny<AT, MT, NW, LOAD, EPI_RESID>), grid, blk, 0, s, a); break;
    case EPI_RESID_SUMSQ:
      hipLaunchKernelGGL((gemm_skinny<AT, MT, NW, LOAD, EPI_RESID_SUMSQ>), grid, blk, 0, s, a);
      *n_part = grid.x;
      break;
    case EPI_SWIGLU:
      if constexpr (AT >= 2) {  // gate and up tiles pair up inside a workgroup
        const int H = BN / 2;
        hipLaunchKernelGGL((gemm_skinny<AT, MT, NW, LOAD, EPI_SWIGLU>), dim3((a.ffn + H - 1) / H), blk, 0, s, a);
        break;
      } else {
        return hipErrorInvalidValue;
      }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Four weight tiles x four waves when that still gives >= ~500 workgroups,
// else one tile x eight waves (K split 8 ways inside the workgroup).
template <int MT, int LOAD>
hipError_t skinny_shape(const GemmArgs& a, int epi, int* n_part, hipStream_t s) {
  const int rows = (epi == EPI_SWIGLU) ? 2 * a.ffn : a.N;
  if (rows / 64 >= 384) return skinny_epi<4, MT, 4, LOAD>(a, epi, n_part, s);
  if (epi == EPI_SWIGLU) return skinny_epi<2, MT, 8, LOAD>(a, epi, n_part, s);
  return skinny_epi<1, MT, 8, LOAD>(a, epi, n_part, s);
}

template <int MT>
hipError_t skinny_load(const GemmArgs& a, int load, int epi, int* n_part, hipStream_t s) {
  if (load == LOAD_F32_NORM && a.K > 8192) return hipErrorInvalidValue;  // gains staged in LDS
  switch (load) {
    case LOAD_F32: return skinny_shape<MT, LOAD_F32>(a, epi, n_part, s);
    case LOAD_F32_NORM: return skinny_shape<MT, LOAD_F32_NORM>(a, epi, n_part, s);
  }
  return hipErrorInvalidValue;
}

struct TiledPlan {
  int mt, mblocks, splits, ntiles;
};

TiledPlan plan_tiled(int M, int N, int K) {
  TiledPlan p;
  // one M block if it fits in 160 rows (weights read once); else blocks of 128
  if (M <= 160) {
    p.mt = (M + 15) / 16;
    p.mt = p.mt <= 4 ? 4 : (p.mt <= 6 ? 6 : (p.mt <= 8 ? 8 : 10));
    p.mblocks = 1;
  } else {
    p.mt = 8;
    p.mblocks = (M + 127) / 128;
  }
  p.ntiles = (N + 127) / 128;
  const int wgs = p.ntiles * p.mblocks;
  int splits = 1;
  while (wgs * splits < 512 && (K % (TL_BK * splits * 2)) == 0 && K / (splits * 2) >= 256) splits *= 2;
  p.splits = splits;
  return p;
}

template <int MT>
hipError_t tiled_launch(const GemmArgs& a, int load, const TiledPlan& p, hipStream_t s) {
  dim3 grid(p.ntiles, p.splits, p.mblocks), blk(256);
  switch (load) {
    case LOAD_F32: hipLaunchKernelGGL((gemm_tiled<2, MT, LOAD_F32>), grid, blk, 0, s, a, 0); break;
    case LOAD_F32_NORM: hipLaunchKernelGGL((gemm_tiled<2, MT, LOAD_F32_NORM>), grid, blk, 0, s, a, 0); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

size_t gemm_bf16_partial_bytes(int M, int N, int K) {
  if (M <= 16) return 0;
  TiledPlan p = plan_tiled(M, N, K);
  return (size_t)p.splits * M * N * sizeof(float);
}

hipError_t launch_gemm_bf16(GemmArgs a, int load, int epi, int* n_part_out, hipStream_t s) {
  if (a.K % SK_KSTEP) return hipErrorInvalidValue;  // both kernels step K in whole 128-element blocks
  if (a.M <= 16) return skinny_load<1>(a, load, epi, n_part_out, s);
  // tiled path; for SwiGLU the logical matrix is [gate; up] with N = 2*ffn
  if (a.part == nullptr) return hipErrorInvalidValue;  // partial buffer is mandatory here
  if (a.K % TL_BK) return hipErrorInvalidValue;
  TiledPlan p = plan_tiled(a.M, a.N, a.K);
  a.splits = p.splits;
  hipError_t e;
  switch (p.mt) {
    case 4: e = tiled_launch<4>(a, load, p, s); break;
    case 6: e = tiled_launch<6>(a, load, p, s); break;
    case 8: e = tiled_launch<8>(a, load, p, s); break;
    default: e = tiled_launch<10>(a, load, p, s); break;
  }
  if (e != hipSuccess) return e;
  const int nout = (epi == EPI_SWIGLU) ? a.ffn : a.N;
  dim3 grid((nout + 1023) / 1024, a.M), blk(256);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_reduce<EPI_STORE>, grid, blk, 0, s, a); break;
    case EPI_BIAS_SUMSQ: hipLaunchKernelGGL(gemm_reduce<EPI_BIAS_SUMSQ>, grid, blk, 0, s, a); *n_part_out = grid.x; break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_reduce<EPI_RESID>, grid, blk, 0, s, a); break;
    case EPI_RESID_SUMSQ: hipLaunchKernelGGL(gemm_reduce<EPI_RESID_SUMSQ>, grid, blk, 0, s, a); *n_part_out = grid.x; break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_reduce<EPI_SWIGLU>, grid, blk, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_f32(GemmArgs a, int load, int epi, int* n_part_out, hipStream_t s) {
  const int nout = (epi == EPI_SWIGLU) ? a.ffn : a.N;
  dim3 grid((nout + 63) / 64, a.M), blk(64);
#define F32_EPI(L)                                                                                   \
  switch (epi) {                                                                                     \
    case EPI_STORE: hipLaunchKernelGGL((gemm_f32<L, EPI_STORE>), grid, blk, 0, s, a); break;         \
    case EPI_BIAS_SUMSQ: hipLaunchKernelGGL((gemm_f32<L, EPI_BIAS_SUMSQ>), grid, blk, 0, s, a); break; \
    case EPI_RESID: hipLaunchKernelGGL((gemm_f32<L, EPI_RESID>), grid, blk, 0, s, a); break;         \
    case EPI_RESID_SUMSQ: hipLaunchKernelGGL((gemm_f32<L, EPI_RESID_SUMSQ>), grid, blk, 0, s, a); break; \
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_f32<L, EPI_SWIGLU>), grid, blk, 0, s, a); break;       \
    default: return hipErrorInvalidValue;                                                            \
  }
  switch (load) {
    case LOAD_F32: F32_EPI(LOAD_F32); break;
    case LOAD_F32_NORM: F32_EPI(LOAD_F32_NORM); break;
    default: return hipErrorInvalidValue;
  }
#undef F32_EPI
  if (epi == EPI_BIAS_SUMSQ || epi == EPI_RESID_SUMSQ) *n_part_out = grid.x;
  return hipGetLastError();
}
