// Draft-head GEMMs on gfx950: y[M, N] = x[M, K] W[N, K]^T.
//
// The draft step's GEMMs stream the whole draft head and the LM head once per
// call; with a few rows they are bound by HBM, not by the matrix units
// (arithmetic intensity ~M flop/byte against a ridge of ~315); the tree-wide
// step over hundreds of rows is bound by the matrix units.  So:
//  * W (bf16) is the MFMA "A" operand and goes straight from HBM to VGPRs, each
//    lane pulling 64 contiguous bytes of a row per step; W is never staged
//    through LDS because every W element is used by exactly one wave.
//  * x (fp32) is the MFMA "B" operand (M padded to 16).  The skinny kernel
//    (M <= 16) loads each k-step's rows of x coalesced and re-reads them in the
//    B layout from the wave's own LDS slice; the large-M kernel stages weight
//    and x tiles through LDS so the waves of a workgroup share both.
//  * Activations enter the matrix units as a pair of bf16 values, hi = x cut
//    to bf16 and lo = bf16(x - hi), two MFMAs into one fp32 accumulator: the
//    product then carries ~16 significant bits of x instead of 8, which keeps a
//    whole draft step within ~1e-3 of an fp64 evaluation.  Weights are exact
//    bf16.
//    In the HBM-bound regime the second MFMA costs nothing, so both MFMAs always
//    run: no MFMA sits under a data-dependent branch (the compiler may drop the
//    execz skip around a short block, and an MFMA does not honour an all-zero
//    EXEC).
//  * RMSNorm(x) * g feeds the next GEMM as (x * g) W^T scaled per row by
//    rsqrt(mean(x^2) + eps): the producing GEMM's epilogue writes x * g next to
//    x and per-tile sums of squares of x; the consuming GEMM applies the row
//    scale in its epilogue.  Its main loop is a plain fp32 stream.
//  * Since the MFMA sums over k, any permutation of k is fine as long as A and
//    B agree: a lane's 8-element group for MFMA j is taken from a contiguous
//    run of 32 (skinny) or 16 (tiled) elements, so the weight loads are wide.
//  * The skinny kernel splits K across the waves of a workgroup and reduces
//    through LDS in a fixed order, then runs the fused epilogue: results are
//    deterministic and need no global atomics.
// MFMA v_mfma_f32_16x16x32_bf16 lane layout (lane l, r = l%16, g = l/16):
// A[r][g*8+i], B[g*8+i][r], D[g*4+v][r].
#include "common.h"
#include "gemm.h"

namespace {

constexpr int SK_KSTEP = 128;  // K covered by one wave iteration (4 lane groups x 32)

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <typename T>
__device__ __forceinline__ const T* wrow(const GemmArgs& a, int n) {
  if (n < a.n_seg0) return (const T*)a.w0 + (size_t)n * a.K;
  n -= a.n_seg0;
  if (n < a.n_seg1) return (const T*)a.w1 + (size_t)n * a.K;
  n -= a.n_seg1;
  return (const T*)a.w2 + (size_t)n * a.K;
}

__device__ __forceinline__ float rms_scale(float sumsq, const GemmArgs& a) {
  return 1.0f / sqrtf(sumsq / (float)a.K + a.eps);
}

// Row scale of RMSNorm from per-tile sums of squares (fixed summation order).
__device__ __forceinline__ float row_scale(const GemmArgs& a, int m) {
  float s = 0.f;
  for (int t = 0; t < a.n_part_in; ++t) s += a.sumsq_in[(size_t)t * a.M + m];
  return rms_scale(s, a);
}

// RMSNorm scales of rows 0 .. BM-1 into LDS, all threads of the workgroup
// cooperating: 32 lanes per row, each summing every 32nd partial, then a fixed
// butterfly across the 32 lanes.  No barrier: readers sync first.
template <int NT>
__device__ __forceinline__ void row_scales_lds(const GemmArgs& a, int BM, float* scale) {
  constexpr int ROWS = NT / 32;
  const int t = threadIdx.x, c = t & 31;
  for (int m0 = 0; m0 < BM; m0 += ROWS) {
    const int m = m0 + t / 32;
    float s = 0.f;
    if (m < BM && m < a.M)
      for (int p = c; p < a.n_part_in; p += 32) s += a.sumsq_in[(size_t)p * a.M + m];
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, WAVE);
    if (c == 0 && m < BM) scale[m] = (m < a.M) ? rms_scale(s, a) : 1.f;
  }
}

// Eight bf16 operand values as (hi, lo) pairs.
struct B8 {
  u32x4 hi, lo;
};

// Two fp32 values as packed bf16 pairs (value a in the low half): hi = x with
// its low 16 bits dropped (so x - hi is exact in fp32), lo = x - hi rounded to
// bf16, ties away from zero.  |x - hi - lo| <= 2^-15 |x|.  Byte permutes and
// three integer/float ops per value: this runs once per operand element per
// wave, so it must stay cheap next to the weight stream.
__device__ __forceinline__ uint32_t split2(float a, float b, uint32_t* lo) {
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  const float ra = a - __uint_as_float(ua & 0xffff0000u), rb = b - __uint_as_float(ub & 0xffff0000u);
  *lo = __builtin_amdgcn_perm(__float_as_uint(rb) + 0x8000u, __float_as_uint(ra) + 0x8000u, 0x07060302u);
  return __builtin_amdgcn_perm(ub, ua, 0x07060302u);
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

__device__ __forceinline__ float4 as_f4(u32x4 v) {
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
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
// Skinny kernel: M <= 16, one workgroup = 16*AT weight rows, NW waves split K.
// Vector-memory loads complete in issue order, so the activations of a k-step
// are loaded in the same register stage as its weights: waiting for a stage
// never waits for a later prefetch.  NS register stages, NS - 1 in flight: the
// deeper the ring, the more of a workgroup's weight stream is requested before
// the first stage returns (with 256 workgroups of 16 rows, a CU owns only a
// few hundred KB of the weights, so the ramp matters).
//
// Activations: a k-step needs 128 fp32 values of each of the M rows, but in
// the MFMA B layout only the 4*M lanes of real rows hold data, 32 values each,
// so loading them in that layout costs 8 load instructions per k-step however
// small M is.  Instead the chunk [M][128] is loaded coalesced, 16 bytes per
// lane (MQ = ceil(M/2) instructions), written to this wave's own LDS slice and
// read back in the B layout: one instruction per two rows in the weight stream.
// A wave's LDS traffic is ordered, so no barrier is involved.
// ---------------------------------------------------------------------------
constexpr int SK_XROW = SK_KSTEP + 4;  // padded LDS row (floats): rows fall in different banks

template <int AT, int MQ>
struct SkStage {
  u32x4 A[AT][4];  // weight fragments
  u32x4 X[MQ];     // coalesced activation chunk: lane l, quad q -> row (q*64+l)/32, 4 floats
};

template <int AT, int NW, int MQ, int NS, int EPI>
__global__ void __launch_bounds__(NW * 64) gemm_skinny(GemmArgs a) {
  constexpr int XR = 2 * MQ;  // activation rows this instance can hold
  constexpr int BN = 16 * AT;
  constexpr int XL = NW * XR * SK_XROW, RED = NW * 16 * (BN + 4);
  // per-wave activation slices during the main loop, then the cross-wave reduction
  __shared__ float smem[XL > RED ? XL : RED];
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
  // coalesced chunk: quad q of lane l covers row xm[q], columns xc..xc+3 of the k-step.
  // Gathered rows: columns below gd from the parent's feature row (fp32), the
  // rest from the token's embedding row (bf16, widened exactly); gd is a
  // multiple of the k-step, so a k-step reads one of the two.
  const int xc = (lane & 31) * 4;
  const bool gather = a.gfeat != nullptr;
  const float* xq[MQ];
  const bf16_t* xe[MQ];
  bool xv[MQ];
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    const int m = 2 * q + (lane >> 5);
    xv[q] = m < a.M;
    if (gather) {
      xq[q] = a.gfeat + (size_t)(xv[q] ? a.gparent[m] : 0) * a.gd + xc;
      xe[q] = (const bf16_t*)a.gembed + (size_t)(xv[q] ? a.gtoken[m] : 0) * a.gd + xc;
    } else {
      const int row = xv[q] ? (a.xrows ? a.xrows[m] : m) : 0;
      xq[q] = a.x + (size_t)row * a.ldx + xc;
      xe[q] = nullptr;
    }
  }
  float* xw = &smem[wv * XR * SK_XROW];
  const bool mv = r < a.M;

  const int nks = a.K / SK_KSTEP;
  SkStage<AT, MQ> S[NS];
  auto issue = [&](SkStage<AT, MQ>& st, int ks) {
#pragma unroll
    for (int at = 0; at < AT; ++at)
#pragma unroll
      for (int j = 0; j < 4; ++j) st.A[at][j] = *(const u32x4*)(ap[at] + (size_t)ks * SK_KSTEP + j * 8);
    const int k0 = ks * SK_KSTEP;
    if (!gather || k0 < a.gd) {  // uniform: ks is the wave's
#pragma unroll
      for (int q = 0; q < MQ; ++q) st.X[q] = xv[q] ? *(const u32x4*)(xq[q] + k0) : u32x4{0, 0, 0, 0};
    } else {
#pragma unroll
      for (int q = 0; q < MQ; ++q) {
        const uint2 e = xv[q] ? *(const uint2*)(xe[q] + (k0 - a.gd)) : make_uint2(0u, 0u);
        st.X[q] = u32x4{e.x << 16, e.x & 0xffff0000u, e.y << 16, e.y & 0xffff0000u};
      }
    }
  };
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (wv + st * NW < nks) issue(S[st], wv + st * NW);

  // RMSNorm row scales of the input rows (applied in the epilogue), summed
  // while the first stages are in flight; visible after the reduction barrier
  __shared__ float scale[16];
  if (a.sumsq_in) row_scales_lds<NW * 64>(a, 16, scale);

  floatx4 acc[AT];
#pragma unroll
  for (int at = 0; at < AT; ++at) acc[at] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](const SkStage<AT, MQ>& st) {
#pragma unroll
    for (int q = 0; q < MQ; ++q) *(u32x4*)&xw[(2 * q + (lane >> 5)) * SK_XROW + xc] = st.X[q];
    const float* xr = &xw[(mv && r < XR ? r : 0) * SK_XROW + g * 32];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float4 v0 = *(const float4*)(xr + j * 8), v1 = *(const float4*)(xr + j * 8 + 4);
      if (!mv) {
        v0 = make_float4(0.f, 0.f, 0.f, 0.f);
        v1 = v0;
      }
      const B8 B = split8(v0, v1);
#pragma unroll
      for (int at = 0; at < AT; ++at) {
        acc[at] = mfma16(st.A[at][j], B.hi, acc[at]);
        acc[at] = mfma16(st.A[at][j], B.lo, acc[at]);
      }
    }
  };

  for (int ks = wv; ks < nks; ks += NS * NW) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int k = ks + st * NW;
      if (k >= nks) break;
      if (k + (NS - 1) * NW < nks) issue(S[(st + NS - 1) % NS], k + (NS - 1) * NW);
      step(S[st]);
    }
  }

  // Cross-wave reduction in a fixed order (over the activation slices: all
  // waves must be done with them first).
  __syncthreads();
  float(*red)[16][BN + 4] = reinterpret_cast<float(*)[16][BN + 4]>(smem);
#pragma unroll
  for (int at = 0; at < AT; ++at)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wv][r][at * 16 + g * 4 + v] = acc[at][v];
  __syncthreads();

  if constexpr (EPI == EPI_SWIGLU) {
    constexpr int H = BN / 2;
    for (int e = threadIdx.x; e < 16 * H; e += NW * 64) {
      const int m = e / H, jl = e % H;
      const int j = tile * H + jl;
      if (m < a.M && j < a.ffn) {
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          gs += red[w][m][jl];
          us += red[w][m][jl + H];
        }
        if (a.sumsq_in) {
          gs *= scale[m];
          us *= scale[m];
        }
        a.yb[(size_t)m * a.ldyb + j] = silu_f(gs) * us;
      }
    }
  } else {
    constexpr int ELEMS = 16 * BN;
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
        if (a.sumsq_in) y *= scale[m];
        if constexpr (EPI == EPI_BIAS_SUMSQ) y += bf2f(((const bf16_t*)a.bias)[n]);
        if constexpr (EPI == EPI_RESID || EPI == EPI_RESID_SUMSQ) y += a.resid[(size_t)m * a.ldr + n];
        a.y[(size_t)m * a.ldy + n] = y;
        if (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ)
          if (a.y2) a.y2[(size_t)m * a.ldy + n] = y * bf2f(((const bf16_t*)a.gain_out)[n]);
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
// Large-M kernel (M > 16): the matrix units are the bound once M reaches a few
// hundred rows.  A workgroup of 8 waves computes 256 weight rows x 128 rows of
// x (64 x 64 per wave, 4 x 4 blocks of v_mfma_f32_16x16x32_bf16, hi and lo).
// Per 64-wide K step the weight tile and the hi/lo split of the x tile are
// staged in LDS (two buffers); the next step's global loads sit in registers
// while the current step is multiplied.  Row blocks of x vary fastest over the
// grid, and consecutive tiles are kept on one XCD, so the workgroups sharing
// a weight tile run together and share an L2.  With a K split the raw
// partial sums go to a.part and gemm_reduce applies the epilogue; otherwise
// the epilogue runs here on the accumulators.
// SwiGLU: the 256 rows of a tile are, per wave quarter, 32 gate rows and the
// 32 up rows of the same ffn columns, so gate and up meet in one lane.
// ---------------------------------------------------------------------------
constexpr int BG_BN = 256, BG_BM = 128, BG_BK = 64;
constexpr int BG_LD = BG_BK + 8;  // LDS row (bf16): 144 B, rows 4 banks apart

struct BigPlan {
  int tiles_n, tiles_m, splits;
};

template <int EPI>
__global__ void __launch_bounds__(512) gemm_big(GemmArgs a, BigPlan p) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BG_BN][BG_LD];
  __shared__ __attribute__((aligned(16))) bf16_t Bh[2][BG_BM][BG_LD];
  __shared__ __attribute__((aligned(16))) bf16_t Bl[2][BG_BM][BG_LD];
  __shared__ float rs_s[BG_BM];
  __shared__ float ssq_s[4][BG_BM];
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int lid = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;  // consecutive tiles on one XCD
  const int mt = lid % p.tiles_m, rest = lid / p.tiles_m;
  const int nt = rest % p.tiles_n, sp = rest / p.tiles_n;
  const int m0 = mt * BG_BM;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wn = wv & 3, wm = wv >> 2;
  const int r = lane & 15, g = lane >> 4;
  const int kper = a.K / p.splits, kbeg = sp * kper, nkb = kper / BG_BK;

  // logical weight row of tile row i (-1 past the end)
  auto wrow_of = [&](int i) -> int {
    if constexpr (EPI == EPI_SWIGLU) {
      const int q = i >> 6, w = i & 63;
      const int j = nt * 128 + q * 32 + (w & 31);
      if (j >= a.ffn) return -1;
      return (w < 32) ? j : a.ffn + j;
    } else {
      const int n = nt * BG_BN + i;
      return n < a.N ? n : -1;
    }
  };
  // staging: weights rows t/8 + 64u, 8 columns at 8*(t%8); x rows t/16 + 32u, 4 columns at 4*(t%16)
  const int ac = (t & 7) * 8, xc = (t & 15) * 4;
  const bf16_t* ap[4];
  const float* xp[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int n = wrow_of((t >> 3) + 64 * u);
    ap[u] = (n >= 0) ? wrow<bf16_t>(a, n) + kbeg + ac : nullptr;
    const int m = m0 + (t >> 4) + 32 * u;
    xp[u] = (m < a.M) ? a.x + (size_t)(a.xrows ? a.xrows[m] : m) * a.ldx + kbeg + xc : nullptr;
  }
  u32x4 areg[4];
  float4 xreg[4];
  auto load_global = [&](int kb) {
    const int k0 = kb * BG_BK;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      areg[u] = ap[u] ? *(const u32x4*)(ap[u] + k0) : u32x4{0, 0, 0, 0};
      xreg[u] = xp[u] ? *(const float4*)(xp[u] + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *(u32x4*)&As[buf][(t >> 3) + 64 * u][ac] = areg[u];
      uint32_t l0, l1;
      const uint32_t h0 = split2(xreg[u].x, xreg[u].y, &l0), h1 = split2(xreg[u].z, xreg[u].w, &l1);
      *(uint2*)&Bh[buf][(t >> 4) + 32 * u][xc] = make_uint2(h0, h1);
      *(uint2*)&Bl[buf][(t >> 4) + 32 * u][xc] = make_uint2(l0, l1);
    }
  };

  const bool fused = (p.splits == 1);
  if (fused && a.sumsq_in && t < BG_BM) rs_s[t] = (m0 + t < a.M) ? row_scale(a, m0 + t) : 1.f;

  floatx4 acc[4][4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load_global(kb + 1);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      u32x4 A[4], Bhf[4], Blf[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) A[nb] = *(const u32x4*)&As[buf][wn * 64 + nb * 16 + r][kc * 32 + g * 8];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        Bhf[mb] = *(const u32x4*)&Bh[buf][wm * 64 + mb * 16 + r][kc * 32 + g * 8];
        Blf[mb] = *(const u32x4*)&Bl[buf][wm * 64 + mb * 16 + r][kc * 32 + g * 8];
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          acc[nb][mb] = mfma16(A[nb], Bhf[mb], acc[nb][mb]);
          acc[nb][mb] = mfma16(A[nb], Blf[mb], acc[nb][mb]);
        }
    }
    if (kb + 1 < nkb) store_lds(buf ^ 1);
    __syncthreads();
  }

  // lane (r, g): acc[nb][mb][v] = tile row wn*64 + nb*16 + 4g + v, x row wm*64 + mb*16 + r
  if (!fused) {
    float* P = a.part + (size_t)sp * a.M * a.N;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + wm * 64 + mb * 16 + r;
      if (m >= a.M) continue;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int n = wrow_of(wn * 64 + nb * 16 + 4 * g);  // 4 consecutive logical rows
        if (n >= 0) *(floatx4*)(P + (size_t)m * a.N + n) = acc[nb][mb];
      }
    }
    return;
  }
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int ml = wm * 64 + mb * 16 + r, m = m0 + ml;
      if (m >= a.M) continue;
      const float sc = a.sumsq_in ? rs_s[ml] : 1.f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int j = nt * 128 + wn * 32 + nb * 16 + 4 * g;
        if (j >= a.ffn) continue;
        float4 o;
        o.x = silu_f(acc[nb][mb][0] * sc) * (acc[nb + 2][mb][0] * sc);
        o.y = silu_f(acc[nb][mb][1] * sc) * (acc[nb + 2][mb][1] * sc);
        o.z = silu_f(acc[nb][mb][2] * sc) * (acc[nb + 2][mb][2] * sc);
        o.w = silu_f(acc[nb][mb][3] * sc) * (acc[nb + 2][mb][3] * sc);
        *(float4*)(a.yb + (size_t)m * a.ldyb + j) = o;
      }
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int ml = wm * 64 + mb * 16 + r, m = m0 + ml;
      const bool mv = m < a.M;
      const float sc = (mv && a.sumsq_in) ? rs_s[ml] : 1.f;
      float ss = 0.f;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int n = nt * BG_BN + wn * 64 + nb * 16 + 4 * g;
        if (!mv || n >= a.N) continue;
        float4 y = make_float4(acc[nb][mb][0] * sc, acc[nb][mb][1] * sc, acc[nb][mb][2] * sc, acc[nb][mb][3] * sc);
        if constexpr (EPI == EPI_BIAS_SUMSQ) {
          const bf16_t* bb = (const bf16_t*)a.bias + n;
          y.x += bf2f(bb[0]); y.y += bf2f(bb[1]); y.z += bf2f(bb[2]); y.w += bf2f(bb[3]);
        }
        if constexpr (EPI == EPI_RESID || EPI == EPI_RESID_SUMSQ) {
          const float4 rr = *(const float4*)(a.resid + (size_t)m * a.ldr + n);
          y.x += rr.x; y.y += rr.y; y.z += rr.z; y.w += rr.w;
        }
        *(float4*)(a.y + (size_t)m * a.ldy + n) = y;
        if (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
          if (a.y2) {
            const bf16_t* gn = (const bf16_t*)a.gain_out + n;
            *(float4*)(a.y2 + (size_t)m * a.ldy + n) =
                make_float4(y.x * bf2f(gn[0]), y.y * bf2f(gn[1]), y.z * bf2f(gn[2]), y.w * bf2f(gn[3]));
          }
          ss += y.x * y.x + y.y * y.y + y.z * y.z + y.w * y.w;
        }
      }
      if constexpr (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
        ss += __shfl_xor(ss, 16, WAVE);
        ss += __shfl_xor(ss, 32, WAVE);
        if (g == 0) ssq_s[wn][ml] = ss;
      }
    }
    if constexpr (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
      __syncthreads();
      if (t < BG_BM && m0 + t < a.M)
        a.sumsq_out[(size_t)nt * a.M + m0 + t] = ssq_s[0][t] + ssq_s[1][t] + ssq_s[2][t] + ssq_s[3][t];
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
  float rs = 1.f;
  if (a.sumsq_in) {
    float s = 0.f;
    for (int p = threadIdx.x; p < a.n_part_in; p += 256) s += a.sumsq_in[(size_t)p * a.M + m];
    rs = rms_scale(block_sum<256>(s, red), a);
  }
  float ss = 0.f;
  if (n < nout) {
    float4 s = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < a.splits; ++sp) {
      const float4 v = *(const float4*)(a.part + sp * stride + (size_t)m * a.N + n);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    s.x *= rs; s.y *= rs; s.z *= rs; s.w *= rs;
    if constexpr (EPI == EPI_SWIGLU) {
      float4 u = {0.f, 0.f, 0.f, 0.f};
      for (int sp = 0; sp < a.splits; ++sp) {
        const float4 v = *(const float4*)(a.part + sp * stride + (size_t)m * a.N + a.ffn + n);
        u.x += v.x; u.y += v.y; u.z += v.z; u.w += v.w;
      }
      u.x *= rs; u.y *= rs; u.z *= rs; u.w *= rs;
      const float4 o = {silu_f(s.x) * u.x, silu_f(s.y) * u.y, silu_f(s.z) * u.z, silu_f(s.w) * u.w};
      *(float4*)(a.yb + (size_t)m * a.ldyb + n) = o;
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
      if (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
        if (a.y2) {
          const bf16_t* gn = (const bf16_t*)a.gain_out + n;
          const float4 o = {s.x * bf2f(gn[0]), s.y * bf2f(gn[1]), s.z * bf2f(gn[2]), s.w * bf2f(gn[3])};
          *(float4*)(a.y2 + (size_t)m * a.ldy + n) = o;
        }
      }
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
// Same interface as the bf16 path; gains and bias are fp32 here.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float load_x1(const GemmArgs& a, int m, int k) {
  const int row = a.xrows ? a.xrows[m] : m;
  return a.x[(size_t)row * a.ldx + k];
}

template <int EPI>
__global__ void __launch_bounds__(64) gemm_f32(GemmArgs a) {
  const int m = blockIdx.y;
  const int n = blockIdx.x * 64 + threadIdx.x;
  const int nout = (EPI == EPI_SWIGLU) ? a.ffn : a.N;
  const float rs = a.sumsq_in ? row_scale(a, m) : 1.f;
  float y = 0.f;
  const bool live = n < nout;
  if (live) {
    if constexpr (EPI == EPI_SWIGLU) {
      const float* wg = wrow<float>(a, n);
      const float* wu = wrow<float>(a, a.ffn + n);
      float gs = 0.f, us = 0.f;
      for (int k = 0; k < a.K; ++k) {
        const float xv = load_x1(a, m, k);
        gs += wg[k] * xv;
        us += wu[k] * xv;
      }
      a.yb[(size_t)m * a.ldyb + n] = silu_f(gs * rs) * (us * rs);
    } else {
      const float* w = wrow<float>(a, n);
      for (int k = 0; k < a.K; ++k) y += w[k] * load_x1(a, m, k);
      y *= rs;
      if constexpr (EPI == EPI_BIAS_SUMSQ) y += ((const float*)a.bias)[n];
      if constexpr (EPI == EPI_RESID || EPI == EPI_RESID_SUMSQ) y += a.resid[(size_t)m * a.ldr + n];
      a.y[(size_t)m * a.ldy + n] = y;
      if (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ)
        if (a.y2) a.y2[(size_t)m * a.ldy + n] = y * ((const float*)a.gain_out)[n];
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
// Register stages of the skinny ring.  Deeper rings (4-6 stages at 8 waves)
// measured no faster on the 7B shapes: with every workgroup resident at once,
// two stages in flight already keep HBM busy.
constexpr int skinny_ns(int, int, int) { return 3; }

template <int AT, int NW, int MQ, int NS = skinny_ns(AT, NW, MQ)>
hipError_t skinny_epi(const GemmArgs& a, int epi, int* n_part, hipStream_t s) {
  const int BN = 16 * AT;
  dim3 blk(NW * 64);
  const dim3 grid((a.N + BN - 1) / BN);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_skinny<AT, NW, MQ, NS, EPI_STORE>), grid, blk, 0, s, a); break;
    case EPI_BIAS_SUMSQ:
      hipLaunchKernelGGL((gemm_skinny<AT, NW, MQ, NS, EPI_BIAS_SUMSQ>), grid, blk, 0, s, a);
      *n_part = grid.x;
      break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_skinny<AT, NW, MQ, NS, EPI_RESID>), grid, blk, 0, s, a); break;
    case EPI_RESID_SUMSQ:
      hipLaunchKernelGGL((gemm_skinny<AT, NW, MQ, NS, EPI_RESID_SUMSQ>), grid, blk, 0, s, a);
      *n_part = grid.x;
      break;
    case EPI_SWIGLU:
      if constexpr (AT >= 2) {  // gate and up tiles pair up inside a workgroup
        const int H = BN / 2;
        hipLaunchKernelGGL((gemm_skinny<AT, NW, MQ, NS, EPI_SWIGLU>), dim3((a.ffn + H - 1) / H), blk, 0, s, a);
        break;
      } else {
        return hipErrorInvalidValue;
      }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int AT, int NW>
hipError_t skinny_mq(const GemmArgs& a, int epi, int* n_part, hipStream_t s) {
  if (a.M <= 2) return skinny_epi<AT, NW, 1>(a, epi, n_part, s);
  if (a.M <= 4) return skinny_epi<AT, NW, 2>(a, epi, n_part, s);
  if (a.M <= 8) return skinny_epi<AT, NW, 4>(a, epi, n_part, s);
  return skinny_epi<AT, NW, 8>(a, epi, n_part, s);
}

// Variant choice, measured on the 7B draft-head shapes (N = 4096, 12288,
// 22016 gate+up, 32000; M = 1..16), weights streamed from HBM:
//  * fewer than 512 row tiles (N = 4096): one tile x 8 waves, so 256
//    workgroups of 8 waves cover the chip;
//  * SwiGLU: a gate and an up tile x 4 waves up to M = 8; x 8 waves above;
//  * wide N with M > 8: four tiles x 4 waves -- each activation chunk then
//    feeds four weight tiles, which matters once x is as large as the weights
//    a wave streams per step;
//  * wide N, M <= 3, >= 1536 tiles (the LM head): one tile x 8 waves (two
//    workgroups per CU, ~4 full rounds of workgroups); else one tile x 4 waves.
hipError_t skinny_launch(const GemmArgs& a, int epi, int* n_part, hipStream_t s) {
  if (epi == EPI_SWIGLU)
    return a.M > 8 ? skinny_mq<2, 8>(a, epi, n_part, s) : skinny_mq<2, 4>(a, epi, n_part, s);
  const int tiles = (a.N + 15) / 16;
  if (tiles < 512) return skinny_mq<1, 8>(a, epi, n_part, s);
  if (a.M > 8) return skinny_mq<4, 4>(a, epi, n_part, s);
  if (a.M <= 3 && tiles >= 1536) return skinny_mq<1, 8>(a, epi, n_part, s);
  return skinny_mq<1, 4>(a, epi, n_part, s);
}

// Tiles of the large-M kernel, plus a K split (powers of 2) while the grid
// has fewer than 256 workgroups (one per CU: the kernel holds 148 KB of LDS).
BigPlan plan_big(int M, int N, int K, bool swiglu) {
  BigPlan p;
  p.tiles_n = swiglu ? (N / 2 + 127) / 128 : (N + BG_BN - 1) / BG_BN;
  p.tiles_m = (M + BG_BM - 1) / BG_BM;
  p.splits = 1;
  while (p.tiles_n * p.tiles_m * p.splits < 256 && K % (BG_BK * p.splits * 2) == 0 && K / (p.splits * 2) >= 512)
    p.splits *= 2;
  return p;
}

}  // namespace

size_t gemm_bf16_partial_bytes(int M, int N, int K) {
  if (M <= 16) return 0;
  const BigPlan p = plan_big(M, N, K, false);  // N/2-wide SwiGLU tiles give no more splits than this
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm_bf16(GemmArgs a, int epi, int* n_part_out, hipStream_t s) {
  if (a.K % SK_KSTEP) return hipErrorInvalidValue;  // both kernels step K in whole 128-element blocks
  if (a.gfeat && (a.M > 16 || a.gd % SK_KSTEP || a.K != 2 * a.gd)) return hipErrorInvalidValue;
  if ((epi == EPI_BIAS_SUMSQ || epi == EPI_RESID_SUMSQ) && a.y2 && !a.gain_out) return hipErrorInvalidValue;
  if (a.M <= 16) return skinny_launch(a, epi, n_part_out, s);
  if (a.N % 4) return hipErrorInvalidValue;  // float4 epilogue stores
  const bool sw = (epi == EPI_SWIGLU);
  const BigPlan p = plan_big(a.M, a.N, a.K, sw);
  a.splits = p.splits;
  if (p.splits > 1 && a.part == nullptr) return hipErrorInvalidValue;  // partial buffer needed for a K split
  const dim3 grid(p.tiles_n * p.tiles_m * p.splits), blk(512);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_big<EPI_STORE>, grid, blk, 0, s, a, p); break;
    case EPI_BIAS_SUMSQ: hipLaunchKernelGGL(gemm_big<EPI_BIAS_SUMSQ>, grid, blk, 0, s, a, p); break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_big<EPI_RESID>, grid, blk, 0, s, a, p); break;
    case EPI_RESID_SUMSQ: hipLaunchKernelGGL(gemm_big<EPI_RESID_SUMSQ>, grid, blk, 0, s, a, p); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_big<EPI_SWIGLU>, grid, blk, 0, s, a, p); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.splits == 1) {
    if (epi == EPI_BIAS_SUMSQ || epi == EPI_RESID_SUMSQ) *n_part_out = p.tiles_n;
    return hipSuccess;
  }
  const int nout = sw ? a.ffn : a.N;
  dim3 rgrid((nout + 1023) / 1024, a.M), rblk(256);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_reduce<EPI_STORE>, rgrid, rblk, 0, s, a); break;
    case EPI_BIAS_SUMSQ: hipLaunchKernelGGL(gemm_reduce<EPI_BIAS_SUMSQ>, rgrid, rblk, 0, s, a); *n_part_out = rgrid.x; break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_reduce<EPI_RESID>, rgrid, rblk, 0, s, a); break;
    case EPI_RESID_SUMSQ: hipLaunchKernelGGL(gemm_reduce<EPI_RESID_SUMSQ>, rgrid, rblk, 0, s, a); *n_part_out = rgrid.x; break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_reduce<EPI_SWIGLU>, rgrid, rblk, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_f32(GemmArgs a, int epi, int* n_part_out, hipStream_t s) {
  if ((epi == EPI_BIAS_SUMSQ || epi == EPI_RESID_SUMSQ) && a.y2 && !a.gain_out) return hipErrorInvalidValue;
  const int nout = (epi == EPI_SWIGLU) ? a.ffn : a.N;
  dim3 grid((nout + 63) / 64, a.M), blk(64);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_f32<EPI_STORE>, grid, blk, 0, s, a); break;
    case EPI_BIAS_SUMSQ: hipLaunchKernelGGL(gemm_f32<EPI_BIAS_SUMSQ>, grid, blk, 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_f32<EPI_RESID>, grid, blk, 0, s, a); break;
    case EPI_RESID_SUMSQ: hipLaunchKernelGGL(gemm_f32<EPI_RESID_SUMSQ>, grid, blk, 0, s, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_f32<EPI_SWIGLU>, grid, blk, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  if (epi == EPI_BIAS_SUMSQ || epi == EPI_RESID_SUMSQ) *n_part_out = grid.x;
  return hipGetLastError();
}
