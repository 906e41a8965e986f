// Draft-head GEMMs on gfx950: y[M, N] = x[M, K] W[N, K]^T.
//
// The draft step's GEMMs stream the whole draft head and the LM head once per
// call; with a few rows they are bound by HBM, not by the matrix units
// (arithmetic intensity ~M flop/byte against a ridge of ~315); the tree-wide
// step over hundreds of rows is bound by the matrix units.  So:
//  * W (bf16) is the MFMA "A" operand.  In the skinny and wide kernels it goes
//    straight from HBM to VGPRs, each lane pulling 64 contiguous bytes of a row
//    per step, never through LDS, because every W element is used by exactly
//    one wave there.
//  * x (fp32) is the MFMA "B" operand (M padded to 16).  The skinny kernel
//    (M <= 16) loads each k-step's rows of x coalesced and re-reads them in the
//    B layout from the wave's own LDS slice.  Above 16 rows the operand arrives
//    in bf16 (hi and lo halves, or one rounded half), written by the producing
//    GEMM's epilogue or a prep pass, and the wide kernel (weights to VGPRs,
//    activation tile shared through LDS: up to 128 and from 161 to 256 rows) or
//    the large-M kernel (both operands loaded straight into LDS, shared by the
//    waves: from 129 to 160 rows with 160-row tiles, from 257 rows with
//    256-row tiles) consumes it.
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
#include <hip/hip_ext.h>

#include "common.h"
#include "gemm.h"

namespace {

// Kernel start/stop events for the next skinny launch (gemm_set_kernel_events).
hipEvent_t g_kev_start = nullptr, g_kev_stop = nullptr;

template <typename K>
void launch_skinny_kernel(K kernel, dim3 grid, dim3 blk, hipStream_t s, const GemmArgs& a) {
  if (g_kev_start) {
    hipExtLaunchKernelGGL(kernel, grid, blk, 0, s, g_kev_start, g_kev_stop, 0, a);
    g_kev_start = g_kev_stop = nullptr;
  } else {
    hipLaunchKernelGGL(kernel, grid, blk, 0, s, a);
  }
}

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

// Logical row n in the blocked copies wb0..wb2: the start of its first 32
// columns in the first block of its 16-row band.  Columns 32 g.. of the row
// are 512 g further, the next k-step's slice one block (2048 values) further;
// lane (r, g) of a 16-row tile thus reads the 64 bytes at 64 (16 g + r) of the
// block, adjacent lanes adjacent bytes.
__device__ __forceinline__ const bf16_t* wrow_blocked(const GemmArgs& a, int n) {
  const void* base;
  if (n < a.n_seg0) {
    base = a.wb0;
  } else if (n - a.n_seg0 < a.n_seg1) {
    base = a.wb1;
    n -= a.n_seg0;
  } else {
    base = a.wb2;
    n -= a.n_seg0 + a.n_seg1;
  }
  return (const bf16_t*)base + (size_t)(n >> 4) * (a.K / 128) * 2048 + (n & 15) * 32;
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
__device__ __forceinline__ void row_scales_lds(const GemmArgs& a, int BM, float* scale, int row0 = 0) {
  constexpr int ROWS = NT / 32;
  const int t = threadIdx.x, c = t & 31;
  for (int m0 = 0; m0 < BM; m0 += ROWS) {
    const int m = m0 + t / 32, mg = row0 + m;
    float s = 0.f;
    if (m < BM && mg < a.M)
      for (int p = c; p < a.n_part_in; p += 32) s += a.sumsq_in[(size_t)p * a.M + mg];
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, WAVE);
    if (c == 0 && m < BM) scale[m] = (mg < a.M) ? rms_scale(s, a) : 1.f;
  }
}

// Eight bf16 operand values as (hi, lo) pairs.
struct B8 {
  u32x4 hi, lo;
};

// Outputs n..n+3 of row m as the next GEMM's split operand: hi at
// xb_out[m][n], lo at xb_out[M + m][n] (rows of `width` values).
__device__ __forceinline__ void put_split4(const GemmArgs& a, int m, int n, int width, float4 v) {
  put_split4((bf16_t*)a.xb_out + (size_t)m * width + n, (size_t)a.M * width, v);
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

// fp32 -> bf16 round to nearest even, two values per instruction
// (v_cvt_pk_bf16_f32; value a in the low half).
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4 round8(float4 v0, float4 v1, float sc) {
  return u32x4{cvt2(v0.x * sc, v0.y * sc), cvt2(v0.z * sc, v0.w * sc), cvt2(v1.x * sc, v1.y * sc),
               cvt2(v1.z * sc, v1.w * sc)};
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
  } else if constexpr (EPI == EPI_ROPE) {
    // a 16-row tile holds 8 rotary pairs (e, e + hd/2) of one head: rows 0-7
    // are columns 8j..8j+7 of the head, rows 8-15 the same plus hd/2
    static_assert(AT == 1, "one 16-row tile per workgroup");
    const int tph = a.rp_hd >> 4, hb = tile / tph, j = tile % tph;
    const int n = hb * a.rp_hd + (r < 8 ? 8 * j + r : (a.rp_hd >> 1) + 8 * j + r - 8);
    *ok = n < a.N;
    return *ok ? n : 0;
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

template <int AT, int NW, int MQ, int NS, bool A16, int EPI>
__global__ void __launch_bounds__(NW * 64) gemm_skinny(GemmArgs a) {
  constexpr int XR = 2 * MQ;  // activation rows this instance can hold
  constexpr int BN = 16 * AT;
  constexpr int XL = NW * XR * SK_XROW, RED = NW * 16 * (BN + 4);
  // per-wave activation slices during the main loop, then the cross-wave reduction
  __shared__ float smem[XL > RED ? XL : RED];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x;

  // weights row-major (a k-step further: 128 values) or blocked (one 4 KB block)
  const bool blocked = a.wb0 != nullptr;
  const size_t kstride = blocked ? 2048 : SK_KSTEP;
  const bf16_t* ap[AT];
#pragma unroll
  for (int at = 0; at < AT; ++at) {
    bool ok;
    const int n = tile_row<AT, EPI>(a, tile, at, r, &ok);
    ap[at] = blocked ? wrow_blocked(a, n) + g * 512 : wrow<bf16_t>(a, n) + g * 32;
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
      for (int j = 0; j < 4; ++j) st.A[at][j] = *(const u32x4*)(ap[at] + (size_t)ks * kstride + j * 8);
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
  // bf16 activations are rounded after the RMSNorm row scale, so the scales
  // are needed before the first product
  float xs = 1.f;
  if constexpr (A16) {
    if (a.sumsq_in) {
      __syncthreads();
      xs = scale[r];
    }
  }

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
      if constexpr (A16) {
        const u32x4 B = round8(v0, v1, xs);
#pragma unroll
        for (int at = 0; at < AT; ++at) acc[at] = mfma16(st.A[at][j], B, acc[at]);
      } else {
        const B8 B = split8(v0, v1);
#pragma unroll
        for (int at = 0; at < AT; ++at) {
          acc[at] = mfma16(st.A[at][j], B.hi, acc[at]);
          acc[at] = mfma16(st.A[at][j], B.lo, acc[at]);
        }
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

  if constexpr (EPI == EPI_ROPE) {
    // rows m, pairs pi: x0 = column 8j + pi of head hb, x1 = its partner hd/2
    // further.  Angles pos * theta^(-2e/hd) in fp64 (a position in the
    // thousands keeps its phase exact to fp32), the rotation in fp32.
    const int hd = a.rp_hd, half = hd >> 1, tph = hd >> 4;
    const int hb = tile / tph, j = tile % tph;
    for (int e = threadIdx.x; e < 16 * 8; e += NW * 64) {
      const int m = e >> 3, pi = e & 7;
      if (m >= a.M || hb * hd >= a.N) continue;
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        x0 += red[w][m][pi];
        x1 += red[w][m][pi + 8];
      }
      if (!A16 && a.sumsq_in) {
        x0 *= scale[m];
        x1 *= scale[m];
      }
      const int ee = 8 * j + pi;
      float y0 = x0, y1 = x1;
      if (hb < a.rp_hq + a.rp_hkv) {
        const double inv = exp2(-2.0 * (double)ee / (double)hd * log2((double)a.rp_theta));
        double sd, cd;
        sincos((double)a.rp_pos[m] * inv, &sd, &cd);
        const float c = (float)cd, sv = (float)sd;
        y0 = x0 * c - x1 * sv;
        y1 = x1 * c + x0 * sv;
      }
      if (hb < a.rp_hq) {
        float* qo = a.y + (size_t)m * a.ldy + (size_t)hb * hd;
        qo[ee] = y0;
        qo[ee + half] = y1;
      } else {
        int b = 0;
        for (int i = 0; i < a.rp_batch; ++i)
          if (a.rp_row_start[i] <= m && m < a.rp_row_start[i + 1]) b = i;
        const bool isk = hb < a.rp_hq + a.rp_hkv;
        const int g = isk ? hb - a.rp_hq : hb - a.rp_hq - a.rp_hkv;
        bf16_t* dst = (bf16_t*)(isk ? a.rp_tree_k : a.rp_tree_v) +
                      (((size_t)b * 64 + a.rp_slot[m]) * a.rp_hkv + g) * hd;
        dst[ee] = f2bf(y0);
        dst[ee + half] = f2bf(y1);
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
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
        if (!A16 && a.sumsq_in) {
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
        if (!A16 && a.sumsq_in) y *= scale[m];
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

// Grid of the large-M kernel: weight tiles x activation tiles x K splits.
// With a split tail, the first `full` tiles (whole weight tiles, a multiple
// of 8 workgroups) run unsplit and the remaining tiles run `splits`-way split,
// so that the last round of workgroups is filled with shorter ones.
struct BigPlan {
  int tiles_n, tiles_m, splits;
  int full;  // tiles launched unsplit before the split ones (0: every tile split `splits` ways)
};

// ---------------------------------------------------------------------------
// Wide kernel: bf16 activations (act_bf16) and M > 16.  Both operands are
// bf16 in memory: a prep pass (act_prep) writes the activation operand once,
// bf16(x * RMSNorm row scale), or bf16 of the gathered [f ; e] rows.
//  * 4 waves; wave w owns 16*AT weight rows (the MFMA A operand), streamed from
//    HBM straight into VGPRs through an NS-stage register ring exactly as in
//    the skinny kernel (lane (r, g) takes 32 contiguous k of row r per k-step).
//  * The activation tile [16*MB rows][128 k] is the B operand, shared by the
//    four waves through LDS (two buffers, one barrier per k-step); each
//    thread prefetches its part of the next-but-one tile into registers.
//  * M is split into tiles of at most 128 rows; consecutive workgroups take
//    the M tiles of one weight tile and are kept on one XCD (shared L2), so
//    the weights leave HBM about once.  K is split over the grid while the
//    grid would leave CUs idle; gemm_reduce then sums the partials.
// ---------------------------------------------------------------------------
constexpr int WD_XLD = SK_KSTEP + 8;  // LDS row of the activation tile (bf16): 272 B, rows 4 banks apart

struct WidePlan {
  int tiles_n, tiles_m, splits;  // K split sp covers k-steps [sp*nks/splits, (sp+1)*nks/splits)
};

template <int NW, int AT, int MB, int NS, bool SPLIT, int EPI>
__global__ void __launch_bounds__(NW * 64) gemm_wide(GemmArgs a, const bf16_t* __restrict__ xb, WidePlan p) {
  constexpr int NT = NW * 64, BM = 16 * MB;
  constexpr int NH = SPLIT ? 2 : 1;  // operand halves: hi (and lo, at xb + M*K)
  constexpr int XCH = (BM * 16 + NT - 1) / NT;  // 16-byte activation chunks per thread per k-step and half
  __shared__ __attribute__((aligned(16))) bf16_t Xs[2][NH][BM][WD_XLD];
  __shared__ float ssq_s[NW][BM];
  __shared__ float rs_s[BM];  // RMSNorm row scales of an operand handed over unscaled (xb_in)
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int lid = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;  // consecutive tiles on one XCD
  const int mt = lid % p.tiles_m, rest = lid / p.tiles_m;
  const int nt = rest % p.tiles_n, sp = rest / p.tiles_n;
  const int m0 = mt * BM;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int r = lane & 15, g = lane >> 4;
  // row scales for the epilogue of an unsplit launch (visible after the main loop's barriers)
  const bool scale_rows = a.sumsq_in != nullptr && p.splits == 1;
  if (scale_rows) row_scales_lds<NT>(a, BM, rs_s, m0);
  const int nks_all = a.K / SK_KSTEP;
  const int ks0 = sp * nks_all / p.splits;
  const int nks = (sp + 1) * nks_all / p.splits - ks0;

  const int wtile = nt * NW + wv;  // this wave's tile of 16*AT weight rows
  // weights row-major (a k-step further: 128 values) or blocked (one 4 KB block)
  const bool blocked = a.wb0 != nullptr;
  const size_t kstride = blocked ? 2048 : SK_KSTEP;
  const bf16_t* ap[AT];
#pragma unroll
  for (int at = 0; at < AT; ++at) {
    bool ok;
    const int n = tile_row<AT, EPI>(a, wtile, at, r, &ok);
    ap[at] = blocked ? wrow_blocked(a, n) + g * 512 : wrow<bf16_t>(a, n) + g * 32;
  }
  // activation chunks: chunk c = t + NT u covers tile row c / 16, columns 8 (c % 16) .. + 7
  const bf16_t* xp[XCH];
  bool xv[XCH], xl[XCH];
#pragma unroll
  for (int u = 0; u < XCH; ++u) {
    const int c = t + NT * u, m = m0 + (c >> 4);
    xl[u] = c < BM * 16;  // chunk inside the tile
    xv[u] = xl[u] && m < a.M;
    xp[u] = xb + (size_t)(xv[u] ? m : 0) * a.K + (c & 15) * 8;
  }
  const size_t lo_off = (size_t)a.M * a.K;
  u32x4 xr[NH][XCH];
  auto load_x = [&](int ks) {
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int u = 0; u < XCH; ++u)
        xr[h][u] = xv[u] ? *(const u32x4*)(xp[u] + h * lo_off + (size_t)ks * SK_KSTEP) : u32x4{0, 0, 0, 0};
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int u = 0; u < XCH; ++u) {
        const int c = t + NT * u;
        if (xl[u]) *(u32x4*)&Xs[buf][h][c >> 4][(c & 15) * 8] = xr[h][u];
      }
  };
  struct Stage {
    u32x4 A[AT][4];
  };
  Stage S[NS];
  auto issue = [&](Stage& st, int ks) {
#pragma unroll
    for (int at = 0; at < AT; ++at)
#pragma unroll
      for (int j = 0; j < 4; ++j) st.A[at][j] = *(const u32x4*)(ap[at] + (size_t)ks * kstride + j * 8);
  };

  floatx4 acc[AT][MB];
#pragma unroll
  for (int at = 0; at < AT; ++at)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[at][mb] = floatx4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nks) issue(S[st], ks0 + st);
  if (nks > 0) {
    load_x(ks0);
    store_x(0);
    if (nks > 1) load_x(ks0 + 1);
  }
  __syncthreads();

  for (int s0 = 0; s0 < nks; s0 += NS) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int s = s0 + st;
      if (s >= nks) break;
      if (s + NS - 1 < nks) issue(S[(st + NS - 1) % NS], ks0 + s + NS - 1);
      const int buf = s & 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          u32x4 B[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) B[mb] = *(const u32x4*)&Xs[buf][h][mb * 16 + r][g * 32 + j * 8];
#pragma unroll
          for (int at = 0; at < AT; ++at)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[at][mb] = mfma16(S[st].A[at][j], B[mb], acc[at][mb]);
        }
      }
      if (s + 1 < nks) {
        store_x(buf ^ 1);
        if (s + 2 < nks) load_x(ks0 + s + 2);
      }
      __syncthreads();
    }
  }

  // lane (r, g): acc[at][mb][v] = output row m0 + 16 mb + r, logical weight row 16 at + 4 g + v of the wave's tile
  if (p.splits > 1) {
    float* P = a.part + (size_t)sp * a.M * a.N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 16 + r;
      if (m >= a.M) continue;
#pragma unroll
      for (int at = 0; at < AT; ++at) {
        bool ok;
        const int n = tile_row<AT, EPI>(a, wtile, at, 4 * g, &ok);  // 4 consecutive logical rows
        if (ok) *(floatx4*)(P + (size_t)m * a.N + n) = acc[at][mb];
      }
    }
    return;
  }
  if constexpr (EPI == EPI_SWIGLU) {
    constexpr int H = AT / 2;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 16 + r;
      if (m >= a.M) continue;
      const float rs = scale_rows ? rs_s[mb * 16 + r] : 1.f;
#pragma unroll
      for (int at = 0; at < H; ++at) {
        const int j = wtile * 16 * H + at * 16 + 4 * g;
        if (j >= a.ffn) continue;
        float4 o;
        o.x = silu_f(acc[at][mb][0] * rs) * (acc[at + H][mb][0] * rs);
        o.y = silu_f(acc[at][mb][1] * rs) * (acc[at + H][mb][1] * rs);
        o.z = silu_f(acc[at][mb][2] * rs) * (acc[at + H][mb][2] * rs);
        o.w = silu_f(acc[at][mb][3] * rs) * (acc[at + H][mb][3] * rs);
        if (a.yb) *(float4*)(a.yb + (size_t)m * a.ldyb + j) = o;
        if (a.xb_out) put_split4(a, m, j, a.ffn, o);
      }
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int ml = mb * 16 + r, m = m0 + ml;
      const bool mv = m < a.M;
      const float rs = (scale_rows && mv) ? rs_s[ml] : 1.f;
      float ss = 0.f;
#pragma unroll
      for (int at = 0; at < AT; ++at) {
        const int n = wtile * 16 * AT + at * 16 + 4 * g;
        if (!mv || n >= a.N) continue;
        float4 y = make_float4(acc[at][mb][0] * rs, acc[at][mb][1] * rs, acc[at][mb][2] * rs, acc[at][mb][3] * rs);
        if constexpr (EPI == EPI_BIAS_SUMSQ) {
          const bf16_t* bb = (const bf16_t*)a.bias + n;
          y.x += bf2f(bb[0]); y.y += bf2f(bb[1]); y.z += bf2f(bb[2]); y.w += bf2f(bb[3]);
        }
        if constexpr (EPI == EPI_RESID || EPI == EPI_RESID_SUMSQ) {
          const float4 rr = *(const float4*)(a.resid + (size_t)m * a.ldr + n);
          y.x += rr.x; y.y += rr.y; y.z += rr.z; y.w += rr.w;
        }
        *(float4*)(a.y + (size_t)m * a.ldy + n) = y;
        float4 nx = y;  // the next GEMM's operand: y2 when written, else y
        if constexpr (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
          if (a.gain_out) {
            const bf16_t* gn = (const bf16_t*)a.gain_out + n;
            nx = make_float4(y.x * bf2f(gn[0]), y.y * bf2f(gn[1]), y.z * bf2f(gn[2]), y.w * bf2f(gn[3]));
            if (a.y2) *(float4*)(a.y2 + (size_t)m * a.ldy + n) = nx;
          }
          ss += y.x * y.x + y.y * y.y + y.z * y.z + y.w * y.w;
        }
        if (a.xb_out) put_split4(a, m, n, a.N, nx);
      }
      if constexpr (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
        ss += __shfl_xor(ss, 16, WAVE);
        ss += __shfl_xor(ss, 32, WAVE);
        if (g == 0) ssq_s[wv][ml] = ss;
      }
    }
    if constexpr (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
      __syncthreads();
      if (t < BM && m0 + t < a.M) {
        float q = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) q += ssq_s[w][t];
        a.sumsq_out[(size_t)nt * a.M + m0 + t] = q;
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Large-M kernel (M above a few hundred rows, where the matrix units are the
// bound): WN x WM waves, each owning TN x TM blocks of 16 x 16 outputs
// (weight rows x activation rows), K staged in blocks of 32 through LDS (two
// buffers, the next block's global loads in flight in registers), both
// operands from the prepared bf16 operand (hi and lo halves: two MFMAs per
// product).  The MFMAs per LDS fragment a wave reads grow with its tile,
// TN*TM / (TN + NH*TM).  Consecutive tiles stay on one XCD so the workgroups
// sharing a weight tile share an L2.  SwiGLU: per wave, TN/2 blocks of gate
// rows, then the up rows of the same ffn columns, so gate and up meet in one
// lane.
// LDS layout: tile rows of 64 bytes (32 bf16 of K, four 16-byte chunks) with
// no padding; chunk c of row r sits in slot c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1),
// so the stores (four lanes per row) stay contiguous: with rows padded to 80
// bytes instead the kernel ran 10-20% slower at the 70B shapes.  (The LDS
// bank-conflict counter still reports ~1.3 cycles per fragment read for this
// layout, as for plain row-major rows; a layout it reports conflict-free for
// both the fragment reads and the stores, chunk c of row r of each 16-row
// block in slot ((r / 8) * 4 + c) * 8 + (r + 2 c) % 8, ran no faster at the
// 13B and 70B shapes, so counted conflicts are not what bounds this kernel.)
// ---------------------------------------------------------------------------
template <int WN_, int WM_, int TN_, int TM_, int BK_>
struct TileCfg {
  static constexpr int WN = WN_, WM = WM_, TN = TN_, TM = TM_, BK = BK_;
  static constexpr int BN = WN * TN * 16, BM = WM * TM * 16;
  static constexpr int NT = WN * WM * 64;  // threads of a workgroup
  static_assert(BK % 32 == 0, "whole MFMA k-steps");
};

__device__ __forceinline__ int swz_slot(int row, int c) { return row * 4 + (c ^ ((row >> 1) & 3) ^ ((row >> 3) & 1)); }
// the chunk of tile row `row` that the layout keeps in that row's slot s
__device__ __forceinline__ int swz_chunk(int row, int s) { return s ^ ((row >> 1) & 3) ^ ((row >> 3) & 1); }
// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr unsigned WAIT_VM0 = 0x0F70;         // vmcnt(0)
constexpr unsigned WAIT_LGKM0_VM0 = 0x0070;   // vmcnt(0) lgkmcnt(0)
constexpr unsigned WAIT_LGKM0 = 0x0070;       // lgkmcnt(0), vmcnt(n) with n in bits 3:0 (n < 16)

template <int EPI, bool SPLIT, class T>
__global__ void __launch_bounds__(T::NT) gemm_tile(GemmArgs a, const bf16_t* __restrict__ xb, BigPlan p) {
  constexpr int NH = SPLIT ? 2 : 1, NT = T::NT;
  constexpr int BN = T::BN, BM = T::BM, BK = T::BK, TN = T::TN, TM = T::TM;
  static_assert(BK == 32, "four 16-byte chunks per tile row");
  constexpr int ASL = BN * 4, BSL = BM * 4;  // 16-byte slots of the weight and activation tiles
  constexpr int SLOTS = ASL + NH * BSL;       // one block
  static_assert(ASL % NT == 0, "whole load rounds of weights");
  constexpr int AR = ASL / NT;                              // loads per thread and block: weights
  constexpr int ROUNDS = (SLOTS + NT - 1) / NT;             // all loads per thread and block
  constexpr int SLOTS_PAD = ROUNDS * NT;  // a buffer: the last round's spare lanes load into the padding
  static_assert(ROUNDS < 16, "vmcnt immediate");
  __shared__ __attribute__((aligned(16))) u32x4 L[3][SLOTS_PAD];
  __shared__ float ssq_s[T::WN][BM];
  __shared__ float rs_s[BM];  // RMSNorm row scales of an operand handed over unscaled (xb_in)
  // workgroups [0, full) take whole tiles, the rest the split tiles; within
  // each part consecutive tiles stay on one XCD (both parts are whole
  // multiples of 8 workgroups when full > 0)
  const int bid = blockIdx.x;
  const bool head = bid < p.full;
  const int nwg = head ? p.full : gridDim.x - p.full, b = head ? bid : bid - p.full;
  const int lid = (nwg % 8 == 0) ? (b % 8) * (nwg / 8) + b / 8 : b;
  const int splits = head ? 1 : p.splits;
  const int ntail = p.tiles_n * p.tiles_m - p.full;  // tiles of the split part
  const int tile = head ? lid : p.full + lid % ntail, sp = head ? 0 : lid / ntail;
  const int mt = tile % p.tiles_m, nt = tile / p.tiles_m;
  const int m0 = mt * BM;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  // row scales for the epilogue of an unsplit launch (visible after the main loop's barriers)
  const bool scale_rows = a.sumsq_in != nullptr && splits == 1;
  if (scale_rows) row_scales_lds<NT>(a, BM, rs_s, m0);
  const int wn = wv % T::WN, wm = wv / T::WN;
  const int r = lane & 15, g = lane >> 4;
  // K blocks of this split: the K / BK blocks spread evenly over the splits
  const int nkb_all = a.K / BK, kb0 = sp * nkb_all / splits;
  const int kbeg = kb0 * BK, nkb = (sp + 1) * nkb_all / splits - kb0;

  auto wrow_of = [&](int i) -> int {
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int WR = TN * 16, HR = TN * 8;
      const int q = i / WR, w = i % WR;
      const int j = nt * (BN / 2) + q * HR + (w % HR);
      if (j >= a.ffn) return -1;
      return (w < HR) ? j : a.ffn + j;
    } else {
      const int n = nt * BN + i;
      return n < a.N ? n : -1;
    }
  };
  // load u of a block: 16-byte slot q = u*NT + t of the buffer, chunk (q & 3)
  // of tile row q >> 2.  Rows past the end of W or x are read from row 0
  // (finite values whose outputs are never stored), so every load is
  // unconditional.
  // Blocked weights: a 32-column block of a 16-row band is 16 rows of 32
  // values, 512 values after the previous one (also across 128-column blocks),
  // so the K blocks of a row step by 512 instead of 32.
  const bool blocked = a.wb0 != nullptr;
  const int wstep = blocked ? 16 : 1;
  const size_t lo_off = (size_t)a.M * a.K;
  const bf16_t* src[ROUNDS];
#pragma unroll
  for (int u = 0; u < ROUNDS; ++u) {
    const int q = u * NT + t;
    if (u < AR) {
      const int row = q >> 2, n = wrow_of(row), nn = n >= 0 ? n : 0;
      src[u] = (blocked ? wrow_blocked(a, nn) : wrow<bf16_t>(a, nn)) + (size_t)kbeg * wstep + swz_chunk(row, q & 3) * 8;
    } else if (q >= SLOTS) {
      src[u] = xb + kbeg;  // padding slot: any readable 16 bytes
    } else {
      const int q2 = q - ASL, h = q2 / BSL, q3 = q2 % BSL;
      const int row = q3 >> 2, m = m0 + row < a.M ? m0 + row : 0;
      src[u] = xb + h * lo_off + (size_t)m * a.K + kbeg + swz_chunk(row, q3 & 3) * 8;
    }
  }
  // Block kb goes straight from memory to LDS (global_load_lds: lane l of a
  // wave writes 16 bytes at the wave's base + 16 l), load u of thread t into
  // slot u*NT + t, so each lane loads the chunk the swizzled layout keeps
  // there.  Nothing passes through registers.
  auto dma = [&](int kb, int buf) {
    const int k0 = kb * BK;
#pragma unroll
    for (int u = 0; u < ROUNDS; ++u)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src[u] + (size_t)k0 * (u < AR ? wstep : 1)),
                                       (__attribute__((address_space(3))) void*)&L[buf][u * NT + wv * 64], 16, 0, 0);
  };

  floatx4 acc[TN][TM];
#pragma unroll
  for (int nb = 0; nb < TN; ++nb)
#pragma unroll
    for (int mb = 0; mb < TM; ++mb) acc[nb][mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // a wave's LDS fragments of one block: TN weight blocks, then TM activation
  // blocks per operand half
  constexpr int NF = TN + NH * TM;
  auto read_frags = [&](u32x4 (&F)[NF], int buf) {
    const u32x4* B0 = L[buf];
#pragma unroll
    for (int nb = 0; nb < TN; ++nb) F[nb] = B0[swz_slot((wn * TN + nb) * 16 + r, g)];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int mb = 0; mb < TM; ++mb) F[TN + h * TM + mb] = B0[ASL + h * BSL + swz_slot((wm * TM + mb) * 16 + r, g)];
  };
  auto mfma_frags = [&](const u32x4 (&F)[NF]) {
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int nb = 0; nb < TN; ++nb)
#pragma unroll
        for (int mb = 0; mb < TM; ++mb) acc[nb][mb] = mfma16(F[nb], F[TN + h * TM + mb], acc[nb][mb]);
  };
  // Three LDS buffers, block kb in buffer kb % 3; blocks 0 and 1 are in flight
  // before the loop.
  if (nkb > 0) dma(0, 0);
  if (nkb > 1) dma(1, 1);
  __builtin_amdgcn_s_waitcnt(WAIT_VM0);  // this thread's loads have landed
  __syncthreads();
  // Two wave groups, one wave of each per SIMD (waves w and w + NW/2 share a
  // SIMD), run a block in two phases separated by barriers: an LDS phase (the
  // block's fragments into registers, block kb + 2 requested into the buffer
  // of block kb - 1) and a matrix phase (the block's MFMAs).  The second group
  // starts one barrier later, so while one wave of a SIMD reads LDS the other
  // keeps the matrix pipe busy.  Every wave passes the same number of barriers
  // (the first group takes its extra one after the loop); the group test is on
  // a wave-uniform scalar, so the skipped barrier is a scalar branch.
  // Ordering (phases counted from the first group's first LDS phase, 2kb + 1
  // for its block kb and 2kb + 2 for the second group's): block kb + 2 is
  // requested in phases 2kb + 1 and 2kb + 2 into the buffer of block kb - 1,
  // whose last reader ran in phase 2kb; each wave ends its LDS phase waiting
  // for all but the loads it has just issued, so block kb + 1 has landed
  // before the barrier that precedes its first reader (phase 2kb + 3).  The
  // in-loop barriers carry no memory fence (a fence would wait for the loads
  // just issued); the explicit waits and scheduling barriers order the LDS
  // traffic instead.
  const bool late = __builtin_amdgcn_readfirstlane(wv) >= T::WN * T::WM / 2;
  if (late) __syncthreads();
  int buf = 0;
  for (int kb = 0; kb < nkb; ++kb) {
    u32x4 F[NF];
    read_frags(F, buf);
    const bool more = kb + 2 < nkb;
    if (more) dma(kb + 2, buf == 0 ? 2 : buf - 1);
    if (more)
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0 | ROUNDS);  // only the block just requested may still fly
    else
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0_VM0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    mfma_frags(F);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    buf = buf == 2 ? 0 : buf + 1;
  }
  if (!late) __syncthreads();

  // lane (r, g): acc[nb][mb][v] = tile row (wn*TN + nb)*16 + 4g + v, activation row (wm*TM + mb)*16 + r
  if (splits > 1) {
    float* P = a.part + (size_t)sp * a.M * a.N;
#pragma unroll
    for (int mb = 0; mb < TM; ++mb) {
      const int m = m0 + (wm * TM + mb) * 16 + r;
      if (m >= a.M) continue;
#pragma unroll
      for (int nb = 0; nb < TN; ++nb) {
        const int n = wrow_of((wn * TN + nb) * 16 + 4 * g);
        if (n >= 0) *(floatx4*)(P + (size_t)m * a.N + n) = acc[nb][mb];
      }
    }
    return;
  }
  if constexpr (EPI == EPI_SWIGLU) {
    constexpr int H = TN / 2;
#pragma unroll
    for (int mb = 0; mb < TM; ++mb) {
      const int ml = (wm * TM + mb) * 16 + r, m = m0 + ml;
      if (m >= a.M) continue;
      const float rs = scale_rows ? rs_s[ml] : 1.f;
#pragma unroll
      for (int nb = 0; nb < H; ++nb) {
        const int j = nt * (BN / 2) + wn * (TN * 8) + nb * 16 + 4 * g;
        if (j >= a.ffn) continue;
        float4 o;
        o.x = silu_f(acc[nb][mb][0] * rs) * (acc[nb + H][mb][0] * rs);
        o.y = silu_f(acc[nb][mb][1] * rs) * (acc[nb + H][mb][1] * rs);
        o.z = silu_f(acc[nb][mb][2] * rs) * (acc[nb + H][mb][2] * rs);
        o.w = silu_f(acc[nb][mb][3] * rs) * (acc[nb + H][mb][3] * rs);
        if (a.yb) *(float4*)(a.yb + (size_t)m * a.ldyb + j) = o;
        if (a.xb_out) put_split4(a, m, j, a.ffn, o);
      }
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < TM; ++mb) {
      const int ml = (wm * TM + mb) * 16 + r, m = m0 + ml;
      const bool mv = m < a.M;
      const float rs = (scale_rows && mv) ? rs_s[ml] : 1.f;
      float ss = 0.f;
#pragma unroll
      for (int nb = 0; nb < TN; ++nb) {
        const int n = nt * BN + (wn * TN + nb) * 16 + 4 * g;
        if (!mv || n >= a.N) continue;
        float4 y = make_float4(acc[nb][mb][0] * rs, acc[nb][mb][1] * rs, acc[nb][mb][2] * rs, acc[nb][mb][3] * rs);
        if constexpr (EPI == EPI_BIAS_SUMSQ) {
          const bf16_t* bb = (const bf16_t*)a.bias + n;
          y.x += bf2f(bb[0]); y.y += bf2f(bb[1]); y.z += bf2f(bb[2]); y.w += bf2f(bb[3]);
        }
        if constexpr (EPI == EPI_RESID || EPI == EPI_RESID_SUMSQ) {
          const float4 rr = *(const float4*)(a.resid + (size_t)m * a.ldr + n);
          y.x += rr.x; y.y += rr.y; y.z += rr.z; y.w += rr.w;
        }
        *(float4*)(a.y + (size_t)m * a.ldy + n) = y;
        float4 nx = y;  // the next GEMM's operand: y2 when written, else y
        if constexpr (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
          if (a.gain_out) {
            const bf16_t* gn = (const bf16_t*)a.gain_out + n;
            nx = make_float4(y.x * bf2f(gn[0]), y.y * bf2f(gn[1]), y.z * bf2f(gn[2]), y.w * bf2f(gn[3]));
            if (a.y2) *(float4*)(a.y2 + (size_t)m * a.ldy + n) = nx;
          }
          ss += y.x * y.x + y.y * y.y + y.z * y.z + y.w * y.w;
        }
        if (a.xb_out) put_split4(a, m, n, a.N, nx);
      }
      if constexpr (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
        ss += __shfl_xor(ss, 16, WAVE);
        ss += __shfl_xor(ss, 32, WAVE);
        if (g == 0) ssq_s[wn][ml] = ss;
      }
    }
    if constexpr (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
      __syncthreads();
      if (t < BM && m0 + t < a.M) {
        float q = 0.f;
#pragma unroll
        for (int w = 0; w < T::WN; ++w) q += ssq_s[w][t];
        a.sumsq_out[(size_t)nt * a.M + m0 + t] = q;
      }
    }
  }
}

// The bf16 activation operand of the wide and large-M kernels, from
// v = x[row(m)][k] * rs(m) (rs the RMSNorm row scale when sumsq_in is set,
// else 1) or from the gathered row [f_parent ; e(token)]:
//   SPLIT: xb[m][k] = hi(v) and xb[M*K + m*K + k] = lo(v), the split2 pair;
//   else:  xb[m][k] = bf16(v), round to nearest even.
// grid (ceil(K / 2048), M), 8 values per thread.
template <bool SPLIT>
__global__ void __launch_bounds__(256) act_prep(GemmArgs a, bf16_t* __restrict__ xb) {
  __shared__ float red[4];
  const int m = blockIdx.y;
  const int k = (blockIdx.x * 256 + threadIdx.x) * 8;
  float rs = 1.f;
  if (a.sumsq_in) {
    float sq = 0.f;
    for (int q = threadIdx.x; q < a.n_part_in; q += 256) sq += a.sumsq_in[(size_t)q * a.M + m];
    rs = rms_scale(block_sum<256>(sq, red), a);
  }
  if (k >= a.K) return;
  float4 v0, v1;
  if (a.gfeat) {
    if (k < a.gd) {
      const float* f = a.gfeat + (size_t)a.gparent[m] * a.gd + k;
      v0 = *(const float4*)f;
      v1 = *(const float4*)(f + 4);
    } else {
      const u32x4 e = *(const u32x4*)((const bf16_t*)a.gembed + (size_t)a.gtoken[m] * a.gd + (k - a.gd));
      v0 = make_float4(__uint_as_float(e[0] << 16), __uint_as_float(e[0] & 0xffff0000u), __uint_as_float(e[1] << 16),
                       __uint_as_float(e[1] & 0xffff0000u));
      v1 = make_float4(__uint_as_float(e[2] << 16), __uint_as_float(e[2] & 0xffff0000u), __uint_as_float(e[3] << 16),
                       __uint_as_float(e[3] & 0xffff0000u));
    }
  } else {
    const float* x = a.x + (size_t)(a.xrows ? a.xrows[m] : m) * a.ldx + k;
    v0 = *(const float4*)x;
    v1 = *(const float4*)(x + 4);
  }
  if constexpr (SPLIT) {
    v0.x *= rs; v0.y *= rs; v0.z *= rs; v0.w *= rs;
    v1.x *= rs; v1.y *= rs; v1.z *= rs; v1.w *= rs;
    const B8 h = split8(v0, v1);
    *(u32x4*)(xb + (size_t)m * a.K + k) = h.hi;
    *(u32x4*)(xb + (size_t)a.M * a.K + (size_t)m * a.K + k) = h.lo;
  } else {
    *(u32x4*)(xb + (size_t)m * a.K + k) = round8(v0, v1, rs);
  }
}

// Sum split-K partials and apply the epilogue.  grid (ceil(Nout/1024), M).
template <int EPI>
__global__ void __launch_bounds__(256) gemm_reduce(GemmArgs a, int n0) {
  __shared__ float red[4];
  const int m = blockIdx.y;
  const int n = n0 + blockIdx.x * 1024 + threadIdx.x * 4;
  const int nout = (EPI == EPI_SWIGLU) ? a.ffn : a.N;
  const size_t stride = (size_t)a.M * a.N;
  float rs = 1.f;
  if (a.sumsq_in && !a.act_bf16) {  // bf16 activations were scaled before rounding
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
      if (a.yb) *(float4*)(a.yb + (size_t)m * a.ldyb + n) = o;
      if (a.xb_out) put_split4(a, m, n, nout, o);
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
      float4 nx = s;  // the next GEMM's operand: y2 when written, else y
      if (EPI == EPI_BIAS_SUMSQ || EPI == EPI_RESID_SUMSQ) {
        if (a.gain_out) {
          const bf16_t* gn = (const bf16_t*)a.gain_out + n;
          nx = {s.x * bf2f(gn[0]), s.y * bf2f(gn[1]), s.z * bf2f(gn[2]), s.w * bf2f(gn[3])};
          if (a.y2) *(float4*)(a.y2 + (size_t)m * a.ldy + n) = nx;
        }
      }
      if (a.xb_out) put_split4(a, m, n, a.N, nx);
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

template <int AT, int NW, int MQ, bool A16, int NS = skinny_ns(AT, NW, MQ)>
hipError_t skinny_epi(const GemmArgs& a, int epi, int* n_part, hipStream_t s) {
  const int BN = 16 * AT;
  dim3 blk(NW * 64);
  const dim3 grid((a.N + BN - 1) / BN);
  switch (epi) {
    case EPI_STORE: launch_skinny_kernel(gemm_skinny<AT, NW, MQ, NS, A16, EPI_STORE>, grid, blk, s, a); break;
    case EPI_BIAS_SUMSQ:
      launch_skinny_kernel(gemm_skinny<AT, NW, MQ, NS, A16, EPI_BIAS_SUMSQ>, grid, blk, s, a);
      *n_part = grid.x;
      break;
    case EPI_RESID: launch_skinny_kernel(gemm_skinny<AT, NW, MQ, NS, A16, EPI_RESID>, grid, blk, s, a); break;
    case EPI_RESID_SUMSQ:
      launch_skinny_kernel(gemm_skinny<AT, NW, MQ, NS, A16, EPI_RESID_SUMSQ>, grid, blk, s, a);
      *n_part = grid.x;
      break;
    case EPI_ROPE:
      if constexpr (AT == 1) {
        if (a.rp_hd % 16 || a.N % a.rp_hd) return hipErrorInvalidValue;  // whole heads of 16-column pairs
        launch_skinny_kernel(gemm_skinny<AT, NW, MQ, NS, A16, EPI_ROPE>, grid, blk, s, a);
        break;
      } else {
        return hipErrorInvalidValue;
      }
    case EPI_SWIGLU:
      if constexpr (AT >= 2) {  // gate and up tiles pair up inside a workgroup
        const int H = BN / 2;
        launch_skinny_kernel(gemm_skinny<AT, NW, MQ, NS, A16, EPI_SWIGLU>, dim3((a.ffn + H - 1) / H), blk, s, a);
        break;
      } else {
        return hipErrorInvalidValue;
      }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int AT, int NW, bool A16>
hipError_t skinny_mq(const GemmArgs& a, int epi, int* n_part, hipStream_t s) {
  if (a.M <= 2) return skinny_epi<AT, NW, 1, A16>(a, epi, n_part, s);
  if (a.M <= 4) return skinny_epi<AT, NW, 2, A16>(a, epi, n_part, s);
  if (a.M <= 6) return skinny_epi<AT, NW, 3, A16>(a, epi, n_part, s);
  if (a.M <= 8) return skinny_epi<AT, NW, 4, A16>(a, epi, n_part, s);
  return skinny_epi<AT, NW, 8, A16>(a, epi, n_part, s);
}

// Variant choice, measured on the 7B draft-head shapes (N = 4096, 12288,
// 22016 gate+up, 32000; M = 1..16), weights streamed from HBM:
//  * fewer than 512 row tiles (N = 4096): one tile x 8 waves, so 256
//    workgroups of 8 waves cover the chip;
//  * SwiGLU: a gate and an up tile x 4 waves up to M = 8; x 8 waves above;
//  * wide N with M > 8: four tiles x 4 waves -- each activation chunk then
//    feeds four weight tiles, which matters once x is as large as the weights
//    a wave streams per step;
//  * the LM head (>= 1536 tiles, no input norm), M <= 4: one tile x 8 waves
//    (two workgroups per CU), with a four-stage ring at M <= 2; else, and
//    for qkv (whose workgroups first sum the input norm's partials), one tile
//    x 4 waves -- x 8 waves measured 15-20% slower for qkv inside the round.
template <bool A16>
hipError_t skinny_launch(const GemmArgs& a, int epi, int* n_part, hipStream_t s) {
  if (epi == EPI_SWIGLU)
    return a.M > 8 ? skinny_mq<2, 8, A16>(a, epi, n_part, s) : skinny_mq<2, 4, A16>(a, epi, n_part, s);
  const int tiles = (a.N + 15) / 16;
  if (tiles < 512) return skinny_mq<1, 8, A16>(a, epi, n_part, s);
  if (epi == EPI_ROPE) return skinny_mq<1, 4, A16>(a, epi, n_part, s);  // one 16-row tile per workgroup
  if (a.M > 8) return skinny_mq<4, 4, A16>(a, epi, n_part, s);
  if (tiles >= 1536 && a.M <= 2) return skinny_epi<1, 8, 1, A16, 4>(a, epi, n_part, s);
  if (tiles >= 1536 && a.M <= 4) return skinny_epi<1, 8, 2, A16>(a, epi, n_part, s);
  return skinny_mq<1, 4, A16>(a, epi, n_part, s);
}



// Wide-kernel shape: NW waves of 16*AT weight rows each, ring depth NS.
template <int NW, int AT, int NS>
struct WideCfg {
  static constexpr int nw = NW, at = AT, ns = NS, bn = 16 * AT * NW;
};
// Measured on the 13B / 70B per-depth shapes (M = 80, 160): 8 waves of 32
// weight rows with a two-stage ring (two waves per SIMD) beat 4 waves of 64
// rows with three stages by 5-10%.
using WideDefault = WideCfg<8, 2, 2>;

// Wide-kernel plan: M tiles of at most 16*mb_max rows (16*MB rows each, MB
// as small as covers M), BN-row weight tiles (BN/2 ffn columns for SwiGLU),
// and a K split of any count that keeps the grid within one workgroup per CU
// (target; the workgroup's LDS allows no second one) and each split at four
// or more k-steps.  Measured at M = 80 (13B shapes): split counts of 12
// instead of the next power of two (8 or 16, the latter a second, mostly
// empty wave of workgroups) make the K = 10240 and 13824 products 25-30%
// faster.
WidePlan plan_wide(int M, int N, int K, bool swiglu, int BN, int mb_max, int* mb, int target = 256,
                   bool pow2 = false) {
  WidePlan p;
  const int blocks16 = (M + 15) / 16;
  p.tiles_m = (blocks16 + mb_max - 1) / mb_max;
  *mb = (blocks16 + p.tiles_m - 1) / p.tiles_m;
  p.tiles_n = swiglu ? (N / 2 + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
  const int nks = K / SK_KSTEP;
  const int base = p.tiles_n * p.tiles_m;
  int splits = 1;
  if (pow2) {
    while (base * splits * 2 <= target && nks / (splits * 2) >= 4) splits *= 2;
  } else {
    while (base * (splits + 1) <= target && nks / (splits + 1) >= 4) ++splits;
  }
  p.splits = splits;
  return p;
}

size_t align_up256(size_t b) { return (b + 255) & ~(size_t)255; }

template <class C, int MB, bool SPLIT>
hipError_t wide_epi(const GemmArgs& a, int epi, const bf16_t* xb, const WidePlan& p, hipStream_t s) {
  constexpr int NS = (C::ns == 3 && MB > 6 && C::at == 4) ? 2 : C::ns;
  const dim3 grid(p.tiles_n * p.tiles_m * p.splits), blk(C::nw * 64);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_wide<C::nw, C::at, MB, NS, SPLIT, EPI_STORE>), grid, blk, 0, s, a, xb, p); break;
    case EPI_BIAS_SUMSQ:
      hipLaunchKernelGGL((gemm_wide<C::nw, C::at, MB, NS, SPLIT, EPI_BIAS_SUMSQ>), grid, blk, 0, s, a, xb, p);
      break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_wide<C::nw, C::at, MB, NS, SPLIT, EPI_RESID>), grid, blk, 0, s, a, xb, p); break;
    case EPI_RESID_SUMSQ:
      hipLaunchKernelGGL((gemm_wide<C::nw, C::at, MB, NS, SPLIT, EPI_RESID_SUMSQ>), grid, blk, 0, s, a, xb, p);
      break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_wide<C::nw, C::at, MB, NS, SPLIT, EPI_SWIGLU>), grid, blk, 0, s, a, xb, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class C, bool SPLIT>
hipError_t wide_mb(const GemmArgs& a, int epi, const bf16_t* xb, const WidePlan& p, int mb, hipStream_t s) {
  switch (mb) {
    case 2: return wide_epi<C, 2, SPLIT>(a, epi, xb, p, s);
    case 3: return wide_epi<C, 3, SPLIT>(a, epi, xb, p, s);
    case 4: return wide_epi<C, 4, SPLIT>(a, epi, xb, p, s);
    case 5: return wide_epi<C, 5, SPLIT>(a, epi, xb, p, s);
    case 6: return wide_epi<C, 6, SPLIT>(a, epi, xb, p, s);
    case 7: return wide_epi<C, 7, SPLIT>(a, epi, xb, p, s);
    case 8: return wide_epi<C, 8, SPLIT>(a, epi, xb, p, s);
    default: return hipErrorInvalidValue;  // M > 16 gives at least two 16-row blocks
  }
}

// Tiles of gemm_tile plus a K split (any count; the K blocks spread evenly,
// at least 16 per split).  A workgroup takes about the same time per K block
// whatever the split, and the grid runs in rounds of one workgroup per CU, so
// the count minimises (rounds x K blocks per split) plus the partial sums'
// write and re-read in gemm_reduce, priced at TILE_BLOCK_US per K block and
// REDUCE_BYTES_PER_US (measured at the 13B / 70B tree-wide shapes: about 1.45
// us per block, the reduce near 4 TB/s).  E.g. the 70B QKV product (160 tiles,
// 256 K blocks) takes 3 splits, 480 workgroups in two rounds of 86 blocks,
// instead of 2 splits in two rounds of 128.
constexpr double TILE_BLOCK_US = 1.45, REDUCE_BYTES_PER_US = 4.0e6;
// tail_ok: the epilogue has no per-tile sums of squares, so a split tail is
// allowed: with R whole rounds of tiles and a partial one, the tiles of the
// last round are split as far as one round holds them (the 70B gate/up
// product: 896 tiles, 768 unsplit and 128 split 2 ways, 3.5 rounds of full-K
// workgroups become 3 of them plus one of half length).
template <class T>
BigPlan plan_tile(int M, int N, int K, bool swiglu, bool tail_ok) {
  BigPlan p;
  p.tiles_n = swiglu ? (N / 2 + T::BN / 2 - 1) / (T::BN / 2) : (N + T::BN - 1) / T::BN;
  p.tiles_m = (M + T::BM - 1) / T::BM;
  p.full = 0;
  const int base = p.tiles_n * p.tiles_m, nkb = K / T::BK;
  p.splits = 1;
  double best = 0.0;
  for (int s = 1; s <= 16 && nkb / s >= 16; ++s) {
    const int rounds = (base * s + 255) / 256, per = (nkb + s - 1) / s;
    const double cost = rounds * per * TILE_BLOCK_US + (s > 1 ? 2.0 * s * M * N * 4 / REDUCE_BYTES_PER_US : 0.0);
    if (s == 1 || cost < best) {
      best = cost;
      p.splits = s;
    }
  }
  const int full = base / 256 * 256, ntail = base - full;
  if (tail_ok && full > 0 && ntail > 0 && full % p.tiles_m == 0) {
    int s2 = 1;
    while ((s2 + 1) * ntail <= 256 && nkb / (s2 + 1) >= 16) ++s2;
    if (s2 > 1) {
      const double cost = (full / 256) * nkb * TILE_BLOCK_US + (nkb + s2 - 1) / s2 * TILE_BLOCK_US +
                          2.0 * s2 * ntail * T::BM * T::BN * 4 / REDUCE_BYTES_PER_US;
      if (cost < best) {
        p.full = full;
        p.splits = s2;
      }
    }
  }
  return p;
}

template <class T, bool SPLIT>
hipError_t tile_epi(const GemmArgs& a, int epi, const bf16_t* xb, const BigPlan& p, hipStream_t s) {
  const dim3 grid(p.full + (p.tiles_n * p.tiles_m - p.full) * p.splits), blk(T::NT);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_tile<EPI_STORE, SPLIT, T>), grid, blk, 0, s, a, xb, p); break;
    case EPI_BIAS_SUMSQ: hipLaunchKernelGGL((gemm_tile<EPI_BIAS_SUMSQ, SPLIT, T>), grid, blk, 0, s, a, xb, p); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_tile<EPI_RESID, SPLIT, T>), grid, blk, 0, s, a, xb, p); break;
    case EPI_RESID_SUMSQ: hipLaunchKernelGGL((gemm_tile<EPI_RESID_SUMSQ, SPLIT, T>), grid, blk, 0, s, a, xb, p); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_tile<EPI_SWIGLU, SPLIT, T>), grid, blk, 0, s, a, xb, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Reduce of the K-split partials and the epilogue, over output columns
// [n0, end): n0 > 0 (a split tail, whose earlier columns were written by the
// unsplit tiles) only for epilogues without per-block sums of squares.
hipError_t reduce_launch(const GemmArgs& a, int epi, int* n_part_out, hipStream_t s, int n0 = 0) {
  const int nout = (epi == EPI_SWIGLU) ? a.ffn : a.N;
  if (n0 && (epi == EPI_BIAS_SUMSQ || epi == EPI_RESID_SUMSQ)) return hipErrorInvalidValue;
  dim3 rgrid((nout - n0 + 1023) / 1024, a.M), rblk(256);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_reduce<EPI_STORE>, rgrid, rblk, 0, s, a, n0); break;
    case EPI_BIAS_SUMSQ: hipLaunchKernelGGL(gemm_reduce<EPI_BIAS_SUMSQ>, rgrid, rblk, 0, s, a, n0); *n_part_out = rgrid.x; break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_reduce<EPI_RESID>, rgrid, rblk, 0, s, a, n0); break;
    case EPI_RESID_SUMSQ: hipLaunchKernelGGL(gemm_reduce<EPI_RESID_SUMSQ>, rgrid, rblk, 0, s, a, n0); *n_part_out = rgrid.x; break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_reduce<EPI_SWIGLU>, rgrid, rblk, 0, s, a, n0); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Row count from which the bf16 path uses the LDS-tiled large-M kernel (at
// M = 480 and 960 it runs 5-15% faster than the wide kernel).  Its tile,
// measured on the 13B / 70B tree-wide shapes: 256 x 256 per workgroup, 8 waves
// of 128 weight rows x 64 activation rows, 32-wide K blocks -- 6-19% faster
// than 256 x 128 with 64 x 64 per wave (fewer LDS fragment reads per MFMA).
constexpr int BIG16_MIN_M = 257;
using LargeTile = TileCfg<2, 4, 8, 4, 32>;
// From 129 to 160 rows (the 70B per-depth steps: 16 sequences x 10 rows) the
// same kernel with 256 weight rows x 160 activation rows per workgroup (8
// waves of 64 x 80): every workgroup streams its weights once, where the wide
// kernel's two 80-row tiles read each weight tile twice through L2.
constexpr int MID16_MIN_M = 129;
using MidTile = TileCfg<4, 2, 4, 5, 32>;

// Launch for M > 16 on a prepared operand: the prep pass (RMSNorm row scale
// applied, then split into hi/lo halves or rounded once to bf16), then the
// wide kernel (weight-stream bound shapes) or the large-M kernel, then the
// K-split reduce.  The prepared operand and the partials live in a.part.
template <bool SPLIT>
hipError_t prepared_launch(GemmArgs a, int epi, int* n_part_out, hipStream_t s) {
  const bool sw = (epi == EPI_SWIGLU);
  if (a.part == nullptr) return hipErrorInvalidValue;  // scratch: bf16 operand (+ partials)
  if (!SPLIT && (a.xb_in || a.xb_out)) return hipErrorInvalidValue;  // hand-over is for split operands
  hipError_t e = hipSuccess;
  const bf16_t* xb;
  if (a.xb_in) {  // written by the previous GEMM's epilogue, unscaled: the row scale goes in this epilogue
    xb = (const bf16_t*)a.xb_in;
  } else {
    bf16_t* prep = (bf16_t*)a.part;
    a.part = (float*)((char*)a.part + align_up256((size_t)a.M * a.K * 2 * (SPLIT ? 2 : 1)));
    hipLaunchKernelGGL(act_prep<SPLIT>, dim3((a.K + 2047) / 2048, a.M), dim3(256), 0, s, a, prep);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.sumsq_in = nullptr;  // the row scale is in the prepared operand
    xb = prep;
  }
  int splits, tiles_n, n0 = 0;
  if (a.M >= BIG16_MIN_M) {
    const BigPlan p = plan_tile<LargeTile>(a.M, a.N, a.K, sw, epi == EPI_STORE || sw);
    a.splits = splits = p.splits;
    tiles_n = p.tiles_n;
    n0 = p.full / p.tiles_m * (sw ? LargeTile::BN / 2 : LargeTile::BN);  // first column of the split tiles
    e = tile_epi<LargeTile, SPLIT>(a, epi, xb, p, s);
  } else if (a.M >= MID16_MIN_M && a.M <= MidTile::BM) {
    const BigPlan p = plan_tile<MidTile>(a.M, a.N, a.K, sw, epi == EPI_STORE || sw);
    a.splits = splits = p.splits;
    tiles_n = p.tiles_n;
    n0 = p.full / p.tiles_m * (sw ? MidTile::BN / 2 : MidTile::BN);
    e = tile_epi<MidTile, SPLIT>(a, epi, xb, p, s);
  } else {
    using C = WideDefault;
    int mb;
    const WidePlan p = plan_wide(a.M, a.N, a.K, sw, C::bn, 8, &mb);
    a.splits = splits = p.splits;
    tiles_n = p.tiles_n;
    e = wide_mb<C, SPLIT>(a, epi, xb, p, mb, s);
  }
  if (e != hipSuccess) return e;
  if (splits == 1) {
    if (epi == EPI_BIAS_SUMSQ || epi == EPI_RESID_SUMSQ) *n_part_out = tiles_n;
    return hipSuccess;
  }
  return reduce_launch(a, epi, n_part_out, s, n0);
}

}  // namespace

namespace {

// The blocked copy: one thread per 16 bytes (8 values) of the output.
__global__ void __launch_bounds__(256) block_weight_kernel(const bf16_t* __restrict__ w, int rows, int cols,
                                                           bf16_t* __restrict__ out, size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const size_t e = i * 8;  // output element: block e / 2048, in it (c / 32, r, c % 32)
  const int b = (int)(e % 2048), r = (b / 32) % 16, c = (b / 512) * 32 + b % 32;
  const size_t blk = e / 2048, nks = (size_t)(cols / 128);
  const size_t row = blk / nks * 16 + r, k = blk % nks * 128 + c;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < (size_t)rows) v = *(const u32x4*)(w + row * cols + k);
  *(u32x4*)(out + e) = v;
}

}  // namespace

size_t blocked_weight_bytes(int rows, int cols) { return (size_t)((rows + 15) / 16) * 16 * cols * 2; }

hipError_t launch_block_weight(const void* w, int rows, int cols, void* out, hipStream_t s) {
  if (!w || !out || rows <= 0 || cols <= 0 || cols % 128 || ((uintptr_t)w & 15) || ((uintptr_t)out & 15))
    return hipErrorInvalidValue;
  const size_t n8 = blocked_weight_bytes(rows, cols) / 16;
  hipLaunchKernelGGL(block_weight_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, (const bf16_t*)w, rows,
                     cols, (bf16_t*)out, n8);
  return hipGetLastError();
}

void gemm_set_kernel_events(hipEvent_t start, hipEvent_t stop) {
  g_kev_start = start;
  g_kev_stop = stop;
}

size_t gemm_bf16_partial_bytes(int M, int N, int K) {
  if (M <= 16) return 0;
  // the prepared operand (hi and lo halves), then the partials of the K split
  int splits;
  if (M >= BIG16_MIN_M || (M >= MID16_MIN_M && M <= MidTile::BM)) {
    splits = 1;  // the most any epilogue's plan (with or without a split tail) takes
    for (int v = 0; v < 4; ++v) {
      const int sv = M >= BIG16_MIN_M ? plan_tile<LargeTile>(M, N, K, v & 1, v >> 1).splits
                                      : plan_tile<MidTile>(M, N, K, v & 1, v >> 1).splits;
      splits = sv > splits ? sv : splits;
    }
  } else {
    int mb;
    const WidePlan w = plan_wide(M, N, K, false, WideDefault::bn, 8, &mb);
    const WidePlan ws = plan_wide(M, N, K, true, WideDefault::bn, 8, &mb);
    splits = w.splits > ws.splits ? w.splits : ws.splits;
  }
  return align_up256((size_t)M * K * 4) + (splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0);
}

hipError_t launch_gemm_bf16(GemmArgs a, int epi, int* n_part_out, hipStream_t s) {
  if (a.K % SK_KSTEP) return hipErrorInvalidValue;  // every kernel steps K in whole 128-element blocks
  if (a.gfeat && (a.gd % SK_KSTEP || a.K != 2 * a.gd)) return hipErrorInvalidValue;
  if ((epi == EPI_BIAS_SUMSQ || epi == EPI_RESID_SUMSQ) && a.y2 && !a.gain_out) return hipErrorInvalidValue;
  if (a.M <= 16 && (a.xb_in || a.xb_out)) return hipErrorInvalidValue;  // operand hand-over: tiled kernels only
  if (epi == EPI_SWIGLU && !a.yb && !a.xb_out) return hipErrorInvalidValue;
  if (a.M <= 16) return a.act_bf16 ? skinny_launch<true>(a, epi, n_part_out, s) : skinny_launch<false>(a, epi, n_part_out, s);
  if (epi == EPI_ROPE) return hipErrorInvalidValue;  // the fused rotary epilogue is the skinny kernel's
  if (a.N % 4 || (epi == EPI_SWIGLU && a.ffn % 4)) return hipErrorInvalidValue;  // float4 epilogue stores
  return a.act_bf16 ? prepared_launch<false>(a, epi, n_part_out, s) : prepared_launch<true>(a, epi, n_part_out, s);
}

hipError_t launch_gemm_f32(GemmArgs a, int epi, int* n_part_out, hipStream_t s) {
  if (a.xb_in || a.xb_out) return hipErrorInvalidValue;
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
