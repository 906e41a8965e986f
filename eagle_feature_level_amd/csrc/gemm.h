// Internal interface of the draft-head GEMMs: y = x W^T with fused operand
// loaders (row gather, RMSNorm, fp32 -> bf16 hi/lo) and epilogues (bias,
// residual, SwiGLU, per-tile sums of squares for the next RMSNorm).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

enum GemmLoad {
  LOAD_F32 = 1,       // x fp32 [M, K] (ldx), optional row gather xrows[m]
  LOAD_F32_NORM = 2   // x fp32 * rsqrt(mean(x^2)+eps) * gain[k]; mean from sumsq partials
};
enum GemmEpi {
  EPI_STORE = 0,        // y = acc
  EPI_BIAS_SUMSQ = 1,   // y = acc + bias[n]; sum of squares partials
  EPI_RESID = 2,        // y = acc + resid[m, n]
  EPI_RESID_SUMSQ = 3,  // y = acc + resid[m, n]; sum of squares partials
  EPI_SWIGLU = 4        // yb[m, j] = silu(gate) * up (fp32), gate row j, up row ffn + j
};

struct GemmArgs {
  // weights: logical rows [0, n_seg0) from w0, [n_seg0, n_seg0+n_seg1) from w1, rest from w2
  const void* w0;
  const void* w1;
  const void* w2;
  int n_seg0, n_seg1;
  int N, K, M;
  // operand loaders
  const void* x;
  int ldx;
  const int32_t* xrows;
  const float* sumsq_in;  // [n_part_in][M]
  int n_part_in;
  const void* gain;
  float eps;
  // epilogue
  float* y;
  int ldy;
  void* yb;  // SwiGLU output (fp32)
  int ldyb;
  const void* bias;
  const float* resid;
  int ldr;
  float* sumsq_out;  // [n_part_out][M]
  int ffn;
  // split-K partials for the tiled kernel
  float* part;
  int splits;
};

// Launch helpers (host).  Return hipSuccess or the launch error.
// bf16 path: chooses the skinny (M <= 16) or tiled kernel; args.part holds
// the tiled kernel's split-K partials.  Sum-of-squares epilogues store their
// number of partial tiles in *n_part_out.
hipError_t launch_gemm_bf16(GemmArgs a, int load, int epi, int* n_part_out, hipStream_t s);
hipError_t launch_gemm_f32(GemmArgs a, int load, int epi, int* n_part_out, hipStream_t s);
size_t gemm_bf16_partial_bytes(int M, int N, int K);
