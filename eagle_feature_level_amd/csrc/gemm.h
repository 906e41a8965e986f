// Internal interface of the draft-head GEMMs: y = x W^T with an fp32 operand
// stream (optional row gather) and fused epilogues (RMSNorm row scale, bias,
// residual, SwiGLU, per-tile sums of squares and gain product for the next
// RMSNorm).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

enum GemmEpi {
  EPI_STORE = 0,        // y = acc
  EPI_BIAS_SUMSQ = 1,   // y = acc + bias[n]; sum of squares partials; y2 = y * gain_out[n] if y2
  EPI_RESID = 2,        // y = acc + resid[m, n]
  EPI_RESID_SUMSQ = 3,  // y = acc + resid[m, n]; sum of squares partials; y2 = y * gain_out[n] if y2
  EPI_SWIGLU = 4,       // yb[m, j] = silu(gate) * up, gate row j, up row ffn + j
  EPI_ROPE = 5          // [q; k; v] rows of whole heads: rotary embedding of q and k at the
                        // row's position, q to y, k and v (bf16) into the row's tree slot
};

struct GemmArgs {
  // weights: logical rows [0, n_seg0) from w0, [n_seg0, n_seg0+n_seg1) from w1, rest from w2
  const void* w0;
  const void* w1;
  const void* w2;
  int n_seg0, n_seg1;
  // optional (bf16): the same segments in the blocked layout of
  // launch_block_weight, read instead of w0..w2 (all of the GEMM's segments,
  // or none)
  const void* wb0;
  const void* wb1;
  const void* wb2;
  int N, K, M;
  // activations: x fp32 [M, K] (ldx), row m read from row xrows[m] if xrows is set
  const float* x;
  int ldx;
  const int32_t* xrows;
  // or, for M <= 16 with K = 2 gd: row m = [gfeat[gparent[m]] (fp32) ; gembed[gtoken[m]] (bf16)]
  const float* gfeat;
  const int32_t* gparent;
  const int32_t* gtoken;
  const void* gembed;
  int gd;
  // RMSNorm of the input rows, when sumsq_in is set: acc[m, :] *= rsqrt(sum_p sumsq_in[p][m] / K + eps)
  // (x then already carries the gain)
  const float* sumsq_in;  // [n_part_in][M]
  int n_part_in;
  float eps;
  // epilogue
  float* y;
  int ldy;
  float* yb;  // SwiGLU output
  int ldyb;
  const void* bias;
  const float* resid;
  int ldr;
  float* sumsq_out;  // [n_part_out][M]
  const void* gain_out;  // next RMSNorm's gain (bf16 or fp32 like the weights)
  float* y2;             // y * gain_out, same layout as y
  int ffn;
  // split-K partials for the tiled kernel
  float* part;
  int splits;
  // M > 16, split operands (act_bf16 == 0) only.  xb_out: the epilogue also
  // writes the next GEMM's operand from this GEMM's output -- y * gain_out when
  // gain_out is set (y2 may then be null), else y (the SwiGLU output, yb may
  // then be null) -- as hi / lo bf16 halves, hi [M][Nout] at xb_out and lo at
  // xb_out + M*Nout.  xb_in: this GEMM's operand so written by the previous
  // one or by attention (the prep pass is skipped); with sumsq_in set, the
  // RMSNorm row scale is then applied in the epilogue.
  uint16_t* xb_out;
  const uint16_t* xb_in;
  // activation precision: 0 = each fp32 activation enters the matrix units as
  // a (hi, lo) pair of bf16 values (two MFMAs per product); 1 = it is rounded
  // once to bf16 (round to nearest even) after the RMSNorm row scale, one MFMA
  int act_bf16;
  // EPI_ROPE (M <= 16, bf16 weights): heads of rp_hd columns, rp_hq query heads
  // then rp_hkv key heads then rp_hkv value heads; row m of sequence b (the b
  // with rp_row_start[b] <= m < rp_row_start[b + 1]) at position rp_pos[m]
  // writes k, v to tree slot rp_slot[m]: rp_tree_k/v[b][slot][head][rp_hd]
  const int32_t* rp_pos;
  const int32_t* rp_slot;
  const int32_t* rp_row_start;
  int rp_batch;
  void* rp_tree_k;
  void* rp_tree_v;
  int rp_hd, rp_hq, rp_hkv;
  float rp_theta;
};

// Launch helpers (host).  Return hipSuccess or the launch error.
// bf16 path: chooses the skinny (M <= 16) or tiled kernel; args.part holds
// the tiled kernel's split-K partials.  Sum-of-squares epilogues store their
// number of partial tiles in *n_part_out.
hipError_t launch_gemm_bf16(GemmArgs a, int epi, int* n_part_out, hipStream_t s);
// Measurement hook: the next bf16 launch with M <= 16 (a single kernel) is
// issued with hipExtLaunchKernelGGL and records its own start and stop into
// these events (kernel execution only, no dispatch gap); then they are cleared.
void gemm_set_kernel_events(hipEvent_t start, hipEvent_t stop);
hipError_t launch_gemm_f32(GemmArgs a, int epi, int* n_part_out, hipStream_t s);
size_t gemm_bf16_partial_bytes(int M, int N, int K);
// Blocked copy of a bf16 matrix W [rows, cols] (cols a multiple of 128): 16-row
// by 128-column blocks of 4 KB, the blocks of a 16-row band in column order,
// inside a block the four 32-column quarters one after the other, each 16 rows
// of 32 values:
// out[(t * (cols / 128) + s) * 2048 + ((c / 32) * 16 + r) * 32 + c % 32] = W[16 t + r][128 s + c],
// rows past the end 0.  out holds blocked_weight_bytes(rows, cols) bytes.
size_t blocked_weight_bytes(int rows, int cols);
hipError_t launch_block_weight(const void* w, int rows, int cols, void* out, hipStream_t s);
