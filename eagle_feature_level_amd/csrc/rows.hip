// Row set-up of an fp32 draft step: the draft layer's input [f_parent ;
// e(token)] as one fp32 row of 2d values (bf16 draft steps gather the two
// halves in the FC GEMM's loader or operand prep pass instead).  Also the
// [l ; m ; h] rows of the three-feature fusion.
//
// The draft head concatenates the parent's feature vector with the embedding
// of the token sampled after it, then reduces the 2d values to d with a fully
// connected layer ("eagle feature-level speculative decoding", the drafting
// section: the shifted token sequence is appended to the feature sequence).
// Writing the concatenation once here keeps the FC GEMM a plain fp32 loader;
// the embedding half converts exactly (bf16 -> fp32), so its lo half is zero.
#include "common.h"
#include "kernels.h"

namespace {

// One workgroup per row.
template <typename T>
__global__ void __launch_bounds__(256) row_setup_kernel(RowSetupArgs a) {
  const int m = blockIdx.x;
  const int d = a.d;
  float* out = a.xin + (size_t)m * 2 * d;
  const float* fr = a.feat + (size_t)a.parent[m] * d;
  const T* e = (const T*)a.embed + (size_t)a.token[m] * d;
  if (d % 8) {  // unaligned widths: element by element
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
      out[i] = fr[i];
      if constexpr (sizeof(T) == 2) out[d + i] = bf2f(e[i]); else out[d + i] = e[i];
    }
    return;
  }
  for (int i = threadIdx.x; i < d / 4; i += blockDim.x) ((float4*)out)[i] = ((const float4*)fr)[i];
  if constexpr (sizeof(T) == 2) {
    // eight bf16 per 16-byte load
    for (int i = threadIdx.x; i < d / 8; i += blockDim.x) {
      const u32x4 v = *(const u32x4*)(e + i * 8);
      float4 lo4, hi4;
      lo4.x = __uint_as_float(v[0] << 16); lo4.y = __uint_as_float(v[0] & 0xffff0000u);
      lo4.z = __uint_as_float(v[1] << 16); lo4.w = __uint_as_float(v[1] & 0xffff0000u);
      hi4.x = __uint_as_float(v[2] << 16); hi4.y = __uint_as_float(v[2] & 0xffff0000u);
      hi4.z = __uint_as_float(v[3] << 16); hi4.w = __uint_as_float(v[3] & 0xffff0000u);
      ((float4*)(out + d))[2 * i] = lo4;
      ((float4*)(out + d))[2 * i + 1] = hi4;
    }
  } else {
    for (int i = threadIdx.x; i < d / 4; i += blockDim.x) ((float4*)(out + d))[i] = ((const float4*)e)[i];
  }
}

// [low ; mid ; high] rows of 3d fp32 values, one workgroup per row.
__global__ void __launch_bounds__(256) concat3_kernel(const float* __restrict__ low, const float* __restrict__ mid,
                                                      const float* __restrict__ high, int d, float* __restrict__ out) {
  const int m = blockIdx.x;
  const float* src[3] = {low + (size_t)m * d, mid + (size_t)m * d, high + (size_t)m * d};
  float* o = out + (size_t)m * 3 * d;
#pragma unroll
  for (int s = 0; s < 3; ++s)
    for (int i = threadIdx.x; i < d; i += blockDim.x) o[s * d + i] = src[s][i];
}

}  // namespace

hipError_t launch_concat3(const float* low, const float* mid, const float* high, int n_rows, int d, float* out,
                          hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(concat3_kernel, dim3(n_rows), dim3(256), 0, s, low, mid, high, d, out);
  return hipGetLastError();
}

hipError_t launch_row_setup(const RowSetupArgs& a, bool bf16, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(row_setup_kernel<bf16_t>, dim3(a.n_rows), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(row_setup_kernel<float>, dim3(a.n_rows), dim3(256), 0, s, a);
  return hipGetLastError();
}
