// Shared device helpers for the gfx950 kernels: bf16 conversion, vector
// types, wave/block reductions.  Wavefronts are 64 lanes wide.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // storage type; arithmetic is fp32
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define WAVE 64

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

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

// Consecutive values of one row as the split operand of the next GEMM: hi at
// hi[0..], lo at hi[lo_off + 0..] (aligned to the store width).
__device__ __forceinline__ void put_split4(bf16_t* hi, size_t lo_off, float4 v) {
  uint32_t l0, l1;
  const uint32_t h0 = split2(v.x, v.y, &l0), h1 = split2(v.z, v.w, &l1);
  *(uint2*)hi = make_uint2(h0, h1);
  *(uint2*)(hi + lo_off) = make_uint2(l0, l1);
}
__device__ __forceinline__ void put_split8(bf16_t* hi, size_t lo_off, float4 v0, float4 v1) {
  u32x4 h, l;
  uint32_t t;
  h[0] = split2(v0.x, v0.y, &t); l[0] = t;
  h[1] = split2(v0.z, v0.w, &t); l[1] = t;
  h[2] = split2(v1.x, v1.y, &t); l[2] = t;
  h[3] = split2(v1.z, v1.w, &t); l[3] = t;
  *(u32x4*)hi = h;
  *(u32x4*)(hi + lo_off) = l;
}
__device__ __forceinline__ void put_split1(bf16_t* hi, size_t lo_off, float v) {
  const uint32_t u = __float_as_uint(v);
  hi[0] = (bf16_t)(u >> 16);
  hi[lo_off] = (bf16_t)((__float_as_uint(v - __uint_as_float(u & 0xffff0000u)) + 0x8000u) >> 16);
}

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11): counter (c0, c1, c2, c3), key (k0, k1), 10 rounds; a
// round maps (x0, x1, x2, x3) to (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3
// ^ k1, lo(M0 x0)) and the key is bumped by the Weyl constants between rounds.
__device__ __forceinline__ void philox4x64_10(uint64_t k0, uint64_t k1, uint64_t c0, uint64_t c1, uint64_t c2,
                                              uint64_t c3, uint64_t (&out)[4]) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = c0, x1 = c1, x2 = c2, x3 = c3;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t hi0 = __umul64hi(M0, x0), lo0 = M0 * x0;
    const uint64_t hi1 = __umul64hi(M1, x2), lo1 = M1 * x2;
    const uint64_t y0 = hi1 ^ x1 ^ k0, y2 = hi0 ^ x3 ^ k1;
    x0 = y0;
    x1 = lo1;
    x2 = y2;
    x3 = lo0;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

// Reductions over a full wave with shuffles (fixed order -> deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, WAVE);
    v = w > v ? w : v;
  }
  return v;
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key);
// -0.0 is folded onto +0.0 first so the two compare equal.
__device__ __forceinline__ uint32_t float_key(float f) {
  f = f + 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
// (value desc, index asc) as one 64-bit key: larger key ranks first.
__device__ __forceinline__ uint64_t topk_key(float v, uint32_t idx) {
  return ((uint64_t)float_key(v) << 32) | (uint64_t)(0xffffffffu - idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return 0xffffffffu - (uint32_t)(k & 0xffffffffu); }
__device__ __forceinline__ float key_value(uint64_t k) { return key_float((uint32_t)(k >> 32)); }

// Block reductions; `red` must hold blockDim.x/64 entries.  All threads get the result.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / WAVE; ++i) s += red[i];
  return s;
}
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = -INFINITY;
#pragma unroll
  for (int i = 0; i < NT / WAVE; ++i) s = fmaxf(s, red[i]);
  return s;
}
