// bl_common.h -- device helpers shared by the gfx950 kernels of the
// FusedBitLinear library: element loads / stores for the three activation
// dtypes, 64-lane wave reductions, and the 2-bit weight unpack.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitlinear.h"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// -------------------------------------------------------------- elements

// 8 consecutive elements of dtype DT kept as raw bits in registers: one
// 16-byte load for fp16 / bf16, two for fp32.
template <int DT> struct Chunk8 {
  uint4 u[DT == BL_F32 ? 2 : 1];
};

// p must be 16-byte aligned.
template <int DT>
__device__ __forceinline__ Chunk8<DT> load_chunk(const void *p) {
  Chunk8<DT> c;
  const uint4 *q = reinterpret_cast<const uint4 *>(p);
  c.u[0] = q[0];
  if constexpr (DT == BL_F32) c.u[1] = q[1];
  return c;
}

// Exact widening of the 8 elements to fp32.
template <int DT>
__device__ __forceinline__ void widen(const Chunk8<DT> &c, float f[8]) {
  if constexpr (DT == BL_F32) {
    f[0] = __uint_as_float(c.u[0].x); f[1] = __uint_as_float(c.u[0].y);
    f[2] = __uint_as_float(c.u[0].z); f[3] = __uint_as_float(c.u[0].w);
    f[4] = __uint_as_float(c.u[1].x); f[5] = __uint_as_float(c.u[1].y);
    f[6] = __uint_as_float(c.u[1].z); f[7] = __uint_as_float(c.u[1].w);
  } else {
    const uint32_t w[4] = {c.u[0].x, c.u[0].y, c.u[0].z, c.u[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = w[i] & 0xFFFFu, hi = w[i] >> 16;
      if constexpr (DT == BL_BF16) {
        f[2 * i] = __uint_as_float(lo << 16);
        f[2 * i + 1] = __uint_as_float(hi << 16);
      } else {
        f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)lo);
        f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)hi);
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void load8(const void *p, float f[8]) {
  widen<DT>(load_chunk<DT>(p), f);
}

// Bytes per element of a dtype code.
__host__ __device__ constexpr int dtype_bytes(int dt) { return dt == BL_F32 ? 4 : 2; }

// Round-to-nearest-even conversion of fp32 to the output dtype bits.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u)           // Inf / NaN: truncate,
    return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));  // keep NaN quiet
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int DT>
__device__ __forceinline__ void store1(void *base, int64_t idx, float v) {
  if constexpr (DT == BL_F32) {
    reinterpret_cast<float *>(base)[idx] = v;
  } else if constexpr (DT == BL_F16) {
    reinterpret_cast<uint16_t *>(base)[idx] = f32_to_f16_bits(v);
  } else {
    reinterpret_cast<uint16_t *>(base)[idx] = f32_to_bf16_bits(v);
  }
}

// ------------------------------------------------------- wave reductions

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ------------------------------------------------------------ quantizers

// Correctly rounded fp32 division: the fp64 quotient is correctly rounded
// (IEEE division on the f64 unit) and rounding it again to fp32 cannot
// change the result, since 53 >= 2*24 + 2.
__device__ __forceinline__ float div_rn(float a, float b) {
  return (float)((double)a / (double)b);
}

// Correctly rounded fp32 square root of a positive finite t.  The fp64
// root gives a candidate within one fp32 ulp; it is then corrected exactly:
// the midpoints between neighbouring floats have at most 25 significant
// bits, so their squares are exact in fp64 and can be compared with t (a
// tie is impossible: t has 24 significant bits, a midpoint square 49-50).
// HIP's __fsqrt_rn is not used because it lowers to the native,
// not correctly rounded, instruction.
__device__ __forceinline__ float sqrt_rn(float t) {
  float q = (float)__builtin_sqrt((double)t);
  const uint32_t u = __float_as_uint(q);
  const double qd = q;
  const double hi = 0.5 * (qd + (double)__uint_as_float(u + 1));
  const double lo = 0.5 * (qd + (double)__uint_as_float(u - 1));
  const double td = t;
  if (td > hi * hi) q = __uint_as_float(u + 1);
  else if (td < lo * lo) q = __uint_as_float(u - 1);
  return q;
}

// r = 1 / sqrt(fp32(sumsq / K) + eps), every step correctly rounded fp32.
__device__ __forceinline__ float rms_inv(double sumsq, int K, float eps) {
  const float ms = (float)(sumsq / (double)K);
  return div_rn(1.0f, sqrt_rn(ms + eps));
}

// s = 127 / max(absmax, 1e-5), correctly rounded fp32.
__device__ __forceinline__ float act_scale(float absmax) {
  return div_rn(127.0f, fmaxf(absmax, 1e-5f));
}

// int8 code of one normalized activation: clamp(rne(xn * s), -128, 127).
__device__ __forceinline__ int quant8(float xn, float s) {
  float q = __builtin_rintf(xn * s);
  q = fminf(fmaxf(q, -128.0f), 127.0f);
  return (int)q;
}

// ---------------------------------------------------------- weight codes

// The 16 two-bit codes of one packed word as the 16 int8 bytes of an MFMA
// operand (values 0, 1, 2 = Wq + 1): byte b of dword q is element 4q + b.
__device__ __forceinline__ v4i unpack_codes(uint32_t w) {
  v4i r;
  r.x = (int)(w & 0x03030303u);
  r.y = (int)((w >> 2) & 0x03030303u);
  r.z = (int)((w >> 4) & 0x03030303u);
  r.w = (int)((w >> 6) & 0x03030303u);
  return r;
}

__device__ __forceinline__ v4i mfma16x16x64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

}  // namespace bl
