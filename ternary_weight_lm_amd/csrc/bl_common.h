// bl_common.h -- device helpers shared by the gfx950 kernels of the
// FusedBitLinear library: element loads / stores for the three activation
// dtypes, 64-lane wave reductions, and the 2-bit weight unpack.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitlinear.h"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// -------------------------------------------------------------- elements

// 8 consecutive elements of dtype DT kept as raw bits in registers: one
// 16-byte load for fp16 / bf16, two for fp32.  (Native int vectors: copies of
// HIP's uint4 struct can be lowered to memcpy through private memory.)
template <int DT> struct Chunk8 {
  v4i u[DT == BL_F32 ? 2 : 1];
};

// p must be 16-byte aligned.
template <int DT>
__device__ __forceinline__ Chunk8<DT> load_chunk(const void *p) {
  Chunk8<DT> c;
  const v4i *q = reinterpret_cast<const v4i *>(p);
  c.u[0] = q[0];
  if constexpr (DT == BL_F32) c.u[1] = q[1];
  return c;
}

// Exact widening of the 8 elements to fp32.
template <int DT>
__device__ __forceinline__ void widen(const Chunk8<DT> &c, float f[8]) {
  if constexpr (DT == BL_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __int_as_float(c.u[0][i]);
      f[4 + i] = __int_as_float(c.u[1][i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wd = (uint32_t)c.u[0][i];
      const uint32_t lo = wd & 0xFFFFu, hi = wd >> 16;
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

// ------------------------------------------------------------ buffer loads
// Raw buffer loads: a scalar base and size, a per-lane byte offset, and an
// optional scalar offset; offsets at or past the size read as zero without
// touching memory, so a load never needs a guarding branch.

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer over `bytes` bytes at base: offsets at or past `bytes` read as
// zero (and touch no memory).
constexpr uint32_t kOob = 0x40000000u;  // a buffer offset past every range

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ v4i bload(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

template <int DT>
__device__ __forceinline__ Chunk8<DT> bload_chunk(rsrc_t r, uint32_t off) {
  Chunk8<DT> c;
  c.u[0] = bload(r, off);
  if constexpr (DT == BL_F32) c.u[1] = bload(r, off + 16);
  return c;
}

// Bytes per element of a dtype code.
__host__ __device__ constexpr int dtype_bytes(int dt) { return dt == BL_F32 ? 4 : 2; }

// fp32 -> fp16, round to nearest even, from the fp32 value as it stands.
// The empty asm pins f as a materialized fp32 value: otherwise the compiler
// folds a preceding fp32 multiply into the conversion (v_fma_mixlo_f16, one
// rounding of the exact product straight to fp16), which differs from
// rounding the fp32 product at every fp16 tie it creates.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  __asm__("" : "+v"(f));
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// The 16-bit pattern of v rounded to a 2-byte output dtype (fp16 / bf16),
// as store1 rounds it.
template <int DT>
__device__ __forceinline__ uint16_t out_bits(float v) {
  if constexpr (DT == BL_F16) return f32_to_f16_bits(v);
  else return __builtin_bit_cast(uint16_t, (__bf16)v);
}

template <int DT>
__device__ __forceinline__ void store1(void *base, int64_t idx, float v) {
  if constexpr (DT == BL_F32) {
    reinterpret_cast<float *>(base)[idx] = v;
  } else if constexpr (DT == BL_F16) {
    reinterpret_cast<uint16_t *>(base)[idx] = f32_to_f16_bits(v);
  } else {
    // gfx950 converts with v_cvt_pk_bf16_f32 (round to nearest even)
    reinterpret_cast<__bf16 *>(base)[idx] = (__bf16)v;
  }
}

// Between LDS writes by some lanes of a wave and reads of that data by other
// lanes of the same wave.  The hardware already runs one wave's LDS
// operations in order, so this emits no instruction; it is a wavefront-scope
// fence for the compiler, which otherwise treats each lane as alone and may
// move a lane's reads ahead of the writes it does not itself depend on.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// XOR swizzle of the 16-byte chunks of a 128-byte LDS row: conflict-free for
// 16-byte accesses by 8 consecutive rows (32 banks) and by 16 consecutive
// rows (64 banks), the two ways gfx9 LDS serves ds_read/write_b128.
__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
}

// ------------------------------------------------------- wave reductions
// All-lane reductions of a 64-lane wave: a DPP butterfly inside each row of
// 16 lanes (quad_perm xor 1, quad_perm xor 2, half-row mirror, row mirror;
// after each step every lane of the group holds the same partial), then the
// four row results are read out of lanes 0, 16, 32, 48 and combined in a
// fixed order ((r0 + r1) + (r2 + r3)).  DPP moves are plain VALU ops, far
// cheaper in latency than LDS-routed shuffles.  The result is identical in
// every lane and the association order is fixed, so every kernel that uses
// these gets bit-identical sums.

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int2 u = __builtin_bit_cast(int2, v);
  return __builtin_bit_cast(double, make_int2(dpp_i32<CTRL>(u.x), dpp_i32<CTRL>(u.y)));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i inside 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i inside 16 lanes

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  const int2 u = __builtin_bit_cast(int2, v);
  auto lane_val = [&](int l) {
    return __builtin_bit_cast(double, make_int2(__builtin_amdgcn_readlane(u.x, l),
                                                __builtin_amdgcn_readlane(u.y, l)));
  };
  return (lane_val(0) + lane_val(16)) + (lane_val(32) + lane_val(48));
}

__device__ __forceinline__ int wave_sum(int v) {
  v += dpp_i32<kDppXor1>(v);
  v += dpp_i32<kDppXor2>(v);
  v += dpp_i32<kDppHalfMirror>(v);
  v += dpp_i32<kDppMirror>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  auto lane_val = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
  return fmaxf(fmaxf(lane_val(0), lane_val(16)), fmaxf(lane_val(32), lane_val(48)));
}

// ------------------------------------------------------------ quantizers

// Correctly rounded fp32 division: the library is compiled with
// -fhip-fp32-correctly-rounded-divide-sqrt, under which fp32 '/' lowers to
// the IEEE division sequence (div_scale / rcp / fma / div_fixup).
__device__ __forceinline__ float div_rn(float a, float b) { return a / b; }

// Correctly rounded fp32 square root of a positive finite t.  The fp32 root
// is a candidate within one ulp; it is then corrected exactly: the midpoints
// between neighbouring floats have at most 25 significant bits, so their
// squares are exact in fp64 and can be compared with t (a tie is
// impossible: t has 24 significant bits, a midpoint square 49-50).  HIP's
// __fsqrt_rn is not used because it lowers to the native instruction.
__device__ __forceinline__ float sqrt_rn(float t) {
  float q = __builtin_sqrtf(t);
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

// int8 code of one normalized activation, clamp(rne(v), -128, 127) with
// v = fp32(xn * s), returned in the LOW BYTE of the result (the other bytes
// are not a sign extension; pack4 and the row sum read the low byte only).
// The clamp never binds: s = fp32(127 / max|xn|) makes |v| <= 127 (1 + 3 *
// 2^-24) < 127.5.  Adding 1.5 * 2^23 puts v where the float spacing is 1,
// so the sum is 1.5 * 2^23 + rne(v) (ties to even, as the mantissa parity
// follows rne(v)), and its low mantissa byte is rne(v) mod 256: two adds'
// worth of work instead of rint, clamp and convert.
__device__ __forceinline__ int quant8(float xn, float s) {
  const float v = xn * s;
  return __float_as_int(v + 12582912.0f);
}

// SiLU in fp32, a / (1 + e^-a) (the activation of the HGRNBit MLP gate),
// from the hardware base-2 exponential and reciprocal: e^-a = 2^(-a log2 e).
// The gate is a floating-point output checked within tolerance, and the
// library expf plus an IEEE division cost ~30 instructions per output --
// in the GEMM epilogue about half the main loop's time.  Relative error
// about 1e-6.  For a very negative a the exponential overflows to +inf, its
// reciprocal is 0 and the result is 0 (the limit); a very positive a gives
// a.
__device__ __forceinline__ float silu(float a) {
  const float e = __builtin_amdgcn_exp2f(-a * 1.4426950408889634f);
  return a * __builtin_amdgcn_rcpf(1.0f + e);
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

// Unpack two consecutive code words of a lane slot (the same 16 output
// rows, both 64-wide k halves) at once: one 64-bit shift moves both words,
// and the bits the low word takes in from the high one land outside the
// mask, so 3 shifts and 8 masks replace 6 shifts and 8 masks.  (Written as
// inline shifts: left to itself the compiler splits a 64-bit shift by a
// constant into two 32-bit ones.)  The unpack is the contraction's VALU
// work; taking a fifth of it off measured 2-4 % faster prefill launches and
// 0.5 % faster one-token decode launches.
__device__ __forceinline__ void unpack_pair(uint32_t x, uint32_t y, v4i &ux, v4i &uy) {
  const uint64_t p = ((uint64_t)y << 32) | x;
  uint64_t p2, p4, p6;
  asm("v_lshrrev_b64 %0, 2, %1" : "=v"(p2) : "v"(p));
  asm("v_lshrrev_b64 %0, 4, %1" : "=v"(p4) : "v"(p));
  asm("v_lshrrev_b64 %0, 6, %1" : "=v"(p6) : "v"(p));
  constexpr uint32_t M = 0x03030303u;
  ux = v4i{(int)(x & M), (int)((uint32_t)p2 & M), (int)((uint32_t)p4 & M), (int)((uint32_t)p6 & M)};
  uy = v4i{(int)(y & M), (int)((uint32_t)(p2 >> 32) & M), (int)((uint32_t)(p4 >> 32) & M),
           (int)((uint32_t)(p6 >> 32) & M)};
}

__device__ __forceinline__ v4i mfma16x16x64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

}  // namespace bl
