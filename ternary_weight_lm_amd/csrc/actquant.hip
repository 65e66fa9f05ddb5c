// actquant.hip -- RMSNorm fused with per-token absmax int8 quantization.
//
// The norm sits inside every FusedBitLinear and runs right before the
// activations are quantized (hysenlabs de review "MatMul-Free LM:
// Ternary-Gewichte statt Matrixmultiplikation im Transformer", section
// "HGRNBit: was in einem Block tatsächlich passiert"; datacamp "MatMul-freie
// LLMs: Zentrale Konzepte erklärt", figure panel 5).  One 64-lane wave owns
// one token row; the row is read in 16-byte chunks (8 elements per lane per
// step, 512 per wave) and reduced with cross-lane shuffles only:
//   pass 1: sum of x^2 in fp64                  -> r = 1/sqrt(ms + eps)
//   pass 2: xn = (x * r) * g, max |xn|          -> s = 127 / max(., 1e-5)
//   pass 3: xq = clamp(rne(xn * s)), 8-byte stores, sum of xq -> rowsum
// Passes 2 and 3 re-read the row from cache (HBM traffic stays one read of
// x and one write of xq).  Four rows per 256-thread workgroup.
#include "bl_common.h"
#include "bl_launch.h"

namespace bl {

template <int DT>
__global__ __launch_bounds__(256) void act_quant_kernel(
    const void *__restrict__ x, const void *__restrict__ gain, int64_t M,
    int64_t K, float eps, int8_t *__restrict__ xq, float *__restrict__ s_out,
    int32_t *__restrict__ rowsum_out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // a whole wave leaves; no workgroup barrier below
  constexpr int EB = dtype_bytes(DT);
  const char *xr = reinterpret_cast<const char *>(x) + row * K * EB;
  const char *gr = reinterpret_cast<const char *>(gain);

  double ss = 0.0;
  for (int64_t k = lane * 8; k < K; k += 512) {
    float f[8];
    load8<DT>(xr + k * EB, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += (double)f[e] * (double)f[e];
  }
  const float r = rms_inv(wave_sum(ss), (int)K, eps);

  float amax = 0.0f;
  for (int64_t k = lane * 8; k < K; k += 512) {
    float f[8], g[8];
    load8<DT>(xr + k * EB, f);
    load8<DT>(gr + k * EB, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((f[e] * r) * g[e]));
  }
  const float sc = act_scale(wave_max(amax));

  int rs = 0;
  int8_t *qr = xq + row * K;
  for (int64_t k = lane * 8; k < K; k += 512) {
    float f[8], g[8];
    load8<DT>(xr + k * EB, f);
    load8<DT>(gr + k * EB, g);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = quant8((f[e] * r) * g[e], sc);
      rs += q;
      if (e < 4) lo |= (uint32_t)(q & 0xFF) << (8 * e);
      else hi |= (uint32_t)(q & 0xFF) << (8 * (e - 4));
    }
    *reinterpret_cast<uint2 *>(qr + k) = make_uint2(lo, hi);
  }
  rs = wave_sum(rs);
  if (lane == 0) {
    s_out[row] = sc;
    rowsum_out[row] = rs;
  }
}

hipError_t launch_act_quant(const void *x, int x_dtype, const void *gain,
                            int64_t M, int64_t K, float eps, int8_t *xq,
                            float *s, int32_t *rowsum, hipStream_t stream) {
  const unsigned blocks = (unsigned)((M + 3) / 4);
  switch (x_dtype) {
    case BL_F32:
      act_quant_kernel<BL_F32><<<blocks, 256, 0, stream>>>(x, gain, M, K, eps, xq, s, rowsum);
      break;
    case BL_F16:
      act_quant_kernel<BL_F16><<<blocks, 256, 0, stream>>>(x, gain, M, K, eps, xq, s, rowsum);
      break;
    default:
      act_quant_kernel<BL_BF16><<<blocks, 256, 0, stream>>>(x, gain, M, K, eps, xq, s, rowsum);
      break;
  }
  return hipGetLastError();
}

}  // namespace bl
