// skinny.hip -- decode-shaped FusedBitLinear (M <= 16 tokens).
//
// At a handful of tokens the layer is a stream over the packed weights
// (N*K/4 bytes): the matrix cores have far more throughput than needed, so
// the design goal is bytes in flight, not arithmetic.  One workgroup owns one
// packed 32-row tile column (32 output features x all of K); its 4 waves
// split the K-blocks round-robin.
//   1. Every wave first issues the 16-byte loads of all its weight tiles
//      (one contiguous 1 KiB per wave per tile), so HBM latency overlaps the
//      prologue.
//   2. Fused variant: the workgroup normalizes and quantizes the M token
//      rows itself (RMSNorm before quantization, as in the hysenlabs de
//      review "MatMul-Free LM: Ternary-Gewichte statt Matrixmultiplikation im
//      Transformer", section "HGRNBit: was in einem Block tatsächlich
//      passiert") into LDS, with fp64 sum of squares and fp32 absmax per row,
//      exactly the arithmetic of actquant.hip.  Pre-quantized variant: xq,
//      s, rowsum come from the act-quant kernel and A operands are read
//      straight from global memory.
//   3. Each tile feeds four v_mfma_i32_16x16x64_i8 (2 output halves x 2
//      k-steps); token rows >= M are zero operands.
//   4. The 4 waves' partial sums are added in LDS; the epilogue subtracts
//      rowsum and rescales by beta / s_m (datacamp "MatMul-freie LLMs:
//      Zentrale Konzepte erklärt", figure panel 4).
#include "bl_common.h"
#include "bl_launch.h"

namespace bl {

constexpr int kSkinnyBatch = 16;  // weight tiles held in registers per wave

struct SkinnyParams {
  const void *x;
  const void *gain;
  float eps;
  const int8_t *xq;
  const float *s;
  const int32_t *rowsum;
  const uint4 *packed;
  const float *beta;
  int M, N, K;
  void *out;
};

template <bool FUSED, int DT, int OUT>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyParams p) {
  extern __shared__ __align__(16) int8_t xs[];  // fused: [M][K + 16] int8
  __shared__ int red[4][8][64];
  __shared__ float s_row[16];
  __shared__ int rs_row[16];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nt = blockIdx.x;
  const int M = p.M, K = p.K, KB = K >> 7;
  const int lds_stride = K + 16;
  const int nmine = w < KB ? (KB - w + 3) / 4 : 0;
  const uint4 *wp = p.packed + (int64_t)nt * KB * 64 + lane;

  // ---- 1. weight loads of the first batch
  uint4 wr[kSkinnyBatch];
#pragma unroll
  for (int t = 0; t < kSkinnyBatch; ++t)
    if (t < nmine) wr[t] = wp[(int64_t)(w + 4 * t) * 64];

  // ---- 2. activations
  if constexpr (FUSED) {
    constexpr int EB = dtype_bytes(DT);
    const char *gr = reinterpret_cast<const char *>(p.gain);
    for (int m = w; m < M; m += 4) {
      const char *xr = reinterpret_cast<const char *>(p.x) + (int64_t)m * K * EB;
      double ss = 0.0;
      for (int k = lane * 8; k < K; k += 512) {
        float f[8];
        load8<DT>(xr + (int64_t)k * EB, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += (double)f[e] * (double)f[e];
      }
      const float r = rms_inv(wave_sum(ss), K, p.eps);
      float amax = 0.0f;
      for (int k = lane * 8; k < K; k += 512) {
        float f[8], g[8];
        load8<DT>(xr + (int64_t)k * EB, f);
        load8<DT>(gr + (int64_t)k * EB, g);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((f[e] * r) * g[e]));
      }
      const float sc = act_scale(wave_max(amax));
      int rs = 0;
      for (int k = lane * 8; k < K; k += 512) {
        float f[8], g[8];
        load8<DT>(xr + (int64_t)k * EB, f);
        load8<DT>(gr + (int64_t)k * EB, g);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int q = quant8((f[e] * r) * g[e], sc);
          rs += q;
          if (e < 4) lo |= (uint32_t)(q & 0xFF) << (8 * e);
          else hi |= (uint32_t)(q & 0xFF) << (8 * (e - 4));
        }
        *reinterpret_cast<uint2 *>(xs + m * lds_stride + k) = make_uint2(lo, hi);
      }
      rs = wave_sum(rs);
      if (lane == 0) {
        s_row[m] = sc;
        rs_row[m] = rs;
      }
    }
  } else {
    if constexpr (OUT != kOutI32) {
      if (tid < M) s_row[tid] = p.s[tid];
    }
    if (tid < M) rs_row[tid] = p.rowsum[tid];
  }
  __syncthreads();

  // ---- 3. contraction
  v4i acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  const int arow = lane & 15;
  const bool arow_ok = arow < M;
  for (int base = 0; base < nmine; base += kSkinnyBatch) {
    if (base > 0) {
#pragma unroll
      for (int t = 0; t < kSkinnyBatch; ++t)
        if (base + t < nmine) wr[t] = wp[(int64_t)(w + 4 * (base + t)) * 64];
    }
#pragma unroll
    for (int t = 0; t < kSkinnyBatch; ++t) {
      if (base + t >= nmine) break;
      const int kb = w + 4 * (base + t);
      const uint4 u = wr[t];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int koff = kb * 128 + 32 * (lane >> 4) + 16 * s2;
        v4i a = {0, 0, 0, 0};
        if (arow_ok) {
          if constexpr (FUSED)
            a = *reinterpret_cast<const v4i *>(xs + arow * lds_stride + koff);
          else
            a = *reinterpret_cast<const v4i *>(p.xq + (int64_t)arow * K + koff);
        }
        const v4i b0 = unpack_codes(s2 ? u.y : u.x);
        const v4i b1 = unpack_codes(s2 ? u.w : u.z);
        acc0 = mfma16x16x64(a, b0, acc0);
        acc1 = mfma16x16x64(a, b1, acc1);
      }
    }
  }

  // ---- 4. cross-wave sum and epilogue
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[w][i][lane] = acc0[i];
    red[w][4 + i][lane] = acc1[i];
  }
  __syncthreads();
  const float bt = OUT == kOutI32 ? 0.0f : *p.beta;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = tid + 256 * q;
    const int j = idx >> 6, L = idx & 63;
    const int h = j >> 2, i = j & 3;
    const int m = 4 * (L >> 4) + i;
    if (m >= M) continue;
    const int n = nt * 32 + 16 * h + (L & 15);
    const int v = red[0][j][L] + red[1][j][L] + red[2][j][L] + red[3][j][L] - rs_row[m];
    const int64_t o = (int64_t)m * p.N + n;
    if constexpr (OUT == kOutI32) {
      reinterpret_cast<int32_t *>(p.out)[o] = v;
    } else {
      store1<OUT>(p.out, o, (float)v * div_rn(bt, s_row[m]));
    }
  }
}

template <bool FUSED, int DT>
static void launch_out(const SkinnyParams &p, int out_kind, size_t lds,
                       hipStream_t stream) {
  const unsigned grid = (unsigned)(p.N / 32);
  switch (out_kind) {
    case BL_F32: skinny_kernel<FUSED, DT, BL_F32><<<grid, 256, lds, stream>>>(p); break;
    case BL_F16: skinny_kernel<FUSED, DT, BL_F16><<<grid, 256, lds, stream>>>(p); break;
    case BL_BF16: skinny_kernel<FUSED, DT, BL_BF16><<<grid, 256, lds, stream>>>(p); break;
    default: skinny_kernel<FUSED, DT, kOutI32><<<grid, 256, lds, stream>>>(p); break;
  }
}

hipError_t launch_skinny(const SkinnyArgs &a, hipStream_t stream) {
  SkinnyParams p;
  p.x = a.x;
  p.gain = a.gain;
  p.eps = a.eps;
  p.xq = a.xq;
  p.s = a.s;
  p.rowsum = a.rowsum;
  p.packed = reinterpret_cast<const uint4 *>(a.packed);
  p.beta = a.beta;
  p.M = (int)a.M;
  p.N = (int)a.N;
  p.K = (int)a.K;
  p.out = a.out;
  if (a.fused) {
    const size_t lds = (size_t)a.M * (size_t)(a.K + 16);
    switch (a.x_dtype) {
      case BL_F32: launch_out<true, BL_F32>(p, a.out_kind, lds, stream); break;
      case BL_F16: launch_out<true, BL_F16>(p, a.out_kind, lds, stream); break;
      default: launch_out<true, BL_BF16>(p, a.out_kind, lds, stream); break;
    }
  } else {
    launch_out<false, BL_F32>(p, a.out_kind, 0, stream);
  }
  return hipGetLastError();
}

}  // namespace bl
