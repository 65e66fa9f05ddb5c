// actquant.hip -- RMSNorm fused with per-token absmax int8 quantization.
//
// The norm sits inside every FusedBitLinear and runs right before the
// activations are quantized (hysenlabs de review "MatMul-Free LM:
// Ternary-Gewichte statt Matrixmultiplikation im Transformer", section
// "HGRNBit: was in einem Block tatsächlich passiert"; datacamp "MatMul-freie
// LLMs: Zentrale Konzepte erklärt", figure panel 5).  One 64-lane wave per
// token row runs the shared row quantizer (rowquant.h): the row is read once
// with 16-byte loads (widened and kept in registers up to K = 6144, kept raw
// up to K = 8192, re-read from cache beyond), the three reductions are
// cross-lane shuffles, and the int8 codes leave as coalesced 8-byte stores.
// Four rows per 256-thread workgroup, no barriers; the grouped kernel takes
// up to three projections' rows in one launch.  HBM traffic: one read of x,
// one write of xq, 8 bytes of scale + row sum.
#include "bl_launch.h"
#include "rowquant.h"

namespace bl {

// Chunks cached per lane when the row fits the float mode (the widened row
// in registers): 2, 4, 6, 8 or 12 rounds of 512 elements, so K <= 6144
// (one wave per row can afford 12: the act-quant kernel holds nothing
// else); 0 beyond that (raw / reload modes).
constexpr int aq_float_nc(int64_t K) { return K <= 4096 ? row_cache((int)K) : (K <= 6144 ? 12 : 0); }

template <int DT, int MODE, int NC>
__device__ __forceinline__ void act_quant_row(
    const void *__restrict__ x, const void *__restrict__ gain, int64_t row, int K, float eps,
    int8_t *__restrict__ xq, float *__restrict__ s_out, int32_t *__restrict__ rowsum_out) {
  constexpr int EB = dtype_bytes(DT);
  const char *xr = reinterpret_cast<const char *>(x) + row * K * EB;
  int8_t *qr = xq + row * K;
  float sc;
  int rs;
  quantize_row<DT, MODE, NC>(
      xr, reinterpret_cast<const char *>(gain), K, eps,
      [&](int k, uint2 codes) { *reinterpret_cast<uint2 *>(qr + k) = codes; }, sc, rs);
  if ((threadIdx.x & 63) == 0) {
    s_out[row] = sc;
    rowsum_out[row] = rs;
  }
}

template <int DT, int MODE, int NC>
__global__ __launch_bounds__(256) void act_quant_kernel(
    const void *__restrict__ x, const void *__restrict__ gain, int64_t M, int K, float eps,
    int8_t *__restrict__ xq, float *__restrict__ s_out, int32_t *__restrict__ rowsum_out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // a whole wave leaves; nothing below synchronizes
  act_quant_row<DT, MODE, NC>(x, gain, row, K, eps, xq, s_out, rowsum_out);
}

// Several projections' rows in one launch: blockIdx.y selects the call.
template <int DT, int MODE, int NC>
__global__ __launch_bounds__(256) void act_quant_group_kernel(int64_t M, int K, float eps,
                                                              AqCalls calls) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const AqCall &c = calls.c[blockIdx.y];
  act_quant_row<DT, MODE, NC>(c.x, c.gain, row, K, eps, c.xq, c.s, c.rowsum);
}

template <int DT>
static void launch_dt(const void *x, const void *gain, int64_t M, int64_t K, float eps,
                      int8_t *xq, float *s, int32_t *rowsum, hipStream_t stream) {
  const unsigned blocks = (unsigned)((M + 3) / 4);
#define BL_AQ(MODE, NC) \
  act_quant_kernel<DT, MODE, NC><<<blocks, 256, 0, stream>>>(x, gain, M, (int)K, eps, xq, s, rowsum)
  // the float mode issues only the chunk loads a row of K needs
  switch (aq_float_nc(K)) {
    case 2: BL_AQ(kRowFloat, 2); break;
    case 4: BL_AQ(kRowFloat, 4); break;
    case 6: BL_AQ(kRowFloat, 6); break;
    case 8: BL_AQ(kRowFloat, 8); break;
    case 12: BL_AQ(kRowFloat, 12); break;
    default:
      if (row_mode((int)K) == kRowRaw) BL_AQ(kRowRaw, kRowCache);
      else BL_AQ(kRowReload, kRowCache);
      break;
  }
#undef BL_AQ
}

template <int DT>
static void launch_group_dt(const AqCalls &calls, int ncalls, int64_t M, int64_t K, float eps,
                            hipStream_t stream) {
  const dim3 grid((unsigned)((M + 3) / 4), (unsigned)ncalls);
#define BL_AQG(MODE, NC) \
  act_quant_group_kernel<DT, MODE, NC><<<grid, 256, 0, stream>>>(M, (int)K, eps, calls)
  switch (aq_float_nc(K)) {
    case 2: BL_AQG(kRowFloat, 2); break;
    case 4: BL_AQG(kRowFloat, 4); break;
    case 6: BL_AQG(kRowFloat, 6); break;
    case 8: BL_AQG(kRowFloat, 8); break;
    case 12: BL_AQG(kRowFloat, 12); break;
    default:
      if (row_mode((int)K) == kRowRaw) BL_AQG(kRowRaw, kRowCache);
      else BL_AQG(kRowReload, kRowCache);
      break;
  }
#undef BL_AQG
}

hipError_t launch_act_quant_group(const AqCalls &calls, int ncalls, int x_dtype, int64_t M,
                                  int64_t K, float eps, hipStream_t stream) {
  switch (x_dtype) {
    case BL_F32: launch_group_dt<BL_F32>(calls, ncalls, M, K, eps, stream); break;
    case BL_F16: launch_group_dt<BL_F16>(calls, ncalls, M, K, eps, stream); break;
    default: launch_group_dt<BL_BF16>(calls, ncalls, M, K, eps, stream); break;
  }
  return hipGetLastError();
}

hipError_t launch_act_quant(const void *x, int x_dtype, const void *gain,
                            int64_t M, int64_t K, float eps, int8_t *xq,
                            float *s, int32_t *rowsum, hipStream_t stream) {
  switch (x_dtype) {
    case BL_F32: launch_dt<BL_F32>(x, gain, M, K, eps, xq, s, rowsum, stream); break;
    case BL_F16: launch_dt<BL_F16>(x, gain, M, K, eps, xq, s, rowsum, stream); break;
    default: launch_dt<BL_BF16>(x, gain, M, K, eps, xq, s, rowsum, stream); break;
  }
  return hipGetLastError();
}

}  // namespace bl
