// actquant.hip -- RMSNorm fused with per-token absmax int8 quantization.
//
// The norm sits inside every FusedBitLinear and runs right before the
// activations are quantized (hysenlabs de review "MatMul-Free LM:
// Ternary-Gewichte statt Matrixmultiplikation im Transformer", section
// "HGRNBit: was in einem Block tatsächlich passiert"; datacamp "MatMul-freie
// LLMs: Zentrale Konzepte erklärt", figure panel 5).  One 64-lane wave per
// token row runs the shared row quantizer (rowquant.h): the row is read once
// with 16-byte loads (widened and kept in registers up to K = 4096, re-read
// from cache per pass beyond K = 8192), the three reductions are
// cross-lane shuffles, and the int8 codes leave as coalesced 8-byte stores.
// Four rows per 256-thread workgroup, no barriers.  Few rows, or rows past
// K = 4096, instead get a workgroup each, split over its four waves with
// the same association of every sum (act_quant_split_row).  The grouped
// kernels take up to three projections' rows in one launch.  HBM traffic:
// one read of x, one write of xq, 8 bytes of scale + row sum.
#include "bl_launch.h"
#include "rowquant.h"

namespace bl {


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

// ---- few rows: one row per workgroup, split over its 4 waves.  A wave
// per row leaves a long row's passes (K = 5632: 11 chunks of 8 per lane)
// in one wave's instruction stream while most CUs idle; here wave w takes
// the chunk rounds c = w + 4 r of the row quantizer's layout (lane L: the 8
// elements 8 L + 512 c), which are exactly its slot group w of the sum of
// squares.  The four per-lane partials meet in LDS and are combined as
// (p0 + p1) + (p2 + p3) before the same DPP tree, so the sum -- and every
// code and scale -- is bit-identical to the one-wave kernel's; the absmax
// and the row sum are exact in any order.  NR: chunk rounds per wave
// (K <= 2048 NR).
template <int DT, int NR>
__device__ __forceinline__ void act_quant_split_row(
    const void *__restrict__ x, const void *__restrict__ gain, int64_t row, int K, float eps,
    int8_t *__restrict__ xq, float *__restrict__ s_out, int32_t *__restrict__ rowsum_out) {
  __shared__ double part_ss[4][64];
  __shared__ float part_max[4];
  __shared__ int part_rs[4];
  constexpr int EB = dtype_bytes(DT);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nch = (K + 511) >> 9;
  const auto kof = [&](int r) { return 8 * lane + 512 * (w + 4 * r); };
  const auto live = [&](int r) { return w + 4 * r < nch && kof(r) < K; };
  const rsrc_t xr = make_rsrc(reinterpret_cast<const char *>(x) + row * K * EB, (uint32_t)(K * EB));
  const rsrc_t gr = make_rsrc(gain, (uint32_t)(K * EB));
  Chunk8<DT> xraw[NR], graw[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) xraw[r] = bload_chunk<DT>(xr, live(r) ? (uint32_t)(kof(r) * EB) : kOob);
#pragma unroll
  for (int r = 0; r < NR; ++r) graw[r] = bload_chunk<DT>(gr, live(r) ? (uint32_t)(kof(r) * EB) : kOob);
  float v[NR][8];
  double ss = 0.0;
#pragma unroll
  for (int r = 0; r < NR; ++r)
    if (live(r)) {
      widen<DT>(xraw[r], v[r]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fma((double)v[r][e], (double)v[r][e], ss);
    }
  part_ss[w][lane] = ss;
  __syncthreads();
  const float rr = rms_inv(wave_sum((part_ss[0][lane] + part_ss[1][lane]) +
                                    (part_ss[2][lane] + part_ss[3][lane])),
                           K, eps);
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < NR; ++r)
    if (live(r)) {
      float g[8];
      widen<DT>(graw[r], g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[r][e] = (v[r][e] * rr) * g[e];
        amax = fmaxf(amax, fabsf(v[r][e]));
      }
    }
  amax = wave_max(amax);
  if (lane == 0) part_max[w] = amax;
  __syncthreads();
  const float sc = act_scale(fmaxf(fmaxf(part_max[0], part_max[1]), fmaxf(part_max[2], part_max[3])));
  int8_t *qr = xq + row * K;
  int rs = 0;
#pragma unroll
  for (int r = 0; r < NR; ++r)
    if (live(r)) {
      int q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = quant8(v[r][e], sc);
      const uint2 codes = make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
      rs = __builtin_amdgcn_sdot4((int)codes.x, 0x01010101, rs, false);
      rs = __builtin_amdgcn_sdot4((int)codes.y, 0x01010101, rs, false);
      *reinterpret_cast<uint2 *>(qr + kof(r)) = codes;
    }
  rs = wave_sum(rs);
  if (lane == 0) part_rs[w] = rs;
  __syncthreads();
  if (threadIdx.x == 0) {
    s_out[row] = sc;
    rowsum_out[row] = (part_rs[0] + part_rs[1]) + (part_rs[2] + part_rs[3]);
  }
}

template <int DT, int NR>
__global__ __launch_bounds__(256) void act_quant_split_kernel(
    const void *__restrict__ x, const void *__restrict__ gain, int K, float eps,
    int8_t *__restrict__ xq, float *__restrict__ s_out, int32_t *__restrict__ rowsum_out) {
  act_quant_split_row<DT, NR>(x, gain, blockIdx.x, K, eps, xq, s_out, rowsum_out);
}

template <int DT, int NR>
__global__ __launch_bounds__(256) void act_quant_split_group_kernel(int K, float eps, AqCalls calls) {
  const AqCall &c = calls.c[blockIdx.y];
  act_quant_split_row<DT, NR>(c.x, c.gain, blockIdx.x, K, eps, c.xq, c.s, c.rowsum);
}

// Rows the split kernel takes: K <= 8192 (at most 4 chunk rounds per wave)
// and either few rows (one wave per row leaves CUs idle: M = 64, K = 7040
// 9.2 -> 3.6 us; M = 512, K = 2560 4.1 -> 3.5 us) or rows past K = 4096,
// whose one-wave passes keep raw chunks (M = 8192, K = 7040: 45 -> 33 us).
// Many short rows stay one per wave (M = 4096, K = 2048: 7.4 us, split 10).
constexpr bool split_fits(int64_t M, int64_t K) { return K <= 8192 && (M <= 1024 || K > 4096); }
constexpr int split_nr(int64_t K) { return (int)((((K + 511) >> 9) + 3) >> 2); }

// Many rows read by up to three projections (HGRN's i/f/g share their
// block input): one wave per row loads the row once, computes its r once
// (row_rms) and runs the gain-dependent passes per call (quantize_scaled),
// with the bits of one call per launch.
template <int DT, int NC>
__global__ __launch_bounds__(256) void act_quant_shared_kernel(int64_t M, int K, float eps,
                                                               int ncalls, AqCalls calls) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // a whole wave leaves; nothing below synchronizes
  constexpr int EB = dtype_bytes(DT);
  const int lane = threadIdx.x & 63;
  const auto kof = [&](int c) { return 8 * lane + 512 * c; };
  const rsrc_t xr = make_rsrc(static_cast<const char *>(calls.c[0].x) + row * K * EB,
                              (uint32_t)(K * EB));
  Chunk8<DT> xraw[NC], graw[kGroupCalls][NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) xraw[c] = bload_chunk<DT>(xr, (uint32_t)(kof(c) * EB));
#pragma unroll
  for (int j = 0; j < kGroupCalls; ++j) {
    const rsrc_t gr = make_rsrc(calls.c[j].gain, j < ncalls ? (uint32_t)(K * EB) : 0u);
#pragma unroll
    for (int c = 0; c < NC; ++c) graw[j][c] = bload_chunk<DT>(gr, (uint32_t)(kof(c) * EB));
  }
  const float r = row_rms<DT, NC>(xraw, K, eps);
#pragma unroll
  for (int j = 0; j < kGroupCalls; ++j) {
    if (j >= ncalls) break;
    const AqCall &cj = calls.c[j];
    int8_t *qr = cj.xq + row * K;
    float sc;
    int rs;
    quantize_scaled<DT, NC>(xraw, graw[j], K, r,
                            [&](int k, uint2 codes) { *reinterpret_cast<uint2 *>(qr + k) = codes; },
                            sc, rs);
    if (lane == 0) {
      cj.s[row] = sc;
      cj.rowsum[row] = rs;
    }
  }
}

template <int DT>
static void launch_dt(const void *x, const void *gain, int64_t M, int64_t K, float eps,
                      int8_t *xq, float *s, int32_t *rowsum, hipStream_t stream) {
  if (split_fits(M, K)) {
#define BL_AQS(NR) act_quant_split_kernel<DT, NR><<<(unsigned)M, 256, 0, stream>>>(x, gain, (int)K, eps, xq, s, rowsum)
    switch (split_nr(K)) {
      case 1: BL_AQS(1); break;
      case 2: BL_AQS(2); break;
      case 3: BL_AQS(3); break;
      default: BL_AQS(4); break;
    }
#undef BL_AQS
    return;
  }
  // many rows of K <= 4096, or K > 8192 (re-read per pass)
  const unsigned blocks = (unsigned)((M + 3) / 4);
#define BL_AQ(MODE, NC) \
  act_quant_kernel<DT, MODE, NC><<<blocks, 256, 0, stream>>>(x, gain, M, (int)K, eps, xq, s, rowsum)
  // the float mode issues only the chunk loads a row of K needs
  if (K > 4096) {
    BL_AQ(kRowReload, kRowCache);
  } else {
    switch (row_cache((int)K)) {
      case 2: BL_AQ(kRowFloat, 2); break;
      case 4: BL_AQ(kRowFloat, 4); break;
      case 6: BL_AQ(kRowFloat, 6); break;
      default: BL_AQ(kRowFloat, 8); break;
    }
  }
#undef BL_AQ
}

// Below this many rows one wave per row per call fills the chip better
// than one wave per row running every call.
constexpr int64_t kSharedMinRows = 3072;

template <int DT>
static void launch_group_dt(const AqCalls &calls, int ncalls, int64_t M, int64_t K, float eps,
                            hipStream_t stream) {
  bool shared = ncalls > 1;
  for (int j = 1; j < ncalls; ++j) shared = shared && calls.c[j].x == calls.c[0].x;
  if (shared && M >= kSharedMinRows && !split_fits(M, K) && K <= 4096) {
    const unsigned blocks = (unsigned)((M + 3) / 4);
#define BL_AQX(NC) \
  act_quant_shared_kernel<DT, NC><<<blocks, 256, 0, stream>>>(M, (int)K, eps, ncalls, calls)
    switch (row_cache((int)K)) {
      case 2: BL_AQX(2); break;
      case 4: BL_AQX(4); break;
      case 6: BL_AQX(6); break;
      default: BL_AQX(8); break;
    }
#undef BL_AQX
    return;
  }
  if (split_fits(M, K)) {
    const dim3 g((unsigned)M, (unsigned)ncalls);
#define BL_AQSG(NR) act_quant_split_group_kernel<DT, NR><<<g, 256, 0, stream>>>((int)K, eps, calls)
    switch (split_nr(K)) {
      case 1: BL_AQSG(1); break;
      case 2: BL_AQSG(2); break;
      case 3: BL_AQSG(3); break;
      default: BL_AQSG(4); break;
    }
#undef BL_AQSG
    return;
  }
  const dim3 grid((unsigned)((M + 3) / 4), (unsigned)ncalls);
#define BL_AQG(MODE, NC) \
  act_quant_group_kernel<DT, MODE, NC><<<grid, 256, 0, stream>>>(M, (int)K, eps, calls)
  if (K > 4096) {
    BL_AQG(kRowReload, kRowCache);
  } else {
    switch (row_cache((int)K)) {
      case 2: BL_AQG(kRowFloat, 2); break;
      case 4: BL_AQG(kRowFloat, 4); break;
      case 6: BL_AQG(kRowFloat, 6); break;
      default: BL_AQG(kRowFloat, 8); break;
    }
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
