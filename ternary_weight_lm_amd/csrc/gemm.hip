// gemm.hip -- tiled ternary contraction on the gfx950 int8 matrix cores.
//
// acc[m, n] = sum_k xq[m, k] * Wq[n, k]: with ternary weights every product
// is a negate / zero / keep of an activation (datacamp "MatMul-freie LLMs:
// Zentrale Konzepte erklärt", section "MatMul durch ternäre Operationen
// ersetzen"), followed by the scaled rescale of figure panel 4.  On gfx950
// the cheapest exact way to add up many int8 values is still the dense i8
// MFMA (v_mfma_i32_16x16x64_i8), so the stored codes c = Wq + 1 in {0,1,2}
// are fed to it as int8 and the signed sum is recovered exactly as
//   sum_k xq * Wq = sum_k xq * c - sum_k xq      (rowsum from act-quant).
//
// Workgroup tile: BM = 32*MI token rows x BN = 128 output rows, K in blocks
// of 128 (one packed tile column).  4 waves as 2 x 2; wave (wm, wn) owns
// 16*MI rows x 64 outputs = MI x 4 MFMA blocks of 16 x 16.
//   A (xq): global -> registers -> LDS, double-buffered, 16-byte chunks of a
//           128-byte row XOR-swizzled with (row & 7) so the 16 lanes that read
//           one column of chunks hit distinct banks.
//   B (packed codes): each wave loads its two 1 KiB tiles per k-block
//           straight into registers (one 16-byte load per lane per tile, the
//           layout was built for exactly this) and unpacks them with
//           shift + mask; no LDS traffic for weights.
// Epilogue: subtract rowsum, multiply by beta / s_m, round to the output
// dtype (or store the exact int32 accumulator).
// Workgroup ids are remapped so each of the 8 XCDs (which receive ids
// round-robin) works on a contiguous range of tiles, keeping A rows and B
// columns of neighbouring tiles in that XCD's L2.
#include <algorithm>

#include "bl_common.h"
#include "bl_launch.h"

namespace bl {

template <int MI, int OUT>
__global__ __launch_bounds__(256, 2) void gemm_mfma_kernel(
    const int8_t *__restrict__ xq, const int32_t *__restrict__ rowsum,
    const float *__restrict__ s, const uint4 *__restrict__ packed,
    const float *__restrict__ beta, int M, int N, int K,
    void *__restrict__ out, int tiles_m, int tiles_n) {
  constexpr int BM = 32 * MI;
  constexpr int BN = 128;
  __shared__ __align__(16) uint8_t lds[2][BM * 128];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile order.
  const int ntiles = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  const int per = ntiles / 8, rem = ntiles % 8;
  const int xcd = bid % 8, local = bid / 8;
  const int t = xcd < rem ? xcd * (per + 1) + local
                          : rem * (per + 1) + (xcd - rem) * per + local;
  const int tm = t / tiles_n, tn = t % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int KB = K >> 7;
  const int NT = N >> 5;

  // ---- A tile: BM rows x 8 chunks of 16 B, MI chunks per thread; thread
  // chunk j covers row (tid + 256 j) / 8, chunk (tid + 256 j) % 8.
  const int8_t *a_src[MI];
  int a_dst[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int c = tid + 256 * j;
    const int row = c >> 3, ch = c & 7;
    a_src[j] = xq + (int64_t)min(m0 + row, M - 1) * K + ch * 16;
    a_dst[j] = row * 128 + ((ch ^ (row & 7)) << 4);
  }
  // ---- B: the wave's two packed 32-row tiles; missing tiles read as zero.
  const int nt0 = (n0 >> 5) + 2 * wn;
  const uint4 *b_src0 = packed + (int64_t)nt0 * KB * 64 + lane;
  const uint4 *b_src1 = b_src0 + (int64_t)KB * 64;
  const bool b_ok0 = nt0 < NT, b_ok1 = nt0 + 1 < NT;

  v4i acc[MI][4];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mi][nb] = v4i{0, 0, 0, 0};

  uint4 areg[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) areg[j] = *reinterpret_cast<const uint4 *>(a_src[j]);
  uint4 b0 = b_ok0 ? b_src0[0] : make_uint4(0, 0, 0, 0);
  uint4 b1 = b_ok1 ? b_src1[0] : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < MI; ++j) *reinterpret_cast<uint4 *>(&lds[0][a_dst[j]]) = areg[j];
  __syncthreads();

  const int arow0 = wm * 16 * MI + (lane & 15);
  for (int kb = 0; kb < KB; ++kb) {
    const uint4 c0 = b0, c1 = b1;
    // prefetch the next k-block (the last iteration re-reads block KB-1; the
    // copy it leaves in the idle LDS buffer is never read)
    const int kn = min(kb + 1, KB - 1);
    {
      const int64_t ko = (int64_t)kn * 128;
#pragma unroll
      for (int j = 0; j < MI; ++j) areg[j] = *reinterpret_cast<const uint4 *>(a_src[j] + ko);
      if (b_ok0) b0 = b_src0[kn * 64];
      if (b_ok1) b1 = b_src1[kn * 64];
    }
    const uint8_t *As = lds[kb & 1];
    v4i a[MI][2];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = arow0 + 16 * mi;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int ch = 2 * (lane >> 4) + s2;
        a[mi][s2] = *reinterpret_cast<const v4i *>(As + row * 128 + ((ch ^ (row & 7)) << 4));
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      // word (h, s2) of a lane slot sits at dword 2h + s2
      const v4i w00 = unpack_codes(s2 ? c0.y : c0.x);
      const v4i w01 = unpack_codes(s2 ? c0.w : c0.z);
      const v4i w10 = unpack_codes(s2 ? c1.y : c1.x);
      const v4i w11 = unpack_codes(s2 ? c1.w : c1.z);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        acc[mi][0] = mfma16x16x64(a[mi][s2], w00, acc[mi][0]);
        acc[mi][1] = mfma16x16x64(a[mi][s2], w01, acc[mi][1]);
        acc[mi][2] = mfma16x16x64(a[mi][s2], w10, acc[mi][2]);
        acc[mi][3] = mfma16x16x64(a[mi][s2], w11, acc[mi][3]);
      }
    }
#pragma unroll
    for (int j = 0; j < MI; ++j)
      *reinterpret_cast<uint4 *>(&lds[(kb + 1) & 1][a_dst[j]]) = areg[j];
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4*(lane/16)+i of each 16x16 block.
  const float bt = OUT == kOutI32 ? 0.0f : *beta;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 16 * MI + 16 * mi + 4 * (lane >> 4) + i;
      if (m >= M) continue;
      const int rs = rowsum[m];
      const float scale = OUT == kOutI32 ? 0.0f : div_rn(bt, s[m]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int n = n0 + 64 * wn + 16 * nb + (lane & 15);
        if (n >= N) continue;
        const int v = acc[mi][nb][i] - rs;
        const int64_t idx = (int64_t)m * N + n;
        if constexpr (OUT == kOutI32) {
          reinterpret_cast<int32_t *>(out)[idx] = v;
        } else {
          store1<OUT>(out, idx, (float)v * scale);
        }
      }
    }
}

template <int MI>
static hipError_t launch_mi(const int8_t *xq, const int32_t *rowsum,
                            const float *s, const void *packed,
                            const float *beta, int64_t M, int64_t N, int64_t K,
                            void *out, int out_kind, hipStream_t stream) {
  const int BM = 32 * MI;
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + 127) / 128);
  const unsigned grid = (unsigned)(tiles_m * tiles_n);
  const uint4 *pk = reinterpret_cast<const uint4 *>(packed);
#define BL_GEMM_CASE(KIND)                                                   \
  gemm_mfma_kernel<MI, KIND><<<grid, 256, 0, stream>>>(                      \
      xq, rowsum, s, pk, beta, (int)M, (int)N, (int)K, out, tiles_m, tiles_n)
  switch (out_kind) {
    case BL_F32: BL_GEMM_CASE(BL_F32); break;
    case BL_F16: BL_GEMM_CASE(BL_F16); break;
    case BL_BF16: BL_GEMM_CASE(BL_BF16); break;
    default: BL_GEMM_CASE(kOutI32); break;
  }
#undef BL_GEMM_CASE
  return hipGetLastError();
}

hipError_t launch_gemm_mfma(const int8_t *xq, const int32_t *rowsum,
                            const float *s, const void *packed,
                            const float *beta, int64_t M, int64_t N,
                            int64_t K, void *out, int out_kind,
                            hipStream_t stream) {
  if (M <= 32) return launch_mi<1>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, stream);
  if (M <= 64) return launch_mi<2>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, stream);
  return launch_mi<4>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, stream);
}

}  // namespace bl
