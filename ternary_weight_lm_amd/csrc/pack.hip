// pack.hip -- offline weight packing for gfx950.
//
// Absmean ternarization (datacamp "MatMul-freie LLMs: Zentrale Konzepte
// erklärt", section "MatMul durch ternäre Operationen ersetzen"): the whole
// matrix is divided by its mean absolute value and every entry is rounded to
// the nearest of -1, 0, +1.  Three launches:
//   1. absum_partial_kernel: fp64 partial sums of |W| per workgroup;
//   2. beta_kernel: one workgroup adds the partials in a fixed order and
//      writes beta = max(fp32(sum / (N*K)), 1e-5);
//   3. pack_kernel: one thread per 16-byte lane slot of the 2-bit tile
//      layout (bitlinear.h) writes four 32-bit code words.
// The rounding rule clamp(rne(fp32(W / beta)), -1, 1) is evaluated as the
// exactly equivalent comparison |W| > beta * (0.5 + 2^-25) in fp64: the fp32
// quotient exceeds 0.5 (and so rounds to +-1) exactly when the real quotient
// is above the midpoint between 0.5 and the next float, and the product is
// exact in fp64 (24-bit times 25-bit mantissa).
#include "bl_common.h"
#include "bl_launch.h"

namespace bl {

constexpr int kAbsBlocks = 1024;

size_t pack_workspace_bytes() { return kAbsBlocks * sizeof(double); }

__global__ __launch_bounds__(256) void absum_partial_kernel(
    const float4 *__restrict__ W, int64_t n4, double *__restrict__ partial) {
  double acc = 0.0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const float4 w = W[i];
    acc += fabs((double)w.x);
    acc += fabs((double)w.y);
    acc += fabs((double)w.z);
    acc += fabs((double)w.w);
  }
  acc = wave_sum(acc);
  __shared__ double red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = ((red[0] + red[1]) + red[2]) + red[3];
}

__global__ __launch_bounds__(256) void beta_kernel(const double *__restrict__ partial,
                                                   int nparts, int64_t count,
                                                   float *__restrict__ beta) {
  double acc = 0.0;
  for (int i = threadIdx.x; i < nparts; i += 256) acc += partial[i];
  acc = wave_sum(acc);
  __shared__ double red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double total = ((red[0] + red[1]) + red[2]) + red[3];
    const float mean = (float)(total / (double)count);
    *beta = fmaxf(mean, 1e-5f);
  }
}

// glu_F > 0: W is a gate_proj [2F, K] packed in the GLU row order (packed
// row 32t + 16h + c holds source row h * F + 16t + c), so that each 32-row
// tile carries 16 SiLU-gated rows and the 16 rows they multiply.
__global__ __launch_bounds__(256) void pack_kernel(const float *__restrict__ W,
                                                   int64_t N, int64_t K,
                                                   const float *__restrict__ beta,
                                                   uint4 *__restrict__ packed,
                                                   int64_t glu_F) {
  const int64_t KB = K / 128;
  const int64_t nslots = (N / 32) * KB * 64;
  const int64_t slot = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (slot >= nslots) return;
  const int64_t tile = slot >> 6;
  const int L = (int)(slot & 63);
  const int64_t nt = tile / KB, kb = tile % KB;
  const double thr = (double)(*beta) * (0.5 + 0x1p-25);
  uint32_t words[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = i >> 1, s = i & 1;
    const int64_t n = glu_F > 0 ? h * glu_F + nt * 16 + (L & 15) : nt * 32 + h * 16 + (L & 15);
    const int64_t k0 = kb * 128 + 16 * (2 * (L >> 4) + s);
    const float4 *src = reinterpret_cast<const float4 *>(W + n * K + k0);
    float w[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = src[q];
      w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
    }
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t code = fabs((double)w[e]) > thr ? (w[e] > 0.0f ? 2u : 0u) : 1u;
      word |= code << (8 * (e & 3) + 2 * (e >> 2));
    }
    words[i] = word;
  }
  packed[slot] = make_uint4(words[0], words[1], words[2], words[3]);
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint4 *__restrict__ packed,
                                                     int64_t N, int64_t K,
                                                     int8_t *__restrict__ Wq) {
  const int64_t KB = K / 128;
  const int64_t nslots = (N / 32) * KB * 64;
  const int64_t slot = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (slot >= nslots) return;
  const int64_t tile = slot >> 6;
  const int L = (int)(slot & 63);
  const int64_t nt = tile / KB, kb = tile % KB;
  const uint4 u = packed[slot];
  const uint32_t words[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = i >> 1, s = i & 1;
    const int64_t n = nt * 32 + h * 16 + (L & 15);
    const int64_t k0 = kb * 128 + 16 * (2 * (L >> 4) + s);
    const v4i c = unpack_codes(words[i]);
    // codes 0,1,2 -> -1,0,+1 in every byte (no byte ever borrows: each
    // byte is >= 0x80 before the subtraction)
    uint4 o;
    o.x = (((uint32_t)c.x | 0x80808080u) - 0x01010101u) ^ 0x80808080u;
    o.y = (((uint32_t)c.y | 0x80808080u) - 0x01010101u) ^ 0x80808080u;
    o.z = (((uint32_t)c.z | 0x80808080u) - 0x01010101u) ^ 0x80808080u;
    o.w = (((uint32_t)c.w | 0x80808080u) - 0x01010101u) ^ 0x80808080u;
    *reinterpret_cast<uint4 *>(Wq + n * K + k0) = o;
  }
}

hipError_t launch_pack(const float *W, int64_t N, int64_t K, void *packed,
                       float *beta, void *ws, int64_t glu_F, hipStream_t stream) {
  const int64_t n4 = N * K / 4;
  const int nparts = (int)std::min<int64_t>(kAbsBlocks, (n4 + 255) / 256);
  double *partial = reinterpret_cast<double *>(ws);
  absum_partial_kernel<<<nparts, 256, 0, stream>>>(
      reinterpret_cast<const float4 *>(W), n4, partial);
  beta_kernel<<<1, 256, 0, stream>>>(partial, nparts, N * K, beta);
  const int64_t nslots = N * K / 64;
  pack_kernel<<<(unsigned)((nslots + 255) / 256), 256, 0, stream>>>(
      W, N, K, beta, reinterpret_cast<uint4 *>(packed), glu_F);
  return hipGetLastError();
}

hipError_t launch_unpack(const void *packed, int64_t N, int64_t K, int8_t *Wq,
                         hipStream_t stream) {
  const int64_t nslots = N * K / 64;
  unpack_kernel<<<(unsigned)((nslots + 255) / 256), 256, 0, stream>>>(
      reinterpret_cast<const uint4 *>(packed), N, K, Wq);
  return hipGetLastError();
}

}  // namespace bl
