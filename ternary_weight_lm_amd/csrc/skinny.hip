// skinny.hip -- decode-shaped FusedBitLinear (M <= 16 tokens).
//
// At a handful of tokens the layer is a stream over the packed weights
// (N*K/4 bytes): the matrix cores have far more throughput than needed, so
// the design goal is bytes in flight, not arithmetic.  One workgroup owns one
// packed 32-row tile column (32 output features x all of K); its 4 waves
// split the K-blocks round-robin.
//   1. Every wave first issues the 16-byte loads of its weight tiles (one
//      contiguous 1 KiB per wave per tile), so HBM latency overlaps the
//      prologue.
//   2. Fused variant: the workgroup normalizes and quantizes the M token
//      rows itself, a wave per row, with the shared row quantizer
//      (rowquant.h) into LDS --
//      RMSNorm right before quantization, as in the hysenlabs de review
//      "MatMul-Free LM: Ternary-Gewichte statt Matrixmultiplikation im
//      Transformer", section "HGRNBit: was in einem Block tatsächlich
//      passiert".  Pre-quantized variant: xq, s, rowsum come from the
//      act-quant kernel and A operands are read straight from memory.
//   3. Each tile feeds four v_mfma_i32_16x16x64_i8 (2 output halves x 2
//      k-steps); token rows >= M are zero operands.
//   4. The 4 waves' partial sums are added in LDS; the epilogue subtracts
//      rowsum and rescales by beta / s_m (datacamp "MatMul-freie LLMs:
//      Zentrale Konzepte erklärt", figure panel 4).
// A launch can carry up to kGroupMax independent calls (grouped entry
// point): workgroups are numbered call after call and each finds its call
// from the prefix table in the kernel arguments.
#include <vector>

#include "bl_launch.h"
#include "rowquant.h"

namespace bl {

constexpr int kSkinnyBatch = 16;  // weight tiles held in registers per wave

struct SkinnyCall {
  const void *x;
  const void *gain;
  const int8_t *xq;
  const float *s;
  const int32_t *rowsum;
  const uint4 *packed;
  const float *beta;
  void *out;
  int M, N, K;
};

template <int MAXC>
struct SkinnyLaunch {
  SkinnyCall call[MAXC];
  int first_block[MAXC + 1];
  int ncalls;
  float eps;
};

template <bool FUSED, int DT, int OUT, int MAXC, int RMODE>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyLaunch<MAXC> L) {
  extern __shared__ __align__(16) int8_t xs[];  // fused: [M][K + 16] int8
  __shared__ int red[4][8][64];
  __shared__ float s_row[16];
  __shared__ int rs_row[16];

  int c = 0;
  if constexpr (MAXC > 1) {
    while (c + 1 < L.ncalls && (int)blockIdx.x >= L.first_block[c + 1]) ++c;
  }
  const SkinnyCall &p = L.call[c];
  const int nt = (int)blockIdx.x - L.first_block[c];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
    for (int m = w; m < M; m += 4) {  // a wave per token row
      const char *xr = reinterpret_cast<const char *>(p.x) + (int64_t)m * K * EB;
      int8_t *dst = xs + m * lds_stride;
      float sc;
      int rs;
      auto sink = [&](int k, uint2 codes) { *reinterpret_cast<uint2 *>(dst + k) = codes; };
      // fused calls have K <= 8192: the row stays in registers (RMODE is
      // chosen on the host from the largest K of the launch)
      quantize_row<DT, RMODE>(xr, reinterpret_cast<const char *>(p.gain), K, L.eps, sink, sc, rs);
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
    const int j = idx >> 6, Lq = idx & 63;
    const int h = j >> 2, i = j & 3;
    const int m = 4 * (Lq >> 4) + i;
    if (m >= M) continue;
    const int n = nt * 32 + 16 * h + (Lq & 15);
    const int v = red[0][j][Lq] + red[1][j][Lq] + red[2][j][Lq] + red[3][j][Lq] - rs_row[m];
    const int64_t o = (int64_t)m * p.N + n;
    if constexpr (OUT == kOutI32) {
      reinterpret_cast<int32_t *>(p.out)[o] = v;
    } else {
      store1<OUT>(p.out, o, (float)v * div_rn(bt, s_row[m]));
    }
  }
}

static SkinnyCall to_call(const SkinnyArgs &a) {
  SkinnyCall c;
  c.x = a.x;
  c.gain = a.gain;
  c.xq = a.xq;
  c.s = a.s;
  c.rowsum = a.rowsum;
  c.packed = reinterpret_cast<const uint4 *>(a.packed);
  c.beta = a.beta;
  c.out = a.out;
  c.M = (int)a.M;
  c.N = (int)a.N;
  c.K = (int)a.K;
  return c;
}

template <bool FUSED, int DT, int MAXC, int RMODE>
static void launch_out(const SkinnyLaunch<MAXC> &L, int out_kind, unsigned grid, size_t lds,
                       hipStream_t stream) {
  switch (out_kind) {
    case BL_F32: skinny_kernel<FUSED, DT, BL_F32, MAXC, RMODE><<<grid, 256, lds, stream>>>(L); break;
    case BL_F16: skinny_kernel<FUSED, DT, BL_F16, MAXC, RMODE><<<grid, 256, lds, stream>>>(L); break;
    case BL_BF16: skinny_kernel<FUSED, DT, BL_BF16, MAXC, RMODE><<<grid, 256, lds, stream>>>(L); break;
    default: skinny_kernel<FUSED, DT, kOutI32, MAXC, RMODE><<<grid, 256, lds, stream>>>(L); break;
  }
}

template <bool FUSED, int DT, int MAXC>
static void launch_mode(const SkinnyLaunch<MAXC> &L, int out_kind, unsigned grid, size_t lds,
                        int64_t kmax, hipStream_t stream) {
  if constexpr (!FUSED) {
    launch_out<FUSED, DT, MAXC, kRowFloat>(L, out_kind, grid, lds, stream);
  } else {
    if (row_mode((int)kmax) == kRowFloat)
      launch_out<FUSED, DT, MAXC, kRowFloat>(L, out_kind, grid, lds, stream);
    else
      launch_out<FUSED, DT, MAXC, kRowRaw>(L, out_kind, grid, lds, stream);
  }
}

template <int MAXC>
static void launch_any(const SkinnyLaunch<MAXC> &L, bool fused, int x_dtype, int out_kind,
                       unsigned grid, size_t lds, int64_t kmax, hipStream_t stream) {
  if (fused) {
    switch (x_dtype) {
      case BL_F32: launch_mode<true, BL_F32, MAXC>(L, out_kind, grid, lds, kmax, stream); break;
      case BL_F16: launch_mode<true, BL_F16, MAXC>(L, out_kind, grid, lds, kmax, stream); break;
      default: launch_mode<true, BL_BF16, MAXC>(L, out_kind, grid, lds, kmax, stream); break;
    }
  } else {
    launch_mode<false, BL_F32, MAXC>(L, out_kind, grid, lds, kmax, stream);
  }
}

static bool decode_ok(const SkinnyArgs &a) {
  return a.fused && decode_fits(a.M, a.K, a.x_dtype);
}

static DecodeArgs decode_args(const SkinnyArgs &a) {
  DecodeArgs d{};
  d.x_dtype = a.x_dtype;
  d.M = a.M;
  d.N = a.N;
  d.K = a.K;
  d.eps = a.eps;
  d.out_kind = a.out_kind;
  d.ncalls = 0;
  return d;
}

static void decode_add(DecodeArgs &d, const SkinnyArgs &a) {
  d.x[d.ncalls] = a.x;
  d.gain[d.ncalls] = a.gain;
  d.packed[d.ncalls] = a.packed;
  d.beta[d.ncalls] = a.beta;
  d.out[d.ncalls] = a.out;
  ++d.ncalls;
}

hipError_t launch_skinny(const SkinnyArgs &a, hipStream_t stream) {
  if (decode_ok(a)) {
    DecodeArgs d = decode_args(a);
    decode_add(d, a);
    return launch_decode(d, stream);
  }
  SkinnyLaunch<1> L;
  L.call[0] = to_call(a);
  L.first_block[0] = 0;
  L.first_block[1] = (int)(a.N / 32);
  L.ncalls = 1;
  L.eps = a.eps;
  const size_t lds = a.fused ? (size_t)a.M * (size_t)(a.K + 16) : 0;
  launch_any<1>(L, a.fused, a.x_dtype, a.out_kind, (unsigned)(a.N / 32), lds, a.K, stream);
  return hipGetLastError();
}

// Consecutive calls of one shape that the decode kernel takes go out in
// launches of up to kDecodeCalls; the others are gathered into launches of
// the skinny kernel of up to kGroupMax calls.
hipError_t launch_skinny_grouped(const SkinnyArgs *calls, int ncalls, hipStream_t stream) {
  std::vector<SkinnyArgs> rest;
  for (int i = 0; i < ncalls;) {
    const SkinnyArgs &a = calls[i];
    if (!decode_ok(a)) {
      rest.push_back(a);
      ++i;
      continue;
    }
    DecodeArgs d = decode_args(a);
    while (i < ncalls && d.ncalls < kDecodeCalls && decode_ok(calls[i]) && calls[i].M == a.M &&
           calls[i].K == a.K && calls[i].N == a.N)
      decode_add(d, calls[i++]);
    const hipError_t e = launch_decode(d, stream);
    if (e != hipSuccess) return e;
  }
  const int nrest = (int)rest.size();
  for (int base = 0; base < nrest; base += kGroupMax) {
    const int n = nrest - base < kGroupMax ? nrest - base : kGroupMax;
    SkinnyLaunch<kGroupMax> L;
    int blocks = 0;
    size_t lds = 0;
    int64_t kmax = 0;
    for (int i = 0; i < n; ++i) {
      const SkinnyArgs &a = rest[base + i];
      L.call[i] = to_call(a);
      L.first_block[i] = blocks;
      blocks += (int)(a.N / 32);
      const size_t l = (size_t)a.M * (size_t)(a.K + 16);
      if (l > lds) lds = l;
      if (a.K > kmax) kmax = a.K;
    }
    for (int i = n; i <= kGroupMax; ++i) L.first_block[i] = blocks;
    L.ncalls = n;
    L.eps = rest[base].eps;
    launch_any<kGroupMax>(L, true, rest[base].x_dtype, rest[base].out_kind, (unsigned)blocks,
                          lds, kmax, stream);
  }
  return hipGetLastError();
}

}  // namespace bl
