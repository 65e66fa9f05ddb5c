// mlgru.hip -- the MLGRU token mixer's recurrence over a sequence.
//
// The pages describe the MLGRU in words only (datacamp "MatMul-freie LLMs:
// Zentrale Konzepte erklärt", section "Kernkomponenten: MLGRU und GLU", the
// MLGRU paragraph and figure panel 2): token by token, the current token
// and the previous hidden state go in, and gates -- vectors of values in
// (0, 1) -- weigh which parts of the previous state and of the current token
// carry on.  Its projections are the block's i_proj and f_proj (hysenlabs ja
// review "matmulfreellm 評価", section "HGRNBit という層構成を読む").  This
// library reads that as
//   a = 1 / (1 + e^-f),   h_t = a h_{t-1} + (1 - a) i_t,   h_{-1} = h0,
// per sequence and channel, in fp32 (the exponential and the reciprocal from
// the hardware exp2 and rcp), h rounded to the activation dtype.
//
// The recurrence is linear in h, so a chunk of L steps maps a start state H
// to P H + S (P the product of the chunk's gates, S the chunk run from
// zero).  Three launches over [B, T, D]:
//   1. per (sequence, chunk, 8 channels): P and S of the chunk;
//   2. per (sequence, channel): the chunk start states, walking the chunks
//      in order (H_{c+1} = P_c H_c + S_c), written over S;
//   3. per (sequence, chunk, 8 channels): the chunk run again from its start
//      state, storing h (and, in the last chunk, the final state hT).
// A sequence of at most L steps is launch 3 alone, from h0.  Each thread
// holds 8 consecutive channels (one 16-byte chunk of a 2-byte dtype), so a
// wave reads 512 channels of a token row per load; the loads of a chunk do
// not depend on the state and run ahead of the recurrence.  HBM traffic:
// i and f twice and h once (10 bytes per element in bf16), plus 24 bytes per
// chunk and channel of P, S and the start states.
#include "bl_common.h"
#include "bl_launch.h"

namespace bl {

namespace {

constexpr int kScanThreads = 256;  // threads per workgroup, 8 channels each

__device__ __forceinline__ float gate_of(float f) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-f * 1.4426950408889634f));
}

template <int DT>
__device__ __forceinline__ void load_token(const void *p, int64_t elem, float v[8]) {
  constexpr int EB = dtype_bytes(DT);
  const char *q = static_cast<const char *>(p) + elem * EB;
  Chunk8<DT> c;
  c.u[0] = *reinterpret_cast<const v4i *>(q);
  if constexpr (DT == BL_F32) c.u[1] = *reinterpret_cast<const v4i *>(q + 16);
  widen<DT>(c, v);
}

template <int DT>
__device__ __forceinline__ void store_token(void *p, int64_t elem, const float v[8]) {
  constexpr int EB = dtype_bytes(DT);
  char *q = static_cast<char *>(p) + elem * EB;
  if constexpr (DT == BL_F32) {
    *reinterpret_cast<v4i *>(q) = v4i{__float_as_int(v[0]), __float_as_int(v[1]),
                                      __float_as_int(v[2]), __float_as_int(v[3])};
    *reinterpret_cast<v4i *>(q + 16) = v4i{__float_as_int(v[4]), __float_as_int(v[5]),
                                           __float_as_int(v[6]), __float_as_int(v[7])};
  } else {
    v4i w;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (int)((uint32_t)out_bits<DT>(v[2 * j]) | ((uint32_t)out_bits<DT>(v[2 * j + 1]) << 16));
    *reinterpret_cast<v4i *>(q) = w;
  }
}

// 1. P and S of chunk blockIdx.y of sequence blockIdx.z.
template <int DT>
__global__ __launch_bounds__(kScanThreads) void mlgru_chunk_kernel(const void *__restrict__ i,
                                                                   const void *__restrict__ f,
                                                                   int T, int D, int L, int C,
                                                                   float *__restrict__ P,
                                                                   float *__restrict__ S) {
  const int d0 = 8 * ((int)blockIdx.x * kScanThreads + (int)threadIdx.x);
  if (d0 >= D) return;
  const int b = (int)blockIdx.z, c = (int)blockIdx.y;
  const int t0 = c * L, t1 = min(T, t0 + L);
  float p[8], s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = 1.0f;
    s[e] = 0.0f;
  }
#pragma unroll 4
  for (int t = t0; t < t1; ++t) {
    const int64_t row = ((int64_t)b * T + t) * D + d0;
    float iv[8], fv[8];
    load_token<DT>(i, row, iv);
    load_token<DT>(f, row, fv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a = gate_of(fv[e]);
      s[e] = a * s[e] + (1.0f - a) * iv[e];
      p[e] = p[e] * a;
    }
  }
  const int64_t o = ((int64_t)b * C + c) * D + d0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    P[o + e] = p[e];
    S[o + e] = s[e];
  }
}

// 2. The chunk start states of sequence b, channel d, written over S.
__global__ __launch_bounds__(kScanThreads) void mlgru_carry_kernel(const float *__restrict__ h0,
                                                                   int B, int D, int C,
                                                                   const float *__restrict__ P,
                                                                   float *__restrict__ S) {
  const int64_t bd = (int64_t)blockIdx.x * kScanThreads + threadIdx.x;
  if (bd >= (int64_t)B * D) return;
  const int64_t b = bd / D, d = bd - b * D;
  float H = h0 ? h0[bd] : 0.0f;
  for (int c = 0; c < C; ++c) {
    const int64_t o = (b * C + c) * D + d;
    const float p = P[o], s = S[o];
    S[o] = H;
    H = p * H + s;
  }
}

// 3. The chunk run from its start state (Hs[(b C + c) D + d], or h0 / zero
// when Hs is null -- one chunk per sequence), storing h and, in the last
// chunk, hT.
template <int DT>
__global__ __launch_bounds__(kScanThreads) void mlgru_apply_kernel(
    const void *__restrict__ i, const void *__restrict__ f, int T, int D, int L, int C,
    const float *__restrict__ Hs, const float *__restrict__ h0, void *__restrict__ h,
    float *__restrict__ hT) {
  const int d0 = 8 * ((int)blockIdx.x * kScanThreads + (int)threadIdx.x);
  if (d0 >= D) return;
  const int b = (int)blockIdx.z, c = (int)blockIdx.y;
  const int t0 = c * L, t1 = min(T, t0 + L);
  float s[8];
  const float *start = Hs ? Hs + ((int64_t)b * C + c) * D + d0 : h0 ? h0 + (int64_t)b * D + d0 : nullptr;
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = start ? start[e] : 0.0f;
#pragma unroll 4
  for (int t = t0; t < t1; ++t) {
    const int64_t row = ((int64_t)b * T + t) * D + d0;
    float iv[8], fv[8];
    load_token<DT>(i, row, iv);
    load_token<DT>(f, row, fv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a = gate_of(fv[e]);
      s[e] = a * s[e] + (1.0f - a) * iv[e];
    }
    store_token<DT>(h, row, s);
  }
  if (hT && c == C - 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) hT[(int64_t)b * D + d0 + e] = s[e];
  }
}

template <int DT>
hipError_t launch_t(const MlgruArgs &a, hipStream_t stream) {
  const int T = (int)a.T, D = (int)a.D, B = (int)a.B;
  const int C = (T + kMlgruChunk - 1) / kMlgruChunk;
  const dim3 grid((unsigned)((D / 8 + kScanThreads - 1) / kScanThreads), (unsigned)C, (unsigned)B);
  if (C == 1) {
    mlgru_apply_kernel<DT><<<grid, kScanThreads, 0, stream>>>(a.i, a.f, T, D, kMlgruChunk, 1,
                                                              nullptr, a.h0, a.h, a.hT);
    return hipGetLastError();
  }
  float *P = static_cast<float *>(a.ws);
  float *S = P + (int64_t)B * C * D;
  mlgru_chunk_kernel<DT><<<grid, kScanThreads, 0, stream>>>(a.i, a.f, T, D, kMlgruChunk, C, P, S);
  const unsigned cgrid = (unsigned)(((int64_t)B * D + kScanThreads - 1) / kScanThreads);
  mlgru_carry_kernel<<<cgrid, kScanThreads, 0, stream>>>(a.h0, B, D, C, P, S);
  mlgru_apply_kernel<DT><<<grid, kScanThreads, 0, stream>>>(a.i, a.f, T, D, kMlgruChunk, C, S,
                                                            a.h0, a.h, a.hT);
  return hipGetLastError();
}

}  // namespace

size_t mlgru_workspace_bytes(int64_t B, int64_t T, int64_t D) {
  const int64_t C = (T + kMlgruChunk - 1) / kMlgruChunk;
  return C <= 1 ? 0 : (size_t)(2 * B * C * D) * sizeof(float);
}

hipError_t launch_mlgru_scan(const MlgruArgs &a, hipStream_t stream) {
  switch (a.dtype) {
    case BL_F32: return launch_t<BL_F32>(a, stream);
    case BL_F16: return launch_t<BL_F16>(a, stream);
    default: return launch_t<BL_BF16>(a, stream);
  }
}

}  // namespace bl
