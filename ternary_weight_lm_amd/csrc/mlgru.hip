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
// zero).  L = 16 for 33..1023 steps, else 32 (mlgru_chunk_len): shorter
// chunks put more independent recurrences on the two streaming launches,
// longer ones shorten the carry (2.7B width, one sequence: 8192 steps 46.1 /
// 44.8 / 45.2 us per scan at L = 16 / 32 / 64, 512 steps 10.4 at L = 16
// against 12.5 at 32; before the carry composed groups of chunks in
// parallel, 64 was the best length at 8192 steps).  Three launches over
// [B, T, D]:
//   1. per (sequence, chunk, 2 channels): P and S of the chunk;
//   2. per (sequence, channel): the chunk start states (H_{c+1} = P_c H_c +
//      S_c), written over S -- up to 32 chunks walked in order, more
//      composed over groups of 32 chunks in parallel and chained across the
//      groups;
//   3. per (sequence, chunk, 2 channels): the chunk run again from its start
//      state, storing h (and, in the last chunk, the final state hT).
// A sequence of at most L steps is launch 3 alone, from h0.  A thread holds
// two consecutive channels, so a wave reads 128 channels of a token row per
// load and a 2560-wide row spreads over 20 waves; the loads of a chunk go
// out in batches ahead of the recurrence, which does not feed them.  HBM
// traffic: i and f twice and h once (10 bytes per element in bf16), plus 24
// bytes per chunk and channel of P, S and the start states.
#include "bl_common.h"
#include "bl_launch.h"

namespace bl {

namespace {

constexpr int kScanThreads = 256;  // threads per workgroup
constexpr int kCpt = 2;            // consecutive channels per thread

__device__ __forceinline__ float gate_of(float f) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-f * 1.4426950408889634f));
}

// The kCpt channels a thread holds in one token row: one dword of a 2-byte
// dtype, two of fp32.
template <int DT>
struct Pair {
  uint32_t w[DT == BL_F32 ? 2 : 1];
};

template <int DT>
__device__ __forceinline__ Pair<DT> load_pair(const void *p, int64_t elem) {
  Pair<DT> v;
  if constexpr (DT == BL_F32) {
    const uint2 q = *reinterpret_cast<const uint2 *>(static_cast<const float *>(p) + elem);
    v.w[0] = q.x;
    v.w[1] = q.y;
  } else {
    v.w[0] = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(p) + elem);
  }
  return v;
}

template <int DT>
__device__ __forceinline__ void widen_pair(const Pair<DT> &v, float f[2]) {
  if constexpr (DT == BL_F32) {
    f[0] = __uint_as_float(v.w[0]);
    f[1] = __uint_as_float(v.w[1]);
  } else if constexpr (DT == BL_BF16) {
    f[0] = __uint_as_float(v.w[0] << 16);
    f[1] = __uint_as_float(v.w[0] & 0xFFFF0000u);
  } else {
    f[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.w[0] & 0xFFFFu));
    f[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.w[0] >> 16));
  }
}

template <int DT>
__device__ __forceinline__ void store_pair(void *p, int64_t elem, const float v[2]) {
  if constexpr (DT == BL_F32) {
    *reinterpret_cast<uint2 *>(static_cast<float *>(p) + elem) =
        make_uint2(__float_as_uint(v[0]), __float_as_uint(v[1]));
  } else {
    *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(p) + elem) =
        (uint32_t)out_bits<DT>(v[0]) | ((uint32_t)out_bits<DT>(v[1]) << 16);
  }
}

// Tokens [t0, t1) of one chunk (t1 - t0 <= L) for kCpt channels of
// one sequence, in batches of U tokens whose 2 U loads (i and f) go out
// together, the next batch's before the current one is computed (the loads
// do not depend on the state).  The batch loop is unrolled over the whole
// chunk with two buffers and no branch around the loads (rows past t1 load
// row t1 - 1 again and are not computed): left to itself the compiler
// waits for each token's pair before requesting the next.  step(t, a, iv)
// receives each token in order.
template <int DT>
struct ScanBatch {
  static constexpr int U = 16;  // tokens per batch
  Pair<DT> i[U], f[U];
};

template <int DT>
__device__ __forceinline__ void scan_load(ScanBatch<DT> &bt, const void *i, const void *f,
                                          int64_t row0, int64_t D, int t, int t1) {
#pragma unroll
  for (int u = 0; u < ScanBatch<DT>::U; ++u) {
    const int64_t r = row0 + (int64_t)min(t + u, t1 - 1) * D;
    bt.i[u] = load_pair<DT>(i, r);
    bt.f[u] = load_pair<DT>(f, r);
  }
}

template <int DT, int L, class Step>
__device__ __forceinline__ void scan_tokens(const void *i, const void *f, int64_t row0, int64_t D,
                                            int t0, int t1, Step step) {
  constexpr int U = ScanBatch<DT>::U;
  static_assert(L % U == 0, "whole batches");
  constexpr int NB = L / U;
  ScanBatch<DT> buf[2];
  scan_load<DT>(buf[0], i, f, row0, D, t0, t1);
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int t = t0 + k * U;
    if (k + 1 < NB) scan_load<DT>(buf[(k + 1) & 1], i, f, row0, D, t + U, t1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t + u < t1) {
        float iv[kCpt], fv[kCpt], a[kCpt];
        widen_pair<DT>(buf[k & 1].i[u], iv);
        widen_pair<DT>(buf[k & 1].f[u], fv);
#pragma unroll
        for (int e = 0; e < kCpt; ++e) a[e] = gate_of(fv[e]);
        step(t + u, a, iv);
      }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// 1. P and S of chunk blockIdx.y (L steps) of sequence blockIdx.z.
template <int DT, int L>
__global__ __launch_bounds__(kScanThreads) void mlgru_chunk_kernel(const void *__restrict__ i,
                                                                   const void *__restrict__ f,
                                                                   int T, int D, int C,
                                                                   float *__restrict__ P,
                                                                   float *__restrict__ S) {
  const int d0 = kCpt * ((int)blockIdx.x * kScanThreads + (int)threadIdx.x);
  if (d0 >= D) return;
  const int b = (int)blockIdx.z, c = (int)blockIdx.y;
  const int t0 = c * L, t1 = min(T, t0 + L);
  float p[kCpt], s[kCpt];
#pragma unroll
  for (int e = 0; e < kCpt; ++e) {
    p[e] = 1.0f;
    s[e] = 0.0f;
  }
  scan_tokens<DT, L>(i, f, (int64_t)b * T * D + d0, D, t0, t1,
                  [&](int, const float *a, const float *iv) {
#pragma unroll
                    for (int e = 0; e < kCpt; ++e) {
                      s[e] = a[e] * s[e] + (1.0f - a[e]) * iv[e];
                      p[e] = p[e] * a[e];
                    }
                  });
  const int64_t o = ((int64_t)b * C + c) * D + d0;
  *reinterpret_cast<float2 *>(P + o) = make_float2(p[0], p[1]);
  *reinterpret_cast<float2 *>(S + o) = make_float2(s[0], s[1]);
}

// 2. (at most kCarryPerGroup chunks) The chunk start states of sequence b,
// channel d, written over S: one thread per pair walks the chunks in order,
// their P and S loaded together first.
constexpr int kCarryPerGroup = 32;   // chunks a thread loads at once
__global__ __launch_bounds__(kScanThreads) void mlgru_carry_short_kernel(
    const float *__restrict__ h0, int B, int D, int C, const float *__restrict__ P,
    float *__restrict__ S) {
  const int64_t bd = (int64_t)blockIdx.x * kScanThreads + threadIdx.x;
  if (bd >= (int64_t)B * D) return;
  const int64_t b = bd / D, d = bd - b * D;
  const float *Pb = P + b * C * D + d;
  float *Sb = S + b * C * D + d;
  float H = h0 ? h0[bd] : 0.0f;
  float p[kCarryPerGroup], s[kCarryPerGroup];
#pragma unroll
  for (int j = 0; j < kCarryPerGroup; ++j) {
    const int c = min(j, C - 1);   // past the end: a repeat, never used
    p[j] = Pb[(int64_t)c * D];
    s[j] = Sb[(int64_t)c * D];
  }
#pragma unroll
  for (int j = 0; j < kCarryPerGroup; ++j)
    if (j < C) {
      Sb[(int64_t)j * D] = H;
      H = p[j] * H + s[j];
    }
}

// 2. (more chunks) The chunk start states, written over S.  A workgroup takes 32
// channels (of the B D sequence-channel pairs) and their chunks in windows
// of kCarryGroups x 32: group g of its threads composes chunks
// 32 g .. 32 g + 31 of the window into one map (their P and S loaded
// together, one memory latency), the window's group maps are chained in
// LDS by the first group (8 steps, carrying each channel's state from the
// window before), and every group then walks its chunks from its start
// state, storing each chunk's.  The carry pays a few memory latencies per
// 256 chunks instead of one per chunk.
constexpr int kCarryGroups = kScanThreads / 32;   // 8
__global__ __launch_bounds__(kScanThreads) void mlgru_carry_kernel(const float *__restrict__ h0,
                                                                   int B, int D, int C,
                                                                   const float *__restrict__ P,
                                                                   float *__restrict__ S) {
  __shared__ float s_p[kCarryGroups][32], s_s[kCarryGroups][32];
  const int g = (int)threadIdx.x >> 5, dl = (int)threadIdx.x & 31;
  const int64_t bd = (int64_t)blockIdx.x * 32 + dl;
  const bool live = bd < (int64_t)B * D;
  const int64_t b = live ? bd / D : 0, d = live ? bd - b * D : 0;
  const float *Pb = P + b * C * D + d;
  float *Sb = S + b * C * D + d;
  float H = (live && h0) ? h0[bd] : 0.0f;   // the running state (group 0's threads)
  for (int w0 = 0; w0 < C; w0 += kCarryGroups * kCarryPerGroup) {
    const int c0 = w0 + g * kCarryPerGroup;
    float p[kCarryPerGroup], s[kCarryPerGroup];
#pragma unroll
    for (int j = 0; j < kCarryPerGroup; ++j) {
      const int c = min(c0 + j, C - 1);   // past the end: a repeat, never used
      p[j] = live ? Pb[(int64_t)c * D] : 1.0f;
      s[j] = live ? Sb[(int64_t)c * D] : 0.0f;
    }
    // this group's map over its chunks: H -> pg H + sg
    float pg = 1.0f, sg = 0.0f;
#pragma unroll
    for (int j = 0; j < kCarryPerGroup; ++j)
      if (c0 + j < C) {
        sg = p[j] * sg + s[j];
        pg = p[j] * pg;
      }
    s_p[g][dl] = pg;
    s_s[g][dl] = sg;
    __syncthreads();
    if (g == 0) {
#pragma unroll
      for (int k = 0; k < kCarryGroups; ++k) {
        const float pk = s_p[k][dl], sk = s_s[k][dl];
        s_s[k][dl] = H;   // group k's start state
        H = pk * H + sk;
      }
    }
    __syncthreads();
    float Hg = s_s[g][dl];
#pragma unroll
    for (int j = 0; j < kCarryPerGroup; ++j)
      if (live && c0 + j < C) {
        Sb[(int64_t)(c0 + j) * D] = Hg;
        Hg = p[j] * Hg + s[j];
      }
    __syncthreads();   // s_s is rewritten by the next window
  }
}

// 3. The chunk run from its start state (Hs[(b C + c) D + d], or h0 / zero
// when Hs is null -- one chunk per sequence), storing h and, in the last
// chunk, hT.
template <int DT, int L>
__global__ __launch_bounds__(kScanThreads) void mlgru_apply_kernel(
    const void *__restrict__ i, const void *__restrict__ f, int T, int D, int C,
    const float *__restrict__ Hs, const float *__restrict__ h0, void *__restrict__ h,
    float *__restrict__ hT) {
  const int d0 = kCpt * ((int)blockIdx.x * kScanThreads + (int)threadIdx.x);
  if (d0 >= D) return;
  const int b = (int)blockIdx.z, c = (int)blockIdx.y;
  const int t0 = c * L, t1 = min(T, t0 + L);
  const float *start = Hs ? Hs + ((int64_t)b * C + c) * D + d0 : h0 ? h0 + (int64_t)b * D + d0 : nullptr;
  float s[kCpt];
#pragma unroll
  for (int e = 0; e < kCpt; ++e) s[e] = start ? start[e] : 0.0f;
  const int64_t row0 = (int64_t)b * T * D + d0;
  scan_tokens<DT, L>(i, f, row0, D, t0, t1, [&](int t, const float *a, const float *iv) {
#pragma unroll
    for (int e = 0; e < kCpt; ++e) s[e] = a[e] * s[e] + (1.0f - a[e]) * iv[e];
    store_pair<DT>(h, row0 + (int64_t)t * D, s);
  });
  if (hT && c == C - 1) {
#pragma unroll
    for (int e = 0; e < kCpt; ++e) hT[(int64_t)b * D + d0 + e] = s[e];
  }
}

template <int DT, int L>
hipError_t launch_l(const MlgruArgs &a, hipStream_t stream) {
  const int T = (int)a.T, D = (int)a.D, B = (int)a.B;
  const int C = (T + L - 1) / L;
  const dim3 grid((unsigned)((D / kCpt + kScanThreads - 1) / kScanThreads), (unsigned)C, (unsigned)B);
  if (C == 1) {
    mlgru_apply_kernel<DT, L><<<grid, kScanThreads, 0, stream>>>(a.i, a.f, T, D, 1, nullptr, a.h0,
                                                                 a.h, a.hT);
    return hipGetLastError();
  }
  float *P = static_cast<float *>(a.ws);
  float *S = P + (int64_t)B * C * D;
  mlgru_chunk_kernel<DT, L><<<grid, kScanThreads, 0, stream>>>(a.i, a.f, T, D, C, P, S);
  if (C <= kCarryPerGroup) {
    const unsigned cgrid = (unsigned)(((int64_t)B * D + kScanThreads - 1) / kScanThreads);
    mlgru_carry_short_kernel<<<cgrid, kScanThreads, 0, stream>>>(a.h0, B, D, C, P, S);
  } else {
    const unsigned cgrid = (unsigned)(((int64_t)B * D + 31) / 32);
    mlgru_carry_kernel<<<cgrid, kScanThreads, 0, stream>>>(a.h0, B, D, C, P, S);
  }
  mlgru_apply_kernel<DT, L><<<grid, kScanThreads, 0, stream>>>(a.i, a.f, T, D, C, S, a.h0, a.h,
                                                               a.hT);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_t(const MlgruArgs &a, hipStream_t stream) {
  return mlgru_chunk_len(a.T) == 16 ? launch_l<DT, 16>(a, stream) : launch_l<DT, 32>(a, stream);
}

}  // namespace

size_t mlgru_workspace_bytes(int64_t B, int64_t T, int64_t D) {
  const int64_t L = mlgru_chunk_len(T);
  const int64_t C = (T + L - 1) / L;
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
