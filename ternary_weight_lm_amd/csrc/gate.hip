// gate.hip -- FusedRMSNormSwishGate in front of o_proj, alone and as the
// prologue of o_proj's act-quant launch.
//
// HGRNBit hands the token mixer's output to o_proj through a gate layer,
// FusedRMSNormSwishGate, a layer of its own that fuses an RMSNorm with the
// gate (hysenlabs ja review "matmulfreellm 評価: 行列積を消した HGRNBit を
// Transformers 互換で読む", sections "HGRNBit という層構成を読む" and
// "代替手段との違い").  The pages give only the name; this library reads it
// as the RMSNorm of the mixer output o (gain w, epsilon eps_gate) times the
// Swish of the gate input g, Swish with unit slope being the SiLU of the GLU
// (datacamp "MatMul-freie LLMs: Zentrale Konzepte erklärt", section
// "Kernkomponenten: MLGRU und GLU"):
//   z = ((o * r) * w) * silu(g),  r = 1 / sqrt(fp32(sum o^2 / K) + eps_gate)
// with the sum of squares in fp64 in the library's fixed association and the
// rest in fp32 (silu from the hardware exp2 and reciprocal), z rounded to
// the activation dtype -- the value a gate layer hands on.
//
// One wave per token row (K <= 4096: the row cached in registers, lane L
// holding elements 8 L + 512 c .. +7).  gate_kernel stores z;
// act_quant_gated_kernel keeps z in registers and quantizes it for o_proj
// with the act-quant passes of rowquant.h, so its codes, scales and row sums
// are those of the act-quant kernel run on the stored z, bit for bit.
#include "bl_launch.h"
#include "rowquant.h"

namespace bl {

namespace {

constexpr int kGateWaves = 4;  // rows (waves) per workgroup

template <int DT, int NC>
__device__ __forceinline__ void load_rows(const void *o, const void *g, const void *w, int m,
                                          int K, Chunk8<DT> (&oc)[NC], Chunk8<DT> (&gc)[NC],
                                          Chunk8<DT> (&wc)[NC]) {
  constexpr int EB = dtype_bytes(DT);
  const int lane = threadIdx.x & 63;
  const rsrc_t ors = make_rsrc(static_cast<const char *>(o) + (int64_t)m * K * EB, (uint32_t)(K * EB));
  const rsrc_t grs = make_rsrc(static_cast<const char *>(g) + (int64_t)m * K * EB, (uint32_t)(K * EB));
  const rsrc_t wrs = make_rsrc(w, (uint32_t)(K * EB));
#pragma unroll
  for (int c = 0; c < NC; ++c) oc[c] = bload_chunk<DT>(ors, (uint32_t)((8 * lane + 512 * c) * EB));
#pragma unroll
  for (int c = 0; c < NC; ++c) gc[c] = bload_chunk<DT>(grs, (uint32_t)((8 * lane + 512 * c) * EB));
#pragma unroll
  for (int c = 0; c < NC; ++c) wc[c] = bload_chunk<DT>(wrs, (uint32_t)((8 * lane + 512 * c) * EB));
}

template <int DT, int NC>
__global__ __launch_bounds__(64 * kGateWaves) void gate_kernel(const void *o, const void *g,
                                                                const void *w, int M, int K,
                                                                float eps, void *z) {
  const int m = (int)blockIdx.x * kGateWaves + (int)(threadIdx.x >> 6);
  if (m >= M) return;
  const int lane = threadIdx.x & 63;
  Chunk8<DT> oc[NC], gc[NC], wc[NC], zc[NC];
  load_rows<DT, NC>(o, g, w, m, K, oc, gc, wc);
  gate_row<DT, NC>(oc, gc, wc, K, eps, zc);
  constexpr int EB = dtype_bytes(DT);
  char *zr = static_cast<char *>(z) + (int64_t)m * K * EB;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int k = 8 * lane + 512 * c;
    if (k < K) {
      *reinterpret_cast<v4i *>(zr + (int64_t)k * EB) = zc[c].u[0];
      if constexpr (DT == BL_F32) *reinterpret_cast<v4i *>(zr + (int64_t)k * EB + 16) = zc[c].u[1];
    }
  }
}

template <int DT, int NC>
__global__ __launch_bounds__(64 * kGateWaves) void act_quant_gated_kernel(
    const void *o, const void *g, const void *w, float gate_eps, const void *gain, int M, int K,
    float eps, int8_t *xq, float *s, int32_t *rowsum) {
  const int m = (int)blockIdx.x * kGateWaves + (int)(threadIdx.x >> 6);
  if (m >= M) return;
  const int lane = threadIdx.x & 63;
  constexpr int EB = dtype_bytes(DT);
  Chunk8<DT> oc[NC], gc[NC], wc[NC], zc[NC], gn[NC];
  load_rows<DT, NC>(o, g, w, m, K, oc, gc, wc);
  {
    const rsrc_t nrs = make_rsrc(gain, (uint32_t)(K * EB));
#pragma unroll
    for (int c = 0; c < NC; ++c) gn[c] = bload_chunk<DT>(nrs, (uint32_t)((8 * lane + 512 * c) * EB));
  }
  gate_row<DT, NC>(oc, gc, wc, K, gate_eps, zc);
  int8_t *dst = xq + (int64_t)m * K;
  float sc;
  int rs;
  quantize_loaded<DT, NC>(zc, gn, K, eps,
                          [&](int k, uint2 codes) { *reinterpret_cast<uint2 *>(dst + k) = codes; },
                          sc, rs);
  if (lane == 0) {
    s[m] = sc;
    rowsum[m] = rs;
  }
}

template <int DT, int NC>
hipError_t launch_gate_t(const GateArgs &a, hipStream_t stream) {
  const unsigned grid = (unsigned)((a.M + kGateWaves - 1) / kGateWaves);
  if (a.xq)
    act_quant_gated_kernel<DT, NC><<<grid, 64 * kGateWaves, 0, stream>>>(
        a.o, a.g, a.w, a.gate_eps, a.gain, (int)a.M, (int)a.K, a.eps, a.xq, a.s, a.rowsum);
  else
    gate_kernel<DT, NC><<<grid, 64 * kGateWaves, 0, stream>>>(a.o, a.g, a.w, (int)a.M, (int)a.K,
                                                             a.gate_eps, a.z);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_gate_dt(const GateArgs &a, hipStream_t stream) {
  switch (row_cache((int)a.K)) {
    case 2: return launch_gate_t<DT, 2>(a, stream);
    case 4: return launch_gate_t<DT, 4>(a, stream);
    case 6: return launch_gate_t<DT, 6>(a, stream);
    default: return launch_gate_t<DT, 8>(a, stream);
  }
}

}  // namespace

hipError_t launch_gate(const GateArgs &a, hipStream_t stream) {
  switch (a.dtype) {
    case BL_F32: return launch_gate_dt<BL_F32>(a, stream);
    case BL_F16: return launch_gate_dt<BL_F16>(a, stream);
    default: return launch_gate_dt<BL_BF16>(a, stream);
  }
}

}  // namespace bl
