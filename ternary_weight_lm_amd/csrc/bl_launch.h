// bl_launch.h -- host-side launchers of the gfx950 kernels.  Each returns
// the hipError_t of its launches; argument checking is done once, in the C
// ABI layer (capi.cpp), before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "bitlinear.h"

namespace bl {

// Output kinds of the contraction kernels: a BL_* dtype code, or kOutI32 for
// the exact int32 accumulator (stage-level entry point).
constexpr int kOutI32 = 3;

// Workspace bytes of the weight packer (partial sums of |W|).
size_t pack_workspace_bytes();

// glu_F > 0: W is a gate_proj [2F, K] (F = glu_F) packed in the GLU row
// order (see pack.hip); 0: plain row order.
hipError_t launch_pack(const float *W, int64_t N, int64_t K, void *packed,
                       float *beta, void *ws, int64_t glu_F, hipStream_t stream);

hipError_t launch_unpack(const void *packed, int64_t N, int64_t K, int8_t *Wq,
                         hipStream_t stream);

hipError_t launch_act_quant(const void *x, int x_dtype, const void *gain,
                            int64_t M, int64_t K, float eps, int8_t *xq,
                            float *s, int32_t *rowsum, hipStream_t stream);

// Up to kGroupCalls same-shape projections per launch on the two-kernel
// path (HGRN's i/f/g at prefill): one act-quant launch and one MFMA launch
// for all of them.  Pointers travel in the argument buffer.
constexpr int kGroupCalls = 3;
struct AqCall {
  const void *x;
  const void *gain;
  int8_t *xq;
  float *s;
  int32_t *rowsum;
};
struct AqCalls {
  AqCall c[kGroupCalls];
};
hipError_t launch_act_quant_group(const AqCalls &calls, int ncalls, int x_dtype, int64_t M,
                                  int64_t K, float eps, hipStream_t stream);

// Tiled MFMA contraction of pre-quantized activations (any M).
// out_kind = BL_* writes y = (acc) * beta / s; kOutI32 writes acc.
// glu: the N = 2F packed rows are a gate_proj in GLU order and out is
// h [M, F] = silu(y_gate) * y_up (out_kind a float dtype).
hipError_t launch_gemm_mfma(const int8_t *xq, const int32_t *rowsum,
                            const float *s, const void *packed,
                            const float *beta, int64_t M, int64_t N,
                            int64_t K, void *out, int out_kind, bool glu,
                            hipStream_t stream);

struct GemmCall {
  const int8_t *xq;
  const int32_t *rowsum;
  const float *s;
  const void *packed;
  const float *beta;
  void *out;
};
struct GemmCalls {
  GemmCall c[kGroupCalls];
};
// ncalls <= kGroupCalls contractions of one shape, out_kind a float dtype.
hipError_t launch_gemm_mfma_group(const GemmCalls &calls, int ncalls, int64_t M, int64_t N,
                                  int64_t K, int out_kind, hipStream_t stream);

// Skinny contraction for M <= kSkinnyMaxM (fused: M <= kFusedMaxM): one
// workgroup per 32 output rows.
// fused = true: x / gain / eps are read and normalized + quantized inside;
// fused = false: xq / s / rowsum come from a previous act-quant launch.
struct SkinnyArgs {
  bool fused;
  const void *x;
  int x_dtype;
  const void *gain;
  float eps;
  const int8_t *xq;
  const float *s;
  const int32_t *rowsum;
  const void *packed;
  const float *beta;
  int64_t M, N, K;
  void *out;
  int out_kind;
  bool glu;  // GLU epilogue (pre-quantized calls, or fused calls the decode kernel takes)
};
hipError_t launch_skinny(const SkinnyArgs &a, hipStream_t stream);

// Up to kGroupCalls pre-quantized, non-GLU calls of one shape (M <= 64) in
// one launch of the skinny kernel; each output as launch_skinny computes it.
hipError_t launch_skinny_pre_grouped(const SkinnyArgs *calls, int ncalls, hipStream_t stream);

// Up to kGroupMax fused skinny calls per launch (more are split into several
// launches).  Every call must be fused-eligible and share x / out dtypes.
constexpr int kGroupMax = 16;
hipError_t launch_skinny_grouped(const SkinnyArgs *calls, int ncalls, hipStream_t stream);

// Fused decode kernel (M <= kDecodeMaxM, K <= kFusedMaxK): up to
// kDecodeCalls projections of one shape (same M, K, N) per launch.
// launch_skinny and launch_skinny_grouped route fused calls here when they
// fit.
constexpr int kDecodeCalls = 3;
constexpr int64_t kDecodeMaxM = 4;
struct DecodeArgs {
  const void *x[kDecodeCalls];
  int x_dtype;
  int64_t M, N, K;
  float eps;
  int ncalls;
  const void *gain[kDecodeCalls];
  const void *packed[kDecodeCalls];
  const float *beta[kDecodeCalls];
  void *out[kDecodeCalls];
  int out_kind;
  bool glu;  // one call only: out = h [M, N/2] = silu(y_gate) * y_up
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
// Contraction unit of the decode kernels at 1 token (split mode) and 2
// tokens (row mode): BL_DECODE_MFMA or BL_DECODE_VALU, from the process-wide
// setting of bitlinear_set_decode_contraction (capi.cpp).
bool decode_use_valu();
// the kernels for one activation dtype (decode_f32.hip, decode_f16.hip,
// decode_bf16.hip); launch_decode picks one
void launch_decode_f32(const DecodeArgs &a, hipStream_t stream);
void launch_decode_f16(const DecodeArgs &a, hipStream_t stream);
void launch_decode_bf16(const DecodeArgs &a, hipStream_t stream);
// Row mode of the decode kernel (8 waves, one token row per wave up to 8
// rows, two up to 16): 2 <= M <= 16, K <= 4096, the codes M (K + 16) bytes
// within the LDS budget; fp32 activations with more than 8 rows K <= 2048.
constexpr int64_t kDecodeRowsMaxM = 16;
constexpr int64_t kDecodeRowsLds = 45056;  // M * (K + 16) bytes of int8 codes in LDS
inline bool decode_rows_fits(int64_t M, int64_t K, int x_dtype) {
  if (M < 2 || K > 4096 || M > kDecodeRowsMaxM || M * (K + 16) > kDecodeRowsLds) return false;
  // fp32 rows hold twice the registers: two rows per wave only up to K = 2048
  return x_dtype != BL_F32 || M <= 8 || K <= 2048;
}
// Split mode (every wave takes a share of each row; up to three calls per
// launch): M <= 4 (fp32 x: M == 1), K <= 8192.
inline bool decode_split_fits(int64_t M, int64_t K, int x_dtype) {
  return M >= 1 && K <= 8192 && (M == 1 || (M <= kDecodeMaxM && x_dtype != BL_F32));
}
// Whether the decode kernel takes a single fused call of this shape/dtype.
inline bool decode_fits(int64_t M, int64_t K, int x_dtype) {
  return decode_split_fits(M, K, x_dtype) || decode_rows_fits(M, K, x_dtype);
}

// Chained decode (chain.hip): dependent calls of 1..4 token rows, 16-bit
// activations, in one persistent launch.  The C ABI layer validates the
// calls and works out which earlier call (if any) each call reads.
struct ChainPlanIn {
  const bl_chain_call *calls;
  int ncalls;
  int64_t M;
  int dtype;
  float eps;
  std::vector<int> dep;        // call whose y is this call's x, or -1
  std::vector<char> consumed;  // a later call reads this call's y
  std::vector<int64_t> n_out;  // output columns (N, or N / 2 for GLU)
};
constexpr int64_t kChainMaxM = 4;
constexpr int kChainMaxCalls = 4096;
size_t chain_workspace_bytes(const ChainPlanIn &in);
hipError_t chain_plan(const ChainPlanIn &in, void *ws, bl_chain &out, hipStream_t stream);
hipError_t chain_run(const bl_chain &p, uint32_t wait_us, hipStream_t stream);
// synchronizes the stream, returns the chain's error word and clears it
hipError_t chain_error(const bl_chain &p, uint32_t *err, hipStream_t stream);

// FusedRMSNormSwishGate (gate.hip), one wave per row, K <= kGateMaxK:
// z = ((o r) w) silu(g) rounded to dtype.  xq == nullptr: store z [M, K];
// else quantize z for the following projection (gain, eps) into xq / s /
// rowsum, as the act-quant kernel would from the stored z.
struct GateArgs {
  const void *o, *g, *w;
  float gate_eps;
  int dtype;
  int64_t M, K;
  void *z;
  const void *gain;
  float eps;
  int8_t *xq;
  float *s;
  int32_t *rowsum;
};
constexpr int64_t kGateMaxK = 4096;
hipError_t launch_gate(const GateArgs &a, hipStream_t stream);

// MLGRU recurrence over [B, T, D] (mlgru.hip): h_t = a h_{t-1} + (1 - a) i_t,
// a = sigmoid(f_t), chunks of mlgru_chunk_len(T) steps; ws holds 2 B C D
// floats (C = ceil(T / chunk length)) when C > 1.
struct MlgruArgs {
  const void *i, *f;
  int dtype;
  int64_t B, T, D;
  const float *h0;  // [B, D] or null (zero start)
  void *h;          // [B, T, D], dtype
  float *hT;        // [B, D] or null
  void *ws;
};
// chunk length: 16 steps for 33..1023 steps (more chunks in flight: 512
// steps 12.5 -> 10.4 us per scan at the 2.7B width), else 32 (8192 steps:
// 45.2 us at 64, 44.8 at 32, 46.1 at 16); a sequence of up to 32 steps is one
// chunk
constexpr int64_t mlgru_chunk_len(int64_t T) { return T > 32 && T < 1024 ? 16 : 32; }
constexpr int64_t kMlgruMaxB = 65535;      // launch grid z
constexpr int64_t kMlgruMaxT = 1 << 20;    // chunks per sequence (grid y) <= 32768
constexpr int64_t kMlgruMaxD = 1 << 16;
size_t mlgru_workspace_bytes(int64_t B, int64_t T, int64_t D);
hipError_t launch_mlgru_scan(const MlgruArgs &a, hipStream_t stream);

// o_proj behind FusedRMSNormSwishGate in one launch of the decode kernel's
// row mode: 1..8 rows of 16-bit activations, K <= 4096, the codes within the
// row mode's LDS budget.
struct DecodeGateArgs {
  const void *o, *g, *gate_w;
  float gate_eps;
  int x_dtype;
  int64_t M, N, K;
  const void *gain;
  float eps;
  const void *packed;
  const float *beta;
  void *out;
  int out_kind;
};
inline bool decode_gated_fits(int64_t M, int64_t K, int x_dtype) {
  return x_dtype != BL_F32 && M >= 1 && M <= 8 && K <= kGateMaxK && M * (K + 16) <= kDecodeRowsLds;
}
hipError_t launch_decode_gated(const DecodeGateArgs &a, hipStream_t stream);
void launch_decode_gated_f16(const DecodeGateArgs &a, hipStream_t stream);
void launch_decode_gated_bf16(const DecodeGateArgs &a, hipStream_t stream);

// Largest M and K the fused skinny kernel accepts.
constexpr int64_t kFusedMaxM = 16;
constexpr int64_t kFusedMaxK = 8192;
constexpr int64_t kSkinnyMaxM = 64;  // pre-quantized skinny calls

}  // namespace bl
