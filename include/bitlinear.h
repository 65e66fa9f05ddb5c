/*
 * bitlinear.h -- C ABI of the MI355X (gfx950) FusedBitLinear library.
 *
 * One FusedBitLinear projection (in_features K -> out_features N, no bias)
 * computes, for every token row x[m, :]:
 *
 *   RMSNorm   r_m  = 1 / sqrt(mean_k x[m,k]^2 + eps),  xn = (x * r_m) * g
 *   act-quant s_m  = 127 / max(max_k |xn[m,k]|, 1e-5),
 *             xq   = clamp(round_half_even(xn * s_m), -128, 127)      (int8)
 *   weights   beta = max(mean |W|, 1e-5) over the whole matrix,
 *             Wq   = clamp(round_half_even(W / beta), -1, +1)         (ternary)
 *   contract  acc[m,n] = sum_k xq[m,k] * Wq[n,k]                      (int32)
 *   rescale   y[m,n]   = acc[m,n] / s_m * beta
 *
 * Where each step comes from (page titles and sections):
 *   - FusedBitLinear(in, out, bias=False) carrying its own RMSNorm with
 *     eps = 1e-08, the norm fused with the ternary projection and applied
 *     right before quantization: hysenlabs ja review "matmulfreellm 評価 ...",
 *     section "HGRNBit という層構成を読む"; hysenlabs fr review "MatMul-Free
 *     LM : un modèle de langage sans multiplication matricielle ...", section
 *     "HGRNBit : ce que la structure du modèle révèle"; hysenlabs de review
 *     "MatMul-Free LM: Ternary-Gewichte statt Matrixmultiplikation im
 *     Transformer", section "HGRNBit: was in einem Block tatsächlich passiert".
 *   - absmean ternary weights, and products by -1/0/+1 reduced to negate /
 *     zero / keep: datacamp "MatMul-freie LLMs: Zentrale Konzepte erklärt",
 *     section "MatMul durch ternäre Operationen ersetzen".
 *   - RMSNorm before quantization and the scaled ternary accumulation:
 *     same datacamp page, section "Kernkomponenten: MLGRU und GLU", figure
 *     panels 5 and 4.
 *   - y = W x orientation of a linear layer (W stored [out, in]): aidev
 *     bluegarage "量子化とは何か？MatMulというAIの計算やモデルサイズの最大の
 *     ネック", section "ニューラルネットにおける実態".
 *   The activation format (8-bit, one absmax scale per token), round half to
 *   even, the 1e-5 floors and eps inside the square root are the readings
 *   this library fixes where the pages are silent.
 *
 * Precision.  The sums of x^2 and |W| are accumulated in fp64; every other
 * step before an integer is decided runs in IEEE fp32 with correctly rounded
 * division and square root; the contraction is exact int32; the rescale is
 * fp32 (acc * (beta / s_m)), rounded to nearest-even into the output dtype.
 *
 * ---------------------------------------------------------------- layout
 * Packed ternary weights (bitlinear_pack_weights output) use N*K/4 bytes:
 *   - 2-bit code per weight: code = Wq + 1 (0 = -1, 1 = 0, 2 = +1; 3 unused).
 *   - The [N, K] matrix is cut into tiles of 32 rows x 128 columns (K index),
 *     1024 bytes each, stored row-tile-major: tile (nt, kb) starts at byte
 *     1024 * (nt * (K/128) + kb).
 *   - In a tile, row n = 32*nt + 16*h + c (h in {0,1}, c in 0..15) and the
 *     16-column group j (k = 128*kb + 16*j + e, j in 0..7, e in 0..15) form
 *     one little-endian 32-bit word at tile byte offset
 *     16 * (16 * (j / 2) + c) + 4 * (2 * h + j % 2).
 *   - In that word the code of element e sits at bits 8*(e%4) + 2*(e/4)
 *     (and the next bit), so (word >> 2q) & 0x03030303 yields the codes of
 *     elements 4q .. 4q+3 as four bytes.
 * With this layout one 16-byte load by lane L of a 64-lane wave returns
 * exactly the four B operands (rows 16h + L%16, k-groups 2*(L/16) + s) that
 * lane feeds to four v_mfma_i32_16x16x64_i8 instructions, and a wave reads a
 * tile as one contiguous 1 KiB.
 * beta is a separate fp32 in device memory.
 *
 * ------------------------------------------------------------ conventions
 * - All pointers to data are DEVICE pointers, caller-allocated and owned; the
 *   library allocates nothing and keeps no per-call state.  Every data
 *   pointer must be 16-byte aligned.
 * - Matrices are dense row-major: x [M, K], gain [K], W [N, K], y [M, N].
 * - Shapes: K % 128 == 0, N % 32 == 0, 128 <= K <= 65536, 32 <= N <= 2^20,
 *   0 <= M <= 2^24.  M == 0 is a no-op that returns BL_OK.
 * - dtypes: BL_F32, BL_F16, BL_BF16 for x / gain (same dtype) and for y.
 * - Calls are asynchronous on `stream` (0 = the null stream); errors from a
 *   kernel surface at the caller's next synchronization.  Every argument is
 *   validated on the host before anything is launched; a rejected call
 *   launches nothing and touches no memory.
 * - Calls that share a workspace must be ordered (same stream).
 * - Inputs must be finite; NaN / Inf give unspecified codes.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype codes */
enum { BL_F32 = 0, BL_F16 = 1, BL_BF16 = 2 };

/* status codes (0 = success) */
enum {
    BL_OK = 0,
    BL_ERR_NULL = -1,        /* a required pointer is NULL                  */
    BL_ERR_DTYPE = -2,       /* unknown dtype code                          */
    BL_ERR_SHAPE = -3,       /* M, N or K outside the supported set         */
    BL_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned            */
    BL_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required  */
    BL_ERR_EPS = -6,         /* eps not finite or not > 0                   */
    BL_ERR_HIP = -7,         /* a HIP launch or query failed                */
    BL_ERR_UNSUPPORTED = -8, /* valid request the library does not implement */
    BL_ERR_PATH = -9,        /* unknown execution path code                 */
    BL_ERR_SCRATCH = -10,    /* beyond bitlinear_forward_noalloc's scratch  */
    BL_ERR_TIMEOUT = -11     /* a chained launch's bounded wait gave up     */
};

/* execution paths for bitlinear_forward_path / bitlinear_gemm_i32 */
enum {
    BL_PATH_AUTO = 0,    /* choose by M (what bitlinear_forward does)        */
    BL_PATH_FUSED = 1,   /* one kernel: norm + quant + skinny contraction    */
    BL_PATH_SKINNY = 2,  /* act-quant kernel, then skinny contraction (M<=64)*/
    BL_PATH_MFMA = 3     /* act-quant kernel, then tiled MFMA contraction    */
};

/* Bytes of packed weights for an [N, K] matrix: N*K/4 (0 for a bad shape). */
size_t bitlinear_packed_bytes(int64_t N, int64_t K);

/* Workspace bytes bitlinear_pack_weights needs (0 for a bad shape). */
size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K);

/* Offline weight packing (absmean ternarization + 2-bit tile layout): the
 * matrix is divided by its mean absolute value and each entry rounded to
 * the nearest of -1, 0, +1 (datacamp page, section "MatMul durch ternäre
 * Operationen ersetzen"); fewer bits per weight mean less memory and
 * bandwidth (aidev bluegarage page, section "量子化とは何か"), hence the
 * 2-bit codes.
 *   W       device fp32 [N, K] latent weights (read only)
 *   packed  device, bitlinear_packed_bytes(N, K) bytes (written)
 *   beta    device fp32 scalar: the per-tensor scale (written)
 *   ws      device scratch of >= bitlinear_pack_workspace_bytes(N, K)
 * beta stays on the device; no host synchronization is needed before a
 * forward call on the same stream. */
int bitlinear_pack_weights(const float *W, int64_t N, int64_t K, void *packed,
                           float *beta, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/* Workspace bytes bitlinear_forward needs for (M, K, N), covering every
 * path (0 for a bad shape). */
size_t bitlinear_workspace_bytes(int64_t M, int64_t K, int64_t N);

/* One FusedBitLinear forward: y = rescale(contract(quant(rmsnorm(x)), Wq)).
 * The layer as the pages state it: FusedBitLinear(in_features, out_features,
 * bias=False) holding its own RMSNorm(eps=1e-08) (hysenlabs fr review,
 * section "HGRNBit : ce que la structure du modèle révèle"; hysenlabs ja
 * review, section "HGRNBit という層構成を読む"), the norm fused with the
 * ternary projection right before quantization (hysenlabs de review,
 * section "HGRNBit: was in einem Block tatsächlich passiert"), the scaled
 * ternary accumulation of datacamp "Kernkomponenten: MLGRU und GLU"
 * (figure panels 4 and 5).
 *   x       device [M, K], dtype x_dtype (read only)
 *   gain    device [K], dtype x_dtype: the RMSNorm weight (read only)
 *   packed  device packed weights of an [N, K] matrix (read only)
 *   beta    device fp32 scalar written by bitlinear_pack_weights
 *   y       device [M, N], dtype y_dtype (written)
 *   eps     RMSNorm epsilon (the layer uses 1e-8)
 *   ws      device scratch of >= bitlinear_workspace_bytes(M, K, N) bytes;
 *           its contents on entry do not matter; it holds the int8
 *           activations, per-row scales and row sums between the stages.
 * Returns BL_OK or a negative BL_ERR_* code (nothing launched on error). */
int bitlinear_forward(const void *x, int x_dtype, int64_t M, int64_t K,
                      const void *gain, const void *packed, const float *beta,
                      int64_t N, void *y, int y_dtype, float eps, void *ws,
                      size_t ws_bytes, hipStream_t stream);

/* Same as bitlinear_forward with an explicit execution path (BL_PATH_*).
 * BL_PATH_FUSED requires M <= 16, K <= 8192 and M * (K + 16) <= 56320 (its
 * int8 activations live in LDS); BL_PATH_SKINNY requires M <= 64 (else
 * BL_ERR_SHAPE).  Every path computes the same function with the same
 * arithmetic in the same order (the fp64 sum of squares included), so the
 * codes, scales, accumulators and y are bit-identical across paths. */
int bitlinear_forward_path(const void *x, int x_dtype, int64_t M, int64_t K,
                           const void *gain, const void *packed,
                           const float *beta, int64_t N, void *y, int y_dtype,
                           float eps, void *ws, size_t ws_bytes, int path,
                           hipStream_t stream);

/* The BL_PATH_FUSED / _SKINNY / _MFMA path bitlinear_forward takes for a
 * token count M and in_features K with 16-bit activations (BL_ERR_SHAPE for
 * an invalid M or K): FUSED for M <= 4 and K <= 8192 and for M <= 16 and
 * K <= 4096 with M * (K + 16) <= 45056, SKINNY up to M = 64, MFMA above.
 * fp32 activations take FUSED for M == 1 (K <= 8192) and M <= 8
 * (K <= 4096), M <= 16 only up to K = 2048, SKINNY otherwise up to
 * M = 64. */
int bitlinear_select_path(int64_t M, int64_t K);

/* One projection of a grouped forward (all pointers device, as in
 * bitlinear_forward). */
typedef struct bl_call {
    const void *x;        /* [M, K], dtype x_dtype                       */
    const void *gain;     /* [K], dtype x_dtype                          */
    const void *packed;   /* packed weights of an [N, K] matrix          */
    const float *beta;    /* per-tensor weight scale                     */
    void *y;              /* [M, N], dtype y_dtype (written)             */
    int64_t M, K, N;
} bl_call;

/* Several independent FusedBitLinear forwards in few launches, for decode
 * steps where each call is too small to fill the GPU on its own -- e.g. the
 * i/f/g/o projections of an HGRNBit block (hysenlabs ja review, section
 * "HGRNBit という層構成を読む").  Consecutive calls of one shape that the
 * decode kernel takes (in its row mode 2 <= M <= 16, K <= 4096, M * (K + 16)
 * <= 45056, fp32 x with M > 8 only K <= 2048; else in its split mode M <= 4
 * and K <= 8192, fp32 x M == 1) go out up to three per launch, the
 * remaining calls up to 16 per launch of the skinny kernel.
 *   calls   HOST array of ncalls descriptors (read during the call only)
 *   Every call must satisfy the BL_PATH_FUSED limits (M <= 16, K <= 8192,
 *   M * (K + 16) <= 56320) and the usual shape / alignment rules, and all
 *   share x_dtype, y_dtype and eps; calls with M == 0 are skipped.  No
 *   workspace is needed.  Results equal bitlinear_forward on each call.
 *   0 <= ncalls <= 4096; any invalid call rejects the whole group before
 *   anything is launched. */
int bitlinear_forward_grouped(const bl_call *calls, int ncalls, int x_dtype,
                              int y_dtype, float eps, hipStream_t stream);

/* Grouped forward of calls of any size, with a workspace.  Each call is
 * independent and gives bitlinear_forward's result bit for bit.  Calls the
 * default path sends to the one-launch kernels (bitlinear_select_path ==
 * BL_PATH_FUSED for that call's M, K and x_dtype) go out as in
 * bitlinear_forward_grouped.  Every other call runs its two-kernel path, and
 * up to three consecutive calls of one shape (M, K, N) on the same path --
 * HGRNBit's i/f/g projections, which read the same block input (hysenlabs
 * ja review, section "HGRNBit という層構成を読む") -- share one act-quant
 * launch; on the MFMA path also one GEMM launch (three 2048-wide
 * projections of 4096 tokens fill the GPU for several rounds instead of one
 * each), on the skinny path (M <= 64) each keeps its contraction launch.
 * When such a run's calls all pass the same x pointer and the rows are many
 * (M >= 3072, K <= 4096), the shared act-quant reads each row once and
 * quantizes it under every call's gain; the results are the same bits.
 *   calls    HOST array of ncalls descriptors (read during the call only);
 *            shapes, pointers and alignment as for bitlinear_forward, all
 *            sharing x_dtype, y_dtype and eps; calls with M == 0 skipped.
 *   ws       device workspace of at least
 *            bitlinear_grouped_workspace_bytes(calls, ncalls, x_dtype)
 *            bytes, 16-byte aligned (may be NULL when that is 0); reused by
 *            the launches one after another, so two grouped calls may share
 *            it only on one stream.
 * 0 <= ncalls <= 4096; any invalid call rejects the group (BL_ERR_*) before
 * anything is launched. */
size_t bitlinear_grouped_workspace_bytes(const bl_call *calls, int ncalls, int x_dtype);
int bitlinear_forward_grouped_ws(const bl_call *calls, int ncalls, int x_dtype, int y_dtype,
                                 float eps, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ GLU MLP
 * The HGRNBit MLP is gate_proj -> SiLU gate -> down_proj (hysenlabs ja
 * review, section "HGRNBit という層構成を読む": gate_proj 2048 -> 11264,
 * down_proj 5632 -> 2048, SiLU).  Its GLU (datacamp page, section
 * "Kernkomponenten: MLGRU und GLU") passes one BitLinear output through SiLU
 * and multiplies the other by it.  Here gate_proj is one FusedBitLinear with
 * 2F outputs (one per-tensor scale): rows 0..F-1 the SiLU-gated half, rows
 * F..2F-1 the multiplied half, and the gate is fused into its epilogue, so
 * the [M, 2F] projection output never reaches memory. */

/* Pack a gate_proj weight W fp32 [2F, K] (device, row-major) in the GLU
 * row order: packed row 32t + 16h + c holds W row h * F + 16t + c, so each
 * 32-row tile carries 16 gated rows and the 16 rows they multiply.  Same
 * tile format, sizes (bitlinear_packed_bytes(2F, K)) and beta as
 * bitlinear_pack_weights of the same W.  F > 0, F % 16 == 0, K % 128 == 0.
 * Returns BL_OK or a negative BL_ERR_* code. */
int bitlinear_pack_glu_weights(const float *W, int64_t F, int64_t K, void *packed, float *beta,
                               void *ws, size_t ws_bytes, hipStream_t stream);

/* gate_proj + GLU gate: h[m, j] = silu(y[m, j]) * y[m, F + j] with y the
 * FusedBitLinear output of x through the GLU-packed gate_proj, computed in
 * fp32 from the exact int32 accumulators and rounded once to h_dtype.
 *   h       device [M, F], dtype h_dtype (written)
 *   ws      device scratch of >= bitlinear_workspace_bytes(M, K, 2F) bytes
 *   path    BL_PATH_* as for bitlinear_forward_path; BL_PATH_FUSED takes
 *           the one-launch decode kernel where it applies (M <= 4, fp32 x:
 *           M == 1) and otherwise falls back to the two-kernel paths.
 * Everything else as bitlinear_forward.  silu(a) = a / (1 + exp(-a)). */
int bitlinear_forward_glu(const void *x, int x_dtype, int64_t M, int64_t K, const void *gain,
                          const void *packed, const float *beta, int64_t F, void *h,
                          int h_dtype, float eps, void *ws, size_t ws_bytes, int path,
                          hipStream_t stream);

/* ------------------------------------------- FusedRMSNormSwishGate
 * The gate in front of o_proj.  The pages name it -- the gate part of an
 * HGRNBit block is FusedRMSNormSwishGate, a layer of its own fusing an
 * RMSNorm with the gate (hysenlabs ja review, sections "HGRNBit という層構成を
 * 読む" and "代替手段との違い") -- but give no formula; this library reads the
 * name as the RMSNorm of the token mixer's output o times the Swish of the
 * gate input g, Swish with unit slope being the SiLU of the GLU (datacamp
 * page, section "Kernkomponenten: MLGRU und GLU"):
 *   z[m,k] = ((o[m,k] * r_m) * w[k]) * silu(g[m,k]),
 *   r_m = 1 / sqrt(mean_k o[m,k]^2 + eps)
 * (sum of squares in fp64, the rest fp32, silu from the hardware exp2 and
 * reciprocal, ~1e-6 relative), z rounded to the activation dtype. */

/* z [M, K] (dtype, written) from o, g [M, K] and the gate gain w [K] (all
 * dtype, device, read only).  K % 128 == 0, K <= 4096 (else
 * BL_ERR_UNSUPPORTED); eps > 0 (this library's workloads use 1e-6). */
int bitlinear_rmsnorm_swish_gate(const void *o, const void *g, const void *w, int dtype,
                                 int64_t M, int64_t K, float eps, void *z, hipStream_t stream);

/* ------------------------------------------------------- MLGRU scan
 * The token mixer's recurrence.  The pages describe the MLGRU in words only
 * (datacamp page, section "Kernkomponenten: MLGRU und GLU", the MLGRU
 * paragraph and figure panel 2: token by token, gates of values in (0, 1)
 * weigh the previous hidden state against the current token; its
 * projections are i_proj and f_proj, hysenlabs ja review, section "HGRNBit
 * という層構成を読む").  This library reads that as
 *   a = 1 / (1 + e^-f[b,t,d]),  h[b,t,d] = a h[b,t-1,d] + (1 - a) i[b,t,d],
 *   h[b,-1,d] = h0[b,d]  (zero when h0 is NULL),
 * in fp32 (hardware exp2 and reciprocal), h rounded to dtype.  Chunks of 16
 * steps (for 33 <= T < 1024) or 32 are scanned in parallel and joined
 * through their start states (three launches; one when T <= 32). */

/* Workspace bytes bitlinear_mlgru_scan needs for [B, T, D]: 2 B C D floats
 * for C = ceil(T / L) chunks of L = 16 steps (33 <= T < 1024) or 32; 0 when
 * T <= 32, or for an invalid shape. */
size_t bitlinear_mlgru_workspace_bytes(int64_t B, int64_t T, int64_t D);

/* h [B, T, D] (dtype, device, written) from i and f [B, T, D] (dtype,
 * device, read only; a sequence's T token rows consecutive, each D wide --
 * the row order of the i_proj and f_proj outputs).
 *   h0  device fp32 [B, D] start state, or NULL for zeros (read only)
 *   hT  device fp32 [B, D] written with the state after step T - 1
 *       (bit-identical to h[:, T-1, :] before rounding), or NULL; it may
 *       be h0 itself (the state carried from call to call in place)
 *   ws  device scratch of >= bitlinear_mlgru_workspace_bytes(B, T, D) bytes
 *       (16-byte aligned; may be NULL when that is 0)
 * Shapes: 0 <= B <= 65535, 0 <= T <= 2^20, 0 <= D <= 65536, D % 8 == 0
 * (else BL_ERR_SHAPE); B, T or D == 0 is a no-op.  i, f, h 16-byte aligned
 * (BL_ERR_ALIGN); h may not overlap i or f.  Returns BL_OK or a negative
 * BL_ERR_* code (nothing launched on error). */
int bitlinear_mlgru_scan(const void *i, const void *f, int dtype, int64_t B, int64_t T, int64_t D,
                         const float *h0, void *h, float *hT, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* o_proj with the gate as its prologue: y = FusedBitLinear(z) for the z of
 * bitlinear_rmsnorm_swish_gate(o, g, gate_w, gate_eps), without z going
 * through memory.  1..8 tokens of 16-bit activations (M (K + 16) <= 45056):
 * one launch of the decode kernel's row mode, each wave gating, normalizing
 * and quantizing its row in registers before the contraction; otherwise the
 * act-quant launch computes z in registers and quantizes it, then the
 * contraction runs on the skinny path (M <= 64) or the MFMA path.  Either
 * way the codes, scales, row sums and y are identical to running the gate
 * and then bitlinear_forward on the stored z.  gain, packed, beta, N, y,
 * y_dtype, eps, ws and ws_bytes as for bitlinear_forward (workspace
 * bitlinear_workspace_bytes(M, K, N)); x_dtype is the dtype of o, g, gate_w
 * and gain; K <= 4096. */
int bitlinear_forward_gated(const void *o, const void *g, const void *gate_w, float gate_eps,
                            int x_dtype, int64_t M, int64_t K, const void *gain,
                            const void *packed, const float *beta, int64_t N, void *y,
                            int y_dtype, float eps, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/* ------------------------------------------------------ chained decode
 * A decode step of an HGRNBit stack is a chain of FusedBitLinear calls: per
 * block i/f/g_proj on the block input, o_proj, the MLP's gate_proj (GLU)
 * and down_proj, whose output the next block reads (hysenlabs ja review,
 * section "HGRNBit という層構成を読む"; hysenlabs de review, section "Die
 * drei vortrainierten Modelle und ihre Trainingsdaten" for the 24- and
 * 32-block stacks).  At 1..4 tokens each call is too small to fill the GPU
 * and a launch per call costs more than its weights take to stream, so the
 * chain runs as ONE persistent launch: workgroups claim the calls' output
 * tile columns in call order, fetch their weights ahead, and wait (bounded)
 * only for the call whose output they read.  Every call's y equals
 * bitlinear_forward's (or bitlinear_forward_glu's) on the same input, bit
 * for bit.
 *
 * Plan once, run every step: bitlinear_chain_plan validates the calls,
 * works out which earlier call each call reads, and writes a call table and
 * counters into the workspace (it copies from the host and synchronizes the
 * stream: not for graph capture); bitlinear_chain_run is one kernel launch
 * (capturable, allocation-free, replayable any number of times). */
typedef struct bl_chain_call {
    const void *x;        /* [M, K]: an earlier call's y (that call's output
                             is then read inside the launch), or an input
                             no call of the chain writes                   */
    const void *gain;     /* [K]                                          */
    const void *packed;   /* packed [N, K] (GLU order when glu)            */
    const float *beta;    /* per-tensor weight scale                       */
    void *y;              /* [M, N], or h [M, N / 2] when glu (written)    */
    int64_t K, N;         /* N = packed rows (2F for a GLU gate_proj)      */
    int32_t glu;          /* 1: y = silu(gate half) * up half, as
                             bitlinear_forward_glu                         */
    int32_t reserved;     /* 0                                             */
} bl_chain_call;

/* A planned chain (filled by bitlinear_chain_plan; plain data, copyable). */
typedef struct bl_chain {
    void *ws;
    int64_t M, items, kmax, grid, lds;
    int32_t dtype, ncalls;
} bl_chain;

/* Workspace bytes of a chain (0 if the calls are invalid). */
size_t bitlinear_chain_workspace_bytes(const bl_chain_call *calls, int ncalls, int64_t M);

/* Validate and plan a chain.
 *   calls   HOST array of ncalls (1..4096) descriptors, read during the call
 *   M       token rows, 1..4; dtype BL_F16 or BL_BF16 (x, gain and y of
 *           every call); eps the RMSNorm epsilon of every call
 *   ws      device workspace of >= bitlinear_chain_workspace_bytes bytes,
 *           256-byte aligned, owned by this plan until it is re-planned
 *   plan    HOST struct, written
 * A call whose x pointer equals an earlier call's y reads that call's
 * output (the latest such call; its output width must equal K).  Any other
 * x is read as it is and must not overlap a y of the chain.  When y buffers
 * of two calls overlap, the later call's values remain only if it depends,
 * directly or through other calls, on the earlier one.  Shapes, alignment
 * and pointers as for bitlinear_forward; K <= 8192.
 * Returns BL_OK, BL_ERR_* for an invalid request (nothing touched), or
 * BL_ERR_UNSUPPORTED for an x that overlaps a y without equalling it, or
 * fp32 activations. */
int bitlinear_chain_plan(const bl_chain_call *calls, int ncalls, int64_t M, int dtype, float eps,
                         void *ws, size_t ws_bytes, bl_chain *plan, hipStream_t stream);

/* Run a planned chain once: one launch on `stream`.  Runs of one plan must
 * be ordered (same stream); each leaves the workspace ready for the next. */
int bitlinear_chain_run(const bl_chain *plan, hipStream_t stream);

/* bitlinear_chain_run with the bounded wait set to wait_us microseconds of
 * wall clock (bitlinear_chain_run uses two seconds; 0 gives up at the
 * first wait that is not already satisfied).  A wait that gives up sets the
 * plan's error word; every other wait then gives up at once, items whose
 * input never came are skipped, and the launch still ends normally. */
int bitlinear_chain_run_ex(const bl_chain *plan, uint32_t wait_us, hipStream_t stream);

/* Synchronize `stream`, then BL_OK, or BL_ERR_TIMEOUT if a run since the
 * last check gave up waiting (its outputs are then incomplete); clears the
 * error word. */
int bitlinear_chain_status(const bl_chain *plan, hipStream_t stream);

/* ------------------------------------------------- no-allocation forward
 * For callers that cannot allocate device memory at all -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc --
 * bitlinear_forward without the workspace argument: the int8 activations,
 * per-row scales and row sums that pass between its act-quant and
 * contraction launches live in a static device array of
 * bitlinear_noalloc_max_scratch_bytes() bytes (32 MiB) inside the library,
 * one per GPU, held until the process ends.  Nothing is allocated per call
 * (no hipMalloc / hipFree); the first call on a device looks the array's
 * address up once.
 *   Arguments, results and errors as bitlinear_forward (same kernels, same
 *   bits), except: a call whose workspace would exceed the scratch (M * K +
 *   8 M bytes, 256-byte aligned pieces, more than 32 MiB) is rejected with
 *   BL_ERR_SCRATCH before anything is launched.
 *   Every call on one GPU shares that GPU's array and overwrites it before
 *   reading it; calls that overlap in time on one GPU (different streams,
 *   host threads) race on it and must be ordered by the caller. */
size_t bitlinear_noalloc_max_scratch_bytes(void);
int bitlinear_forward_noalloc(const void *x, int x_dtype, int64_t M, int64_t K, const void *gain,
                              const void *packed, const float *beta, int64_t N, void *y,
                              int y_dtype, float eps, hipStream_t stream);

/* Test hook, for callers' failure-path tests: the next n kernel launches the
 * library would issue (any entry point) return BL_ERR_HIP instead, as a
 * failed HIP launch does, without launching or touching memory; n <= 0
 * clears it.  Process-wide; launches that are not forced are unaffected. */
void bitlinear_test_fail_launches(int n);

/* The unit that contracts the decode kernels' 1-token (split mode) and
 * 2-token (row mode) calls -- bitlinear_forward, _forward_glu, _grouped and
 * _grouped_ws on BL_PATH_FUSED.  The datacamp page (section "MatMul durch
 * ternäre Operationen ersetzen") reduces the ternary product to additions
 * and subtractions of activations.  The MFMA path multiplies 16-row blocks
 * of which 1 or 2 rows are live; the VALU path dots each lane's unpacked
 * codes with the activation codes (v_dot4_i32_i8).  Both compute the same
 * exact int32 sums, so outputs are identical bit for bit; only speed
 * differs (the VALU path measured 2-7 % slower on the 2.7B decode calls).
 *   BL_DECODE_AUTO  the library's choice (the MFMA path)
 *   BL_DECODE_MFMA  matrix cores
 *   BL_DECODE_VALU  vector ALU
 * Process-wide, read when a launch is issued (a captured graph keeps the
 * unit it was captured with).  Returns BL_OK, or BL_ERR_PATH for an unknown
 * unit (the setting is then unchanged). */
enum { BL_DECODE_AUTO = 0, BL_DECODE_MFMA = 1, BL_DECODE_VALU = 2 };
int bitlinear_set_decode_contraction(int unit);
int bitlinear_get_decode_contraction(void);

/* Human-readable name of a status code (static string, never NULL). */
const char *bitlinear_status_string(int status);

/* ------------------------------------------------ stage-level entry points
 * These expose the stages of the path one at a time so each can be checked
 * on its own (bit-exact integer outputs). */

/* RMSNorm + per-token int8 quantization: the normalization that keeps the
 * activations in a usable range right before they are quantized (hysenlabs
 * de review, section "HGRNBit: was in einem Block tatsächlich passiert";
 * datacamp page, figure panel 5 of "Kernkomponenten: MLGRU und GLU").  The
 * 8-bit width and one absmax scale per token are this library's reading.
 *   xq [M, K] int8, s [M] fp32, rowsum [M] int32 = sum_k xq[m, k]
 *   (all device, written); x, gain as for bitlinear_forward. */
int bitlinear_act_quant(const void *x, int x_dtype, const void *gain,
                        int64_t M, int64_t K, float eps, int8_t *xq, float *s,
                        int32_t *rowsum, hipStream_t stream);

/* Exact contraction acc[m, n] = sum_k xq[m, k] * Wq[n, k] from int8
 * activations and packed weights (datacamp page above, section "MatMul
 * durch ternäre Operationen ersetzen"; C_ij = sum_p A_ip B_pj as the aidev
 * bluegarage page, section "MatMulとは具体的にどんな計算か", writes it).
 * Beyond the plain contraction this takes a `path`, so each contraction
 * kernel can be checked on its own.
 *   xq      device int8 [M, K] (read only)
 *   rowsum  device int32 [M] = sum_k xq[m, k] (as written by
 *           bitlinear_act_quant); the kernels use it to turn the sum over
 *           the stored codes (Wq + 1) back into the signed sum, so a wrong
 *           rowsum gives a wrong acc.
 *   acc     device int32 [M, N] (written)
 *   path    BL_PATH_AUTO, BL_PATH_SKINNY (M <= 64) or BL_PATH_MFMA;
 *           BL_PATH_FUSED is BL_ERR_PATH here. */
int bitlinear_gemm_i32(const int8_t *xq, const int32_t *rowsum, int64_t M,
                       int64_t K, const void *packed, int64_t N, int32_t *acc,
                       int path, hipStream_t stream);

/* Contraction + rescale from already quantized activations:
 *   y[m, n] = (sum_k xq[m, k] * Wq[n, k]) * beta / s[m]
 * (datacamp page above, section "MatMul durch ternäre Operationen
 * ersetzen" and figure panel 4).  xq, s and rowsum are what
 * bitlinear_act_quant writes; with them this is the second half of
 * bitlinear_forward, so one quantized input can feed several projections.
 *   path    BL_PATH_AUTO, BL_PATH_SKINNY (M <= 64) or BL_PATH_MFMA. */
int bitlinear_contract(const int8_t *xq, const float *s, const int32_t *rowsum,
                       int64_t M, int64_t K, const void *packed,
                       const float *beta, int64_t N, void *y, int y_dtype,
                       int path, hipStream_t stream);

/* bitlinear_contract with the GLU gate in the epilogue: from quantized
 * activations (xq, s, rowsum as bitlinear_act_quant writes them) and a
 * gate_proj packed by bitlinear_pack_glu_weights (2F rows),
 *   h[m, j] = silu(y[m, j]) * y[m, F + j],  y[m, n] = acc[m, n] * beta / s[m]
 * -- the second half of bitlinear_forward_glu, bit for bit (datacamp page,
 * section "Kernkomponenten: MLGRU und GLU": one BitLinear output through
 * SiLU times the other).
 *   h       device [M, F], dtype h_dtype (written)
 *   path    BL_PATH_AUTO, BL_PATH_SKINNY (M <= 64) or BL_PATH_MFMA.
 * F > 0, F % 16 == 0; everything else as bitlinear_contract. */
int bitlinear_contract_glu(const int8_t *xq, const float *s, const int32_t *rowsum, int64_t M,
                           int64_t K, const void *packed, const float *beta, int64_t F, void *h,
                           int h_dtype, int path, hipStream_t stream);

/* One contraction of bitlinear_contract_grouped (device pointers as in
 * bitlinear_contract). */
typedef struct bl_contract_call {
    const int8_t *xq;        /* [M, K]                                     */
    const float *s;          /* [M]                                        */
    const int32_t *rowsum;   /* [M]                                        */
    const void *packed;      /* packed weights of an [N, K] matrix         */
    const float *beta;       /* per-tensor weight scale                    */
    void *y;                 /* [M, N], dtype y_dtype (written)            */
    int64_t M, K, N;
} bl_contract_call;

/* bitlinear_contract on the MFMA kernel for several independent calls, with
 * up to three consecutive calls of one shape (M, K, N) in one launch (the
 * stage-level counterpart of bitlinear_forward_grouped_ws's runs).  Each
 * call's y equals bitlinear_contract(..., BL_PATH_MFMA) bit for bit.
 *   calls   HOST array of ncalls descriptors; shapes, pointers and alignment
 *           as for bitlinear_contract; calls with M == 0 are skipped.
 * 0 <= ncalls <= 4096; any invalid call rejects the group before anything
 * is launched. */
int bitlinear_contract_grouped(const bl_contract_call *calls, int ncalls, int y_dtype,
                               hipStream_t stream);

/* bitlinear_contract_grouped with a path, as bitlinear_contract takes it:
 * BL_PATH_MFMA is bitlinear_contract_grouped; BL_PATH_SKINNY (every call
 * M <= 64, else BL_ERR_SHAPE) runs each group of up to three same-shape
 * calls as one launch of the skinny kernel (the contraction
 * bitlinear_forward_grouped_ws runs for HGRN's i/f/g at 9..64 tokens);
 * BL_PATH_AUTO takes SKINNY for groups with M <= 64, else MFMA.  Each
 * call's y equals bitlinear_contract(..., same path) bit for bit.  Unknown
 * path: BL_ERR_PATH before anything is launched. */
int bitlinear_contract_grouped_path(const bl_contract_call *calls, int ncalls, int y_dtype,
                                    int path, hipStream_t stream);

/* Decode packed weights back to int8 Wq [N, K] in {-1, 0, +1} (device):
 * the ternary matrix of datacamp page, section "MatMul durch ternäre
 * Operationen ersetzen", for checking a pack.  packed as written by
 * bitlinear_pack_weights (N*K/4 bytes, read only); Wq written. */
int bitlinear_unpack_weights(const void *packed, int64_t N, int64_t K,
                             int8_t *Wq, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
