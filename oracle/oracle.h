/*
 * oracle.h -- plain, slow, single-threaded CPU oracle of the FusedBitLinear
 * hot path (RMSNorm -> per-token absmax int8 activations -> per-tensor
 * absmean ternary weights -> integer ternary contraction -> rescale).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library under
 * ternary_weight_lm_amd/ includes, links or calls this code; only the tests,
 * the smoke check and the CPU-baseline leg of the benchmark do.  It shares no
 * header, helper, table or constant with the GPU path.
 *
 * Sources (titles and sections of the pages this follows):
 *   [p1] hysenlabs ja review "matmulfreellm 評価: 行列積を消した HGRNBit を
 *        Transformers 互換で読む", section "HGRNBit という層構成を読む"
 *        (FusedBitLinear holds its own RMSNorm with eps=1e-08).
 *   [p2] hysenlabs fr review "MatMul-Free LM : un modèle de langage sans
 *        multiplication matricielle ...", section "HGRNBit : ce que la
 *        structure du modèle révèle" (bias=False projections).
 *   [p3] hysenlabs de review "MatMul-Free LM: Ternary-Gewichte statt
 *        Matrixmultiplikation im Transformer", section "HGRNBit: was in einem
 *        Block tatsächlich passiert" (norm fused with the ternary projection,
 *        normalization right before quantization).
 *   [p4] datacamp "MatMul-freie LLMs: Zentrale Konzepte erklärt", section
 *        "MatMul durch ternäre Operationen ersetzen" (absmean ternarization,
 *        multiply by -1/0/+1 = negate/zero/keep) and section "Kernkomponenten:
 *        MLGRU und GLU", figure panels 4 (scaled ternary accumulation) and 5
 *        (RMSNorm before quantization).
 *   [p5] aidev.bluegarage "量子化とは何か？MatMulというAIの計算やモデルサイズの
 *        最大のネック", section "MatMulとは具体的にどんな計算か" (C_ij =
 *        sum_p A_ip B_pj and its 2x3 by 3x2 worked example).
 *
 * The pages fix neither the activation bit width nor the rounding details;
 * the readings used here are: 8-bit per-token absmax activations (Qmax 127,
 * clamp [-128,127]); round half to even for both quantizers; eps added to the
 * mean square inside the square root; gain applied after the 1/rms scale;
 * weight scale = mean |W| over the whole matrix, floored at 1e-5; absmax
 * floored at 1e-5.
 *
 * Precision: every value that decides an integer (ternary code, int8 code)
 * is computed in IEEE fp32 with correctly rounded operations, the precision
 * the kernels decide in, except the two long sums (sum of x^2, sum of |W|),
 * which are accumulated in fp64.  The rescale of the integer accumulator is
 * done in fp64.  Build with -O2 -ffp-contract=off, no fast-math.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_pins.py
 * and tests/test_oracle_glu.py (printed worked example, brute force, closed
 * forms, invariants).  Two
 * conventions have no pin on the pages: the 1e-5 floors of the two scales
 * (they never bind on the benchmark data) -- parity unpinned for those
 * floors only.
 */
#ifndef TERNARY_ORACLE_H
#define TERNARY_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Generic integer product C[m,n] = sum_p A[m,p] * B[p,n], all row-major
 * int64 ([p5] "MatMulとは具体的にどんな計算か").  The contraction below is
 * this product with B = Wq transposed. */
void oracle_matmul_i64(const int64_t *A, const int64_t *B, int64_t m,
                       int64_t k, int64_t n, int64_t *C);

/* Sum of |W| over n elements, sequential, fp64. */
double oracle_abs_sum(const float *W, int64_t n);

/* Per-tensor weight scale beta = max(fp32(sum|W| / (N*K)), 1e-5)  ([p4]
 * absmean: the matrix is scaled by its mean absolute value). */
float oracle_weight_scale(const float *W, int64_t N, int64_t K);

/* Ternarize with a given scale: Wq = clamp(rne(fp32(W / beta)), -1, +1)
 * ([p4]: each scaled element is rounded to the nearest of -1, 0, +1). */
void oracle_ternarize(const float *W, int64_t count, float beta, int8_t *Wq);

/* Packed byte size of an [N,K] ternary matrix: N*K/4. */
int64_t oracle_packed_bytes(int64_t N, int64_t K);

/* Pack Wq [N,K] into the 2-bit tile layout (N % 32 == 0, K % 128 == 0).
 * Returns 0, or -1 on a bad shape or a code outside {-1,0,+1}. */
int oracle_pack(const int8_t *Wq, int64_t N, int64_t K, uint8_t *packed);

/* Inverse of oracle_pack.  Returns 0, or -1 on a bad shape or an invalid
 * code (bit pattern 3). */
int oracle_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *Wq);

/* Full offline pack: beta, then Wq, then the 2-bit tiles. */
int oracle_pack_weights(const float *W, int64_t N, int64_t K,
                        uint8_t *packed, float *beta, int8_t *Wq_out);

/* RMSNorm of each row ([p1], [p3]): Q = sum x^2 (fp64, in order),
 * ms = fp32(Q / K), r = 1 / sqrt(ms + eps) (fp32, correctly rounded),
 * xn = (x * r) * g (fp32).  x [M,K] and g [K] are fp32 (inputs stored in
 * fp16 / bf16 are widened exactly by the caller).  r_out may be NULL. */
void oracle_rmsnorm(const float *x, const float *g, int64_t M, int64_t K,
                    float eps, float *xn, float *r_out);

/* Per-token absmax 8-bit quantization of the normalized rows:
 * gamma = max(max|xn|, 1e-5), s = fp32(127 / gamma), v = fp32(xn * s),
 * xq = clamp(rne(v), -128, 127).  v_out (pre-rounding values) may be NULL. */
void oracle_act_quant(const float *xn, int64_t M, int64_t K, int8_t *xq,
                      float *s, float *v_out);

/* Ternary contraction acc[m,n] = sum_k xq[m,k] * Wq[n,k], exact in int64
 * ([p4]: a ternary product is a negate / zero / keep, so only adds and
 * subtracts remain).  Returns 0, or -1 if a sum does not fit int32. */
int oracle_contract(const int8_t *xq, const int8_t *Wq, int64_t M, int64_t N,
                    int64_t K, int32_t *acc);

/* Rescale ([p4] figure panel 4, scaled ternary accumulation):
 * y[m,n] = (acc[m,n] / s[m]) * beta, in fp64. */
void oracle_epilogue(const int32_t *acc, const float *s, float beta,
                     int64_t M, int64_t N, double *y);

/* Whole forward of one FusedBitLinear given its ternary weights.
 * Writes y [M,N] (fp64) and, when non-NULL, xq [M,K], s [M], v [M,K],
 * acc [M,N].  Returns 0 or -1. */
int oracle_forward(const float *x, const float *g, int64_t M, int64_t K,
                   const int8_t *Wq, float beta, int64_t N, float eps,
                   double *y, int8_t *xq, float *s, float *v, int32_t *acc);

/* ------------------------------------------------------------ GLU MLP
 * The MLP of an HGRNBit block is gate_proj -> SiLU gate -> down_proj ([p1]
 * "HGRNBit という層構成を読む", [p2], [p3]: gate_proj 2048 -> 11264, down_proj
 * 5632 -> 2048, SiLU activation).  [p4] "Kernkomponenten: MLGRU und GLU":
 * the input goes through two BitLinear layers, one output passes SiLU and
 * multiplies the other elementwise, and the gated signal goes through a
 * third BitLinear.  Reading (the pages do not say which half is which):
 * gate_proj is those two layers stacked, 2F outputs with F = 5632 = 11264/2;
 * its first F outputs are the SiLU-gated half, the last F the multiplied
 * half; one per-tensor weight scale covers all 2F rows (gate_proj is one
 * FusedBitLinear). */

/* SiLU: a * sigmoid(a) = a / (1 + exp(-a)), fp64. */
double oracle_silu(double a);

/* h[m,j] = silu(y[m,j]) * y[m,F+j] for y [M, 2F] (fp64). */
void oracle_glu(const double *y, int64_t M, int64_t F, double *h);

/* Source row of each packed row of a gate_proj weight [2F, K] in the GLU
 * packed order: packed row 32t + 16h + c holds row 16t + c of the gated half
 * (h = 0) or row F + 16t + c of the multiplied half (h = 1), so each 32-row
 * tile carries 16 gated rows and the 16 rows they multiply.  src [2F].
 * Returns 0, or -1 unless F > 0 and F % 16 == 0. */
int oracle_glu_rows(int64_t F, int64_t *src);

/* FusedRMSNormSwishGate, as the module's name reads (see oracle.c):
 * z [M, K] (fp64) = (o * r_m) * w * silu(g), r_m = 1/sqrt(mean_k o^2 + eps).
 * o, g [M, K] and w [K] fp32 (exact widening of the stored dtype). */
void oracle_rmsnorm_swish_gate(const float *o, const float *g, const float *w, int64_t M,
                               int64_t K, double eps, double *z);

/* The MLGRU scan, as the pages' description reads (see oracle.c):
 * h[b,t,d] = a h[b,t-1,d] + (1 - a) i[b,t,d], a = sigmoid(f[b,t,d]),
 * h[b,-1,:] = h0[b,:] (zero if h0 is NULL).  i, f [B, T, D] fp32; h [B, T, D]
 * and hT [B, D] (may be NULL) fp64. */
void oracle_mlgru_scan(const float *i, const float *f, int64_t B, int64_t T, int64_t D,
                       const double *h0, double *h, double *hT);

#ifdef __cplusplus
}
#endif

#endif
