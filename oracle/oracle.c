/*
 * oracle.c -- plain single-threaded CPU oracle of the FusedBitLinear path.
 * TEST INFRASTRUCTURE ONLY (see oracle.h for the sources, the readings of the
 * pages and the precision rules).  Every loop here is the textbook loop of
 * the step it implements: no blocking, no fusion, no reordering.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- matmul */

void oracle_matmul_i64(const int64_t *A, const int64_t *B, int64_t m,
                       int64_t k, int64_t n, int64_t *C)
{
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            int64_t acc = 0;
            for (int64_t p = 0; p < k; ++p)
                acc += A[i * k + p] * B[p * n + j];
            C[i * n + j] = acc;
        }
}

/* ------------------------------------------------------- weight quantizer */

double oracle_abs_sum(const float *W, int64_t n)
{
    double sum = 0.0;
    for (int64_t i = 0; i < n; ++i)
        sum += fabs((double)W[i]);
    return sum;
}

float oracle_weight_scale(const float *W, int64_t N, int64_t K)
{
    double total = oracle_abs_sum(W, N * K);
    float mean = (float)(total / (double)(N * K));
    return mean > 1e-5f ? mean : 1e-5f;
}

/* rintf rounds half to even in the default rounding mode. */
static int8_t ternary_of(float w, float beta)
{
    float q = rintf(w / beta);
    if (q > 1.0f) q = 1.0f;
    if (q < -1.0f) q = -1.0f;
    return (int8_t)q;
}

void oracle_ternarize(const float *W, int64_t count, float beta, int8_t *Wq)
{
    for (int64_t i = 0; i < count; ++i)
        Wq[i] = ternary_of(W[i], beta);
}

/* ------------------------------------------------------------ 2-bit tiles
 * Layout (the library header states the same rule in prose; this is an
 * independent implementation of that statement):
 *   tile (nt, kb) holds rows 32*nt .. 32*nt+31 and columns 128*kb .. +127;
 *   tiles are stored nt-major, kb-minor, 1024 bytes each;
 *   inside a tile, row 32*nt + 16*h + c and 16-column group j (k = 128*kb +
 *   16*j + e) live in the little-endian 32-bit word at byte offset
 *   16*(16*(j/2) + c) + 4*(2*h + j%2);
 *   inside that word, element e uses bits 8*(e%4) + 2*(e/4) and +1;
 *   the 2-bit value is Wq + 1 (0 -> -1, 1 -> 0, 2 -> +1; 3 is never used). */

int64_t oracle_packed_bytes(int64_t N, int64_t K) { return N * K / 4; }

static int layout_ok(int64_t N, int64_t K)
{
    return N > 0 && K > 0 && N % 32 == 0 && K % 128 == 0;
}

/* Byte offset of the word holding (n, j) and the bit of element e. */
static void locate(int64_t n, int64_t k, int64_t K, int64_t *byte_off,
                   int *bit)
{
    int64_t nt = n / 32, kb = k / 128;
    int64_t h = (n % 32) / 16, c = n % 16;
    int64_t j = (k % 128) / 16, e = k % 16;
    int64_t tile = nt * (K / 128) + kb;
    int64_t word_off = 16 * (16 * (j / 2) + c) + 4 * (2 * h + j % 2);
    int bitpos = (int)(8 * (e % 4) + 2 * (e / 4));
    *byte_off = tile * 1024 + word_off + bitpos / 8;
    *bit = bitpos % 8;
}

int oracle_pack(const int8_t *Wq, int64_t N, int64_t K, uint8_t *packed)
{
    if (!layout_ok(N, K)) return -1;
    memset(packed, 0, (size_t)oracle_packed_bytes(N, K));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int8_t w = Wq[n * K + k];
            if (w < -1 || w > 1) return -1;
            int64_t off;
            int bit;
            locate(n, k, K, &off, &bit);
            packed[off] |= (uint8_t)((w + 1) << bit);
        }
    return 0;
}

int oracle_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *Wq)
{
    if (!layout_ok(N, K)) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t off;
            int bit;
            locate(n, k, K, &off, &bit);
            int code = (packed[off] >> bit) & 3;
            if (code == 3) return -1;
            Wq[n * K + k] = (int8_t)(code - 1);
        }
    return 0;
}

int oracle_pack_weights(const float *W, int64_t N, int64_t K,
                        uint8_t *packed, float *beta, int8_t *Wq_out)
{
    if (!layout_ok(N, K)) return -1;
    int8_t *Wq = Wq_out ? Wq_out : (int8_t *)malloc((size_t)(N * K));
    if (!Wq) return -1;
    float b = oracle_weight_scale(W, N, K);
    oracle_ternarize(W, N * K, b, Wq);
    int rc = oracle_pack(Wq, N, K, packed);
    if (!Wq_out) free(Wq);
    *beta = b;
    return rc;
}

/* ------------------------------------------------------------- activations */

void oracle_rmsnorm(const float *x, const float *g, int64_t M, int64_t K,
                    float eps, float *xn, float *r_out)
{
    for (int64_t m = 0; m < M; ++m) {
        const float *row = x + m * K;
        double sumsq = 0.0;
        for (int64_t k = 0; k < K; ++k)
            sumsq += (double)row[k] * (double)row[k];
        float ms = (float)(sumsq / (double)K);
        float r = 1.0f / sqrtf(ms + eps);
        for (int64_t k = 0; k < K; ++k) {
            float t = row[k] * r;
            xn[m * K + k] = t * g[k];
        }
        if (r_out) r_out[m] = r;
    }
}

void oracle_act_quant(const float *xn, int64_t M, int64_t K, int8_t *xq,
                      float *s, float *v_out)
{
    for (int64_t m = 0; m < M; ++m) {
        const float *row = xn + m * K;
        float gamma = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(row[k]);
            if (a > gamma) gamma = a;
        }
        if (gamma < 1e-5f) gamma = 1e-5f;
        float scale = 127.0f / gamma;
        s[m] = scale;
        for (int64_t k = 0; k < K; ++k) {
            float v = row[k] * scale;
            float q = rintf(v);
            if (q > 127.0f) q = 127.0f;
            if (q < -128.0f) q = -128.0f;
            xq[m * K + k] = (int8_t)q;
            if (v_out) v_out[m * K + k] = v;
        }
    }
}

/* -------------------------------------------------------------- contraction */

int oracle_contract(const int8_t *xq, const int8_t *Wq, int64_t M, int64_t N,
                    int64_t K, int32_t *acc)
{
    /* acc = xq (M x K) times Wq^T (K x N), through the generic product. */
    int64_t *A = (int64_t *)malloc((size_t)(M * K) * sizeof(int64_t));
    int64_t *B = (int64_t *)malloc((size_t)(K * N) * sizeof(int64_t));
    int64_t *C = (int64_t *)malloc((size_t)(M * N) * sizeof(int64_t));
    int rc = 0;
    if (!A || !B || !C) { rc = -1; goto done; }
    for (int64_t i = 0; i < M * K; ++i) A[i] = xq[i];
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            B[k * N + n] = Wq[n * K + k];
    oracle_matmul_i64(A, B, M, K, N, C);
    for (int64_t i = 0; i < M * N; ++i) {
        if (C[i] > INT32_MAX || C[i] < INT32_MIN) { rc = -1; goto done; }
        acc[i] = (int32_t)C[i];
    }
done:
    free(A);
    free(B);
    free(C);
    return rc;
}

void oracle_epilogue(const int32_t *acc, const float *s, float beta,
                     int64_t M, int64_t N, double *y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = ((double)acc[m * N + n] / (double)s[m]) * (double)beta;
}

/* ----------------------------------------------------------------- forward */

int oracle_forward(const float *x, const float *g, int64_t M, int64_t K,
                   const int8_t *Wq, float beta, int64_t N, float eps,
                   double *y, int8_t *xq_out, float *s_out, float *v_out,
                   int32_t *acc_out)
{
    float *xn = (float *)malloc((size_t)(M * K) * sizeof(float));
    int8_t *xq = xq_out ? xq_out : (int8_t *)malloc((size_t)(M * K));
    float *s = s_out ? s_out : (float *)malloc((size_t)M * sizeof(float));
    int32_t *acc = acc_out ? acc_out
                           : (int32_t *)malloc((size_t)(M * N) * sizeof(int32_t));
    int rc = -1;
    if (!xn || !xq || !s || !acc) goto done;
    oracle_rmsnorm(x, g, M, K, eps, xn, NULL);
    oracle_act_quant(xn, M, K, xq, s, v_out);
    if (oracle_contract(xq, Wq, M, N, K, acc) != 0) goto done;
    oracle_epilogue(acc, s, beta, M, N, y);
    rc = 0;
done:
    free(xn);
    if (!xq_out) free(xq);
    if (!s_out) free(s);
    if (!acc_out) free(acc);
    return rc;
}

/* --------------------------------------------------------------- GLU MLP */

double oracle_silu(double a)
{
    return a / (1.0 + exp(-a));
}

void oracle_glu(const double *y, int64_t M, int64_t F, double *h)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < F; ++j)
            h[m * F + j] = oracle_silu(y[m * 2 * F + j]) * y[m * 2 * F + F + j];
}

int oracle_glu_rows(int64_t F, int64_t *src)
{
    if (F <= 0 || F % 16 != 0) return -1;
    for (int64_t r = 0; r < 2 * F; ++r) {
        const int64_t t = r / 32, half = (r % 32) / 16, c = r % 16;
        src[r] = (half == 0 ? 0 : F) + 16 * t + c;
    }
    return 0;
}

/* ------------------------------------- FusedRMSNormSwishGate (a reading) */

/* The gate in front of o_proj.  The pages name the module and its role only:
 * the gate part of the block is FusedRMSNormSwishGate, a layer of its own
 * that fuses an RMSNorm with the gate (hysenlabs ja review, sections
 * "HGRNBit という層構成を読む" and "代替手段との違い").  The reading is what the
 * name says: the RMSNorm of the token mixer's output o (gain w, epsilon eps)
 * multiplied elementwise by the Swish of the gate input g, Swish with unit
 * slope being the SiLU a / (1 + e^-a) of the GLU (datacamp "MatMul-freie
 * LLMs: Zentrale Konzepte erklärt", section "Kernkomponenten: MLGRU und GLU"):
 *   z[m,k] = (o[m,k] * r_m) * w[k] * silu(g[m,k]),
 *   r_m    = 1 / sqrt(sum_k o[m,k]^2 / K + eps).
 * Everything in fp64; z is a floating-point value held to a tolerance. */
void oracle_rmsnorm_swish_gate(const float *o, const float *g, const float *w, int64_t M,
                               int64_t K, double eps, double *z)
{
    for (int64_t m = 0; m < M; ++m) {
        const float *orow = o + m * K;
        const float *grow = g + m * K;
        double sumsq = 0.0;
        for (int64_t k = 0; k < K; ++k)
            sumsq += (double)orow[k] * (double)orow[k];
        const double r = 1.0 / sqrt(sumsq / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            z[m * K + k] = ((double)orow[k] * r) * (double)w[k] * oracle_silu((double)grow[k]);
    }
}

/* ------------------------------------------------ MLGRU scan (a reading) */

/* The token mixer of the HGRNBit block.  The pages describe the MLGRU in
 * words only (datacamp "MatMul-freie LLMs: Zentrale Konzepte erklärt",
 * section "Kernkomponenten: MLGRU und GLU", the MLGRU paragraph and figure
 * panel 2): it runs over the sequence token by token; each step takes the
 * current token and the previous hidden state and updates the state with
 * elementwise operations and gates, vectors of values between 0 and 1 that
 * weigh which parts of the previous state and of the current token carry
 * on.  Its projections are the block's i_proj and f_proj (hysenlabs ja
 * review, section "HGRNBit という層構成を読む").  The reading taken here is
 * the plainest one those words support: the forget gate is the logistic
 * sigmoid of f_proj's output, the candidate is i_proj's output, and the new
 * state is their gate-weighted mix,
 *   a = 1 / (1 + e^-f[b,t,d]),
 *   h[b,t,d] = a * h[b,t-1,d] + (1 - a) * i[b,t,d],   h[b,-1,d] = h0[b,d],
 * per sequence b, time step t and channel d; the state starts at h0 (zero
 * when h0 is NULL) and hT receives h[b,T-1,:].  i, f, h are [B, T, D] with
 * the tokens of one sequence consecutive; everything in fp64. */
void oracle_mlgru_scan(const float *i, const float *f, int64_t B, int64_t T, int64_t D,
                       const double *h0, double *h, double *hT)
{
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d) {
            double state = h0 ? h0[b * D + d] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t e = (b * T + t) * D + d;
                const double a = 1.0 / (1.0 + exp(-(double)f[e]));
                state = a * state + (1.0 - a) * (double)i[e];
                h[e] = state;
            }
            if (hT) hT[b * D + d] = state;
        }
}
