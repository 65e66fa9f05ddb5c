// decode_kernels.h -- the whole FusedBitLinear in one launch for M <= 16 tokens.
//
// RMSNorm right before the quantizers (hysenlabs de review "MatMul-Free LM:
// Ternary-Gewichte statt Matrixmultiplikation im Transformer", section
// "HGRNBit: was in einem Block tatsächlich passiert"), per-token absmax int8
// codes, the ternary contraction and the rescale of datacamp "MatMul-freie
// LLMs: Zentrale Konzepte erklärt", figure panels 4 and 5.
//
// At decode the layer moves N*K/4 bytes of packed weights and almost nothing
// else, and at the sizes of a single layer it is latency-bound: the design
// removes every serial step it can from the path launch -> last store.
//   * Arguments are plain scalars, so gfx950 preloads them into SGPRs
//     (kernel-argument preloading) instead of the waves fetching them (the
//     three-call kernels fetch what does not fit: gain, beta, output).
//   * All loads of a wave are issued at once, first the activation row and
//     the gain, then the wave's weight tiles.  They are buffer loads whose
//     out-of-range lanes / tiles read as zero, so none is conditional and the
//     compiler's wait for the activations does not also wait for the weights.
//   * The kernels are compiled for a few K capacities (1024 KC, KC = 1 .. 8)
//     and the launch takes the smallest that covers K: each load instruction
//     costs the CU's address unit a slot even where every lane is out of
//     range, and loads sized for the largest K made a short row spend most
//     of its time issuing them.
//   * One workgroup owns one packed 32-row tile column; its waves take the
//     K-blocks round-robin, each feeding v_mfma_i32_16x16x64_i8 from
//     registers (weights) and LDS (codes), and the partial sums meet in LDS.
//   * Split mode (1..4 rows, K <= 8192): the normalization of a row is
//     split over the waves.  The sum of squares stays on waves 0..3 (wave w
//     owns the 8-element chunks 64w + lane + 256r) and meets per lane in LDS
//     ((p0 + p1) + (p2 + p3)) before one DPP tree: the association of the
//     act-quant kernel, so codes and scales are bit-identical across paths.
//     Absmax and codes (exact in any order) are split over all waves.  4
//     waves up to K = 1024, 8 above.
//   * Row mode (2..16 rows, K <= 4096): 8 waves (16 from 13 rows), wave w
//     normalizes and quantizes rows w (and w + 8 at 9..12 rows) alone with
//     the shared row passes of rowquant.h (no cross-wave reduction, one
//     barrier), then the waves share the contraction.
// Up to kDecodeCalls projections of the same shape (HGRN's i/f/g) can share
// one launch in either mode: workgroup b works on call b / tiles.
// At 1 token (split mode) and 2 tokens (row mode) the contraction can run on
// the vector ALU instead (v_dot4_i32_i8 on the unpacked codes, valu_contract)
// -- same integers, same output bits; bitlinear_set_decode_contraction
// picks the unit.
//
// The templates are instantiated once per activation dtype (decode_f32.hip,
// decode_f16.hip, decode_bf16.hip), so the three compile in parallel.
#pragma once
#include "bl_launch.h"
#include "rowquant.h"

namespace bl {


// K capacity of a kernel instance in units of 1024: the smallest of 1, 2, 3,
// 4, 6, 8 with 1024 * KC >= K.  A wave's share of a row follows from it.
constexpr int dec_kc(int64_t K) {
  return K <= 1024 ? 1 : K <= 2048 ? 2 : K <= 3072 ? 3 : K <= 4096 ? 4 : K <= 6144 ? 6 : 8;
}

// Waves per workgroup in the split mode.  More waves share the tile
// column's contraction and the per-element passes; the sum of squares stays
// on waves 0..3 (its fp64 association, below, is fixed).
constexpr int dec_nw(int64_t K) { return K <= 1024 ? 4 : 8; }

// The body of both kernels below: NW waves own one 32-row tile column.
//   * Sum of squares (waves 0..3): lane `l` of wave w owns the 8-element
//     chunks q = 64 w + l + 256 r, r = 0, 1, ... (slot q mod 256, summed in r
//     order); the slots meet per lane in LDS ((p0 + p1) + (p2 + p3) over
//     the 4 waves) before one DPP tree -- the association of the act-quant
//     kernel, so codes and scales are bit-identical across paths.
//   * Absmax and codes (all waves, order-free): wave w takes the rounds
//     r = (NW / 4) c + w / 4 of wave w mod 4's chunks.
//   * Contraction: wave w takes the K-blocks w, w + NW, ...
// The call's packed / gain / beta / out pointers are selected only after
// the activation loads are issued: in the three-call kernel some of them are
// not preloaded and must first be fetched from the argument buffer, and that
// wait must not hold up the first loads.
// The contraction on the vector ALU, for VR <= 2 token rows (the MFMA path
// multiplies 16-row blocks of which VR rows are live).  Lane l holds, per
// tile and k-step s2, the 16 codes of output rows 16 h + l % 16 at k = 32
// (l / 16) + 16 s2 + 0..15 -- the MFMA B operand -- and dots each with the
// same 16 activation codes of every token row (LDS, one broadcast 16-byte
// read per row) by v_dot4_i32_i8, four int8 products per instruction, exact
// in int32.  The four lane groups l / 16 hold disjoint k, so two cross-lane
// additions leave lanes 0..15 with the wave's sums: out[m][h] of output row
// 16 h + lane.  Same integers as the MFMA path, so the same output bits.
template <int VR, int TPW, int NW>
__device__ __forceinline__ void valu_contract(const v4i (&wt)[TPW], const int8_t *xs,
                                              int lds_stride, int w, int nmine, int lane,
                                              int (&out)[VR][2]) {
  int acc[VR][2];
#pragma unroll
  for (int m = 0; m < VR; ++m) acc[m][0] = acc[m][1] = 0;
  const int8_t *abase = xs + 32 * (lane >> 4);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if (t >= nmine) break;
    const v4i u = wt[t];
    const int kofs = (w + NW * t) * 128;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const v4i c0 = unpack_codes((uint32_t)(s2 ? u.y : u.x));  // output rows 0..15
      const v4i c1 = unpack_codes((uint32_t)(s2 ? u.w : u.z));  // output rows 16..31
#pragma unroll
      for (int m = 0; m < VR; ++m) {
        const v4i a = *reinterpret_cast<const v4i *>(abase + m * lds_stride + kofs + 16 * s2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[m][0] = __builtin_amdgcn_sdot4(c0[i], a[i], acc[m][0], false);
          acc[m][1] = __builtin_amdgcn_sdot4(c1[i], a[i], acc[m][1], false);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < VR; ++m)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int v = acc[m][h];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      out[m][h] = v;
    }
}

template <int DT, int OUT, int MR, bool GAIN_LATE, bool GLU, int KC, int NW, bool VALU = false>
__device__ __forceinline__ void decode_body(
    const void *x, int K, int M, int tiles, int nt, float eps, int call, const uint4 *p0,
    const uint4 *p1, const uint4 *p2, const void *g0, const void *g1, const void *g2,
    const float *b0, const float *b1, const float *b2, void *o0, void *o1, void *o2) {
  extern __shared__ __align__(16) int8_t xs[];  // [M][K + 16] int8 codes
  __shared__ double part_ss[MR][4][64];
  __shared__ float part_max[MR][NW];
  __shared__ int part_rs[MR][NW];
  __shared__ int red[NW][MR][2][16];

  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int EB = dtype_bytes(DT);
  constexpr int R = NW / 4;                      // rounds stride of the per-element passes
  constexpr int TPW = (8 * KC + NW - 1) / NW;     // weight tiles per wave
  constexpr int C4 = (KC + 1) / 2;                // sum-of-squares rounds (waves 0..3)
  constexpr int CA = (2 * KC + NW - 1) / NW;      // absmax / code rounds per wave
  constexpr int CO = R == 2 ? C4 / 2 : 0;         // odd rounds loaded only for the sum
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int w4 = w & 3, wh = w >> 2;
  const int KB = K >> 7, nq = K >> 3;
  const int lds_stride = K + 16;

  // ---- 1. every load of the wave, activations first
  const rsrc_t xr = make_rsrc(x, (uint32_t)(M * K * EB));
  // chunk index of round r of wave w mod 4 (past nq: out of range)
  const auto qof = [&](int r) { return 64 * w4 + lane + 256 * r; };
  const auto off = [&](int r) { return qof(r) < nq ? (uint32_t)(8 * qof(r) * EB) : kOob; };
  // Order matters: x needs only preloaded arguments and goes out first; the
  // gain comes next (it is needed right after the first row reduction), the
  // weights last: they are not needed until the contraction, thousands of
  // cycles later.  Waits are in issue order, so whatever is issued later
  // never holds up the wait for what was issued earlier.
  Chunk8<DT> xa[MR][CA], xo[MR][CO > 0 ? CO : 1];
#pragma unroll
  for (int c = 0; c < CA; ++c)
#pragma unroll
    for (int m = 0; m < MR; ++m)
      xa[m][c] = bload_chunk<DT>(xr, m < M ? off(R * c + wh) + (uint32_t)(m * K * EB) : kOob);
  if constexpr (CO > 0) {
    if (w < 4) {
#pragma unroll
      for (int c = 0; c < CO; ++c)
#pragma unroll
        for (int m = 0; m < MR; ++m)
          xo[m][c] = bload_chunk<DT>(xr, m < M ? off(2 * c + 1) + (uint32_t)(m * K * EB) : kOob);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint4 *pk = call == 0 ? p0 : (call == 1 ? p1 : p2);
  const rsrc_t wr = make_rsrc(pk + (int64_t)nt * KB * 64, (uint32_t)KB * 1024u);
  const void *gain = call == 0 ? g0 : (call == 1 ? g1 : g2);
  Chunk8<DT> gc[CA];
  v4i wt[TPW];
  // GAIN_LATE: the gain pointer has to come from the argument buffer, so
  // the weights are issued before waiting for it
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    if constexpr (GAIN_LATE) wt[t] = bload(wr, (uint32_t)((w + NW * t) * 1024 + lane * 16));
  __builtin_amdgcn_sched_barrier(0);
  {
    const rsrc_t gr = make_rsrc(gain, (uint32_t)(K * EB));
#pragma unroll
    for (int c = 0; c < CA; ++c) gc[c] = bload_chunk<DT>(gr, off(R * c + wh));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    if constexpr (!GAIN_LATE) wt[t] = bload(wr, (uint32_t)((w + NW * t) * 1024 + lane * 16));
  __builtin_amdgcn_sched_barrier(0);
  const float *bp = call == 0 ? b0 : (call == 1 ? b1 : b2);
  void *out = call == 0 ? o0 : (call == 1 ? o1 : o2);
  const float beta = *bp;

  // round r of wave w mod 4 holds at least one element of the row
  const auto live = [&](int r) { return 256 * r + 64 * w4 < nq; };

  // Rows past M read as zeros and are carried through every step (their
  // results are never stored): the MR row chains stay free of branches and
  // interleave.
  // ---- 2. sum of squares (waves 0..3): rounds in order, exchanged per lane
  if (w < 4) {
    double ss[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) ss[m] = 0.0;
#pragma unroll
    for (int r = 0; r < C4; ++r)
      if (live(r)) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          float f[8];
          // round r: xa[r / R] if this wave's per-element passes own it, else
          // the odd round loaded for the sum alone
          widen<DT>(R == 1 || (r & 1) == 0 ? xa[m][r / R] : xo[m][CO > 0 ? r >> 1 : 0], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss[m] = __builtin_fma((double)f[e], (double)f[e], ss[m]);
        }
      }
#pragma unroll
    for (int m = 0; m < MR; ++m) part_ss[m][w][lane] = ss[m];
  }
  __syncthreads();

  // ---- 3. absmax of the normalized row
  float r[MR], amax[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const double lsum = (part_ss[m][0][lane] + part_ss[m][1][lane]) +
                        (part_ss[m][2][lane] + part_ss[m][3][lane]);
    r[m] = rms_inv(wave_sum(lsum), K, eps);
    amax[m] = 0.0f;
  }
#pragma unroll
  for (int c = 0; c < CA; ++c)
    if (live(R * c + wh)) {
      float g[8];
      widen<DT>(gc[c], g);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float f[8];
        widen<DT>(xa[m][c], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax[m] = fmaxf(amax[m], fabsf((f[e] * r[m]) * g[e]));
      }
    }
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const float t = wave_max(amax[m]);
    if (lane == 0) part_max[m][w] = t;
  }
  __syncthreads();

  // ---- 4. int8 codes into LDS, row sums of the codes
  float sc[MR], fscale[MR];
  int rs[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float mx = part_max[m][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) mx = fmaxf(mx, part_max[m][i]);
    sc[m] = act_scale(mx);
    fscale[m] = div_rn(beta, sc[m]);
    rs[m] = 0;
  }
#pragma unroll
  for (int c = 0; c < CA; ++c)
    if (live(R * c + wh)) {
      const int q = qof(R * c + wh);
      float g[8];
      widen<DT>(gc[c], g);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float f[8];
        widen<DT>(xa[m][c], f);
        int qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = quant8((f[e] * r[m]) * g[e], sc[m]);
        const uint2 codes = make_uint2(pack4(qv[0], qv[1], qv[2], qv[3]),
                                       pack4(qv[4], qv[5], qv[6], qv[7]));
        rs[m] = __builtin_amdgcn_sdot4((int)codes.x, 0x01010101, rs[m], false);
        rs[m] = __builtin_amdgcn_sdot4((int)codes.y, 0x01010101, rs[m], false);
        if (q < nq && m < M) *reinterpret_cast<uint2 *>(xs + m * lds_stride + 8 * q) = codes;
      }
    }
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const int t = wave_sum(rs[m]);
    if (lane == 0) part_rs[m][w] = t;
  }
  __syncthreads();

  // ---- 5. contraction: the wave's tiles kb = w + NW t
  const int nmine = w < KB ? (KB - w + NW - 1) / NW : 0;
  if constexpr (VALU) {
    static_assert(MR <= 2, "the VALU contraction takes 1 or 2 rows");
    int vs[MR][2];
    valu_contract<MR, TPW, NW>(wt, xs, lds_stride, w, nmine, lane, vs);
    if (lane < 16) {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        red[w][m][0][lane] = vs[m][0];
        red[w][m][1][lane] = vs[m][1];
      }
    }
  } else {
  const int arow = lane & 15;
  const bool arow_ok = arow < M;
  const int8_t *abase = xs + arow * lds_stride + 32 * (lane >> 4);
  // two accumulators per output half (s2 = 0 / 1): each MFMA depends on the
  // one two steps back, not on the previous one
  v4i acc0[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}}, acc1[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  constexpr int kBatch = TPW < 4 ? TPW : 4;  // A operands read from LDS together
#pragma unroll
  for (int t0 = 0; t0 < TPW; t0 += kBatch) {
    if (t0 >= nmine) break;
    v4i a[kBatch][2];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        a[j][s2] = v4i{0, 0, 0, 0};
        if (t0 + j < TPW && arow_ok && t0 + j < nmine)
          a[j][s2] = *reinterpret_cast<const v4i *>(abase + (w + NW * (t0 + j)) * 128 + 16 * s2);
      }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (t0 + j >= TPW || t0 + j >= nmine) break;
      const v4i u = wt[t0 + j];
      // word (h, s2) of a lane slot sits at dword 2h + s2
      v4i c[2][2];
      unpack_pair((uint32_t)u.x, (uint32_t)u.y, c[0][0], c[1][0]);
      unpack_pair((uint32_t)u.z, (uint32_t)u.w, c[0][1], c[1][1]);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        acc0[s2] = mfma16x16x64(a[j][s2], c[s2][0], acc0[s2]);
        acc1[s2] = mfma16x16x64(a[j][s2], c[s2][1], acc1[s2]);
      }
    }
  }

  // ---- 6. partial sums meet in LDS; rescale and store
  // lanes 0..15 hold rows 0..3 (acc[i] = row i) of columns lane / 16 + lane
  if (lane < 16) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      red[w][m][0][lane] = acc0[0][m] + acc0[1][m];
      red[w][m][1][lane] = acc1[0][m] + acc1[1][m];
    }
  }
  }
  __syncthreads();
  const auto tile_sum = [&](int m, int h, int l) {
    int v = red[0][m][h][l];
#pragma unroll
    for (int i = 1; i < NW; ++i) v += red[i][m][h][l];
    return v;
  };
  const auto row_sum = [&](int m) {
    int v = part_rs[m][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) v += part_rs[m][i];
    return v;
  };
  if constexpr (GLU) {
    // GLU order: tile rows 0..15 are gated, 16..31 the rows they multiply;
    // output h[m, 16 nt + l] = silu(y[m, l]) * y[m, 16 + l]
    if (tid < 16 * M) {
      const int m = tid >> 4, l = tid & 15;
      const int rsum = row_sum(m);
      const int vg = tile_sum(m, 0, l) - rsum;
      const int vu = tile_sum(m, 1, l) - rsum;
      float fs = 0.0f;
#pragma unroll
      for (int i = 0; i < MR; ++i)
        if (i == m) fs = fscale[i];
      store1<OUT>(out, (int64_t)m * tiles * 16 + nt * 16 + l, silu((float)vg * fs) * ((float)vu * fs));
    }
    return;
  }
  if (tid < 32 * M) {
    const int m = tid >> 5, n = tid & 31;
    const int h = n >> 4, l = n & 15;
    const int v = tile_sum(m, h, l) - row_sum(m);
    float fs = 0.0f;
#pragma unroll
    for (int i = 0; i < MR; ++i)
      if (i == m) fs = fscale[i];
    store1<OUT>(out, (int64_t)m * tiles * 32 + nt * 32 + n, (float)v * fs);
  }
}

// One call.  Every argument fits the 14 preloaded SGPRs.
// shape = K/128 | M << 7 | tiles << 10.  GLU: the packed rows are a
// gate_proj in GLU order and out is h [M, tiles * 16].
template <int DT, int OUT, int MR, bool GLU, int KC, int NW, bool VALU = false>
__global__ __launch_bounds__(64 * NW, 8 / NW) void decode_kernel(const void *x, uint32_t shape,
                                                                 float eps, const uint4 *packed,
                                                                 const void *gain,
                                                                 const float *beta, void *out) {
  const int K = (int)(shape & 127u) << 7, M = (int)(shape >> 7) & 7;
  decode_body<DT, OUT, MR, false, GLU, KC, NW, VALU>(x, K, M, (int)(shape >> 10), (int)blockIdx.x, eps, 0,
                                               packed, packed, packed, gain, gain, gain, beta, beta,
                                               beta, out, out, out);
}

// Up to three calls of one shape; workgroup b works on call b / tiles.  The
// activation and weight pointers are preloaded, the rest is fetched.
template <int DT, int OUT, int MR, int KC, int NW, bool VALU = false>
__global__ __launch_bounds__(64 * NW, 8 / NW) void decode3_kernel(
    const void *x0, const void *x1, const void *x2, uint32_t shape, float eps,
    const uint4 *p0, const uint4 *p1, const uint4 *p2, const void *g0, const void *g1,
    const void *g2, const float *b0, const float *b1, const float *b2, void *o0, void *o1,
    void *o2) {
  const int K = (int)(shape & 127u) << 7, M = (int)(shape >> 7) & 7;
  const int tiles = (int)(shape >> 10);
  const int bid = (int)blockIdx.x;
  const int call = (bid >= tiles) + (bid >= 2 * tiles);
  const void *x = call == 0 ? x0 : (call == 1 ? x1 : x2);
  decode_body<DT, OUT, MR, true, false, KC, NW, VALU>(x, K, M, tiles, bid - call * tiles, eps, call, p0,
                                                p1, p2, g0, g1, g2, b0, b1, b2, o0, o1, o2);
}

// ---------------------------------------------------------------- row mode
// 2 <= M <= RPW * NW tokens, K <= 4096: wave w normalizes and quantizes
// rows w, w + NW, ... by itself (the shared float-mode row passes of
// rowquant.h, bit-identical to the act-quant kernel), so no row reduction
// crosses a wave and one barrier (the codes in LDS) suffices; then the NW
// waves share the tile column's contraction (rows 0..15: one MFMA block).  Loads go out x row -> gain -> weights; every
// argument is preloaded.  KC: K capacity 1024 KC; a lane caches 2 KC chunks
// of its row.
// GAIN_LATE (three-call kernel): the gain pointer comes from the argument
// buffer, so the weights are issued before waiting for it.
// GATE (one call): x is the token mixer's output o, and each row is first
// put through FusedRMSNormSwishGate with the gate input gin, the gate's gain
// gw and epsilon gate_eps (gate_row, as the gated act-quant kernel does).
template <int DT, int OUT, bool GLU, int KC, int NW, int RPW, bool GAIN_LATE, bool VALU = false,
          bool GATE = false>
__device__ __forceinline__ void decode_rows_body(
    const void *x, uint32_t shape, float eps, int nt, int call, const uint4 *p0, const uint4 *p1,
    const uint4 *p2, const void *g0, const void *g1, const void *g2, const float *b0,
    const float *b1, const float *b2, void *o0, void *o1, void *o2,
    const void *gin = nullptr, const void *gw = nullptr, float gate_eps = 0.0f) {
  extern __shared__ __align__(16) int8_t xs[];  // [M][K + 16] int8 codes
  __shared__ int red[NW][8][64];
  __shared__ float f_row[16];
  __shared__ int rs_row[16];

  constexpr int EB = dtype_bytes(DT);
  constexpr int RC = 2 * KC;                    // chunks of 512 elements per row
  constexpr int TPW = (8 * KC + NW - 1) / NW;   // weight tiles per wave
  const int K = (int)(shape & 127u) << 7, M = (int)(shape >> 7) & 31;
  const int tiles = (int)(shape >> 12);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = K >> 7;
  const int lds_stride = K + 16;

  // ---- 1. loads: this wave's rows, the gain, then the weight tiles
  const rsrc_t xr = make_rsrc(x, (uint32_t)(M * K * EB));
  Chunk8<DT> xraw[RPW][RC];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int m = w + NW * j;
#pragma unroll
    for (int c = 0; c < RC; ++c) {
      const int k = 8 * lane + 512 * c;
      xraw[j][c] = bload_chunk<DT>(xr, m < M && k < K ? (uint32_t)((m * K + k) * EB) : kOob);
    }
  }
  // GATE: the rows' gate inputs and the gate's gain, right behind o
  Chunk8<DT> gate_in[GATE ? RPW : 1][GATE ? RC : 1], gate_w[GATE ? RC : 1];
  if constexpr (GATE) {
    const rsrc_t gir = make_rsrc(gin, (uint32_t)(M * K * EB));
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int m = w + NW * j;
#pragma unroll
      for (int c = 0; c < RC; ++c) {
        const int k = 8 * lane + 512 * c;
        gate_in[j][c] = bload_chunk<DT>(gir, m < M && k < K ? (uint32_t)((m * K + k) * EB) : kOob);
      }
    }
    const rsrc_t gwr = make_rsrc(gw, (uint32_t)(K * EB));
#pragma unroll
    for (int c = 0; c < RC; ++c) gate_w[c] = bload_chunk<DT>(gwr, (uint32_t)((8 * lane + 512 * c) * EB));
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint4 *packed = call == 0 ? p0 : (call == 1 ? p1 : p2);
  const rsrc_t wr = make_rsrc(packed + (int64_t)nt * KB * 64, (uint32_t)KB * 1024u);
  const void *gain = call == 0 ? g0 : (call == 1 ? g1 : g2);
  Chunk8<DT> graw[RC];
  v4i wt[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    if constexpr (GAIN_LATE) wt[t] = bload(wr, (uint32_t)((w + NW * t) * 1024 + lane * 16));
  __builtin_amdgcn_sched_barrier(0);
  {
    const rsrc_t gr = make_rsrc(gain, (uint32_t)(K * EB));
#pragma unroll
    for (int c = 0; c < RC; ++c)
      graw[c] = bload_chunk<DT>(gr, (uint32_t)((8 * lane + 512 * c) * EB));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    if constexpr (!GAIN_LATE) wt[t] = bload(wr, (uint32_t)((w + NW * t) * 1024 + lane * 16));
  __builtin_amdgcn_sched_barrier(0);
  const float *bp = call == 0 ? b0 : (call == 1 ? b1 : b2);
  void *out = call == 0 ? o0 : (call == 1 ? o1 : o2);
  const float beta = *bp;

  // ---- 2. the wave's rows: codes into LDS, scale factor and row sum
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int m = w + NW * j;
    if (m >= M) break;
    int8_t *dst = xs + m * lds_stride;
    float sc;
    int rs;
    const auto sink = [&](int k, uint2 codes) { *reinterpret_cast<uint2 *>(dst + k) = codes; };
    if constexpr (GATE) {
      Chunk8<DT> z[RC];
      gate_row<DT, RC>(xraw[j], gate_in[j], gate_w, K, gate_eps, z);
      quantize_loaded<DT, RC>(z, graw, K, eps, sink, sc, rs);
    } else {
      quantize_loaded<DT, RC>(xraw[j], graw, K, eps, sink, sc, rs);
    }
    if (lane == 0) {
      f_row[m] = div_rn(beta, sc);
      rs_row[m] = rs;
    }
  }
  __syncthreads();

  // ---- 3. contraction: tiles kb = w + NW t, rows 0..15 as one MFMA block
  // (VALU: the 2 rows of a 2-token call on the vector ALU)
  const int nmine = w < KB ? (KB - w + NW - 1) / NW : 0;
  if constexpr (VALU) {
    int vs[2][2];
    valu_contract<2, TPW, NW>(wt, xs, lds_stride, w, nmine, lane, vs);
    // red[w][4 h + i][L] holds row 4 (L / 16) + i: rows 0, 1 at L = 0..15
    if (lane < 16) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        red[w][m][lane] = vs[m][0];
        red[w][4 + m][lane] = vs[m][1];
      }
    }
  } else {
  const int arow = lane & 15;
  const int8_t *abase = xs + arow * lds_stride + 32 * (lane >> 4);
  v4i acc0[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}}, acc1[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  constexpr int kBatch = TPW < 4 ? TPW : 4;
#pragma unroll
  for (int t0 = 0; t0 < TPW; t0 += kBatch) {
    if (t0 >= nmine) break;
    v4i a[kBatch][2];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        a[j][s2] = v4i{0, 0, 0, 0};
        if (t0 + j < TPW && arow < M && t0 + j < nmine)
          a[j][s2] = *reinterpret_cast<const v4i *>(abase + (w + NW * (t0 + j)) * 128 + 16 * s2);
      }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (t0 + j >= TPW || t0 + j >= nmine) break;
      const v4i u = wt[t0 + j];
      v4i c[2][2];
      unpack_pair((uint32_t)u.x, (uint32_t)u.y, c[0][0], c[1][0]);
      unpack_pair((uint32_t)u.z, (uint32_t)u.w, c[0][1], c[1][1]);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        acc0[s2] = mfma16x16x64(a[j][s2], c[s2][0], acc0[s2]);
        acc1[s2] = mfma16x16x64(a[j][s2], c[s2][1], acc1[s2]);
      }
    }
  }

  // ---- 4. partial sums meet in LDS; rescale and store.  red[w][4 h + i][L]
  // holds row 4 (L / 16) + i, column 16 h + L % 16 of the tile.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[w][i][lane] = acc0[0][i] + acc0[1][i];
    red[w][4 + i][lane] = acc1[0][i] + acc1[1][i];
  }
  }
  __syncthreads();
  const auto wsum = [&](int j, int L) {
    int v = red[0][j][L];
#pragma unroll
    for (int i = 1; i < NW; ++i) v += red[i][j][L];
    return v;
  };
  if constexpr (GLU) {
    const int m = tid >> 4, c = tid & 15;  // 16 rows x 16 outputs
    if (m < M) {
      const int Lq = 16 * (m >> 2) + c, jg = m & 3, ju = jg + 4;
      const int vg = wsum(jg, Lq) - rs_row[m];
      const int vu = wsum(ju, Lq) - rs_row[m];
      store1<OUT>(out, (int64_t)m * tiles * 16 + nt * 16 + c,
                  silu((float)vg * f_row[m]) * ((float)vu * f_row[m]));
    }
  } else {
#pragma unroll
    for (int q = 0; q < (512 + 64 * NW - 1) / (64 * NW); ++q) {
      const int idx = tid + 64 * NW * q;
      if (NW > 8 && idx >= 512) break;  // 16 waves: half the threads store
      const int j = idx >> 6, Lq = idx & 63;
      const int h = j >> 2, i = j & 3;
      const int m = 4 * (Lq >> 4) + i;
      if (m >= M) continue;
      const int v = wsum(j, Lq) - rs_row[m];
      store1<OUT>(out, (int64_t)m * tiles * 32 + nt * 32 + 16 * h + (Lq & 15), (float)v * f_row[m]);
    }
  }
}

template <int DT, int OUT, bool GLU, int KC, int NW, int RPW, bool VALU = false>
__global__ __launch_bounds__(64 * NW, NW <= 8 ? 8 / NW : 4) void decode_rows_kernel(const void *x, uint32_t shape,
                                                                      float eps,
                                                                      const uint4 *packed,
                                                                      const void *gain,
                                                                      const float *bp, void *out) {
  decode_rows_body<DT, OUT, GLU, KC, NW, RPW, false, VALU>(x, shape, eps, (int)blockIdx.x, 0, packed, packed,
                                                packed, gain, gain, gain, bp, bp, bp, out, out,
                                                out);
}

// One gated call (o_proj behind FusedRMSNormSwishGate) in row mode, 1..8
// rows: the gate, o_proj's norm, quantization, contraction and rescale in
// one launch.
template <int DT, int OUT, int KC, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void decode_rows_gated_kernel(
    const void *o, const void *gin, const void *gw, float gate_eps, uint32_t shape, float eps,
    const uint4 *packed, const void *gain, const float *bp, void *out) {
  decode_rows_body<DT, OUT, false, KC, NW, 1, false, false, true>(
      o, shape, eps, (int)blockIdx.x, 0, packed, packed, packed, gain, gain, gain, bp, bp, bp,
      out, out, out, gin, gw, gate_eps);
}

// Up to three row-mode calls of one shape; workgroup b works on call
// b / tiles.  The activation and weight pointers are preloaded, the rest is
// fetched.
template <int DT, int OUT, int KC, int NW, int RPW, bool VALU = false>
__global__ __launch_bounds__(64 * NW, NW <= 8 ? 8 / NW : 4) void decode_rows3_kernel(
    const void *x0, const void *x1, const void *x2, uint32_t shape, float eps, const uint4 *p0,
    const uint4 *p1, const uint4 *p2, const void *g0, const void *g1, const void *g2,
    const float *b0, const float *b1, const float *b2, void *o0, void *o1, void *o2) {
  const int tiles = (int)(shape >> 12);
  const int bid = (int)blockIdx.x;
  const int call = (bid >= tiles) + (bid >= 2 * tiles);
  const void *x = call == 0 ? x0 : (call == 1 ? x1 : x2);
  decode_rows_body<DT, OUT, false, KC, NW, RPW, true, VALU>(x, shape, eps, bid - call * tiles, call, p0, p1,
                                                 p2, g0, g1, g2, b0, b1, b2, o0, o1, o2);
}

// Waves per workgroup in the row mode: 8 (one per row; the contraction is
// split 8 ways -- measured faster than 4 waves from 2 rows and K = 1024 up),
// 16 from 13 rows.
constexpr int kRowsNW = 8;

template <int DT, int OUT, bool GLU, int KC, int NW, int RPW, bool VALU = false>
static void launch_rows_rpw(const DecodeArgs &a, hipStream_t stream) {
  const unsigned tiles = (unsigned)(a.N / 32);
  const size_t lds = (size_t)a.M * (size_t)(a.K + 16);
  const uint32_t shape = (uint32_t)(a.K >> 7) | ((uint32_t)a.M << 7) | (tiles << 12);
  const uint4 *pk = reinterpret_cast<const uint4 *>(a.packed[0]);
  if (a.ncalls > 1) {
    const uint4 *p[3];
    for (int i = 0; i < 3; ++i) p[i] = reinterpret_cast<const uint4 *>(a.packed[i]);
    const unsigned grid = tiles * (unsigned)a.ncalls;
    decode_rows3_kernel<DT, OUT, KC, NW, RPW, VALU><<<grid, 64 * NW, lds, stream>>>(
        a.x[0], a.x[1], a.x[2], shape, a.eps, p[0], p[1], p[2], a.gain[0], a.gain[1], a.gain[2],
        a.beta[0], a.beta[1], a.beta[2], a.out[0], a.out[1], a.out[2]);
    return;
  }
  decode_rows_kernel<DT, OUT, GLU, KC, NW, RPW, VALU><<<tiles, 64 * NW, lds, stream>>>(
      a.x[0], shape, a.eps, pk, a.gain[0], a.beta[0], a.out[0]);
}

// one row per wave up to 8 rows, two up to 16
template <int DT, int OUT, bool GLU, int KC>
static void launch_rows_t(const DecodeArgs &a, hipStream_t stream) {
  // 9..12 rows: 8 waves, two rows on some; 13..16 rows: 16 waves of one row
  // each, so no wave runs two row chains in a row (16 rows: 6-12 % faster;
  // at 9 rows the wider workgroup was 5 % slower).  fp32 rows past K = 2048
  // do not fit 16 waves' registers; decode_rows_fits never sends them more
  // than 8 rows, and the 8-wave kernel stands in for that instance.
  if (a.M == 2 && decode_use_valu()) launch_rows_rpw<DT, OUT, GLU, KC, kRowsNW, 1, true>(a, stream);
  else if (a.M <= kRowsNW) launch_rows_rpw<DT, OUT, GLU, KC, kRowsNW, 1>(a, stream);
  else if (a.M <= 12) launch_rows_rpw<DT, OUT, GLU, KC, kRowsNW, 2>(a, stream);
  else if constexpr (DT == BL_F32 && KC > 2) launch_rows_rpw<DT, OUT, GLU, KC, kRowsNW, 2>(a, stream);
  else launch_rows_rpw<DT, OUT, GLU, KC, 2 * kRowsNW, 1>(a, stream);
}

// row mode: K <= 4096 (decode_rows_fits)
template <int DT, int OUT, bool GLU>
static void launch_rows(const DecodeArgs &a, hipStream_t stream) {
  switch (dec_kc(a.K)) {
    case 1: launch_rows_t<DT, OUT, GLU, 1>(a, stream); break;
    case 2: launch_rows_t<DT, OUT, GLU, 2>(a, stream); break;
    case 3: launch_rows_t<DT, OUT, GLU, 3>(a, stream); break;
    default: launch_rows_t<DT, OUT, GLU, 4>(a, stream); break;
  }
}

template <int DT, int OUT, int KC>
static void launch_mr_t(const DecodeArgs &a, hipStream_t stream) {
  constexpr int NW = dec_nw(1024 * KC);
  const unsigned tiles = (unsigned)(a.N / 32);
  const unsigned grid = tiles * (unsigned)a.ncalls;
  const size_t lds = (size_t)a.M * (size_t)(a.K + 16);
  const uint32_t shape = (uint32_t)(a.K >> 7) | ((uint32_t)a.M << 7) | (tiles << 10);
  const uint4 *p[3];
  for (int i = 0; i < 3; ++i) p[i] = reinterpret_cast<const uint4 *>(a.packed[i]);
  // fp32 activations decode one row per launch (decode_fits)
  constexpr int MR4 = DT == BL_F32 ? 1 : (int)kDecodeMaxM;
  const bool valu = a.M == 1 && decode_use_valu();
  if (a.ncalls == 1) {
#define BL_DECODE1(MR_, G, V)                                                               \
  decode_kernel<DT, OUT, MR_, G, KC, NW, V><<<grid, 64 * NW, lds, stream>>>(                 \
      a.x[0], shape, a.eps, p[0], a.gain[0], a.beta[0], a.out[0])
    if (valu) {
      if (a.glu) BL_DECODE1(1, true, true); else BL_DECODE1(1, false, true);
    } else if (a.M == 1) {
      if (a.glu) BL_DECODE1(1, true, false); else BL_DECODE1(1, false, false);
    } else {
      if (a.glu) BL_DECODE1(MR4, true, false); else BL_DECODE1(MR4, false, false);
    }
#undef BL_DECODE1
    return;
  }
#define BL_DECODE3(MR_, V)                                                                  \
  decode3_kernel<DT, OUT, MR_, KC, NW, V><<<grid, 64 * NW, lds, stream>>>(                   \
      a.x[0], a.x[1], a.x[2], shape, a.eps, p[0], p[1], p[2], a.gain[0], a.gain[1],          \
      a.gain[2], a.beta[0], a.beta[1], a.beta[2], a.out[0], a.out[1], a.out[2])
  if (valu) BL_DECODE3(1, true);
  else if (a.M == 1) BL_DECODE3(1, false);
  else BL_DECODE3(MR4, false);
#undef BL_DECODE3
}

// split mode: K <= 8192 (decode_split_fits)
template <int DT, int OUT>
static void launch_mr(const DecodeArgs &a, hipStream_t stream) {
  switch (dec_kc(a.K)) {
    case 1: launch_mr_t<DT, OUT, 1>(a, stream); break;
    case 2: launch_mr_t<DT, OUT, 2>(a, stream); break;
    case 3: launch_mr_t<DT, OUT, 3>(a, stream); break;
    case 4: launch_mr_t<DT, OUT, 4>(a, stream); break;
    case 6: launch_mr_t<DT, OUT, 6>(a, stream); break;
    default: launch_mr_t<DT, OUT, 8>(a, stream); break;
  }
}

// The gated row mode (decode_gated_fits): 8 waves, one row per wave.
template <int DT, int OUT, int KC>
static void launch_rows_gated_t(const DecodeGateArgs &a, hipStream_t stream) {
  const unsigned tiles = (unsigned)(a.N / 32);
  const size_t lds = (size_t)a.M * (size_t)(a.K + 16);
  const uint32_t shape = (uint32_t)(a.K >> 7) | ((uint32_t)a.M << 7) | (tiles << 12);
  decode_rows_gated_kernel<DT, OUT, KC, kRowsNW><<<tiles, 64 * kRowsNW, lds, stream>>>(
      a.o, a.g, a.gate_w, a.gate_eps, shape, a.eps, reinterpret_cast<const uint4 *>(a.packed),
      a.gain, a.beta, a.out);
}

template <int DT, int OUT>
static void launch_rows_gated(const DecodeGateArgs &a, hipStream_t stream) {
  switch (dec_kc(a.K)) {
    case 1: launch_rows_gated_t<DT, OUT, 1>(a, stream); break;
    case 2: launch_rows_gated_t<DT, OUT, 2>(a, stream); break;
    case 3: launch_rows_gated_t<DT, OUT, 3>(a, stream); break;
    default: launch_rows_gated_t<DT, OUT, 4>(a, stream); break;
  }
}

template <int DT>
static void launch_decode_gated_dt(const DecodeGateArgs &a, hipStream_t stream) {
  switch (a.out_kind) {
    case BL_F32: launch_rows_gated<DT, BL_F32>(a, stream); break;
    case BL_F16: launch_rows_gated<DT, BL_F16>(a, stream); break;
    default: launch_rows_gated<DT, BL_BF16>(a, stream); break;
  }
}

// Row mode whenever it fits (one call, or up to three of one shape without
// the GLU epilogue), else split mode.
template <int DT>
static void launch_decode_dt(const DecodeArgs &a, hipStream_t stream) {
  if (decode_rows_fits(a.M, a.K, a.x_dtype) && (a.ncalls == 1 || !a.glu)) {
#define BL_ROWS(O)                                                   \
  (a.glu ? launch_rows<DT, O, true>(a, stream) : launch_rows<DT, O, false>(a, stream))
    switch (a.out_kind) {
      case BL_F32: BL_ROWS(BL_F32); break;
      case BL_F16: BL_ROWS(BL_F16); break;
      default: BL_ROWS(BL_BF16); break;
    }
#undef BL_ROWS
    return;
  }
  switch (a.out_kind) {
    case BL_F32: launch_mr<DT, BL_F32>(a, stream); break;
    case BL_F16: launch_mr<DT, BL_F16>(a, stream); break;
    default: launch_mr<DT, BL_BF16>(a, stream); break;
  }
}

}  // namespace bl
