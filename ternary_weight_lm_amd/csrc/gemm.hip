// gemm.hip -- tiled ternary contraction on the gfx950 int8 matrix cores.
//
// acc[m, n] = sum_k xq[m, k] * Wq[n, k]: with ternary weights every product
// is a negate / zero / keep of an activation (datacamp "MatMul-freie LLMs:
// Zentrale Konzepte erklärt", section "MatMul durch ternäre Operationen
// ersetzen"), followed by the scaled rescale of figure panel 4.  On gfx950
// the cheapest exact way to add up many int8 values is still the dense i8
// MFMA (v_mfma_i32_16x16x64_i8), so the stored codes c = Wq + 1 in {0,1,2}
// are fed to it as int8 and the signed sum is recovered exactly as
//   sum_k xq * Wq = sum_k xq * c - sum_k xq      (rowsum from act-quant).
//
// Workgroup tile: BM = 32*MI token rows x BN = 128 output rows, K in blocks
// of 128 (one packed tile column).  4 waves as 2 x 2; wave (wm, wn) owns
// 16*MI rows x 64 outputs = MI x 4 MFMA blocks of 16 x 16.
//   A (xq): global -> registers -> LDS, double-buffered, 16-byte chunks of a
//           128-byte row XOR-swizzled (swz) so the lanes that read one column
//           of chunks hit distinct banks.
//   B (packed codes): each wave loads its two 1 KiB tiles per k-block
//           straight into registers (one 16-byte load per lane per tile, the
//           layout was built for exactly this) and unpacks them with
//           shift + mask; no LDS traffic for weights.
//   Loads run two k-blocks ahead of the MFMAs.
// Epilogue: subtract rowsum, multiply by beta / s_m, round to the output
// dtype (or store the exact int32 accumulator); long launches stage 2-byte
// output tiles through LDS for whole-row-segment stores.
// Workgroup ids are remapped so each of the 8 XCDs (which receive ids
// round-robin) works on a contiguous range of a banded column-major tile
// order, keeping the A rows and B columns of the tiles it runs together in
// that XCD's L2.  A grouped launch (gemm_mfma_group_kernel) runs up to three
// same-shape contractions as one tile sequence.
#include <algorithm>

#include "bl_common.h"
#include "bl_launch.h"

namespace bl {

// One k-block of 128: request k-block kb+2 (A into a_load, B into b0/b1
// once they are consumed), stage k-block kb+1 (a_store) into `next`, and
// multiply the A tile in `cur` (LDS) by the B codes in b0/b1.  Called twice per
// loop trip with the register sets swapped, so no register is ever copied
// (a copy would have to wait for its load and serialize the pipeline).
// Loads are buffer loads: a per-lane offset fixed for the whole loop plus a
// k-block offset in a scalar register, so no vector address arithmetic runs
// per k-block; rows and tiles past the matrix read as zero.
template <int MI, int TPW>
__device__ __forceinline__ void gemm_kblock(int kb, int KB, const uint8_t *cur, uint8_t *next,
                                            v4i (&acc)[MI][2 * TPW], v4i (&a_store)[MI],
                                            v4i (&a_load)[MI], v4i (&b)[TPW],
                                            rsrc_t ars, const int (&a_voff)[MI],
                                            const int (&a_dst)[MI], rsrc_t brs, int b_voff,
                                            int b_tile_bytes, int arow0, int lane) {
  const int k2 = min(kb + 2, KB - 1);  // the tail re-reads the last block (unused)
  // scheduling fences keep each k-block's work in its own slot: without
  // them the scheduler pulls the next block's unpack (and so its wait for
  // the B loads) forward, shortening the prefetch distance
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < MI; ++j)
    a_load[j] = __builtin_bit_cast(
        v4i, __builtin_amdgcn_raw_buffer_load_b128(ars, a_voff[j], k2 * 128, 0));
  __builtin_amdgcn_sched_barrier(0);
  v4i a[MI][2];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int row = arow0 + 16 * mi;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int ch = 2 * (lane >> 4) + s2;
      a[mi][s2] = *reinterpret_cast<const v4i *>(cur + row * 128 + (swz(row, ch) << 4));
    }
  }
  // Stage k-block kb+1 into `next` now: every wave finished reading that
  // buffer before the barrier that ended the previous k-block, and writing
  // it here takes the LDS write latency off the barrier below.
#pragma unroll
  for (int j = 0; j < MI; ++j) *reinterpret_cast<v4i *>(next + a_dst[j]) = a_store[j];
  // all 2*MI LDS reads go out before the first MFMA: left to itself the
  // scheduler reads two operands at a time and waits for each pair, which
  // exposes the LDS latency 2*MI/2 times per k-block
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      // word (h, s2) of a lane slot sits at dword 2h + s2: h = 0 is the
      // tile's first 16 rows (block 2t), h = 1 its last 16 (block 2t + 1)
      const v4i w0 = unpack_codes(s2 ? b[t].y : b[t].x);
      const v4i w1 = unpack_codes(s2 ? b[t].w : b[t].z);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        acc[mi][2 * t] = mfma16x16x64(a[mi][s2], w0, acc[mi][2 * t]);
        acc[mi][2 * t + 1] = mfma16x16x64(a[mi][s2], w1, acc[mi][2 * t + 1]);
      }
    }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    b[t] = __builtin_bit_cast(
        v4i, __builtin_amdgcn_raw_buffer_load_b128(brs, b_voff + t * b_tile_bytes, k2 * 1024, 0));
  __syncthreads();
}

constexpr int kBandRows = 4;  // tile rows per band of the tile order
constexpr int64_t kWideTiles = 768;  // 128 x 256 tiles from which a launch takes them

// Tile t of the XCD-aware order for workgroup `bid` of a launch of `ntiles`
// tiles: workgroup ids reach the 8 XCDs round-robin, so XCD x gets the
// contiguous range of the sequence that starts at x * ntiles / 8.
__device__ __forceinline__ int xcd_tile(int bid, int ntiles) {
  const int per = ntiles / 8, rem = ntiles % 8;
  const int xcd = bid % 8, local = bid / 8;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// One tile of one contraction.  t: the tile's place in the sequence of this
// contraction's tiles; work: tiles x k-blocks of the whole launch (picks the
// epilogue).  GLU: the packed rows are a gate_proj in GLU order (each 32-row
// tile = 16 gated rows + the 16 rows they multiply) and out is h [M, N/2].
template <int MI, int OUT, bool GLU, int TPW>
__device__ __forceinline__ void gemm_body(
    const int8_t *__restrict__ xq, const int32_t *__restrict__ rowsum,
    const float *__restrict__ s, const uint4 *__restrict__ packed,
    const float *__restrict__ beta, int M, int N, int K,
    void *__restrict__ out, int tiles_m, int tiles_n, int t, int work) {
  constexpr int BM = 32 * MI;
  constexpr int BN = 64 * TPW;  // a wave: 16 MI rows x 32 TPW outputs (TPW packed tiles)
  __shared__ __align__(16) uint8_t lds[2][BM * 128];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;

  // Inside the sequence, tiles go column by column through bands of
  // kBandRows tile rows, so the ~64 workgroups an XCD runs at once share a
  // few A row tiles and a few B column tiles (about 1 MiB each) in its L2
  // instead of sweeping every B column tile once per tile row.
  const int band = t / (kBandRows * tiles_n), r = t - band * kBandRows * tiles_n;
  const int rows_here = min(kBandRows, tiles_m - band * kBandRows);
  const int tm = band * kBandRows + r % rows_here, tn = r / rows_here;
  const int m0 = tm * BM, n0 = tn * BN;
  const int KB = K >> 7;
  const int NT = N >> 5;

  // ---- A tile: BM rows x 8 chunks of 16 B, MI chunks per thread; thread
  // chunk j covers row (tid + 256 j) / 8, chunk (tid + 256 j) % 8.  The
  // buffer covers the tile's rows that exist (rows past M read as zero and
  // their outputs are never stored).
  const rsrc_t ars = make_rsrc(xq + (int64_t)m0 * K, (uint32_t)(min(BM, M - m0) * K));
  int a_voff[MI], a_dst[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int c = tid + 256 * j;
    const int row = c >> 3, ch = c & 7;
    a_voff[j] = row * K + ch * 16;
    a_dst[j] = row * 128 + (swz(row, ch) << 4);
  }
  // ---- B: the wave's two packed 32-row tiles (tiles past N read as zero:
  // their columns are never stored).
  const int nt0 = (n0 >> 5) + TPW * wn;
  const int tile_bytes = KB * 1024;
  // (readfirstlane: tell the compiler these are wave-uniform, so the buffer
  // descriptor lives in scalar registers)
  const int b_first = __builtin_amdgcn_readfirstlane(min(nt0, NT));
  const int b_bytes = __builtin_amdgcn_readfirstlane(max(0, min(TPW, NT - nt0)) * tile_bytes);
  const rsrc_t brs = make_rsrc(packed + (int64_t)b_first * KB * 64, (uint32_t)b_bytes);
  const int b_voff = lane * 16;

  v4i acc[MI][2 * TPW];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int nb = 0; nb < 2 * TPW; ++nb) acc[mi][nb] = v4i{0, 0, 0, 0};

  // Prefetch distance 2: the A chunks and B tiles of k-block kb+2 are
  // requested while k-block kb is multiplied, so each load has about two
  // iterations of MFMA work to arrive; A goes through a double-buffered LDS
  // stage one iteration before use.  (Native int vectors, not uint4: struct
  // copies are lowered to memcpy through private memory.)
  v4i P[MI], Q[MI];     // A staging sets
  v4i X[TPW], Y[TPW];   // B of even / odd k-blocks
  {
    const int k1 = min(1, KB - 1);
#pragma unroll
    for (int j = 0; j < MI; ++j)
      Q[j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ars, a_voff[j], 0, 0));
#pragma unroll
    for (int j = 0; j < MI; ++j)
      P[j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ars, a_voff[j], k1 * 128, 0));
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      X[t] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(brs, b_voff + t * tile_bytes, 0, 0));
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      Y[t] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(brs, b_voff + t * tile_bytes, k1 * 1024, 0));
#pragma unroll
    for (int j = 0; j < MI; ++j) *reinterpret_cast<v4i *>(&lds[0][a_dst[j]]) = Q[j];
  }
  __syncthreads();

  const int arow0 = wm * 16 * MI + (lane & 15);
  // Both halves of a trip are unconditional: a conditional second half would
  // let the compiler sink the first half's prefetch loads into it.
  int kb = 0;
  for (; kb + 1 < KB; kb += 2) {
    gemm_kblock<MI, TPW>(kb, KB, lds[0], lds[1], acc, P, Q, X, ars, a_voff, a_dst, brs, b_voff,
                         tile_bytes, arow0, lane);
    gemm_kblock<MI, TPW>(kb + 1, KB, lds[1], lds[0], acc, Q, P, Y, ars, a_voff, a_dst, brs,
                         b_voff, tile_bytes, arow0, lane);
  }
  if (kb < KB)
    gemm_kblock<MI, TPW>(kb, KB, lds[0], lds[1], acc, P, Q, X, ars, a_voff, a_dst, brs, b_voff,
                         tile_bytes, arow0, lane);

  // ---- epilogue: lane holds rows 4*(lane/16)+i of each 16x16 block.  The
  // row sums and rescale factors of the wave's 16*MI rows go through a small
  // LDS table (lane l fetches row l; one division per lane), from which each
  // lane reads its four consecutive rows with one 16-byte read (the table is
  // the wave's own: a wavefront fence, no barrier).
  __shared__ __align__(16) int e_rs[4][64];
  __shared__ __align__(16) float e_sc[4][64];
  const int wrow0 = m0 + wm * 16 * MI;
  if (lane < 16 * MI) {
    const int mrow = min(wrow0 + lane, M - 1);
    e_rs[wave][lane] = rowsum[mrow];
    if constexpr (OUT != kOutI32) e_sc[wave][lane] = div_rn(*beta, s[mrow]);
  }
  wave_lds_sync();
  const int q4 = 4 * (lane >> 4);
  const int ncol0 = n0 + 32 * TPW * wn + (lane & 15);
  v4i rs4[MI];
  float sc4[MI][4];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    rs4[mi] = *reinterpret_cast<const v4i *>(&e_rs[wave][16 * mi + q4]);
    const v4i t = *reinterpret_cast<const v4i *>(&e_sc[wave][16 * mi + q4]);
#pragma unroll
    for (int i = 0; i < 4; ++i) sc4[mi][i] = __int_as_float(t[i]);
  }
  const auto put = [&](int mi, int i, int nb, int64_t idx) {
    const int v = acc[mi][nb][i] - rs4[mi][i];
    if constexpr (OUT == kOutI32)
      reinterpret_cast<int32_t *>(out)[idx] = v;
    else
      store1<OUT>(out, idx, (float)v * sc4[mi][i]);
  };
  if constexpr (GLU) {
    // tiles t0 and t0 + 1 of the wave: nb = 2p holds the gated rows of tile
    // t0 + p, nb = 2p + 1 the rows they multiply; output column 16 (t0 + p) + c
    const int t0 = (n0 >> 5) + TPW * wn;
    const int64_t F = N >> 1;
    const bool full = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wrow0 + 16 * mi + q4 + i;
        if (!full && m >= M) continue;
#pragma unroll
        for (int pr = 0; pr < TPW; ++pr) {
          if (!full && 32 * (t0 + pr) >= N) continue;
          const float yg = (float)(acc[mi][2 * pr][i] - rs4[mi][i]) * sc4[mi][i];
          const float yu = (float)(acc[mi][2 * pr + 1][i] - rs4[mi][i]) * sc4[mi][i];
          store1<OUT>(out, (int64_t)m * F + 16 * (t0 + pr) + (lane & 15), silu(yg) * yu);
        }
      }
    return;
  }
  if constexpr ((OUT == BL_F16 || OUT == BL_BF16) && TPW == 2) {
    // Whole tile of 2-byte outputs in a long launch: the wave's 16 MI x 64
    // block goes through the A buffers (idle since the barrier that ended
    // the last k-block), row-major with each row's 16-byte chunks XOR-
    // swizzled by (row / 4) mod 4 so the 2-byte writes are conflict-free,
    // and leaves as 16-byte stores covering whole 128-byte row segments:
    // 2 MI store instructions per wave instead of 16 MI.  In a launch whose
    // tiles all run at once the LDS round trip lengthens the tail that no
    // other tile overlaps, so short launches store directly (measured
    // threshold: tiles x k-blocks > 16384).
    if (m0 + BM <= M && n0 + BN <= N && work > 16384) {
      uint8_t *st = &lds[0][0] + wave * (16 * MI * 128);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * mi + q4 + i;
          const int sw = ((row >> 2) & 3) << 1;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int col = 16 * nb + (lane & 15);
            const float y = (float)(acc[mi][nb][i] - rs4[mi][i]) * sc4[mi][i];
            *reinterpret_cast<uint16_t *>(st + row * 128 + (((col >> 3) ^ sw) << 4) + (col & 7) * 2) =
                out_bits<OUT>(y);
          }
        }
      wave_lds_sync();
      const rsrc_t ors =
          make_rsrc(reinterpret_cast<uint16_t *>(out) + (int64_t)wrow0 * N + n0 + 64 * wn,
                    (uint32_t)((16 * MI - 1) * N + 64) * 2u);
#pragma unroll
      for (int r8 = 0; r8 < 2 * MI; ++r8) {
        const int row = 8 * r8 + (lane >> 3), chunk = lane & 7;
        const int sw = ((row >> 2) & 3) << 1;
        const v4i v = *reinterpret_cast<const v4i *>(st + row * 128 + ((chunk ^ sw) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), ors,
                                               (row * N + chunk * 8) * 2, 0, 0);
      }
      return;
    }
  }
  if (m0 + BM <= M && n0 + BN <= N) {
    // whole tile (all but the ragged edges): no per-element checks, one row
    // offset per (mi, i) and constant column offsets
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t rowbase = (int64_t)(wrow0 + 16 * mi + q4 + i) * N + ncol0;
#pragma unroll
        for (int nb = 0; nb < 2 * TPW; ++nb) put(mi, i, nb, rowbase + 16 * nb);
      }
  } else {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wrow0 + 16 * mi + q4 + i;
        if (m >= M) continue;
        const int64_t rowbase = (int64_t)m * N + ncol0;
#pragma unroll
        for (int nb = 0; nb < 2 * TPW; ++nb)
          if (ncol0 + 16 * nb < N) put(mi, i, nb, rowbase + 16 * nb);
      }
  }
}

template <int MI, int OUT, bool GLU, int TPW = 2>
__global__ __launch_bounds__(256, TPW == 2 ? 3 : 2) void gemm_mfma_kernel(
    const int8_t *__restrict__ xq, const int32_t *__restrict__ rowsum,
    const float *__restrict__ s, const uint4 *__restrict__ packed,
    const float *__restrict__ beta, int M, int N, int K,
    void *__restrict__ out, int tiles_m, int tiles_n) {
  const int ntiles = tiles_m * tiles_n;
  gemm_body<MI, OUT, GLU, TPW>(xq, rowsum, s, packed, beta, M, N, K, out, tiles_m, tiles_n,
                               xcd_tile((int)blockIdx.x, ntiles), ntiles * (K >> 7));
}

// Up to kGemmCalls contractions of one shape in one launch (HGRN's i/f/g at
// prefill): the tile sequence is call 0's tiles, then call 1's, ..., so a
// launch of three one-round contractions runs as several rounds whose
// epilogues overlap other tiles' main loops.  The pointers come from the
// argument buffer.
template <int MI, int OUT, int TPW = 2>
__global__ __launch_bounds__(256, TPW == 2 ? 3 : 2) void gemm_mfma_group_kernel(int ncalls, int M, int N, int K,
                                                                 int tiles_m, int tiles_n,
                                                                 GemmCalls calls) {
  const int ntiles = tiles_m * tiles_n;
  const int tg = xcd_tile((int)blockIdx.x, ncalls * ntiles);
  const int call = __builtin_amdgcn_readfirstlane(tg / ntiles);
  const GemmCall &c = calls.c[call];
  gemm_body<MI, OUT, false, TPW>(c.xq, c.rowsum, c.s, reinterpret_cast<const uint4 *>(c.packed), c.beta,
                            M, N, K, c.out, tiles_m, tiles_n, tg - call * ntiles,
                            ncalls * ntiles * (K >> 7));
}

template <int MI, int TPW = 2>
static hipError_t launch_mi(const int8_t *xq, const int32_t *rowsum,
                            const float *s, const void *packed,
                            const float *beta, int64_t M, int64_t N, int64_t K,
                            void *out, int out_kind, bool glu, hipStream_t stream) {
  const int BM = 32 * MI, BN = 64 * TPW;
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const unsigned grid = (unsigned)(tiles_m * tiles_n);
  const uint4 *pk = reinterpret_cast<const uint4 *>(packed);
#define BL_GEMM_CASE(KIND, G)                                                \
  gemm_mfma_kernel<MI, KIND, G, TPW><<<grid, 256, 0, stream>>>(              \
      xq, rowsum, s, pk, beta, (int)M, (int)N, (int)K, out, tiles_m, tiles_n)
  if (glu) {
    switch (out_kind) {
      case BL_F32: BL_GEMM_CASE(BL_F32, true); break;
      case BL_F16: BL_GEMM_CASE(BL_F16, true); break;
      default: BL_GEMM_CASE(BL_BF16, true); break;
    }
  } else {
    switch (out_kind) {
      case BL_F32: BL_GEMM_CASE(BL_F32, false); break;
      case BL_F16: BL_GEMM_CASE(BL_F16, false); break;
      case BL_BF16: BL_GEMM_CASE(BL_BF16, false); break;
      default: BL_GEMM_CASE(kOutI32, false); break;
    }
  }
#undef BL_GEMM_CASE
  return hipGetLastError();
}

// Tile height among 128 and 96 rows (32 MI, MI = 4 or 3) for a launch of
// t128 resp. t96 tiles of either: the CUs take the tiles in turn, so the
// busiest one runs ceil(tiles / 256) of them, and the height with fewer
// rows on it wins.  96 rows win where 128-row tiles leave half the CUs a
// tile short (M = 3072, N = 2048: 384 tiles of 128 rows against 512 of 96,
// two per CU: 18.5 -> 16.1 us; M = 3000, K = 5632: 38.2 -> 33.8 us); a tie
// keeps 128 rows, whose unpacked weight operands feed four MFMAs instead of
// three (M = 4096, N = 2048: 512 tiles, two per CU, against 688 of 96 rows:
// 20.6 vs 21.6 us).
constexpr int64_t kCUs = 256;
constexpr int tall_mi(int64_t t128, int64_t t96) {
  return ((t96 + kCUs - 1) / kCUs) * 3 < ((t128 + kCUs - 1) / kCUs) * 4 ? 3 : 4;
}

hipError_t launch_gemm_mfma(const int8_t *xq, const int32_t *rowsum,
                            const float *s, const void *packed,
                            const float *beta, int64_t M, int64_t N,
                            int64_t K, void *out, int out_kind, bool glu,
                            hipStream_t stream) {
  // The tallest tile that still gives every CU a workgroup: 128-row tiles
  // reuse each unpacked weight operand four times, but below one tile per
  // CU the idle CUs cost more than the extra unpacking of shorter tiles
  // (measured at M = 512: 32-row tiles beat 64-row ones up to 256 tiles).
  const int64_t tn = (N + 127) / 128;
  const auto tiles = [&](int64_t bm) { return ((M + bm - 1) / bm) * tn; };
  // Wide launches: 128 x 256 tiles, a wave holding 4 packed tiles, so each
  // A operand read from LDS feeds twice the MFMAs (2 waves per SIMD: 246
  // VGPRs).  From 768 such tiles (gate_proj at M = 4096: 87 -> 84 us, at
  // M = 8192: 254 -> 238 us; i/f/g grouped at M = 4096: 51 -> 49 us); with
  // fewer, the tiles do not fill the rounds (2048-wide projections at M =
  // 4096: 20.4 -> 22.7 us, 2560-wide at M = 8192: 49 -> 52 us) and 128 x 128
  // stays.
  if (M > 64 && ((M + 127) / 128) * ((N + 255) / 256) >= kWideTiles)
    return launch_mi<4, 4>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, glu, stream);
  if (M > 64 && tiles(128) >= 256)
    return tall_mi(tiles(128), tiles(96)) == 3
               ? launch_mi<3>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, glu, stream)
               : launch_mi<4>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, glu, stream);
  if (M > 32 && tiles(64) >= 256)
    return launch_mi<2>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, glu, stream);
  return launch_mi<1>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, glu, stream);
}

template <int MI, int TPW = 2>
static hipError_t launch_group_mi(const GemmCalls &calls, int ncalls, int64_t M, int64_t N,
                                  int64_t K, int out_kind, hipStream_t stream) {
  const int BM = 32 * MI, BN = 64 * TPW;
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const unsigned grid = (unsigned)(tiles_m * tiles_n * ncalls);
#define BL_GEMMG_CASE(KIND)                                                     \
  gemm_mfma_group_kernel<MI, KIND, TPW><<<grid, 256, 0, stream>>>(ncalls, (int)M, (int)N, (int)K, \
                                                             tiles_m, tiles_n, calls)
  switch (out_kind) {
    case BL_F32: BL_GEMMG_CASE(BL_F32); break;
    case BL_F16: BL_GEMMG_CASE(BL_F16); break;
    default: BL_GEMMG_CASE(BL_BF16); break;
  }
#undef BL_GEMMG_CASE
  return hipGetLastError();
}

hipError_t launch_gemm_mfma_group(const GemmCalls &calls, int ncalls, int64_t M, int64_t N,
                                  int64_t K, int out_kind, hipStream_t stream) {
  // tile height as for one call, over the tiles of all the calls
  const int64_t tn = (N + 127) / 128;
  const auto tiles = [&](int64_t bm) { return ((M + bm - 1) / bm) * tn * ncalls; };
  if (M > 64 && ((M + 127) / 128) * ((N + 255) / 256) * ncalls >= kWideTiles)
    return launch_group_mi<4, 4>(calls, ncalls, M, N, K, out_kind, stream);
  if (M > 64 && tiles(128) >= 256)
    return tall_mi(tiles(128), tiles(96)) == 3
               ? launch_group_mi<3>(calls, ncalls, M, N, K, out_kind, stream)
               : launch_group_mi<4>(calls, ncalls, M, N, K, out_kind, stream);
  if (M > 32 && tiles(64) >= 256) return launch_group_mi<2>(calls, ncalls, M, N, K, out_kind, stream);
  return launch_group_mi<1>(calls, ncalls, M, N, K, out_kind, stream);
}

}  // namespace bl
