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
// Workgroup tile: BM = 32*MI token rows x BN = 128 (or 256) output rows, K
// in blocks of 128 (one packed tile column).  4 waves, either side by side
// over all the tile's rows, each owning one (or, in 256-wide tiles, two)
// packed 32-row tiles -- so every code word is unpacked once per workgroup
// -- or, for the 96- and 128-row tiles 128 wide, as 2 x 2 waves of 16*MI
// rows x two packed tiles each.
//   A (xq): global -> LDS (straight, by the buffer->LDS load, or through
//           registers), 16-byte chunks of a 128-byte row XOR-swizzled (swz)
//           so the lanes that read one column of chunks hit distinct banks.
//   B (packed codes): each wave loads its 1 KiB tiles per k-block straight
//           into registers (one 16-byte load per lane per tile, the layout
//           was built for exactly this) and unpacks them with shift + mask;
//           no LDS traffic for weights.
//   Loads run two (A) or three (B) k-blocks ahead of the MFMAs.
// Epilogue: subtract rowsum, multiply by beta / s_m, round to the output
// dtype (or store the exact int32 accumulator); long launches stage 2-byte
// output tiles through LDS for whole-row-segment stores.
// Launches with few tiles split K inside the workgroup: KG groups of 4
// waves (KG = 2 or 4) each run the whole tile over a contiguous range of
// k-blocks with their own A stage, then the groups' int32 accumulators are
// added through LDS into group 0, which runs the epilogue.  Integer sums do
// not depend on the order, so the result is the same bits; the serial chain
// of k-blocks per wave (the latency that bounds a one-round launch) shrinks
// KG-fold and each CU holds KG times the waves.
// Workgroup ids are remapped so each of the 8 XCDs (which receive ids
// round-robin) works on a contiguous range of a banded column-major tile
// order, keeping the A rows and B columns of the tiles it runs together in
// that XCD's L2.  A grouped launch (gemm_mfma_group_kernel) runs up to three
// same-shape contractions as one tile sequence.
#include <algorithm>
#include <type_traits>

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
// kb: the k-block multiplied now; kend: one past the last k-block of this
// wave's range (loads clamp to it, k-blocks at or past it are trips that
// only keep the barriers in step with the other groups: CHECK = KG > 1).
template <int MI, int WR, int TPW, bool CHECK>
__device__ __forceinline__ void gemm_kblock(int kb, int kend, const uint8_t *cur, uint8_t *next,
                                            v4i (&acc)[WR][2 * TPW], v4i (&a_store)[MI],
                                            v4i (&a_load)[MI], v4i (&b)[TPW],
                                            rsrc_t ars, const int (&a_voff)[MI],
                                            const int (&a_dst)[MI], rsrc_t brs, int b_voff,
                                            int b_tile_bytes, int arow0, int lane) {
  const int k2 = min(kb + 2, kend - 1);  // the tail re-reads the last block (unused)
  // scheduling fences keep each k-block's work in its own slot: without
  // them the scheduler pulls the next block's unpack (and so its wait for
  // the B loads) forward, shortening the prefetch distance
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < MI; ++j)
    a_load[j] = __builtin_bit_cast(
        v4i, __builtin_amdgcn_raw_buffer_load_b128(ars, a_voff[j], k2 * 128, 0));
  __builtin_amdgcn_sched_barrier(0);
  v4i a[WR][2];
#pragma unroll
  for (int mi = 0; mi < WR; ++mi) {
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
  if (!CHECK || kb < kend) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      // word (h, s2) of a lane slot sits at dword 2h + s2: h = 0 is the
      // tile's first 16 rows (block 2t), h = 1 its last 16 (block 2t + 1)
      v4i w[2][2];
      unpack_pair(b[t].x, b[t].y, w[0][0], w[1][0]);
      unpack_pair(b[t].z, b[t].w, w[0][1], w[1][1]);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int mi = 0; mi < WR; ++mi) {
          acc[mi][2 * t] = mfma16x16x64(a[mi][s2], w[s2][0], acc[mi][2 * t]);
          acc[mi][2 * t + 1] = mfma16x16x64(a[mi][s2], w[s2][1], acc[mi][2 * t + 1]);
        }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    b[t] = __builtin_bit_cast(
        v4i, __builtin_amdgcn_raw_buffer_load_b128(brs, b_voff + t * b_tile_bytes, k2 * 1024, 0));
  __syncthreads();
}

// 16 bytes per lane from a buffer straight into LDS: lane L's bytes land at
// lds + 16 L (lds is wave-uniform, taken through M0).  Kept out of the
// templates: the host pass of the compiler rejects the LDS address-space
// cast inside a template instantiation.
__device__ __forceinline__ void lds_load16(rsrc_t r, uint8_t *lds, int voffset, int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void *)lds, 16, voffset, soffset, 0, 0);
}

// The k-block body of launches without K groups: A goes from global memory
// straight into LDS (the 16-byte buffer->LDS load; lane L writes the 16
// bytes at base + 16 L) through a ring of three stages, two k-blocks ahead,
// so no registers stage it; the weights come three k-blocks ahead through
// three register sets.  At k-block kb: request A(kb+2) into stage
// (kb+2) mod 3 (last read at kb-1, before the barrier that ended it), read
// A(kb) from stage kb mod 3, multiply by the codes in bc (then reloaded with
// k-block kb+3), and before the closing barrier wait only for A(kb+1) --
// the loads issued after it (B(kb+2), A(kb+2), B(kb+3)) stay in flight.
// The barrier is a plain s_barrier: a workgroup fence would also wait for
// every load still in flight.
template <int MI, int WR, int TPW, bool TAIL>
__device__ __forceinline__ void gemm_kblock_dma(int kb, int kend, const uint8_t *cur,
                                                uint8_t *dst, v4i (&acc)[WR][2 * TPW],
                                                v4i (&bc)[TPW], rsrc_t ars,
                                                const int (&a_dma)[MI], int a_lds0, rsrc_t brs,
                                                int b_voff, int b_tile_bytes, int arow0, int lane) {
  const int k2 = min(kb + 2, kend - 1), k3 = min(kb + 3, kend - 1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < MI; ++j)
    lds_load16(ars, dst + a_lds0 + 32 * 128 * j, a_dma[j], k2 * 128);
  __builtin_amdgcn_sched_barrier(0);
  v4i a[WR][2];
#pragma unroll
  for (int mi = 0; mi < WR; ++mi) {
    const int row = arow0 + 16 * mi;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int ch = 2 * (lane >> 4) + s2;
      a[mi][s2] = *reinterpret_cast<const v4i *>(cur + row * 128 + (swz(row, ch) << 4));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    v4i w[2][2];
    unpack_pair(bc[t].x, bc[t].y, w[0][0], w[1][0]);
    unpack_pair(bc[t].z, bc[t].w, w[0][1], w[1][1]);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int mi = 0; mi < WR; ++mi) {
        acc[mi][2 * t] = mfma16x16x64(a[mi][s2], w[s2][0], acc[mi][2 * t]);
        acc[mi][2 * t + 1] = mfma16x16x64(a[mi][s2], w[s2][1], acc[mi][2 * t + 1]);
      }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!TAIL) {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      bc[t] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(brs, b_voff + t * b_tile_bytes, k3 * 1024, 0));
  }
  __builtin_amdgcn_sched_barrier(0);
  // A(kb+1) has landed when at most B(kb+2), A(kb+2) and B(kb+3) remain.
  // The count holds only where all three are issued, i.e. inside the loop,
  // whose code loads are all live; in the last k-blocks the compiler may
  // drop or move the code loads, and only A(kb+2) is sure to follow A(kb+1).
  constexpr int kAfter = TAIL ? MI : 2 * TPW + MI;
  static_assert(kAfter < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(kAfter | (7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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
// KG: groups of 4 waves splitting K (256 KG threads).
template <int MI, int OUT, bool GLU, int TPW, int KG>
__device__ __forceinline__ void gemm_body(
    const int8_t *__restrict__ xq, const int32_t *__restrict__ rowsum,
    const float *__restrict__ s, const uint4 *__restrict__ packed,
    const float *__restrict__ beta, int M, int N, int K,
    void *__restrict__ out, int tiles_m, int tiles_n, int t, int work) {
  // Waves: WM x WN over the tile, each 16 WR rows x 32 TW outputs (TW
  // packed tiles).  TPW = 2 (128 x 128 tiles): 2 x 2 waves of two tiles,
  // WR = MI.  TPW = 1 (32- and 64-row tiles) and TPW = 4 (128 x 256 tiles):
  // 1 x 4 waves side by side, each over all the tile's rows and one resp.
  // two packed tiles, WR = 2 MI: every code word is unpacked by one wave
  // instead of two, for twice the LDS reads of A.  The unpack is VALU work
  // beside the MFMAs, and halving it measured faster wherever the LDS keeps
  // up: the 32- and 64-row tiles (M = 128..1024, 9-18 %) and the 128 x 256
  // tiles (2.7B prefill launches at M = 8192 2.3 %, the 1.3B layer at
  // M = 4096 1.9 %, on top of the paired unpack).
  constexpr bool SIDE = TPW == 1 || TPW == 4;  // waves side by side (1 x 4)
  constexpr int TW = TPW == 4 ? 2 : TPW;        // packed tiles per wave
  constexpr int WN = SIDE ? 4 : 2;
  constexpr int WR = SIDE ? 2 * MI : MI;
  constexpr int BM = 32 * MI;
  constexpr int BN = 32 * TW * WN;
  static_assert(KG == 1 || KG == 2 || KG == 4, "K groups");
  static_assert(KG == 1 || TPW <= 2, "the K-group reduction fits 1- and 2-tile waves only");
  static_assert(16 * WR <= 128, "the epilogue's row table holds 128 rows per wave");
  // A stages: 2 per K group (filled through registers), or without K groups
  // a ring of 3 filled by buffer->LDS loads and kept as three separate
  // arrays: the compiler tells LDS objects apart, not offsets inside one,
  // so a read of one stage does not wait for the loads into another
  constexpr int NST = KG == 1 ? 1 : 2;
  __shared__ __align__(16) uint8_t lds[KG][NST][BM * 128];
  __shared__ __align__(16) uint8_t lds_r1[KG == 1 ? BM * 128 : 16];
  __shared__ __align__(16) uint8_t lds_r2[KG == 1 ? BM * 128 : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int kg = KG == 1 ? 0 : wave >> 2;                    // K group
  const int wq = wave & 3;                                    // wave in its group
  const int gtid = tid & 255;                                 // thread in its group
  const int wm = wq / WN, wn = wq % WN;

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
  // this group's k-blocks [kb0, kend); every group runs `trips` k-blocks so
  // the barriers stay in step (the surplus trips multiply nothing)
  const int trips = KG == 1 ? KB : (KB + KG - 1) / KG;
  const int kb0 = KG == 1 ? 0 : min(kg * trips, KB);
  const int kend = KG == 1 ? KB : min(KB, kb0 + trips);
  const int klast = max(kend - 1, 0);

  // ---- A tile: BM rows x 8 chunks of 16 B, MI chunks per thread; thread
  // chunk j covers row (tid + 256 j) / 8, chunk (tid + 256 j) % 8.  The
  // buffer covers the tile's rows that exist (rows past M read as zero and
  // their outputs are never stored).
  const rsrc_t ars = make_rsrc(xq + (int64_t)m0 * K, (uint32_t)(min(BM, M - m0) * K));
  int a_voff[MI], a_dst[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int c = gtid + 256 * j;
    const int row = c >> 3, ch = c & 7;
    a_voff[j] = row * K + ch * 16;
    a_dst[j] = row * 128 + (swz(row, ch) << 4);
  }
  // ---- B: the wave's TW packed 32-row tiles (tiles past N read as zero:
  // their columns are never stored).
  const int nt0 = (n0 >> 5) + TW * wn;
  const int tile_bytes = KB * 1024;
  // (readfirstlane: tell the compiler these are wave-uniform, so the buffer
  // descriptor lives in scalar registers)
  const int b_first = __builtin_amdgcn_readfirstlane(min(nt0, NT));
  const int b_bytes = __builtin_amdgcn_readfirstlane(max(0, min(TW, NT - nt0)) * tile_bytes);
  const rsrc_t brs = make_rsrc(packed + (int64_t)b_first * KB * 64, (uint32_t)b_bytes);
  const int b_voff = lane * 16;

  v4i acc[WR][2 * TW];
#pragma unroll
  for (int mi = 0; mi < WR; ++mi)
#pragma unroll
    for (int nb = 0; nb < 2 * TW; ++nb) acc[mi][nb] = v4i{0, 0, 0, 0};

  // Without K groups A is loaded straight into a ring of three LDS stages,
  // two k-blocks ahead, and the codes three k-blocks ahead (gemm_kblock_dma;
  // measured 3-5 % faster on the prefill shapes than staging A through
  // registers).  With K groups (where the LDS holds two stages per group)
  // prefetch distance 2: the A chunks and B tiles of k-block kb+2 are
  // requested while k-block kb is multiplied, and A goes through a double-
  // buffered LDS stage one iteration before use.  (Native int vectors, not
  // uint4: struct copies are lowered to memcpy through private memory.)
  const int arow0 = wm * 16 * WR + (lane & 15);
  const int kstop = kb0 + trips;
  int kb = kb0;
  if constexpr (KG == 1) {
    // wave wq fills rows 8 wq + 32 j .. +7 of a stage (1 KiB per load):
    // lane L lands at row 8 wq + 32 j + L / 8, 16-byte slot L % 8, so it
    // fetches the row's chunk that the swizzle puts in that slot
    int a_dma[MI];
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      const int row = 8 * wq + 32 * j + (lane >> 3);
      const int ch = swz(row, lane & 7);  // the swizzle is an involution
      a_dma[j] = row * K + ch * 16;
    }
    const int a_lds0 = 8 * wq * 128;
    uint8_t *const s0 = lds[0][0];
    uint8_t *const s1 = lds_r1;
    uint8_t *const s2 = lds_r2;
    v4i U[TW], V[TW], W[TW];  // codes of k-blocks = 0, 1, 2 mod 3
    {
      // issued in the loop's own order (B(0), A(0), B(1), A(1), B(2)), so
      // the compiler's wait counts at the loop head match the steady state
      const int k1 = __builtin_amdgcn_readfirstlane(min(1, klast));
      const int k2 = __builtin_amdgcn_readfirstlane(min(2, klast));
      const auto load_b = [&](v4i(&b)[TW], int k) {
#pragma unroll
        for (int t = 0; t < TW; ++t)
          b[t] = __builtin_bit_cast(
              v4i, __builtin_amdgcn_raw_buffer_load_b128(brs, b_voff + t * tile_bytes, k * 1024, 0));
      };
      const auto load_a = [&](uint8_t *stage, int k) {
#pragma unroll
        for (int j = 0; j < MI; ++j)
          lds_load16(ars, stage + a_lds0 + 32 * 128 * j, a_dma[j], k * 128);
      };
      load_b(U, 0);
      __builtin_amdgcn_sched_barrier(0);
      load_a(s0, 0);
      __builtin_amdgcn_sched_barrier(0);
      load_b(V, k1);
      __builtin_amdgcn_sched_barrier(0);
      load_a(s1, k1);
      __builtin_amdgcn_sched_barrier(0);
      load_b(W, k2);
      __builtin_amdgcn_sched_barrier(0);
      // A(0) has landed when at most A(1) remains (the code loads may be
      // moved past this point by the compiler: only A(1) is sure to follow
      // A(0)); the kernel-argument loads are drained too, so no wait on
      // them lingers into the loop
      __builtin_amdgcn_s_waitcnt(MI | (7 << 4) | (0 << 8));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    for (; kb + 2 < kstop; kb += 3) {
      gemm_kblock_dma<MI, WR, TW, false>(kb, kend, s0, s2, acc, U, ars, a_dma, a_lds0, brs, b_voff,
                               tile_bytes, arow0, lane);
      gemm_kblock_dma<MI, WR, TW, false>(kb + 1, kend, s1, s0, acc, V, ars, a_dma, a_lds0, brs, b_voff,
                               tile_bytes, arow0, lane);
      gemm_kblock_dma<MI, WR, TW, false>(kb + 2, kend, s2, s1, acc, W, ars, a_dma, a_lds0, brs, b_voff,
                               tile_bytes, arow0, lane);
    }
    if (kb < kstop)
      gemm_kblock_dma<MI, WR, TW, true>(kb, kend, s0, s2, acc, U, ars, a_dma, a_lds0, brs, b_voff,
                               tile_bytes, arow0, lane);
    if (kb + 1 < kstop)
      gemm_kblock_dma<MI, WR, TW, true>(kb + 1, kend, s1, s0, acc, V, ars, a_dma, a_lds0, brs, b_voff,
                               tile_bytes, arow0, lane);
    // the loads of the last k-blocks (clamped repeats) may still be writing
    // the stages: drain them before the epilogue reuses the LDS
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (0xF << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  } else {
  v4i P[MI], Q[MI];     // A staging sets
  v4i X[TW], Y[TW];   // B of even / odd k-blocks
  uint8_t *const st0 = lds[kg][0];
  uint8_t *const st1 = lds[kg][1];
  {
    const int k0 = min(kb0, klast), k1 = min(kb0 + 1, klast);
#pragma unroll
    for (int j = 0; j < MI; ++j)
      Q[j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ars, a_voff[j], k0 * 128, 0));
#pragma unroll
    for (int j = 0; j < MI; ++j)
      P[j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ars, a_voff[j], k1 * 128, 0));
#pragma unroll
    for (int t = 0; t < TW; ++t)
      X[t] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(brs, b_voff + t * tile_bytes, k0 * 1024, 0));
#pragma unroll
    for (int t = 0; t < TW; ++t)
      Y[t] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(brs, b_voff + t * tile_bytes, k1 * 1024, 0));
#pragma unroll
    for (int j = 0; j < MI; ++j) *reinterpret_cast<v4i *>(st0 + a_dst[j]) = Q[j];
  }
  __syncthreads();

  // Both halves of a trip are unconditional: a conditional second half would
  // let the compiler sink the first half's prefetch loads into it.
  constexpr bool CHECK = KG > 1;
  for (; kb + 1 < kstop; kb += 2) {
    gemm_kblock<MI, WR, TW, CHECK>(kb, kend, st0, st1, acc, P, Q, X, ars, a_voff, a_dst, brs, b_voff,
                                tile_bytes, arow0, lane);
    gemm_kblock<MI, WR, TW, CHECK>(kb + 1, kend, st1, st0, acc, Q, P, Y, ars, a_voff, a_dst, brs,
                                b_voff, tile_bytes, arow0, lane);
  }
  if (kb < kstop)
    gemm_kblock<MI, WR, TW, CHECK>(kb, kend, st0, st1, acc, P, Q, X, ars, a_voff, a_dst, brs, b_voff,
                                tile_bytes, arow0, lane);
  }

  if constexpr (KG > 1) {
    // Add the groups' accumulators into group 0 through the A stages (free:
    // the last k-block ended with a barrier).  A slot holds one group's
    // accumulators, lane-contiguous per register; KG = 4 uses two slots and
    // a two-level tree (2 -> 0 and 3 -> 1, then 1 -> 0).  Every wave passes
    // every barrier.
    constexpr int NREG = WR * 2 * TW;
    static_assert(KG * NST * BM * 128 >= (KG / 2) * 4 * NREG * 64 * 16, "reduction slots fit");
    v4i *const red = reinterpret_cast<v4i *>(&lds[0][0][0]);
    const auto slot = [&](int gs, int mi, int nb) -> v4i * {
      return red + ((gs * 4 + wq) * NREG + mi * 2 * TW + nb) * 64 + lane;
    };
    const auto put_acc = [&](int gs) {
#pragma unroll
      for (int mi = 0; mi < WR; ++mi)
#pragma unroll
        for (int nb = 0; nb < 2 * TW; ++nb) *slot(gs, mi, nb) = acc[mi][nb];
    };
    const auto add_acc = [&](int gs) {
#pragma unroll
      for (int mi = 0; mi < WR; ++mi)
#pragma unroll
        for (int nb = 0; nb < 2 * TW; ++nb) acc[mi][nb] += *slot(gs, mi, nb);
    };
    if constexpr (KG == 2) {
      if (kg == 1) put_acc(0);
      __syncthreads();
      if (kg == 1) return;
      add_acc(0);
    } else {
      if (kg >= 2) put_acc(kg - 2);
      __syncthreads();
      if (kg < 2) add_acc(kg);
      __syncthreads();
      if (kg == 1) put_acc(0);
      __syncthreads();
      if (kg != 0) return;
      add_acc(0);
    }
  }

  // ---- epilogue: lane holds rows 4*(lane/16)+i of each 16x16 block.  The
  // row sums and rescale factors of the wave's 16*WR rows go through a small
  // LDS table (lane l fetches row l; one division per lane), from which each
  // lane reads its four consecutive rows with one 16-byte read (the table is
  // the wave's own: a wavefront fence, no barrier).
  constexpr int ER = 16 * WR < 64 ? 64 : 16 * WR;
  __shared__ __align__(16) int e_rs[4][ER];
  __shared__ __align__(16) float e_sc[4][ER];
  const int wrow0 = m0 + wm * 16 * WR;
#pragma unroll
  for (int r0 = 0; r0 < 16 * WR; r0 += 64) {
    const int r = r0 + lane;
    if (r < 16 * WR) {
      const int mrow = min(wrow0 + r, M - 1);
      e_rs[wq][r] = rowsum[mrow];
      if constexpr (OUT != kOutI32) e_sc[wq][r] = div_rn(*beta, s[mrow]);
    }
  }
  wave_lds_sync();
  const int q4 = 4 * (lane >> 4);
  const int ncol0 = n0 + 32 * TW * wn + (lane & 15);
  v4i rs4[WR];
  float sc4[WR][4];
#pragma unroll
  for (int mi = 0; mi < WR; ++mi) {
    rs4[mi] = *reinterpret_cast<const v4i *>(&e_rs[wq][16 * mi + q4]);
    const v4i t = *reinterpret_cast<const v4i *>(&e_sc[wq][16 * mi + q4]);
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
    const int t0 = (n0 >> 5) + TW * wn;
    const int64_t F = N >> 1;
    const bool full = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
    for (int mi = 0; mi < WR; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wrow0 + 16 * mi + q4 + i;
        if (!full && m >= M) continue;
#pragma unroll
        for (int pr = 0; pr < TW; ++pr) {
          if (!full && 32 * (t0 + pr) >= N) continue;
          const float yg = (float)(acc[mi][2 * pr][i] - rs4[mi][i]) * sc4[mi][i];
          const float yu = (float)(acc[mi][2 * pr + 1][i] - rs4[mi][i]) * sc4[mi][i];
          store1<OUT>(out, (int64_t)m * F + 16 * (t0 + pr) + (lane & 15), silu(yg) * yu);
        }
      }
    return;
  }
  if constexpr ((OUT == BL_F16 || OUT == BL_BF16) && TPW == 2 && KG == 1) {
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
      uint8_t *st = (wq < 2 ? &lds[0][0][0] : lds_r1) + (wq & 1) * (16 * MI * 128);
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
    for (int mi = 0; mi < WR; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t rowbase = (int64_t)(wrow0 + 16 * mi + q4 + i) * N + ncol0;
#pragma unroll
        for (int nb = 0; nb < 2 * TW; ++nb) put(mi, i, nb, rowbase + 16 * nb);
      }
  } else {
#pragma unroll
    for (int mi = 0; mi < WR; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wrow0 + 16 * mi + q4 + i;
        if (m >= M) continue;
        const int64_t rowbase = (int64_t)m * N + ncol0;
#pragma unroll
        for (int nb = 0; nb < 2 * TW; ++nb)
          if (ncol0 + 16 * nb < N) put(mi, i, nb, rowbase + 16 * nb);
      }
  }
}

// workgroups per CU the register budget is set for
constexpr int gemm_occupancy(int TPW, int KG) { return TPW == 4 ? 2 : KG == 1 ? 3 : KG == 2 ? 2 : 1; }

template <int MI, int OUT, bool GLU, int TPW = 2, int KG = 1>
__global__ __launch_bounds__(256 * KG, gemm_occupancy(TPW, KG)) void gemm_mfma_kernel(
    const int8_t *__restrict__ xq, const int32_t *__restrict__ rowsum,
    const float *__restrict__ s, const uint4 *__restrict__ packed,
    const float *__restrict__ beta, int M, int N, int K,
    void *__restrict__ out, int tiles_m, int tiles_n) {
  const int ntiles = tiles_m * tiles_n;
  gemm_body<MI, OUT, GLU, TPW, KG>(xq, rowsum, s, packed, beta, M, N, K, out, tiles_m, tiles_n,
                                   xcd_tile((int)blockIdx.x, ntiles), ntiles * (K >> 7));
}

// Up to kGemmCalls contractions of one shape in one launch (HGRN's i/f/g at
// prefill): the tile sequence is call 0's tiles, then call 1's, ..., so a
// launch of three one-round contractions runs as several rounds whose
// epilogues overlap other tiles' main loops.  The pointers come from the
// argument buffer.
template <int MI, int OUT, int TPW = 2, int KG = 1>
__global__ __launch_bounds__(256 * KG, gemm_occupancy(TPW, KG)) void gemm_mfma_group_kernel(
    int ncalls, int M, int N, int K, int tiles_m, int tiles_n, GemmCalls calls) {
  const int ntiles = tiles_m * tiles_n;
  const int tg = xcd_tile((int)blockIdx.x, ncalls * ntiles);
  const int call = __builtin_amdgcn_readfirstlane(tg / ntiles);
  const GemmCall &c = calls.c[call];
  gemm_body<MI, OUT, false, TPW, KG>(c.xq, c.rowsum, c.s, reinterpret_cast<const uint4 *>(c.packed),
                                     c.beta, M, N, K, c.out, tiles_m, tiles_n, tg - call * ntiles,
                                     ncalls * ntiles * (K >> 7));
}

template <int MI, int TPW = 2, int KG = 1>
static hipError_t launch_mi(const int8_t *xq, const int32_t *rowsum,
                            const float *s, const void *packed,
                            const float *beta, int64_t M, int64_t N, int64_t K,
                            void *out, int out_kind, bool glu, hipStream_t stream) {
  const int BM = 32 * MI, BN = TPW == 1 ? 128 : 64 * TPW;
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const unsigned grid = (unsigned)(tiles_m * tiles_n);
  const uint4 *pk = reinterpret_cast<const uint4 *>(packed);
#define BL_GEMM_CASE(KIND, G)                                                \
  gemm_mfma_kernel<MI, KIND, G, TPW, KG><<<grid, 256 * KG, 0, stream>>>(     \
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
// Packed tiles per wave of the 32- and 64-row tiles: one, the waves side by
// side over the tile's rows (1 x 4), so each code word is unpacked once per
// workgroup instead of twice.  Those k-blocks have few MFMAs per unpacked
// word, and halving the unpacking measured 9-18 % faster at M = 128..1024
// on the 2.7B and 1.3B projections (o_proj at M = 512: 9.7 -> 8.3 us,
// down_proj 19.9 -> 16.3, i/f/g grouped 13.5 -> 12.2; c5 M = 512 +6.7 %)
// than 2 x 2 waves of two tiles.
constexpr int kShortTpw = 1;
constexpr int tall_mi(int64_t t128, int64_t t96) {
  return ((t96 + kCUs - 1) / kCUs) * 3 < ((t128 + kCUs - 1) / kCUs) * 4 ? 3 : 4;
}

// K groups per workgroup for a launch of `tiles` workgroups of 32 MI rows
// over KB k-blocks of 128.  A split pays only while the launch leaves a CU
// about one workgroup (its waves then wait on every k-block's loads): up to
// one tile per CU, 4 groups from 8 k-blocks per group, else 2 groups from
// 4.  Past one tile per CU the unsplit waves already overlap each other's
// loads and a split only adds the reduction.  Measured on 2.7B and 1.3B
// shapes with the 1 x 4 wave layout (us, K groups 1 / 2 / 4): M = 128
// down_proj (KB = 55, 80 tiles) 14.0 / 12.1 / 10.2, o_proj (KB = 20) 6.4 /
// 6.0 / 6.2; M = 512 1.3B down_proj (KB = 44, 256 tiles) 11.2 / 10.0 / 9.2,
// 1.3B o_proj (KB = 16) 5.8 / 5.9 / 6.0; M = 512 o_proj (320 tiles) 7.6 /
// 8.1 / 9.1; M = 1024 o_proj (320 tiles of 64 rows) 10.2 / 12.1 / 15.9,
// down_proj 22.2 / 25.6 / 29.0; M = 256 gate_proj (440 tiles) 12.8 / 13.9
// / 17.9.  Taller tiles (MI >= 3) never split.
constexpr int k_groups(int64_t tiles, int64_t KB, int MI) {
  return MI > 2 || tiles > kCUs ? 1 : KB >= 32 ? 4 : KB >= 8 ? 2 : 1;
}

template <int MI>
static hipError_t launch_mi_kg(int kg, const int8_t *xq, const int32_t *rowsum, const float *s,
                               const void *packed, const float *beta, int64_t M, int64_t N,
                               int64_t K, void *out, int out_kind, bool glu, hipStream_t stream) {
  constexpr int TP = MI <= 2 ? kShortTpw : 2;
  if constexpr (MI <= 2) {
    if (kg == 4)
      return launch_mi<MI, TP, 4>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, glu, stream);
    if (kg == 2)
      return launch_mi<MI, TP, 2>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, glu, stream);
  }
  return launch_mi<MI, TP, 1>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, glu, stream);
}

hipError_t launch_gemm_mfma(const int8_t *xq, const int32_t *rowsum,
                            const float *s, const void *packed,
                            const float *beta, int64_t M, int64_t N,
                            int64_t K, void *out, int out_kind, bool glu,
                            hipStream_t stream) {
  // 128-row tiles reuse each unpacked weight operand four times, but with
  // fewer than two of them per CU the rounds run part-empty and 64-row
  // tiles (waves side by side, each code unpacked once) win: at 256..511
  // 128-row tiles, o_proj 2048 x 2048 at M = 2048 12.2 -> 9.6 us, down_proj
  // 2560 x 7040 at M = 2048 36.7 -> 35.1, gate_proj 14080 x 2560 at M = 512
  // 21.9 -> 20.6.  Below one 64-row tile per CU the same holds for 32-row
  // tiles (measured at M = 512).
  const int64_t tn = (N + 127) / 128;
  const auto tiles = [&](int64_t bm) { return ((M + bm - 1) / bm) * tn; };
  // Wide launches: 128 x 256 tiles, the waves side by side over the 128
  // rows with two packed tiles each, so every code word is unpacked once per
  // workgroup and feeds eight MFMAs (2 waves per SIMD: 254 VGPRs).  From 768
  // such tiles (first built as 2 x 2 waves of four tiles: gate_proj at M =
  // 4096 87 -> 84 us, at M = 8192 254 -> 238 us; i/f/g grouped at M = 4096
  // 51 -> 49 us); with fewer, the tiles do not fill the rounds (2048-wide
  // projections at M = 4096: 20.4 -> 22.7 us, 2560-wide at M = 8192: 49 ->
  // 52 us, measured again with the side-by-side waves: no faster) and
  // 128 x 128 stays.
  if (M > 64 && ((M + 127) / 128) * ((N + 255) / 256) >= kWideTiles)
    return launch_mi<4, 4>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, glu, stream);
  if (M > 64 && tiles(128) >= 512)
    return tall_mi(tiles(128), tiles(96)) == 3
               ? launch_mi<3>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, glu, stream)
               : launch_mi<4>(xq, rowsum, s, packed, beta, M, N, K, out, out_kind, glu, stream);
  const int64_t KB = K / 128;
  if (M > 32 && tiles(64) >= 256)
    return launch_mi_kg<2>(k_groups(tiles(64), KB, 2), xq, rowsum, s, packed, beta, M, N, K, out,
                           out_kind, glu, stream);
  return launch_mi_kg<1>(k_groups(tiles(32), KB, 1), xq, rowsum, s, packed, beta, M, N, K, out,
                         out_kind, glu, stream);
}

template <int MI, int TPW = 2, int KG = 1>
static hipError_t launch_group_mi(const GemmCalls &calls, int ncalls, int64_t M, int64_t N,
                                  int64_t K, int out_kind, hipStream_t stream) {
  const int BM = 32 * MI, BN = TPW == 1 ? 128 : 64 * TPW;
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const unsigned grid = (unsigned)(tiles_m * tiles_n * ncalls);
#define BL_GEMMG_CASE(KIND)                                                         \
  gemm_mfma_group_kernel<MI, KIND, TPW, KG><<<grid, 256 * KG, 0, stream>>>(         \
      ncalls, (int)M, (int)N, (int)K, tiles_m, tiles_n, calls)
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
  if (M > 64 && tiles(128) >= 512)
    return tall_mi(tiles(128), tiles(96)) == 3
               ? launch_group_mi<3>(calls, ncalls, M, N, K, out_kind, stream)
               : launch_group_mi<4>(calls, ncalls, M, N, K, out_kind, stream);
  const int64_t KB = K / 128;
  const auto go = [&](auto mi_tag, int kg) {
    constexpr int MI = decltype(mi_tag)::value;
    constexpr int TP = MI <= 2 ? kShortTpw : 2;
    if (kg == 4) return launch_group_mi<MI, TP, 4>(calls, ncalls, M, N, K, out_kind, stream);
    if (kg == 2) return launch_group_mi<MI, TP, 2>(calls, ncalls, M, N, K, out_kind, stream);
    return launch_group_mi<MI, TP, 1>(calls, ncalls, M, N, K, out_kind, stream);
  };
  if (M > 32 && tiles(64) >= 256)
    return go(std::integral_constant<int, 2>{}, k_groups(tiles(64), KB, 2));
  return go(std::integral_constant<int, 1>{}, k_groups(tiles(32), KB, 1));
}

}  // namespace bl
