// skinny.hip -- FusedBitLinear for a few tokens: the contraction of up to 64
// pre-quantized rows, or up to 16 rows normalized and quantized in place.
//
// At a handful of tokens the layer is a stream over the packed weights
// (N*K/4 bytes): the matrix cores have far more throughput than needed, so
// the design goal is bytes in flight, not arithmetic.  One workgroup owns one
// packed 32-row tile column (32 output features x all of K); its 4 waves
// split the K-blocks round-robin.
//   1. Every wave first issues the 16-byte loads of its weight tiles (one
//      contiguous 1 KiB per wave per tile; 4, 8 or 16 tiles by the largest K
//      of the launch), so HBM latency overlaps the prologue.
//   2. Fused variant: the workgroup normalizes and quantizes the M token
//      rows itself, a wave per row, with the shared row quantizer
//      (rowquant.h) into LDS --
//      RMSNorm right before quantization, as in the hysenlabs de review
//      "MatMul-Free LM: Ternary-Gewichte statt Matrixmultiplikation im
//      Transformer", section "HGRNBit: was in einem Block tatsächlich
//      passiert".  Pre-quantized variant: xq, s, rowsum come from the
//      act-quant kernel and A operands are read straight from memory.
//   3. Each tile feeds four v_mfma_i32_16x16x64_i8 (2 output halves x 2
//      k-steps); token rows >= M are zero operands.
//   4. The 4 waves' partial sums are added in LDS; the epilogue subtracts
//      rowsum and rescales by beta / s_m (datacamp "MatMul-freie LLMs:
//      Zentrale Konzepte erklärt", figure panel 4).
// A launch can carry up to kGroupMax independent calls (grouped entry
// point): workgroups are numbered call after call and each finds its call
// from the prefix table in the kernel arguments.
#include <vector>

#include "bl_launch.h"
#include "rowquant.h"

namespace bl {

// weight tiles a wave holds in registers: TB = 4, 8 or 16, the smallest that
// covers a wave's share of the largest K of the launch (every issued load
// instruction costs the CU's address unit a slot, in range or not)
constexpr int skinny_tb(int64_t kmax) {
  return kmax <= 2048 ? 4 : (kmax <= 4096 ? 8 : 16);
}

struct SkinnyCall {
  const void *x;
  const void *gain;
  const int8_t *xq;
  const float *s;
  const int32_t *rowsum;
  const uint4 *packed;
  const float *beta;
  void *out;
  int M, N, K;
};

template <int MAXC>
struct SkinnyLaunch {
  SkinnyCall call[MAXC];
  int first_block[MAXC + 1];
  int ncalls;
  float eps;
};

// MB: 16-row MFMA blocks (pre-quantized calls take up to 4, i.e. M <= 64;
// fused calls 1).
// GLU (pre-quantized calls): the packed rows are a gate_proj in GLU order
// and the output is h [M, N/2] = silu(y_gate) * y_up (tile rows 0..15 are
// gated, 16..31 the rows they multiply).
// NW: waves per workgroup, splitting the K-blocks round-robin (4; the
// pre-quantized path takes 8 from K = 2048 in launches of fewer workgroups
// than CUs, halving each wave's chain of tiles).
template <bool FUSED, int DT, int OUT, int MAXC, int RMODE, int MB, int TB, bool GLU = false,
          int NW = 4>
__global__ __launch_bounds__(64 * NW) void skinny_kernel(SkinnyLaunch<MAXC> L) {
  static_assert(!FUSED || MB == 1, "fused calls have at most 16 rows");
  static_assert(!FUSED || NW == 4, "fused calls run 4 waves");
  static_assert(!GLU || (!FUSED && OUT != kOutI32), "GLU: pre-quantized, float output");
  extern __shared__ __align__(16) int8_t xs[];  // fused: [M][K + 16] int8
  // per-wave LDS region: the pre-quantized path's A stage during the
  // contraction, then the wave's partial sums
  constexpr int kStage = 16 * MB * 128;
  constexpr int kRed = MB * 8 * 64 * 4;
  constexpr int kWave = FUSED ? kRed : (kStage > kRed ? kStage : kRed);
  __shared__ __align__(16) int8_t wbuf[NW][kWave];
  const auto red = [&](int ww, int j, int l) -> int & {
    return reinterpret_cast<int *>(wbuf[ww])[j * 64 + l];
  };
  __shared__ float s_row[16 * MB];
  __shared__ int rs_row[16 * MB];

  int c = 0;
  if constexpr (MAXC > 1) {
    while (c + 1 < L.ncalls && (int)blockIdx.x >= L.first_block[c + 1]) ++c;
  }
  const SkinnyCall &p = L.call[c];
  const int nt = (int)blockIdx.x - L.first_block[c];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int M = p.M, K = p.K, KB = K >> 7;
  const int lds_stride = K + 16;
  const int nmine = w < KB ? (KB - w + NW - 1) / NW : 0;

  // ---- 1. loads.  Buffer loads whose out-of-range offsets read as zero:
  // none is conditional, so each wait below is for exactly the loads it
  // needs (waits are in issue order).  Pre-quantized calls fetch the row
  // scale and row sum first (tiny, used only by the epilogue), then the
  // weight tiles of the first batch.
  float s_reg = 0.0f;
  int rs_reg = 0;
  if constexpr (!FUSED) {
    const uint32_t ro = tid < M ? (uint32_t)(4 * tid) : 0x40000000u;
    rs_reg = __builtin_amdgcn_raw_buffer_load_b32(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(p.rowsum), (short)0, 4 * M, 0x00020000),
        (int)ro, 0, 0);
    if constexpr (OUT != kOutI32)
      s_reg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
          __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p.s), (short)0, 4 * M, 0x00020000),
          (int)ro, 0, 0));
  }
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4 *>(p.packed + (int64_t)nt * KB * 64), (short)0, KB * 1024, 0x00020000);
  const auto w_load = [&](int tile) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                       wrs, (w + NW * tile) * 1024 + lane * 16, 0, 0));
  };
  v4i wr[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) wr[t] = w_load(t);

  // ---- 2. activations
  if constexpr (FUSED) {
    constexpr int EB = dtype_bytes(DT);
    for (int m = w; m < M; m += NW) {  // a wave per token row
      const char *xr = reinterpret_cast<const char *>(p.x) + (int64_t)m * K * EB;
      int8_t *dst = xs + m * lds_stride;
      float sc;
      int rs;
      auto sink = [&](int k, uint2 codes) { *reinterpret_cast<uint2 *>(dst + k) = codes; };
      // fused calls have K <= 8192: the row stays in registers (RMODE is
      // chosen on the host from the largest K of the launch)
      quantize_row<DT, RMODE>(xr, reinterpret_cast<const char *>(p.gain), K, L.eps, sink, sc, rs);
      if (lane == 0) {
        s_row[m] = sc;
        rs_row[m] = rs;
      }
    }
    __syncthreads();
    // rescale factor beta / s_m once per row
    if (OUT != kOutI32 && tid < M) s_row[tid] = div_rn(*p.beta, s_row[tid]);
  }

  // ---- 3. contraction
  v4i acc0[MB], acc1[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc0[mb] = acc1[mb] = v4i{0, 0, 0, 0};
  const int arow = lane & 15;
  // Pre-quantized A.  The MFMA operand layout (lane l: row l mod 16, 16
  // bytes of chunk 2 (l / 16) + s2) gathered straight from memory puts every
  // lane of a load in another row, and such loads cost the address and
  // cache units several times what row-contiguous ones do (the contraction
  // of 64 rows at K = 7040 ran 17 us that way, 10.4 us staged).  So a wave
  // loads its k-block's 16 MB x 128-byte slice with row-contiguous 16-byte
  // loads (load j: rows 8 j + l / 8, chunk l mod 8; rows >= M read as zero),
  // one tile ahead of its MFMAs, and turns it into operands through its own
  // LDS stage (XOR-swizzled rows, conflict-free both ways).  Every load is
  // issued (past the wave's last tile the offset is out of range: zeros, no
  // memory traffic), so the wait for a tile's slice never waits for the
  // loads issued after it.  (A deeper ring of slices in registers was
  // slower: more loads in flight per wave, more registers.)
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t *>(p.xq), (short)0, FUSED ? 0 : M * K, 0x00020000);
  const int crow = lane >> 3, cch = lane & 7;
  const auto a_load = [&](int tile, int j) {
    const int kb = w + NW * tile;
    const uint32_t off = tile < nmine ? (uint32_t)((8 * j + crow) * K + kb * 128 + 16 * cch)
                                      : 0x40000000u;
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(xr, (int)off, 0, 0));
  };
  v4i an[2 * MB];
  if constexpr (!FUSED) {
#pragma unroll
    for (int j = 0; j < 2 * MB; ++j) an[j] = a_load(0, j);
  }
  for (int base = 0; base < nmine; base += TB) {
    if (base > 0) {
#pragma unroll
      for (int t = 0; t < TB; ++t) wr[t] = w_load(base + t);
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if (base + t >= nmine) break;
      const int kb = w + NW * (base + t);
      const v4i u = wr[t];
      v4i a[MB][2];
      if constexpr (FUSED) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          a[0][s2] = v4i{0, 0, 0, 0};
          if (arow < M)
            a[0][s2] = *reinterpret_cast<const v4i *>(xs + arow * lds_stride + kb * 128 +
                                                      32 * (lane >> 4) + 16 * s2);
        }
      } else {
        int8_t *st = wbuf[w];
        // the previous tile's operand reads are done before this overwrite
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < 2 * MB; ++j) {
          const int row = 8 * j + crow;
          *reinterpret_cast<v4i *>(st + row * 128 + (swz(row, cch) << 4)) = an[j];
        }
        wave_lds_sync();
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int row = 16 * mb + arow, ch = 2 * (lane >> 4) + s2;
            a[mb][s2] = *reinterpret_cast<const v4i *>(st + row * 128 + (swz(row, ch) << 4));
          }
#pragma unroll
        for (int j = 0; j < 2 * MB; ++j) an[j] = a_load(base + t + 1, j);
      }
      // word (h, s2) of a lane slot sits at dword 2h + s2
      v4i b[2][2];
      unpack_pair((uint32_t)u[0], (uint32_t)u[1], b[0][0], b[1][0]);
      unpack_pair((uint32_t)u[2], (uint32_t)u[3], b[0][1], b[1][1]);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          acc0[mb] = mfma16x16x64(a[mb][s2], b[s2][0], acc0[mb]);
          acc1[mb] = mfma16x16x64(a[mb][s2], b[s2][1], acc1[mb]);
        }
      }
    }
  }

  // ---- 4. cross-wave sum and epilogue
  if constexpr (!FUSED) {
    if (tid < M) {
      if constexpr (OUT != kOutI32) s_row[tid] = div_rn(*p.beta, s_reg);
      rs_row[tid] = rs_reg;
    }
  }
  // red(w, 8 mb + 4 h + i, lane): row 16 mb + 4 (lane / 16) + i, column
  // 16 h + lane % 16 of the tile; it overwrites the wave's own A stage,
  // whose last operand reads come first
  wave_lds_sync();
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red(w, 8 * mb + i, lane) = acc0[mb][i];
      red(w, 8 * mb + 4 + i, lane) = acc1[mb][i];
    }
  __syncthreads();
  constexpr int T = 64 * NW;
  // sum of the NW waves' partial sums at one place of the table (int32:
  // exact in any order)
  const auto total = [&](int j, int l) {
    int v = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += red(ww, j, l);
    return v;
  };
  if constexpr (GLU) {
    // output (m, c), c < 16: row m's gated value sits at red(., 8 mb + i, L)
    // and the value it multiplies at red(., 8 mb + 4 + i, L), with
    // L = 16 (r / 4) + c, i = r % 4 for r = m % 16
#pragma unroll
    for (int q = 0; q < (256 * MB + T - 1) / T; ++q) {
      const int idx = tid + T * q;
      const int m = idx >> 4, c = idx & 15;
      if (m >= M) continue;
      const int mb = m >> 4, r = m & 15;
      const int Lq = 16 * (r >> 2) + c, jg = 8 * mb + (r & 3), ju = jg + 4;
      const int vg = total(jg, Lq) - rs_row[m];
      const int vu = total(ju, Lq) - rs_row[m];
      const float yg = (float)vg * s_row[m], yu = (float)vu * s_row[m];
      store1<OUT>(p.out, (int64_t)m * (p.N >> 1) + nt * 16 + c, silu(yg) * yu);
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < 512 * MB / T; ++q) {
    const int idx = tid + T * q;
    const int j = idx >> 6, Lq = idx & 63;
    const int mb = j >> 3, h = (j >> 2) & 1, i = j & 3;
    const int m = 16 * mb + 4 * (Lq >> 4) + i;
    if (m >= M) continue;
    const int n = nt * 32 + 16 * h + (Lq & 15);
    const int v = total(j, Lq) - rs_row[m];
    const int64_t o = (int64_t)m * p.N + n;
    if constexpr (OUT == kOutI32) {
      reinterpret_cast<int32_t *>(p.out)[o] = v;
    } else {
      store1<OUT>(p.out, o, (float)v * s_row[m]);
    }
  }
}

static SkinnyCall to_call(const SkinnyArgs &a) {
  SkinnyCall c;
  c.x = a.x;
  c.gain = a.gain;
  c.xq = a.xq;
  c.s = a.s;
  c.rowsum = a.rowsum;
  c.packed = reinterpret_cast<const uint4 *>(a.packed);
  c.beta = a.beta;
  c.out = a.out;
  c.M = (int)a.M;
  c.N = (int)a.N;
  c.K = (int)a.K;
  return c;
}

template <bool FUSED, int DT, int MAXC, int RMODE, int MB, int TB, int NW = 4>
static void launch_out(const SkinnyLaunch<MAXC> &L, int out_kind, unsigned grid, size_t lds,
                       bool glu, hipStream_t stream) {
  constexpr unsigned T = 64 * NW;
  if constexpr (!FUSED && MAXC == 1) {
    if (glu) {
      switch (out_kind) {
        case BL_F32: skinny_kernel<false, DT, BL_F32, 1, RMODE, MB, TB, true, NW><<<grid, T, lds, stream>>>(L); break;
        case BL_F16: skinny_kernel<false, DT, BL_F16, 1, RMODE, MB, TB, true, NW><<<grid, T, lds, stream>>>(L); break;
        default: skinny_kernel<false, DT, BL_BF16, 1, RMODE, MB, TB, true, NW><<<grid, T, lds, stream>>>(L); break;
      }
      return;
    }
  }
  switch (out_kind) {
    case BL_F32: skinny_kernel<FUSED, DT, BL_F32, MAXC, RMODE, MB, TB, false, NW><<<grid, T, lds, stream>>>(L); break;
    case BL_F16: skinny_kernel<FUSED, DT, BL_F16, MAXC, RMODE, MB, TB, false, NW><<<grid, T, lds, stream>>>(L); break;
    case BL_BF16: skinny_kernel<FUSED, DT, BL_BF16, MAXC, RMODE, MB, TB, false, NW><<<grid, T, lds, stream>>>(L); break;
    default: skinny_kernel<FUSED, DT, kOutI32, MAXC, RMODE, MB, TB, false, NW><<<grid, T, lds, stream>>>(L); break;
  }
}

// Fused calls: row-quantizer mode from the largest K of the launch.
template <int DT, int MAXC, int TB>
static void launch_fused(const SkinnyLaunch<MAXC> &L, int out_kind, unsigned grid, size_t lds,
                         int64_t kmax, hipStream_t stream) {
  if (row_mode((int)kmax) == kRowFloat)
    launch_out<true, DT, MAXC, kRowFloat, 1, TB>(L, out_kind, grid, lds, false, stream);
  else
    launch_out<true, DT, MAXC, kRowRaw, 1, TB>(L, out_kind, grid, lds, false, stream);
}

template <int MAXC, int TB>
static void launch_any_tb(const SkinnyLaunch<MAXC> &L, bool fused, int x_dtype, int out_kind,
                          unsigned grid, size_t lds, int64_t kmax, int64_t M, bool glu,
                          hipStream_t stream) {
  if (fused) {
    switch (x_dtype) {
      case BL_F32: launch_fused<BL_F32, MAXC, TB>(L, out_kind, grid, lds, kmax, stream); break;
      case BL_F16: launch_fused<BL_F16, MAXC, TB>(L, out_kind, grid, lds, kmax, stream); break;
      default: launch_fused<BL_BF16, MAXC, TB>(L, out_kind, grid, lds, kmax, stream); break;
    }
  }
}

// Pre-quantized calls (never grouped): 16-row blocks by M, NW waves.
template <int TB, int NW>
static void launch_pre(const SkinnyLaunch<1> &L, int out_kind, unsigned grid, int64_t M, bool glu,
                       hipStream_t stream) {
  if (M <= 16)
    launch_out<false, BL_F32, 1, kRowFloat, 1, TB, NW>(L, out_kind, grid, 0, glu, stream);
  else if (M <= 32)
    launch_out<false, BL_F32, 1, kRowFloat, 2, TB, NW>(L, out_kind, grid, 0, glu, stream);
  else
    launch_out<false, BL_F32, 1, kRowFloat, 4, TB, NW>(L, out_kind, grid, 0, glu, stream);
}

template <int MAXC>
static void launch_any(const SkinnyLaunch<MAXC> &L, bool fused, int x_dtype, int out_kind,
                       unsigned grid, size_t lds, int64_t kmax, int64_t M, bool glu,
                       hipStream_t stream) {
  if constexpr (MAXC == 1) {
    if (!fused) {
      // Fewer tile columns than CUs and K >= 2048: 8 waves per workgroup (4
      // or 8 tiles each) halve each wave's chain of tiles (N = 2048 at M =
      // 32, K = 5632: 6.8 -> 5.5 us).  Wider launches keep 4 waves: more
      // workgroups fit a CU, and 8 were 1-5 % slower there.
      if (kmax >= 2048 && grid < 256) {
        if (kmax <= 4096) launch_pre<4, 8>(L, out_kind, grid, M, glu, stream);
        else launch_pre<8, 8>(L, out_kind, grid, M, glu, stream);
      } else {
        switch (skinny_tb(kmax)) {
          case 4: launch_pre<4, 4>(L, out_kind, grid, M, glu, stream); break;
          case 8: launch_pre<8, 4>(L, out_kind, grid, M, glu, stream); break;
          default: launch_pre<16, 4>(L, out_kind, grid, M, glu, stream); break;
        }
      }
      return;
    }
  }
  switch (skinny_tb(kmax)) {
    case 4: launch_any_tb<MAXC, 4>(L, fused, x_dtype, out_kind, grid, lds, kmax, M, glu, stream); break;
    case 8: launch_any_tb<MAXC, 8>(L, fused, x_dtype, out_kind, grid, lds, kmax, M, glu, stream); break;
    default: launch_any_tb<MAXC, 16>(L, fused, x_dtype, out_kind, grid, lds, kmax, M, glu, stream); break;
  }
}

static bool decode_ok(const SkinnyArgs &a) {
  return a.fused && decode_fits(a.M, a.K, a.x_dtype);
}

static DecodeArgs decode_args(const SkinnyArgs &a) {
  DecodeArgs d{};
  d.x_dtype = a.x_dtype;
  d.M = a.M;
  d.N = a.N;
  d.K = a.K;
  d.eps = a.eps;
  d.out_kind = a.out_kind;
  d.glu = a.glu;
  d.ncalls = 0;
  return d;
}

static void decode_add(DecodeArgs &d, const SkinnyArgs &a) {
  d.x[d.ncalls] = a.x;
  d.gain[d.ncalls] = a.gain;
  d.packed[d.ncalls] = a.packed;
  d.beta[d.ncalls] = a.beta;
  d.out[d.ncalls] = a.out;
  ++d.ncalls;
}

hipError_t launch_skinny(const SkinnyArgs &a, hipStream_t stream) {
  if (decode_ok(a)) {
    DecodeArgs d = decode_args(a);
    decode_add(d, a);
    return launch_decode(d, stream);
  }
  if (!a.fused && !a.glu && a.M > 16 && a.N / 32 < 256) {
    // Fewer tile columns than CUs: the 16-row blocks go to workgroups of
    // their own, as calls of one launch whose pointers start at the block's
    // first row, so the launch has up to four times the workgroups and each
    // stages and multiplies a quarter of the rows (the weights are read once
    // per block, mostly from cache).  Same operations per output, same bits.
    // M = 64, N = 2560, K = 7040: 9.3 -> 7.2 us; M = 48: 5.2 -> 3.7 us; M =
    // 32, N = 2048, K = 5632: 5.5 -> 4.9 us.
    SkinnyLaunch<4> R;
    const int nrb = (int)((a.M + 15) / 16), nt = (int)(a.N / 32);
    const size_t esz = (a.out_kind == BL_F16 || a.out_kind == BL_BF16) ? 2 : 4;
    for (int r = 0; r < 4; ++r) {
      R.call[r] = to_call(a);
      if (r < nrb) {
        R.call[r].xq += (int64_t)16 * r * a.K;
        R.call[r].s += 16 * r;
        R.call[r].rowsum += 16 * r;
        R.call[r].out = static_cast<char *>(R.call[r].out) + (size_t)16 * r * (size_t)a.N * esz;
        R.call[r].M = (int)(a.M - 16 * r < 16 ? a.M - 16 * r : 16);
      }
      R.first_block[r] = (r < nrb ? r : nrb) * nt;
    }
    R.first_block[4] = nrb * nt;
    R.ncalls = nrb;
    R.eps = a.eps;
    const unsigned grid = (unsigned)(nrb * nt);
    // 8 waves (each wave's chain of tiles halves) below a workgroup per CU,
    // and at K > 4096 also above: the 2.7B down_proj at M = 64 (K = 7040,
    // 320 workgroups) runs 14 tiles per wave with 4 waves; 8 made the 2.7B
    // stack at M = 64 3.4 % faster.
    if (a.K >= 2048 && (grid < 256 || a.K > 4096)) {
      if (a.K <= 4096) launch_out<false, BL_F32, 4, kRowFloat, 1, 4, 8>(R, a.out_kind, grid, 0, false, stream);
      else launch_out<false, BL_F32, 4, kRowFloat, 1, 8, 8>(R, a.out_kind, grid, 0, false, stream);
    } else {
      switch (skinny_tb(a.K)) {
        case 4: launch_out<false, BL_F32, 4, kRowFloat, 1, 4, 4>(R, a.out_kind, grid, 0, false, stream); break;
        case 8: launch_out<false, BL_F32, 4, kRowFloat, 1, 8, 4>(R, a.out_kind, grid, 0, false, stream); break;
        default: launch_out<false, BL_F32, 4, kRowFloat, 1, 16, 4>(R, a.out_kind, grid, 0, false, stream); break;
      }
    }
    return hipGetLastError();
  }
  SkinnyLaunch<1> L;
  L.call[0] = to_call(a);
  L.first_block[0] = 0;
  L.first_block[1] = (int)(a.N / 32);
  L.ncalls = 1;
  L.eps = a.eps;
  const size_t lds = a.fused ? (size_t)a.M * (size_t)(a.K + 16) : 0;
  launch_any<1>(L, a.fused, a.x_dtype, a.out_kind, (unsigned)(a.N / 32), lds, a.K, a.M, a.glu,
                stream);
  return hipGetLastError();
}

// Pre-quantized calls of one shape (HGRN's i/f/g at 9..64 tokens) as one
// launch: the calls' 16-row blocks (or the whole calls, when the launch
// already has a tile column per CU or M <= 16) are the sub-calls of the
// launch, numbered call after call, each computed exactly as launch_skinny
// computes it alone.  One launch instead of three: the 2.7B i/f/g at M = 64
// take one launch of 960 workgroups.
constexpr int kPreSub = kGroupCalls * 4;

template <int MB, int TB, int NW>
static void launch_pre_sub(const SkinnyLaunch<kPreSub> &R, int out_kind, unsigned grid,
                           hipStream_t stream) {
  launch_out<false, BL_F32, kPreSub, kRowFloat, MB, TB, NW>(R, out_kind, grid, 0, false, stream);
}

template <int MB>
static void launch_pre_mb(const SkinnyLaunch<kPreSub> &R, int out_kind, unsigned grid, int64_t K,
                          hipStream_t stream) {
  if (K >= 2048 && grid < 256) {
    if (K <= 4096) launch_pre_sub<MB, 4, 8>(R, out_kind, grid, stream);
    else launch_pre_sub<MB, 8, 8>(R, out_kind, grid, stream);
  } else {
    switch (skinny_tb(K)) {
      case 4: launch_pre_sub<MB, 4, 4>(R, out_kind, grid, stream); break;
      case 8: launch_pre_sub<MB, 8, 4>(R, out_kind, grid, stream); break;
      default: launch_pre_sub<MB, 16, 4>(R, out_kind, grid, stream); break;
    }
  }
}

hipError_t launch_skinny_pre_grouped(const SkinnyArgs *calls, int ncalls, hipStream_t stream) {
  const SkinnyArgs &a = calls[0];
  const int nt = (int)(a.N / 32);
  const int nrb = (int)((a.M + 15) / 16);
  const bool split = a.M > 16 && nt * ncalls < 256;  // as launch_skinny, over the launch
  const size_t esz = (a.out_kind == BL_F16 || a.out_kind == BL_BF16) ? 2 : 4;
  SkinnyLaunch<kPreSub> R;
  int sub = 0, blocks = 0;
  for (int j = 0; j < ncalls; ++j) {
    const int parts = split ? nrb : 1;
    for (int r = 0; r < parts; ++r) {
      SkinnyCall c = to_call(calls[j]);
      if (split) {
        c.xq += (int64_t)16 * r * a.K;
        c.s += 16 * r;
        c.rowsum += 16 * r;
        c.out = static_cast<char *>(c.out) + (size_t)16 * r * (size_t)a.N * esz;
        c.M = (int)(a.M - 16 * r < 16 ? a.M - 16 * r : 16);
      }
      R.call[sub] = c;
      R.first_block[sub] = blocks;
      blocks += nt;
      ++sub;
    }
  }
  for (int i = sub; i <= kPreSub; ++i) R.first_block[i] = blocks;
  R.ncalls = sub;
  R.eps = a.eps;
  const unsigned grid = (unsigned)blocks;
  const int64_t M = split ? 16 : a.M;
  if (M <= 16) launch_pre_mb<1>(R, a.out_kind, grid, a.K, stream);
  else if (M <= 32) launch_pre_mb<2>(R, a.out_kind, grid, a.K, stream);
  else launch_pre_mb<4>(R, a.out_kind, grid, a.K, stream);
  return hipGetLastError();
}

// Consecutive calls of one shape that the decode kernel takes go out in
// launches of up to kDecodeCalls; the others are gathered into launches of
// the skinny kernel of up to kGroupMax calls.
hipError_t launch_skinny_grouped(const SkinnyArgs *calls, int ncalls, hipStream_t stream) {
  std::vector<SkinnyArgs> rest;
  for (int i = 0; i < ncalls;) {
    const SkinnyArgs &a = calls[i];
    if (!decode_ok(a)) {
      rest.push_back(a);
      ++i;
      continue;
    }
    DecodeArgs d = decode_args(a);
    // up to kDecodeCalls consecutive calls of one shape per launch (row mode
    // or split mode alike: the shape decides the mode)
    const auto same = [&](const SkinnyArgs &c) {
      return c.fused && !c.glu && !a.glu && decode_ok(c) && c.M == a.M && c.K == a.K &&
             c.N == a.N;
    };
    decode_add(d, calls[i++]);
    while (i < ncalls && d.ncalls < kDecodeCalls && same(calls[i])) decode_add(d, calls[i++]);
    const hipError_t e = launch_decode(d, stream);
    if (e != hipSuccess) return e;
  }
  const int nrest = (int)rest.size();
  for (int base = 0; base < nrest; base += kGroupMax) {
    const int n = nrest - base < kGroupMax ? nrest - base : kGroupMax;
    SkinnyLaunch<kGroupMax> L;
    int blocks = 0;
    size_t lds = 0;
    int64_t kmax = 0;
    for (int i = 0; i < n; ++i) {
      const SkinnyArgs &a = rest[base + i];
      L.call[i] = to_call(a);
      L.first_block[i] = blocks;
      blocks += (int)(a.N / 32);
      const size_t l = (size_t)a.M * (size_t)(a.K + 16);
      if (l > lds) lds = l;
      if (a.K > kmax) kmax = a.K;
    }
    for (int i = n; i <= kGroupMax; ++i) L.first_block[i] = blocks;
    L.ncalls = n;
    L.eps = rest[base].eps;
    launch_any<kGroupMax>(L, true, rest[base].x_dtype, rest[base].out_kind, (unsigned)blocks,
                          lds, kmax, 16, false, stream);
  }
  return hipGetLastError();
}

}  // namespace bl
