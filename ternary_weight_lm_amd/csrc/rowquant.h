// rowquant.h -- RMSNorm + per-token absmax int8 quantization of one token
// row by one 64-lane wave.  Used by the act-quant kernel (a wave per row)
// and by the fused decode prologue, so both paths produce bit-identical
// codes and scales.
//
// Lane L owns the 8-element chunks k = 8L + 512c (c = 0, 1, ...), read with
// 16-byte loads.  Up to K = 8192 the chunks are loaded once, all in flight
// together, and kept in registers (widened when K <= 4096, raw above);
// longer rows are re-read for each pass, four chunks in flight.
// Sum of squares, association fixed for every kernel of the library: the
// chunks form 256 slots (chunk index mod 256); each slot adds its x^2 terms
// in chunk order (fma with an exact fp64 square is the plain product-then-
// add); slots l, l+64, l+128, l+192 are combined as (p0 + p1) + (p2 + p3)
// into lane l's value, and the 64 lane values are reduced by the DPP tree of
// wave_sum.  Here one wave holds all four slots of a lane (slot group =
// chunk index mod 4); the decode kernel gives each group its own wave and
// exchanges the per-lane partials through LDS.  Either way the result is the
// same bits.  The row and the gain are read with buffer loads (chunks past K
// read as zero), issued together and unconditionally, so the wait for x
// never waits for the gain.  No LDS, no barriers.
//   pass 1: sum of x^2 (fp64)            -> r = 1/sqrt(fp32(sum/K) + eps)
//   pass 2: max |(x * r) * g|            -> s = 127 / max(., 1e-5)
//   pass 3: xq = clamp(rne(xn * s)), handed to the sink 8 at a time; the
//           row sum of the codes is reduced exactly in int32.
#pragma once

#include "bl_common.h"

namespace bl {

constexpr int kRowCache = 8;  // cached chunks per lane: K <= 4096

// Chunks a lane caches for a row of K elements in the float mode: the
// smallest of 2, 4, 6, 8 rounds of 512 elements that covers K.  Every load
// instruction costs the CU's address unit a slot even where all its lanes
// are out of range, so a short row issues only the loads it needs.
__host__ __device__ constexpr int row_cache(int K) {
  return K <= 1024 ? 2 : (K <= 2048 ? 4 : (K <= 3072 ? 6 : 8));
}

// The low bytes of four words (int8 codes from quant8) -> one dword of
// int8 (byte i = code i), three byte permutes.
__device__ __forceinline__ uint32_t pack4(int q0, int q1, int q2, int q3) {
  const uint32_t t01 = __builtin_amdgcn_perm((uint32_t)q1, (uint32_t)q0, 0x0c0c0400u);
  const uint32_t t23 = __builtin_amdgcn_perm((uint32_t)q3, (uint32_t)q2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(t23, t01, 0x05040100u);
}

// The row's sum of squares from the four per-lane slot partials:
// (p0 + p1) + (p2 + p3) in each lane, then the wave's DPP tree.
__device__ __forceinline__ double group_sum(const double (&ss)[4]) {
  return wave_sum((ss[0] + ss[1]) + (ss[2] + ss[3]));
}

// How a lane holds its chunks of the row between the three passes.
enum RowMode {
  kRowFloat = 0,  // widened once, xn kept in registers: K <= 512 * kRowCache
  kRowRaw = 1,    // raw 16-byte chunks kept, widened per pass: K <= 512 * kRowRawCache
  kRowReload = 2  // re-read from memory every pass, 4 chunks in flight
};
constexpr int kRowRawCache = 16;  // K <= 8192

__host__ __device__ constexpr int row_mode(int K) {
  return K <= 512 * kRowCache ? kRowFloat : (K <= 512 * kRowRawCache ? kRowRaw : kRowReload);
}

// Pass 1 of the float mode on a row already in registers (chunk c of the
// lane: elements 8 lane + 512 c .. +7, c < NC, in xraw[c]; chunks past K read
// as zero): r = 1 / sqrt(fp32(sum x^2 / K) + eps), the sum in the library's
// association.
template <int DT, int NC>
__device__ __forceinline__ float row_rms(const Chunk8<DT> (&xraw)[NC], int K, float eps) {
  const int lane = threadIdx.x & 63;
  const int nch = (K + 511) >> 9;  // chunk rounds (some lanes idle in the last)
  double ss[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c < nch && 8 * lane + 512 * c < K) {
      float v[8];
      widen<DT>(xraw[c], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss[c & 3] = __builtin_fma((double)v[e], (double)v[e], ss[c & 3]);
    }
  return rms_inv(group_sum(ss), K, eps);
}

// FusedRMSNormSwishGate of one row held in registers (chunk c of the lane:
// elements 8 lane + 512 c .. +7): z = ((o r) w) silu(g), r = 1 / sqrt(fp32(sum
// o^2 / K) + eps) in the library's association, every product in fp32, z
// rounded to the activation dtype -- the value a gate layer hands on.  Used by
// the gate kernels and by the decode kernel's gated row mode, so the two give
// the same bits.
template <int DT, int NC>
__device__ __forceinline__ void gate_row(const Chunk8<DT> (&o)[NC], const Chunk8<DT> (&g)[NC],
                                         const Chunk8<DT> (&w)[NC], int K, float eps,
                                         Chunk8<DT> (&z)[NC]) {
  const float r = row_rms<DT, NC>(o, K, eps);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float fo[8], fg[8], fw[8], v[8];
    widen<DT>(o[c], fo);
    widen<DT>(g[c], fg);
    widen<DT>(w[c], fw);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = ((fo[e] * r) * fw[e]) * silu(fg[e]);
    if constexpr (DT == BL_F32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[c].u[0][i] = __float_as_int(v[i]);
        z[c].u[1][i] = __float_as_int(v[4 + i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        z[c].u[0][i] = (int)((uint32_t)out_bits<DT>(v[2 * i]) |
                             ((uint32_t)out_bits<DT>(v[2 * i + 1]) << 16));
    }
  }
}

// Passes 2 and 3 of the float mode for one gain (its matching chunks in
// graw[c]) and the row's r: xn = (x r) g, s = 127 / max(max |xn|, 1e-5),
// codes.  `sink(k, codes)` receives the 8 codes of elements k..k+7 as two
// dwords; on return every lane holds s and the row sum.  row_rms followed by
// quantize_scaled runs exactly the operations of quantize_loaded below (kept
// separate for the kernels that quantize one row under several gains, so
// the one-row kernels keep their register allocation); a test holds the two
// to the same bits.
template <int DT, int NC, class Sink>
__device__ __forceinline__ void quantize_scaled(const Chunk8<DT> (&xraw)[NC],
                                                const Chunk8<DT> (&graw)[NC], int K, float r,
                                                Sink sink, float &s_out, int &rowsum_out) {
  const int lane = threadIdx.x & 63;
  const int nch = (K + 511) >> 9;
  const auto kof = [&](int c) { return 8 * lane + 512 * c; };
  float v[NC][8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c < nch && kof(c) < K) {
      float g[8];
      widen<DT>(xraw[c], v[c]);
      widen<DT>(graw[c], g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[c][e] = (v[c][e] * r) * g[e];
        amax = fmaxf(amax, fabsf(v[c][e]));
      }
    }
  const float sc = act_scale(wave_max(amax));
  int rs = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c < nch && kof(c) < K) {
      int q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = quant8(v[c][e], sc);
      const uint2 codes = make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
      rs = __builtin_amdgcn_sdot4((int)codes.x, 0x01010101, rs, false);
      rs = __builtin_amdgcn_sdot4((int)codes.y, 0x01010101, rs, false);
      sink(kof(c), codes);
    }
  s_out = sc;
  rowsum_out = wave_sum(rs);
}

// The three passes of the float mode on a row already in registers: chunk
// c of the lane (elements 8 lane + 512 c .. +7, c < NC) in xraw[c],
// the gain's matching chunk in graw[c] (chunks past K read as zero).
// `sink(k, codes)` receives the 8 codes of elements k..k+7 as two dwords; on
// return every lane holds s and the row sum.  Shared by quantize_row and by
// kernels that issue the row's loads themselves, so both give the same bits.
template <int DT, int NC, class Sink>
__device__ __forceinline__ void quantize_loaded(const Chunk8<DT> (&xraw)[NC],
                                                const Chunk8<DT> (&graw)[NC], int K,
                                                float eps, Sink sink, float &s_out,
                                                int &rowsum_out) {
  const int lane = threadIdx.x & 63;
  const int nch = (K + 511) >> 9;  // chunk rounds (some lanes idle in the last)
  const auto kof = [&](int c) { return 8 * lane + 512 * c; };
  // x widened once; after pass 2 the same registers hold xn
  float v[NC][8];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c < nch) widen<DT>(xraw[c], v[c]);
  double ss[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c < nch && kof(c) < K) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        ss[c & 3] = __builtin_fma((double)v[c][e], (double)v[c][e], ss[c & 3]);
    }
  const float r = rms_inv(group_sum(ss), K, eps);
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c < nch && kof(c) < K) {
      float g[8];
      widen<DT>(graw[c], g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[c][e] = (v[c][e] * r) * g[e];
        amax = fmaxf(amax, fabsf(v[c][e]));
      }
    }
  const float sc = act_scale(wave_max(amax));
  int rs = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c < nch && kof(c) < K) {
      int q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = quant8(v[c][e], sc);
      const uint2 codes = make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
      rs = __builtin_amdgcn_sdot4((int)codes.x, 0x01010101, rs, false);
      rs = __builtin_amdgcn_sdot4((int)codes.y, 0x01010101, rs, false);
      sink(kof(c), codes);
    }
  s_out = sc;
  rowsum_out = wave_sum(rs);
}

// Quantizes one row with the calling wave.  `sink(k, codes)` receives the 8
// codes of elements k..k+7 as two dwords.  On return every lane holds s and
// the row sum.  The three modes run the same operations in the same order.
// NC: chunks cached per lane in the float mode (K <= 512 * NC).
template <int DT, int MODE, int NC_FLOAT = kRowCache, class Sink>
__device__ __forceinline__ void quantize_row(const char *__restrict__ xr,
                                             const char *__restrict__ gr, int K,
                                             float eps, Sink sink, float &s_out,
                                             int &rowsum_out) {
  constexpr int EB = dtype_bytes(DT);
  const int lane = threadIdx.x & 63;
  const int nch = (K + 511) >> 9;  // chunk rounds (some lanes idle in the last)
  const auto kof = [&](int c) { return 8 * lane + 512 * c; };
  const rsrc_t xrs = make_rsrc(xr, (uint32_t)(K * EB));
  const rsrc_t grs = make_rsrc(gr, (uint32_t)(K * EB));
  // chunk c of the lane; zeros past K
  const auto ld = [&](int c) { return bload_chunk<DT>(xrs, (uint32_t)(kof(c) * EB)); };
  const auto ldg = [&](int c) { return bload_chunk<DT>(grs, (uint32_t)(kof(c) * EB)); };

  auto emit = [&](int k, const float *xn, float sc, int &rs) {
    int q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = quant8(xn[e], sc);
    const uint2 codes = make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
    rs = __builtin_amdgcn_sdot4((int)codes.x, 0x01010101, rs, false);
    rs = __builtin_amdgcn_sdot4((int)codes.y, 0x01010101, rs, false);
    sink(k, codes);
  };

  if constexpr (MODE == kRowFloat) {
    Chunk8<DT> xraw[NC_FLOAT], graw[NC_FLOAT];
#pragma unroll
    for (int c = 0; c < NC_FLOAT; ++c) xraw[c] = ld(c);
#pragma unroll
    for (int c = 0; c < NC_FLOAT; ++c) graw[c] = ldg(c);
    quantize_loaded<DT, NC_FLOAT>(xraw, graw, K, eps, sink, s_out, rowsum_out);
  } else {
    // raw chunks (kRowRaw) or batches of 4 re-read chunks (kRowReload)
    constexpr int NC = MODE == kRowRaw ? kRowRawCache : 4;
    // the gain is re-read (from cache) in each pass: keeping it in registers
    // too would cost the raw mode half of its occupancy
    constexpr bool GCACHE = false;
    Chunk8<DT> raw[NC];
    Chunk8<DT> graw[GCACHE ? NC : 1];
    // for_each(fn): fn(k, c, x[8]) for every chunk of the lane, in order; c
    // is the chunk's slot in raw[] (a constant once unrolled), and c mod 4 its
    // slot group (NC and the reload step are multiples of 4)
    static_assert(NC % 4 == 0, "chunk groups");
    auto for_each = [&](auto &&fn) {
      if constexpr (MODE == kRowRaw) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
          if (c < nch && kof(c) < K) {
            float f[8];
            widen<DT>(raw[c], f);
            fn(kof(c), c, f);
          }
      } else {
        for (int c0 = 0; c0 < nch; c0 += NC) {
#pragma unroll
          for (int c = 0; c < NC; ++c) raw[c] = ld(c0 + c);
#pragma unroll
          for (int c = 0; c < NC; ++c)
            if (c0 + c < nch && kof(c0 + c) < K) {
              float f[8];
              widen<DT>(raw[c], f);
              fn(kof(c0 + c), c, f);
            }
        }
      }
    };
    const auto gain8 = [&](int k, int c, float *g) {
      if constexpr (GCACHE)
        widen<DT>(graw[c], g);
      else
        load8<DT>(gr + (int64_t)k * EB, g);
    };
    if constexpr (MODE == kRowRaw) {
#pragma unroll
      for (int c = 0; c < NC; ++c) raw[c] = ld(c);
    }
    if constexpr (GCACHE) {
#pragma unroll
      for (int c = 0; c < NC; ++c) graw[c] = ldg(c);
    }
    double ss[4] = {0.0, 0.0, 0.0, 0.0};
    for_each([&](int, int c, const float *f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss[c & 3] = __builtin_fma((double)f[e], (double)f[e], ss[c & 3]);
    });
    const float r = rms_inv(group_sum(ss), K, eps);
    float amax = 0.0f;
    for_each([&](int k, int c, const float *f) {
      float g[8];
      gain8(k, c, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((f[e] * r) * g[e]));
    });
    const float sc = act_scale(wave_max(amax));
    int rs = 0;
    for_each([&](int k, int c, const float *f) {
      float g[8], xn[8];
      gain8(k, c, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) xn[e] = (f[e] * r) * g[e];
      emit(k, xn, sc, rs);
    });
    s_out = sc;
    rowsum_out = wave_sum(rs);
  }
}

}  // namespace bl
