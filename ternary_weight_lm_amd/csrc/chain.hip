// chain.hip -- a sequence of dependent FusedBitLinear calls at decode sizes
// (1..4 token rows) in one persistent launch.
//
// A decode step of an HGRNBit stack is a chain: per block, i/f/g_proj read
// the block input, o_proj reads what the token mixer makes of them, the MLP's
// gate_proj and down_proj follow, and the next block reads the result
// (hysenlabs ja review "matmulfreellm 評価: 行列積を消した HGRNBit を
// Transformers 互換で読む", section "HGRNBit という層構成を読む").  One launch
// per call pays a launch floor of about 1.5 us and leaves the CUs idle while
// each call's first weights arrive; at one token the weights of a 2.7B layer
// stream in well under that.  Here one launch runs the whole chain:
//   * Work items are (call, 32-row tile column) pairs in call order.  A
//     workgroup claims items from a device counter in that order (one claim
//     ahead), issues the item's weight and gain loads at once, and only then
//     waits for the item's input -- so the weights of later calls stream in
//     while earlier calls finish.
//   * A call whose input is an earlier call's output reads it from a tagged
//     copy: every element is one 32-bit word, value in the high half and the
//     launch's tag in the low half, stored and loaded with agent-scope
//     coherent accesses.  A word is valid when its tag is the launch's, so no
//     fence is needed: the consumer polls the producer call's done counter
//     (one relaxed atomic add per finished item), then loads its rows and
//     re-reads them until every tag matches.
//   * Every wait is bounded: it gives up past a wall-clock limit (or at once
//     when another wait already gave up), sets the chain's error word, and
//     the workgroup goes on claiming and skipping items, so every workgroup
//     reaches the exit.  The host reads the error word with
//     bitlinear_chain_status.
//   * No deadlock: a workgroup holds one item it works on (plus one claimed
//     ahead, whose index is larger), items wait only on items of earlier
//     calls, i.e. of smaller index, and items are claimed in index order by
//     running workgroups -- so the smallest unfinished item always has its
//     input and is held by a running workgroup.
//   * The last workgroup to exit resets the counters and advances the tag,
//     so the next launch starts clean without a memset in a captured graph.
// Per item the arithmetic is exactly the decode kernel's split mode (the
// norm's fp64 sum of squares in the library's fixed association on waves
// 0..3, absmax and codes over all 8 waves, v_mfma_i32_16x16x64_i8 on the
// offset codes, the rescale epilogue, the GLU gate for a GLU-packed
// gate_proj), so a chain call gives bitlinear_forward's bits.
#include "bl_launch.h"
#include "rowquant.h"

namespace bl {

namespace {

constexpr int kNW = 8;  // waves per workgroup

// K capacity of an item body in units of 1024 (the smallest of 1, 2, 3, 4,
// 6, 8 covering K): a body issues only the loads a row of that length needs.
__device__ __forceinline__ int chain_kc(uint32_t K) {
  return K <= 1024 ? 1 : K <= 2048 ? 2 : K <= 3072 ? 3 : K <= 4096 ? 4 : K <= 6144 ? 6 : 8;
}

struct ChainHdr {
  uint32_t work, exits, epoch, error;
  uint32_t ncalls, total, M, kmax;
  float eps;
  uint32_t pad[55];
};
static_assert(sizeof(ChainHdr) == 256, "header is 256 bytes");

struct ChainCall {
  const void *x;        // plain input [M, K] (nullptr when xt is used)
  const uint32_t *xt;   // tagged input: an earlier call's tagged output
  const void *gain;     // [K]
  const uint4 *packed;  // packed [N, K]
  const float *beta;
  void *y;              // plain output [M, N] (GLU: [M, N / 2])
  uint32_t *yt;         // tagged output, or nullptr when no later call reads it
  uint32_t K, N, item0, glu;
  int32_t dep;          // call that writes xt, -1 for a plain input
  uint32_t dep_items;   // its item count
  uint32_t pad[12];
};
static_assert(sizeof(ChainCall) == 128, "call descriptor is 128 bytes");

constexpr uint32_t kSc1 = 16;  // buffer cache-policy bit: agent-coherent access

__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Tag of launch `epoch` (never 0, so a zeroed buffer is never valid).
__device__ __forceinline__ uint32_t tag_of(uint32_t epoch) { return epoch % 65535u + 1u; }

// Eight tagged words (two 16-byte coherent loads) -> the raw 16-bit chunk of
// 8 elements; ok is cleared when any word carries another launch's tag.
template <int DT>
__device__ __forceinline__ Chunk8<DT> tagged_chunk(rsrc_t r, uint32_t off, uint32_t tag2,
                                                   bool check, bool &ok) {
  const v4i a = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kSc1));
  const v4i b = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off + 16, 0, kSc1));
  Chunk8<DT> c;
  const uint32_t w[8] = {(uint32_t)a.x, (uint32_t)a.y, (uint32_t)a.z, (uint32_t)a.w,
                         (uint32_t)b.x, (uint32_t)b.y, (uint32_t)b.z, (uint32_t)b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c.u[0][i] = (int)__builtin_amdgcn_perm(w[2 * i + 1], w[2 * i], 0x07060302u);
    if (check && __builtin_amdgcn_perm(w[2 * i + 1], w[2 * i], 0x05040100u) != tag2) ok = false;
  }
  return c;
}

// The 16-bit pattern of an output value in the tagged word of launch tag.
template <int DT>
__device__ __forceinline__ void store_tagged(uint32_t *yt, int64_t idx, float v, uint32_t tag) {
  const uint32_t w = ((uint32_t)out_bits<DT>(v) << 16) | tag;
  __hip_atomic_store(yt + idx, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct ItemShared {
  double part_ss[4][4][64];
  float part_max[4][kNW];
  int part_rs[4][kNW];
  int red[kNW][4][2][16];
  int flag[kNW];
  int abort_;
};

// One item: tile column nt of call cp.  MR rows (1, or 4 for 2..4 tokens),
// K capacity 1024 KC.  Returns after the item's outputs are stored (or the
// wait gave up).
template <int DT, int MR, int KC>
__device__ __forceinline__ void chain_item(const ChainCall *cp, int nt, int M, float eps,
                                           uint32_t tag, ChainHdr *hdr, const uint32_t *done,
                                           uint64_t wait_ticks, int8_t *xs, ItemShared &sh) {
  constexpr int NW = kNW;
  constexpr int EB = 2;
  constexpr int R = NW / 4;
  constexpr int TPW = (8 * KC + NW - 1) / NW;
  constexpr int C4 = (KC + 1) / 2;
  constexpr int CA = (2 * KC + NW - 1) / NW;
  constexpr int CO = C4 / 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w4 = w & 3, wh = w >> 2;
  const int K = (int)cp->K;
  const int N = (int)cp->N;
  const bool glu = cp->glu != 0;
  const int KB = K >> 7, nq = K >> 3;
  const int lds_stride = K + 16;
  const int tiles = N / 32;

  // ---- 1. weights and gain first: they do not depend on the input
  const rsrc_t wr = make_rsrc(cp->packed + (int64_t)nt * KB * 64, (uint32_t)KB * 1024u);
  v4i wt[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) wt[t] = bload(wr, (uint32_t)((w + NW * t) * 1024 + lane * 16));
  const auto qof = [&](int r) { return 64 * w4 + lane + 256 * r; };
  const auto off = [&](int r) { return qof(r) < nq ? (uint32_t)(8 * qof(r) * EB) : kOob; };
  Chunk8<DT> gc[CA];
  {
    const rsrc_t gr = make_rsrc(cp->gain, (uint32_t)(K * EB));
#pragma unroll
    for (int c = 0; c < CA; ++c) gc[c] = bload_chunk<DT>(gr, off(R * c + wh));
  }
  const float beta = *cp->beta;

  // ---- 2. the input rows: plain, or tagged once the producer is done
  Chunk8<DT> xa[MR][CA], xo[MR][CO > 0 ? CO : 1];
  const uint32_t *xt = cp->xt;
  if (xt == nullptr) {
    const rsrc_t xr = make_rsrc(cp->x, (uint32_t)(M * K * EB));
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
  } else {
    // 2a. one lane polls the producer's done counter
    if (tid == 0) {
      const uint32_t *cnt = done + cp->dep;
      const uint32_t need = cp->dep_items;
      const uint64_t t0 = now_ticks();
      int ab = 0;
      while (ld_agent(cnt) < need) {
        if (ld_agent(&hdr->error) != 0u) { ab = 1; break; }
        if (now_ticks() - t0 > wait_ticks) {
          __hip_atomic_fetch_or(&hdr->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ab = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      sh.abort_ = ab;
    }
    __syncthreads();
    if (sh.abort_) return;
    // 2b. every wave loads its chunks until all tags are this launch's
    const rsrc_t xr = make_rsrc(xt, (uint32_t)(M * K * 4));
    const uint32_t tag2 = tag * 0x10001u;
    const uint64_t t0 = now_ticks();
    while (true) {
      bool ok = true;
#pragma unroll
      for (int c = 0; c < CA; ++c)
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const bool in = m < M && qof(R * c + wh) < nq;
          xa[m][c] = tagged_chunk<DT>(xr, in ? (uint32_t)((m * K + 8 * qof(R * c + wh)) * 4) : kOob,
                                      tag2, in, ok);
        }
      if constexpr (CO > 0) {
        if (w < 4) {
#pragma unroll
          for (int c = 0; c < CO; ++c)
#pragma unroll
            for (int m = 0; m < MR; ++m) {
              const bool in = m < M && qof(2 * c + 1) < nq;
              xo[m][c] = tagged_chunk<DT>(xr, in ? (uint32_t)((m * K + 8 * qof(2 * c + 1)) * 4) : kOob,
                                          tag2, in, ok);
            }
        }
      }
      const bool wave_ok = __builtin_amdgcn_ballot_w64(!ok) == 0;
      if (lane == 0) sh.flag[w] = wave_ok ? 1 : 0;
      __syncthreads();
      int all = 1;
#pragma unroll
      for (int i = 0; i < NW; ++i) all &= sh.flag[i];
      if (all) break;
      if (tid == 0) {
        int ab = 0;
        if (ld_agent(&hdr->error) != 0u) ab = 1;
        else if (now_ticks() - t0 > wait_ticks) {
          __hip_atomic_fetch_or(&hdr->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ab = 1;
        }
        sh.abort_ = ab;
      }
      __syncthreads();
      if (sh.abort_) return;
      __builtin_amdgcn_s_sleep(1);
    }
  }

  const auto live = [&](int r) { return 256 * r + 64 * w4 < nq; };

  // ---- 3. sum of squares (waves 0..3), the library's fixed association
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
          widen<DT>(R == 1 || (r & 1) == 0 ? xa[m][r / R] : xo[m][CO > 0 ? r >> 1 : 0], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss[m] = __builtin_fma((double)f[e], (double)f[e], ss[m]);
        }
      }
#pragma unroll
    for (int m = 0; m < MR; ++m) sh.part_ss[m][w][lane] = ss[m];
  }
  __syncthreads();

  // ---- 4. absmax of the normalized rows
  float r[MR], amax[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const double lsum = (sh.part_ss[m][0][lane] + sh.part_ss[m][1][lane]) +
                        (sh.part_ss[m][2][lane] + sh.part_ss[m][3][lane]);
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
    if (lane == 0) sh.part_max[m][w] = t;
  }
  __syncthreads();

  // ---- 5. int8 codes into LDS, row sums of the codes
  float sc[MR], fscale[MR];
  int rs[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float mx = sh.part_max[m][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) mx = fmaxf(mx, sh.part_max[m][i]);
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
    if (lane == 0) sh.part_rs[m][w] = t;
  }
  __syncthreads();

  // ---- 6. contraction: the wave's tiles kb = w + NW t
  const int nmine = w < KB ? (KB - w + NW - 1) / NW : 0;
  const int arow = lane & 15;
  const bool arow_ok = arow < M;
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
        if (t0 + j < TPW && arow_ok && t0 + j < nmine)
          a[j][s2] = *reinterpret_cast<const v4i *>(abase + (w + NW * (t0 + j)) * 128 + 16 * s2);
      }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (t0 + j >= TPW || t0 + j >= nmine) break;
      const v4i u = wt[t0 + j];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        acc0[s2] = mfma16x16x64(a[j][s2], unpack_codes((uint32_t)(s2 ? u.y : u.x)), acc0[s2]);
        acc1[s2] = mfma16x16x64(a[j][s2], unpack_codes((uint32_t)(s2 ? u.w : u.z)), acc1[s2]);
      }
    }
  }

  // ---- 7. partial sums meet in LDS; rescale, store plain and tagged
  if (lane < 16) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      sh.red[w][m][0][lane] = acc0[0][m] + acc0[1][m];
      sh.red[w][m][1][lane] = acc1[0][m] + acc1[1][m];
    }
  }
  __syncthreads();
  const auto tile_sum = [&](int m, int h, int l) {
    int v = sh.red[0][m][h][l];
#pragma unroll
    for (int i = 1; i < NW; ++i) v += sh.red[i][m][h][l];
    return v;
  };
  const auto row_sum = [&](int m) {
    int v = sh.part_rs[m][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) v += sh.part_rs[m][i];
    return v;
  };
  void *out = cp->y;
  uint32_t *yt = cp->yt;
  if (glu) {
    if (tid < 16 * M) {
      const int m = tid >> 4, l = tid & 15;
      const int rsum = row_sum(m);
      const int vg = tile_sum(m, 0, l) - rsum;
      const int vu = tile_sum(m, 1, l) - rsum;
      float fs = 0.0f;
#pragma unroll
      for (int i = 0; i < MR; ++i)
        if (i == m) fs = fscale[i];
      const float v = silu((float)vg * fs) * ((float)vu * fs);
      const int64_t idx = (int64_t)m * tiles * 16 + nt * 16 + l;
      store1<DT>(out, idx, v);
      if (yt) store_tagged<DT>(yt, idx, v, tag);
    }
  } else if (tid < 32 * M) {
    const int m = tid >> 5, n = tid & 31;
    const int h = n >> 4, l = n & 15;
    const int v = tile_sum(m, h, l) - row_sum(m);
    float fs = 0.0f;
#pragma unroll
    for (int i = 0; i < MR; ++i)
      if (i == m) fs = fscale[i];
    const float yv = (float)v * fs;
    const int64_t idx = (int64_t)m * tiles * 32 + nt * 32 + n;
    store1<DT>(out, idx, yv);
    if (yt) store_tagged<DT>(yt, idx, yv, tag);
  }
}

template <int DT, int MR>
__global__ __launch_bounds__(64 * kNW) void chain_kernel(ChainHdr *hdr, const ChainCall *calls,
                                                        const uint32_t *item0_g, uint32_t *done,
                                                        uint32_t wait_us) {
  extern __shared__ __align__(16) int8_t dyn[];
  __shared__ ItemShared sh;
  __shared__ uint32_t s_item, s_call, s_last;

  const int tid = threadIdx.x;
  const uint32_t ncalls = hdr->ncalls, total = hdr->total, kmax = hdr->kmax;
  const int M = (int)hdr->M;
  const float eps = hdr->eps;
  const uint32_t epoch = __builtin_amdgcn_readfirstlane(ld_agent(&hdr->epoch));
  const uint32_t tag = tag_of(epoch);
  const uint64_t wait_ticks = (uint64_t)wait_us * 100u;  // s_memrealtime runs at 100 MHz
  int8_t *xs = dyn;
  uint32_t *item0 = reinterpret_cast<uint32_t *>(dyn + (((size_t)M * (kmax + 16) + 15) & ~size_t(15)));
  for (uint32_t i = tid; i <= ncalls; i += 64 * kNW) item0[i] = item0_g[i];
  if (tid == 0) s_item = __hip_atomic_fetch_add(&hdr->work, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  uint32_t item = s_item;
  while (item < total) {
    uint32_t next = 0;
    if (tid == 0) next = __hip_atomic_fetch_add(&hdr->work, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (uint32_t j = tid; j < ncalls; j += 64 * kNW)
      if (item0[j] <= item && item < item0[j + 1]) s_call = j;
    __syncthreads();
    const uint32_t c = __builtin_amdgcn_readfirstlane(s_call);
    const ChainCall *cp = calls + c;
    const int nt = (int)(item - cp->item0);
    switch (chain_kc(cp->K)) {
      case 1: chain_item<DT, MR, 1>(cp, nt, M, eps, tag, hdr, done, wait_ticks, xs, sh); break;
      case 2: chain_item<DT, MR, 2>(cp, nt, M, eps, tag, hdr, done, wait_ticks, xs, sh); break;
      case 3: chain_item<DT, MR, 3>(cp, nt, M, eps, tag, hdr, done, wait_ticks, xs, sh); break;
      case 4: chain_item<DT, MR, 4>(cp, nt, M, eps, tag, hdr, done, wait_ticks, xs, sh); break;
      case 6: chain_item<DT, MR, 6>(cp, nt, M, eps, tag, hdr, done, wait_ticks, xs, sh); break;
      default: chain_item<DT, MR, 8>(cp, nt, M, eps, tag, hdr, done, wait_ticks, xs, sh); break;
    }
    // every thread is past the item (its stores issued); count it done
    __syncthreads();
    if (tid == 0) {
      __hip_atomic_fetch_add(done + c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_item = next;
    }
    __syncthreads();
    item = s_item;
  }
  // the last workgroup out resets the counters and advances the tag
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&hdr->exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             gridDim.x - 1;
  __syncthreads();
  if (s_last) {
    for (uint32_t i = tid; i < ncalls; i += 64 * kNW)
      __hip_atomic_store(done + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
      __hip_atomic_store(&hdr->work, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&hdr->exits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&hdr->epoch, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Workspace layout: header | call table | item0[ncalls + 1] | done[ncalls] |
// tagged outputs of the calls a later call reads.
struct ChainLayout {
  size_t calls, item0, done, tagged, total;
};

ChainLayout layout(int ncalls, const std::vector<size_t> &tagged_bytes) {
  ChainLayout L;
  L.calls = 256;
  L.item0 = L.calls + align256((size_t)ncalls * sizeof(ChainCall));
  L.done = L.item0 + align256(((size_t)ncalls + 1) * 4);
  L.tagged = L.done + align256((size_t)ncalls * 4);
  size_t t = L.tagged;
  for (size_t b : tagged_bytes) t += align256(b);
  L.total = t;
  return L;
}

// Resident workgroups of a chain kernel on the current device.
template <int DT, int MR>
int resident_groups(size_t lds) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, chain_kernel<DT, MR>, 64 * kNW, lds) !=
      hipSuccess)
    return 0;
  return cus * std::max(per, 1);
}

}  // namespace

size_t chain_workspace_bytes(const ChainPlanIn &in) {
  std::vector<size_t> tb;
  for (int i = 0; i < in.ncalls; ++i)
    if (in.consumed[i]) tb.push_back((size_t)in.M * (size_t)in.n_out[i] * 4);
  return layout(in.ncalls, tb).total;
}

hipError_t chain_plan(const ChainPlanIn &in, void *ws, bl_chain &out, hipStream_t stream) {
  std::vector<size_t> tb;
  for (int i = 0; i < in.ncalls; ++i)
    if (in.consumed[i]) tb.push_back((size_t)in.M * (size_t)in.n_out[i] * 4);
  const ChainLayout L = layout(in.ncalls, tb);
  char *base = static_cast<char *>(ws);
  std::vector<char> img(L.tagged, 0);
  ChainHdr *h = reinterpret_cast<ChainHdr *>(img.data());
  h->epoch = 1;
  h->ncalls = (uint32_t)in.ncalls;
  h->M = (uint32_t)in.M;
  h->eps = in.eps;
  ChainCall *cc = reinterpret_cast<ChainCall *>(img.data() + L.calls);
  uint32_t *item0 = reinterpret_cast<uint32_t *>(img.data() + L.item0);
  std::vector<uint32_t *> tagged(in.ncalls, nullptr);
  size_t t = L.tagged;
  for (int i = 0; i < in.ncalls; ++i)
    if (in.consumed[i]) {
      tagged[i] = reinterpret_cast<uint32_t *>(base + t);
      t += align256((size_t)in.M * (size_t)in.n_out[i] * 4);
    }
  uint32_t items = 0, kmax = 0;
  for (int i = 0; i < in.ncalls; ++i) {
    const bl_chain_call &c = in.calls[i];
    ChainCall &d = cc[i];
    d.x = in.dep[i] < 0 ? c.x : nullptr;
    d.xt = in.dep[i] < 0 ? nullptr : tagged[in.dep[i]];
    d.gain = c.gain;
    d.packed = reinterpret_cast<const uint4 *>(c.packed);
    d.beta = c.beta;
    d.y = c.y;
    d.yt = tagged[i];
    d.K = (uint32_t)c.K;
    d.N = (uint32_t)c.N;
    d.glu = c.glu ? 1u : 0u;
    d.item0 = items;
    d.dep = in.dep[i];
    d.dep_items = in.dep[i] < 0 ? 0u : (uint32_t)(in.calls[in.dep[i]].N / 32);
    item0[i] = items;
    items += (uint32_t)(c.N / 32);
    kmax = std::max(kmax, (uint32_t)c.K);
  }
  item0[in.ncalls] = items;
  h->total = items;
  h->kmax = kmax;
  hipError_t e = hipMemcpyAsync(ws, img.data(), img.size(), hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return e;
  if (L.total > L.tagged) {
    e = hipMemsetAsync(base + L.tagged, 0, L.total - L.tagged, stream);
    if (e != hipSuccess) return e;
  }
  e = hipStreamSynchronize(stream);  // the host image goes out of scope
  if (e != hipSuccess) return e;
  const size_t lds = (((size_t)in.M * (size_t)(kmax + 16) + 15) & ~size_t(15)) +
                     ((size_t)in.ncalls + 1) * 4;
  int res = 0;
  if (in.dtype == BL_F16) res = in.M == 1 ? resident_groups<BL_F16, 1>(lds) : resident_groups<BL_F16, 4>(lds);
  else res = in.M == 1 ? resident_groups<BL_BF16, 1>(lds) : resident_groups<BL_BF16, 4>(lds);
  if (res <= 0) return hipErrorInvalidConfiguration;
  out.ws = ws;
  out.M = in.M;
  out.dtype = in.dtype;
  out.ncalls = in.ncalls;
  out.items = items;
  out.kmax = kmax;
  out.grid = std::min<int64_t>(res, items);
  out.lds = (int64_t)lds;
  return hipSuccess;
}

hipError_t chain_run(const bl_chain &p, uint32_t wait_us, hipStream_t stream) {
  std::vector<size_t> none;
  const ChainLayout L = layout(p.ncalls, none);
  char *base = static_cast<char *>(p.ws);
  ChainHdr *hdr = reinterpret_cast<ChainHdr *>(base);
  const ChainCall *calls = reinterpret_cast<const ChainCall *>(base + L.calls);
  const uint32_t *item0 = reinterpret_cast<const uint32_t *>(base + L.item0);
  uint32_t *done = reinterpret_cast<uint32_t *>(base + L.done);
  const size_t lds = (size_t)p.lds;
  const unsigned grid = (unsigned)p.grid;
#define BL_CHAIN(DT_, MR_) \
  chain_kernel<DT_, MR_><<<grid, 64 * kNW, lds, stream>>>(hdr, calls, item0, done, wait_us)
  if (p.dtype == BL_F16) {
    if (p.M == 1) BL_CHAIN(BL_F16, 1); else BL_CHAIN(BL_F16, 4);
  } else {
    if (p.M == 1) BL_CHAIN(BL_BF16, 1); else BL_CHAIN(BL_BF16, 4);
  }
#undef BL_CHAIN
  return hipGetLastError();
}

hipError_t chain_error(const bl_chain &p, uint32_t *err, hipStream_t stream) {
  ChainHdr *hdr = static_cast<ChainHdr *>(p.ws);
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  e = hipMemcpy(err, &hdr->error, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  if (*err) {
    const uint32_t zero = 0;
    e = hipMemcpy(&hdr->error, &zero, 4, hipMemcpyHostToDevice);
  }
  return e;
}

}  // namespace bl
