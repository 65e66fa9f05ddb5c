// capi.cpp -- the extern "C" boundary of libbitlinear.so.
//
// Every entry point validates all of its arguments on the host before it
// launches anything (so a rejected call touches no memory and needs no GPU),
// then dispatches to the kernel launchers in bl_launch.h.  No exception
// crosses the boundary; every failure is a negative status code.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "bitlinear.h"
#include "bl_launch.h"

namespace {

constexpr int64_t kMaxK = 65536;
constexpr int64_t kMaxN = int64_t(1) << 20;
constexpr int64_t kMaxM = int64_t(1) << 24;
// dynamic LDS the fused skinny kernel may use: 64 KiB minus its static part
// (8320 bytes) and some slack
constexpr int64_t kFusedLdsBytes = 65536 - 9216;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(int dt) { return dt == BL_F32 || dt == BL_F16 || dt == BL_BF16; }

bool nk_ok(int64_t N, int64_t K) {
  return K >= 128 && K <= kMaxK && K % 128 == 0 && N >= 32 && N <= kMaxN && N % 32 == 0;
}

bool m_ok(int64_t M) { return M >= 0 && M <= kMaxM; }

bool eps_ok(float eps) { return std::isfinite(eps) && eps > 0.0f; }

int hip_status(hipError_t e) { return e == hipSuccess ? BL_OK : BL_ERR_HIP; }

// Test hook (bitlinear_test_fail_launches): the next n launcher calls report
// a launch failure instead of launching, so the path of a failed HIP launch
// to the caller can be driven from the host without a GPU.
std::atomic<int> g_fail_launches{0};

bool forced_failure() {
  int n = g_fail_launches.load(std::memory_order_relaxed);
  while (n > 0)
    if (g_fail_launches.compare_exchange_weak(n, n - 1, std::memory_order_relaxed)) return true;
  return false;
}

#define BL_LAUNCH(call) (forced_failure() ? hipErrorLaunchFailure : (call))

// Forward workspace: xq [M, K] int8 | s [M] fp32 | rowsum [M] int32.
struct FwdWs {
  int8_t *xq;
  float *s;
  int32_t *rowsum;
};

size_t fwd_ws_bytes(int64_t M, int64_t K) {
  return align256((size_t)(M * K)) + 2 * align256((size_t)M * 4);
}

FwdWs carve(void *ws, int64_t M, int64_t K) {
  char *b = static_cast<char *>(ws);
  FwdWs w;
  w.xq = reinterpret_cast<int8_t *>(b);
  b += align256((size_t)(M * K));
  w.s = reinterpret_cast<float *>(b);
  b += align256((size_t)M * 4);
  w.rowsum = reinterpret_cast<int32_t *>(b);
  return w;
}

// The contraction half of the two-kernel path on the skinny kernel: a call
// from pre-quantized activations (xq, s, rowsum as the act-quant writes them).
bl::SkinnyArgs pre_call(const int8_t *xq, const float *s, const int32_t *rowsum,
                        const void *packed, const float *beta, int64_t M, int64_t N, int64_t K,
                        void *out, int out_kind, bool glu = false) {
  bl::SkinnyArgs a{};
  a.fused = false;
  a.xq = xq;
  a.s = s;
  a.rowsum = rowsum;
  a.packed = packed;
  a.beta = beta;
  a.M = M;
  a.N = N;
  a.K = K;
  a.out = out;
  a.out_kind = out_kind;
  a.glu = glu;
  return a;
}

bool fused_fits(int64_t M, int64_t K) {
  return M >= 1 && M <= bl::kFusedMaxM && K <= bl::kFusedMaxK && M * (K + 16) <= kFusedLdsBytes;
}

// Default path by token count: the one-launch decode kernel wherever it
// applies (split mode M <= 4 up to K = 8192, fp32 activations M == 1; row
// mode up to 16 rows as decode_rows_fits allows), then the act-quant +
// skinny pair up to 64 tokens, then the MFMA GEMM.
int auto_path(int64_t M, int64_t K, int x_dtype) {
  if (M <= 4 && fused_fits(M, K) && (x_dtype != BL_F32 || bl::decode_fits(M, K, x_dtype)))
    return BL_PATH_FUSED;
  if (bl::decode_rows_fits(M, K, x_dtype)) return BL_PATH_FUSED;
  if (M <= bl::kSkinnyMaxM) return BL_PATH_SKINNY;
  return BL_PATH_MFMA;
}

}  // namespace

namespace {

// bitlinear_set_decode_contraction's process-wide setting.  BL_DECODE_AUTO
// takes the matrix cores: on the 2.7B decode calls the VALU contraction ran
// 2-3 % slower at 1 token and 5-7 % at 2 (it adds 16 v_dot4 per tile to the
// unpack both units pay, while the MFMAs overlap that VALU stream).
std::atomic<int> g_decode_unit{BL_DECODE_AUTO};
constexpr bool kAutoDecodeValu = false;

}  // namespace

namespace bl {
bool decode_use_valu() {
  const int u = g_decode_unit.load(std::memory_order_relaxed);
  return u == BL_DECODE_VALU || (u == BL_DECODE_AUTO && kAutoDecodeValu);
}
}  // namespace bl

extern "C" {

void bitlinear_test_fail_launches(int n) { g_fail_launches.store(n > 0 ? n : 0); }

int bitlinear_set_decode_contraction(int unit) {
  if (unit != BL_DECODE_AUTO && unit != BL_DECODE_MFMA && unit != BL_DECODE_VALU)
    return BL_ERR_PATH;
  g_decode_unit.store(unit, std::memory_order_relaxed);
  return BL_OK;
}

int bitlinear_get_decode_contraction(void) { return g_decode_unit.load(std::memory_order_relaxed); }

const char *bitlinear_status_string(int status) {
  switch (status) {
    case BL_OK: return "ok";
    case BL_ERR_NULL: return "null pointer";
    case BL_ERR_DTYPE: return "unsupported dtype";
    case BL_ERR_SHAPE: return "unsupported shape";
    case BL_ERR_ALIGN: return "pointer not 16-byte aligned";
    case BL_ERR_WORKSPACE: return "workspace missing or too small";
    case BL_ERR_EPS: return "eps must be finite and > 0";
    case BL_ERR_HIP: return "HIP launch failed";
    case BL_ERR_UNSUPPORTED: return "unsupported request";
    case BL_ERR_PATH: return "unknown or inapplicable execution path";
    case BL_ERR_SCRATCH: return "request needs more than the library's static scratch (32 MiB)";
    case BL_ERR_TIMEOUT: return "a chained launch gave up waiting for an input";
    default: return "unknown status";
  }
}

int bitlinear_select_path(int64_t M, int64_t K) {
  if (!m_ok(M) || M == 0 || K < 128 || K > kMaxK || K % 128 != 0) return BL_ERR_SHAPE;
  return auto_path(M, K, BL_BF16);
}

size_t bitlinear_packed_bytes(int64_t N, int64_t K) {
  return nk_ok(N, K) ? (size_t)(N * K / 4) : 0;
}

size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K) {
  return nk_ok(N, K) ? bl::pack_workspace_bytes() : 0;
}

int bitlinear_pack_weights(const float *W, int64_t N, int64_t K, void *packed,
                           float *beta, void *ws, size_t ws_bytes,
                           hipStream_t stream) {
  if (!nk_ok(N, K)) return BL_ERR_SHAPE;
  if (!W || !packed || !beta) return BL_ERR_NULL;
  if (!ws || ws_bytes < bl::pack_workspace_bytes()) return BL_ERR_WORKSPACE;
  if (!aligned16(W) || !aligned16(packed) || !aligned16(ws) ||
      (reinterpret_cast<uintptr_t>(beta) & 3u))
    return BL_ERR_ALIGN;
  return hip_status(BL_LAUNCH(bl::launch_pack(W, N, K, packed, beta, ws, 0, stream)));
}

int bitlinear_pack_glu_weights(const float *W, int64_t F, int64_t K, void *packed, float *beta,
                               void *ws, size_t ws_bytes, hipStream_t stream) {
  if (F <= 0 || F % 16 != 0 || !nk_ok(2 * F, K)) return BL_ERR_SHAPE;
  if (!W || !packed || !beta) return BL_ERR_NULL;
  if (!ws || ws_bytes < bl::pack_workspace_bytes()) return BL_ERR_WORKSPACE;
  if (!aligned16(W) || !aligned16(packed) || !aligned16(ws) ||
      (reinterpret_cast<uintptr_t>(beta) & 3u))
    return BL_ERR_ALIGN;
  return hip_status(BL_LAUNCH(bl::launch_pack(W, 2 * F, K, packed, beta, ws, F, stream)));
}

size_t bitlinear_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (!nk_ok(N, K) || !m_ok(M)) return 0;
  return fwd_ws_bytes(M, K);
}

}  // extern "C"

namespace {

// The forward of bitlinear_forward_path (glu = false: y [M, N]) and of
// bitlinear_forward_glu (glu = true: N = 2F packed rows in GLU order, y is
// h [M, F]).  The fused path takes a GLU call only where the decode kernel
// does (decode_fits).
int forward_impl(const void *x, int x_dtype, int64_t M, int64_t K, const void *gain,
                 const void *packed, const float *beta, int64_t N, void *y, int y_dtype,
                 float eps, void *ws, size_t ws_bytes, int path, bool glu, hipStream_t stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return BL_ERR_DTYPE;
  if (!nk_ok(N, K) || !m_ok(M)) return BL_ERR_SHAPE;
  if (!eps_ok(eps)) return BL_ERR_EPS;
  if (path < BL_PATH_AUTO || path > BL_PATH_MFMA) return BL_ERR_PATH;
  if (M == 0) return BL_OK;
  if (!x || !gain || !packed || !beta || !y) return BL_ERR_NULL;
  if (!ws || ws_bytes < fwd_ws_bytes(M, K)) return BL_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(gain) || !aligned16(packed) || !aligned16(y) ||
      !aligned16(ws) || (reinterpret_cast<uintptr_t>(beta) & 3u))
    return BL_ERR_ALIGN;
  if (path == BL_PATH_AUTO) path = auto_path(M, K, x_dtype);
  if (glu && path == BL_PATH_FUSED && !bl::decode_fits(M, K, x_dtype))
    path = M <= bl::kSkinnyMaxM ? BL_PATH_SKINNY : BL_PATH_MFMA;
  if (path == BL_PATH_FUSED && !fused_fits(M, K)) return BL_ERR_SHAPE;
  if (path == BL_PATH_SKINNY && M > bl::kSkinnyMaxM) return BL_ERR_SHAPE;

  if (path == BL_PATH_FUSED) {
    bl::SkinnyArgs a{};
    a.fused = true;
    a.x = x;
    a.x_dtype = x_dtype;
    a.gain = gain;
    a.eps = eps;
    a.packed = packed;
    a.beta = beta;
    a.M = M;
    a.N = N;
    a.K = K;
    a.out = y;
    a.out_kind = y_dtype;
    a.glu = glu;
    return hip_status(BL_LAUNCH(bl::launch_skinny(a, stream)));
  }
  const FwdWs w = carve(ws, M, K);
  hipError_t e = BL_LAUNCH(bl::launch_act_quant(x, x_dtype, gain, M, K, eps, w.xq, w.s, w.rowsum, stream));
  if (e != hipSuccess) return BL_ERR_HIP;
  if (path == BL_PATH_SKINNY)
    return hip_status(BL_LAUNCH(bl::launch_skinny(
        pre_call(w.xq, w.s, w.rowsum, packed, beta, M, N, K, y, y_dtype, glu), stream)));
  return hip_status(BL_LAUNCH(bl::launch_gemm_mfma(w.xq, w.rowsum, w.s, packed, beta, M, N, K, y,
                                         y_dtype, glu, stream)));
}

}  // namespace

extern "C" {

int bitlinear_forward_path(const void *x, int x_dtype, int64_t M, int64_t K,
                           const void *gain, const void *packed,
                           const float *beta, int64_t N, void *y, int y_dtype,
                           float eps, void *ws, size_t ws_bytes, int path,
                           hipStream_t stream) {
  return forward_impl(x, x_dtype, M, K, gain, packed, beta, N, y, y_dtype, eps, ws, ws_bytes,
                      path, false, stream);
}

int bitlinear_forward_glu(const void *x, int x_dtype, int64_t M, int64_t K, const void *gain,
                          const void *packed, const float *beta, int64_t F, void *h,
                          int h_dtype, float eps, void *ws, size_t ws_bytes, int path,
                          hipStream_t stream) {
  if (F <= 0 || F % 16 != 0) return BL_ERR_SHAPE;
  return forward_impl(x, x_dtype, M, K, gain, packed, beta, 2 * F, h, h_dtype, eps, ws,
                      ws_bytes, path, true, stream);
}

int bitlinear_forward(const void *x, int x_dtype, int64_t M, int64_t K,
                      const void *gain, const void *packed, const float *beta,
                      int64_t N, void *y, int y_dtype, float eps, void *ws,
                      size_t ws_bytes, hipStream_t stream) {
  return bitlinear_forward_path(x, x_dtype, M, K, gain, packed, beta, N, y, y_dtype, eps, ws,
                                ws_bytes, BL_PATH_AUTO, stream);
}

int bitlinear_forward_grouped(const bl_call *calls, int ncalls, int x_dtype,
                              int y_dtype, float eps, hipStream_t stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return BL_ERR_DTYPE;
  if (!eps_ok(eps)) return BL_ERR_EPS;
  if (ncalls < 0 || ncalls > 4096) return BL_ERR_SHAPE;
  if (ncalls == 0) return BL_OK;
  if (!calls) return BL_ERR_NULL;
  std::vector<bl::SkinnyArgs> args;
  args.reserve((size_t)ncalls);
  for (int i = 0; i < ncalls; ++i) {
    const bl_call &c = calls[i];
    if (!nk_ok(c.N, c.K) || !m_ok(c.M)) return BL_ERR_SHAPE;
    if (c.M == 0) continue;
    if (!fused_fits(c.M, c.K)) return BL_ERR_SHAPE;
    if (!c.x || !c.gain || !c.packed || !c.beta || !c.y) return BL_ERR_NULL;
    if (!aligned16(c.x) || !aligned16(c.gain) || !aligned16(c.packed) || !aligned16(c.y) ||
        (reinterpret_cast<uintptr_t>(c.beta) & 3u))
      return BL_ERR_ALIGN;
    bl::SkinnyArgs a{};
    a.fused = true;
    a.x = c.x;
    a.x_dtype = x_dtype;
    a.gain = c.gain;
    a.eps = eps;
    a.packed = c.packed;
    a.beta = c.beta;
    a.M = c.M;
    a.N = c.N;
    a.K = c.K;
    a.out = c.y;
    a.out_kind = y_dtype;
    args.push_back(a);
  }
  if (args.empty()) return BL_OK;
  return hip_status(BL_LAUNCH(bl::launch_skinny_grouped(args.data(), (int)args.size(), stream)));
}

}  // extern "C"

namespace {

// The plan of bitlinear_forward_grouped_ws: calls the fused kernels take
// (default path FUSED) go out together as in bitlinear_forward_grouped;
// every other call runs its two-kernel path, and up to kGroupCalls
// consecutive calls of one shape (M, K, N) and path form one run that shares
// an act-quant launch (and, on the MFMA path, a GEMM launch; skinny-path
// calls keep one contraction launch each).  Runs execute one after another
// on the stream, so they share the workspace.
struct GroupRun {
  int first, n, path;
};

int plan_grouped(const bl_call *calls, int ncalls, int x_dtype, std::vector<GroupRun> &runs,
                 std::vector<int> &fused, size_t &ws_need) {
  if (!dtype_ok(x_dtype)) return BL_ERR_DTYPE;
  if (ncalls < 0 || ncalls > 4096) return BL_ERR_SHAPE;
  if (ncalls > 0 && !calls) return BL_ERR_NULL;
  ws_need = 0;
  for (int i = 0; i < ncalls; ++i) {
    const bl_call &c = calls[i];
    if (!nk_ok(c.N, c.K) || !m_ok(c.M)) return BL_ERR_SHAPE;
    if (c.M == 0) continue;
    const int path = auto_path(c.M, c.K, x_dtype);
    if (path == BL_PATH_FUSED) {
      fused.push_back(i);
      continue;
    }
    if (!runs.empty()) {
      GroupRun &r = runs.back();
      const bl_call &p = calls[r.first];
      if (r.path == path && r.first + r.n == i && r.n < bl::kGroupCalls && p.M == c.M &&
          p.K == c.K && p.N == c.N) {
        ++r.n;
        ws_need = std::max(ws_need, (size_t)r.n * fwd_ws_bytes(c.M, c.K));
        continue;
      }
    }
    runs.push_back(GroupRun{i, 1, path});
    ws_need = std::max(ws_need, fwd_ws_bytes(c.M, c.K));
  }
  return BL_OK;
}

}  // namespace

extern "C" {

size_t bitlinear_grouped_workspace_bytes(const bl_call *calls, int ncalls, int x_dtype) {
  std::vector<GroupRun> runs;
  std::vector<int> fused;
  size_t need = 0;
  return plan_grouped(calls, ncalls, x_dtype, runs, fused, need) == BL_OK ? need : 0;
}

int bitlinear_forward_grouped_ws(const bl_call *calls, int ncalls, int x_dtype, int y_dtype,
                                 float eps, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return BL_ERR_DTYPE;
  if (!eps_ok(eps)) return BL_ERR_EPS;
  std::vector<GroupRun> runs;
  std::vector<int> fused;
  size_t need = 0;
  const int st = plan_grouped(calls, ncalls, x_dtype, runs, fused, need);
  if (st != BL_OK) return st;
  for (int i = 0; i < ncalls; ++i) {
    const bl_call &c = calls[i];
    if (c.M == 0) continue;
    if (!c.x || !c.gain || !c.packed || !c.beta || !c.y) return BL_ERR_NULL;
    if (!aligned16(c.x) || !aligned16(c.gain) || !aligned16(c.packed) || !aligned16(c.y) ||
        (reinterpret_cast<uintptr_t>(c.beta) & 3u))
      return BL_ERR_ALIGN;
  }
  if (need > 0) {
    if (!ws || ws_bytes < need) return BL_ERR_WORKSPACE;
    if (!aligned16(ws)) return BL_ERR_ALIGN;
  }
  for (const GroupRun &r : runs) {
    const bl_call &c0 = calls[r.first];
    if (r.n == 1) {
      const int e = forward_impl(c0.x, x_dtype, c0.M, c0.K, c0.gain, c0.packed, c0.beta, c0.N,
                                 c0.y, y_dtype, eps, ws, ws_bytes, r.path, false, stream);
      if (e != BL_OK) return e;
      continue;
    }
    const size_t stride = fwd_ws_bytes(c0.M, c0.K);
    bl::AqCalls aq{};
    bl::GemmCalls gm{};
    for (int j = 0; j < r.n; ++j) {
      const bl_call &c = calls[r.first + j];
      const FwdWs w = carve(static_cast<char *>(ws) + j * stride, c.M, c.K);
      aq.c[j] = bl::AqCall{c.x, c.gain, w.xq, w.s, w.rowsum};
      gm.c[j] = bl::GemmCall{w.xq, w.rowsum, w.s, c.packed, c.beta, c.y};
    }
    if (BL_LAUNCH(bl::launch_act_quant_group(aq, r.n, x_dtype, c0.M, c0.K, eps, stream)) != hipSuccess)
      return BL_ERR_HIP;
    if (r.path == BL_PATH_MFMA) {
      if (BL_LAUNCH(bl::launch_gemm_mfma_group(gm, r.n, c0.M, c0.N, c0.K, y_dtype, stream)) != hipSuccess)
        return BL_ERR_HIP;
      continue;
    }
    bl::SkinnyArgs sk[bl::kGroupCalls];
    for (int j = 0; j < r.n; ++j)
      sk[j] = pre_call(gm.c[j].xq, gm.c[j].s, gm.c[j].rowsum, gm.c[j].packed, gm.c[j].beta, c0.M,
                       c0.N, c0.K, gm.c[j].out, y_dtype);
    if (BL_LAUNCH(bl::launch_skinny_pre_grouped(sk, r.n, stream)) != hipSuccess) return BL_ERR_HIP;
  }
  if (!fused.empty()) {
    std::vector<bl::SkinnyArgs> args;
    for (const int i : fused) {
      const bl_call &c = calls[i];
      bl::SkinnyArgs a{};
      a.fused = true;
      a.x = c.x;
      a.x_dtype = x_dtype;
      a.gain = c.gain;
      a.eps = eps;
      a.packed = c.packed;
      a.beta = c.beta;
      a.M = c.M;
      a.N = c.N;
      a.K = c.K;
      a.out = c.y;
      a.out_kind = y_dtype;
      args.push_back(a);
    }
    return hip_status(BL_LAUNCH(bl::launch_skinny_grouped(args.data(), (int)args.size(), stream)));
  }
  return BL_OK;
}

int bitlinear_act_quant(const void *x, int x_dtype, const void *gain,
                        int64_t M, int64_t K, float eps, int8_t *xq, float *s,
                        int32_t *rowsum, hipStream_t stream) {
  if (!dtype_ok(x_dtype)) return BL_ERR_DTYPE;
  if (!m_ok(M) || K < 128 || K > kMaxK || K % 128 != 0) return BL_ERR_SHAPE;
  if (!eps_ok(eps)) return BL_ERR_EPS;
  if (M == 0) return BL_OK;
  if (!x || !gain || !xq || !s || !rowsum) return BL_ERR_NULL;
  if (!aligned16(x) || !aligned16(gain) || !aligned16(xq) ||
      (reinterpret_cast<uintptr_t>(s) & 3u) || (reinterpret_cast<uintptr_t>(rowsum) & 3u))
    return BL_ERR_ALIGN;
  return hip_status(BL_LAUNCH(bl::launch_act_quant(x, x_dtype, gain, M, K, eps, xq, s, rowsum, stream)));
}

int bitlinear_gemm_i32(const int8_t *xq, const int32_t *rowsum, int64_t M,
                       int64_t K, const void *packed, int64_t N, int32_t *acc,
                       int path, hipStream_t stream) {
  if (!nk_ok(N, K) || !m_ok(M)) return BL_ERR_SHAPE;
  if (path != BL_PATH_AUTO && path != BL_PATH_SKINNY && path != BL_PATH_MFMA) return BL_ERR_PATH;
  if (M == 0) return BL_OK;
  if (!xq || !rowsum || !packed || !acc) return BL_ERR_NULL;
  if (!aligned16(xq) || !aligned16(packed) || !aligned16(acc) ||
      (reinterpret_cast<uintptr_t>(rowsum) & 3u))
    return BL_ERR_ALIGN;
  if (path == BL_PATH_AUTO) path = M <= bl::kSkinnyMaxM ? BL_PATH_SKINNY : BL_PATH_MFMA;
  if (path == BL_PATH_SKINNY && M > bl::kSkinnyMaxM) return BL_ERR_SHAPE;
  if (path == BL_PATH_SKINNY)
    return hip_status(BL_LAUNCH(bl::launch_skinny(
        pre_call(xq, nullptr, rowsum, packed, nullptr, M, N, K, acc, bl::kOutI32), stream)));
  return hip_status(BL_LAUNCH(bl::launch_gemm_mfma(xq, rowsum, nullptr, packed, nullptr, M, N, K, acc,
                                         bl::kOutI32, false, stream)));
}

int bitlinear_contract(const int8_t *xq, const float *s, const int32_t *rowsum,
                       int64_t M, int64_t K, const void *packed,
                       const float *beta, int64_t N, void *y, int y_dtype,
                       int path, hipStream_t stream) {
  if (!dtype_ok(y_dtype)) return BL_ERR_DTYPE;
  if (!nk_ok(N, K) || !m_ok(M)) return BL_ERR_SHAPE;
  if (path != BL_PATH_AUTO && path != BL_PATH_SKINNY && path != BL_PATH_MFMA) return BL_ERR_PATH;
  if (M == 0) return BL_OK;
  if (!xq || !s || !rowsum || !packed || !beta || !y) return BL_ERR_NULL;
  if (!aligned16(xq) || !aligned16(packed) || !aligned16(y) ||
      (reinterpret_cast<uintptr_t>(s) & 3u) || (reinterpret_cast<uintptr_t>(rowsum) & 3u) ||
      (reinterpret_cast<uintptr_t>(beta) & 3u))
    return BL_ERR_ALIGN;
  if (path == BL_PATH_AUTO) path = M <= bl::kSkinnyMaxM ? BL_PATH_SKINNY : BL_PATH_MFMA;
  if (path == BL_PATH_SKINNY && M > bl::kSkinnyMaxM) return BL_ERR_SHAPE;
  if (path == BL_PATH_SKINNY)
    return hip_status(BL_LAUNCH(bl::launch_skinny(
        pre_call(xq, s, rowsum, packed, beta, M, N, K, y, y_dtype), stream)));
  return hip_status(BL_LAUNCH(bl::launch_gemm_mfma(xq, rowsum, s, packed, beta, M, N, K, y, y_dtype, false,
                                         stream)));
}

int bitlinear_contract_glu(const int8_t *xq, const float *s, const int32_t *rowsum, int64_t M,
                           int64_t K, const void *packed, const float *beta, int64_t F, void *h,
                           int h_dtype, int path, hipStream_t stream) {
  if (!dtype_ok(h_dtype)) return BL_ERR_DTYPE;
  if (F <= 0 || F % 16 != 0 || !nk_ok(2 * F, K) || !m_ok(M)) return BL_ERR_SHAPE;
  if (path != BL_PATH_AUTO && path != BL_PATH_SKINNY && path != BL_PATH_MFMA) return BL_ERR_PATH;
  if (M == 0) return BL_OK;
  if (!xq || !s || !rowsum || !packed || !beta || !h) return BL_ERR_NULL;
  if (!aligned16(xq) || !aligned16(packed) || !aligned16(h) ||
      (reinterpret_cast<uintptr_t>(s) & 3u) || (reinterpret_cast<uintptr_t>(rowsum) & 3u) ||
      (reinterpret_cast<uintptr_t>(beta) & 3u))
    return BL_ERR_ALIGN;
  if (path == BL_PATH_AUTO) path = M <= bl::kSkinnyMaxM ? BL_PATH_SKINNY : BL_PATH_MFMA;
  if (path == BL_PATH_SKINNY && M > bl::kSkinnyMaxM) return BL_ERR_SHAPE;
  if (path == BL_PATH_SKINNY)
    return hip_status(BL_LAUNCH(bl::launch_skinny(
        pre_call(xq, s, rowsum, packed, beta, M, 2 * F, K, h, h_dtype, true), stream)));
  return hip_status(BL_LAUNCH(bl::launch_gemm_mfma(xq, rowsum, s, packed, beta, M, 2 * F, K, h, h_dtype,
                                         true, stream)));
}

int bitlinear_contract_grouped(const bl_contract_call *calls, int ncalls, int y_dtype,
                               hipStream_t stream) {
  return bitlinear_contract_grouped_path(calls, ncalls, y_dtype, BL_PATH_MFMA, stream);
}

int bitlinear_contract_grouped_path(const bl_contract_call *calls, int ncalls, int y_dtype,
                                    int path, hipStream_t stream) {
  if (!dtype_ok(y_dtype)) return BL_ERR_DTYPE;
  if (path != BL_PATH_AUTO && path != BL_PATH_SKINNY && path != BL_PATH_MFMA) return BL_ERR_PATH;
  if (ncalls < 0 || ncalls > 4096) return BL_ERR_SHAPE;
  if (ncalls == 0) return BL_OK;
  if (!calls) return BL_ERR_NULL;
  for (int i = 0; i < ncalls; ++i) {
    const bl_contract_call &c = calls[i];
    if (!nk_ok(c.N, c.K) || !m_ok(c.M)) return BL_ERR_SHAPE;
    if (path == BL_PATH_SKINNY && c.M > bl::kSkinnyMaxM) return BL_ERR_SHAPE;
    if (c.M == 0) continue;
    if (!c.xq || !c.s || !c.rowsum || !c.packed || !c.beta || !c.y) return BL_ERR_NULL;
    if (!aligned16(c.xq) || !aligned16(c.packed) || !aligned16(c.y) ||
        (reinterpret_cast<uintptr_t>(c.s) & 3u) || (reinterpret_cast<uintptr_t>(c.rowsum) & 3u) ||
        (reinterpret_cast<uintptr_t>(c.beta) & 3u))
      return BL_ERR_ALIGN;
  }
  for (int i = 0; i < ncalls;) {
    const bl_contract_call &c0 = calls[i];
    if (c0.M == 0) {
      ++i;
      continue;
    }
    int n = 1;
    while (n < bl::kGroupCalls && i + n < ncalls && calls[i + n].M == c0.M &&
           calls[i + n].K == c0.K && calls[i + n].N == c0.N)
      ++n;
    const bool skinny =
        path == BL_PATH_SKINNY || (path == BL_PATH_AUTO && c0.M <= bl::kSkinnyMaxM);
    bl::GemmCalls gm{};
    bl::SkinnyArgs sk[bl::kGroupCalls];
    for (int j = 0; j < n; ++j) {
      const bl_contract_call &c = calls[i + j];
      gm.c[j] = bl::GemmCall{c.xq, c.rowsum, c.s, c.packed, c.beta, c.y};
      sk[j] = pre_call(c.xq, c.s, c.rowsum, c.packed, c.beta, c.M, c.N, c.K, c.y, y_dtype);
    }
    hipError_t e;
    if (skinny)
      e = n == 1 ? BL_LAUNCH(bl::launch_skinny(sk[0], stream))
                 : BL_LAUNCH(bl::launch_skinny_pre_grouped(sk, n, stream));
    else
      e = n == 1 ? BL_LAUNCH(bl::launch_gemm_mfma(c0.xq, c0.rowsum, c0.s, c0.packed, c0.beta, c0.M,
                                                 c0.N, c0.K, c0.y, y_dtype, false, stream))
                 : BL_LAUNCH(bl::launch_gemm_mfma_group(gm, n, c0.M, c0.N, c0.K, y_dtype, stream));
    if (e != hipSuccess) return BL_ERR_HIP;
    i += n;
  }
  return BL_OK;
}

int bitlinear_unpack_weights(const void *packed, int64_t N, int64_t K,
                             int8_t *Wq, hipStream_t stream) {
  if (!nk_ok(N, K)) return BL_ERR_SHAPE;
  if (!packed || !Wq) return BL_ERR_NULL;
  if (!aligned16(packed) || !aligned16(Wq)) return BL_ERR_ALIGN;
  return hip_status(BL_LAUNCH(bl::launch_unpack(packed, N, K, Wq, stream)));
}

}  // extern "C"

namespace {

// Scratch of bitlinear_forward_noalloc: the int8 activations, per-row scales
// and row sums its act-quant launch writes and its contraction launch reads,
// held in a file-scope device array instead of a caller workspace.  Every
// GPU the library runs on holds its own copy until the process ends.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of each device's copy of `scratch`, looked up once per
// device (the host-side name is only a stand-in for the symbol).
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];

void *scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t bitlinear_noalloc_max_scratch_bytes(void) { return kScratchBytes; }

int bitlinear_forward_noalloc(const void *x, int x_dtype, int64_t M, int64_t K, const void *gain,
                              const void *packed, const float *beta, int64_t N, void *y,
                              int y_dtype, float eps, hipStream_t stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return BL_ERR_DTYPE;
  if (!nk_ok(N, K) || !m_ok(M)) return BL_ERR_SHAPE;
  if (!eps_ok(eps)) return BL_ERR_EPS;
  if (M == 0) return BL_OK;
  if (!x || !gain || !packed || !beta || !y) return BL_ERR_NULL;
  if (!aligned16(x) || !aligned16(gain) || !aligned16(packed) || !aligned16(y) ||
      (reinterpret_cast<uintptr_t>(beta) & 3u))
    return BL_ERR_ALIGN;
  if (fwd_ws_bytes(M, K) > kScratchBytes) return BL_ERR_SCRATCH;
  void *ws = scratch_address();
  if (!ws) return BL_ERR_HIP;
  return forward_impl(x, x_dtype, M, K, gain, packed, beta, N, y, y_dtype, eps, ws,
                      kScratchBytes, BL_PATH_AUTO, false, stream);
}

}  // extern "C"

namespace {

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Validation and dependency analysis of a chain (host only).
int chain_analyse(const bl_chain_call *calls, int ncalls, int64_t M, int dtype,
                  bl::ChainPlanIn &in) {
  if (dtype != BL_F16 && dtype != BL_BF16) return dtype == BL_F32 ? BL_ERR_UNSUPPORTED : BL_ERR_DTYPE;
  if (ncalls < 1 || ncalls > bl::kChainMaxCalls) return BL_ERR_SHAPE;
  if (M < 1 || M > bl::kChainMaxM) return BL_ERR_SHAPE;
  if (!calls) return BL_ERR_NULL;
  in.calls = calls;
  in.ncalls = ncalls;
  in.M = M;
  in.dtype = dtype;
  in.dep.assign(ncalls, -1);
  in.consumed.assign(ncalls, 0);
  in.n_out.assign(ncalls, 0);
  for (int i = 0; i < ncalls; ++i) {
    const bl_chain_call &c = calls[i];
    if (c.glu != 0 && c.glu != 1) return BL_ERR_SHAPE;
    if (!nk_ok(c.N, c.K) || c.K > bl::kFusedMaxK) return BL_ERR_SHAPE;
    if (c.glu && c.N % 64 != 0) return BL_ERR_SHAPE;
    if (!c.x || !c.gain || !c.packed || !c.beta || !c.y) return BL_ERR_NULL;
    if (!aligned16(c.x) || !aligned16(c.gain) || !aligned16(c.packed) || !aligned16(c.y) ||
        (reinterpret_cast<uintptr_t>(c.beta) & 3u))
      return BL_ERR_ALIGN;
    in.n_out[i] = c.glu ? c.N / 2 : c.N;
  }
  const size_t eb = 2;
  for (int i = 0; i < ncalls; ++i) {
    const bl_chain_call &c = calls[i];
    for (int j = i - 1; j >= 0; --j)
      if (calls[j].y == c.x) {
        if (in.n_out[j] != c.K) return BL_ERR_SHAPE;
        in.dep[i] = j;
        in.consumed[j] = 1;
        break;
      }
    if (in.dep[i] >= 0) continue;
    // a plain input must not be written by any call of the chain
    for (int j = 0; j < ncalls; ++j)
      if (overlaps(c.x, (size_t)(M * c.K) * eb, calls[j].y, (size_t)(M * in.n_out[j]) * eb))
        return BL_ERR_UNSUPPORTED;
  }
  return BL_OK;
}

}  // namespace

extern "C" {

size_t bitlinear_chain_workspace_bytes(const bl_chain_call *calls, int ncalls, int64_t M) {
  bl::ChainPlanIn in;
  if (chain_analyse(calls, ncalls, M, BL_BF16, in) != BL_OK) return 0;
  return bl::chain_workspace_bytes(in);
}

int bitlinear_chain_plan(const bl_chain_call *calls, int ncalls, int64_t M, int dtype, float eps,
                         void *ws, size_t ws_bytes, bl_chain *plan, hipStream_t stream) {
  if (!eps_ok(eps)) return BL_ERR_EPS;
  if (!plan) return BL_ERR_NULL;
  bl::ChainPlanIn in;
  const int st = chain_analyse(calls, ncalls, M, dtype, in);
  if (st != BL_OK) return st;
  in.eps = eps;
  if (!ws || ws_bytes < bl::chain_workspace_bytes(in)) return BL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return BL_ERR_ALIGN;
  return hip_status(BL_LAUNCH(bl::chain_plan(in, ws, *plan, stream)));
}

int bitlinear_chain_run_ex(const bl_chain *plan, uint32_t wait_us, hipStream_t stream) {
  if (!plan || !plan->ws) return BL_ERR_NULL;
  if (plan->M < 1 || plan->M > bl::kChainMaxM || plan->ncalls < 1 || plan->grid < 1 ||
      (plan->dtype != BL_F16 && plan->dtype != BL_BF16))
    return BL_ERR_SHAPE;
  return hip_status(BL_LAUNCH(bl::chain_run(*plan, wait_us, stream)));
}

int bitlinear_chain_run(const bl_chain *plan, hipStream_t stream) {
  return bitlinear_chain_run_ex(plan, 2000000u, stream);
}

int bitlinear_chain_status(const bl_chain *plan, hipStream_t stream) {
  if (!plan || !plan->ws) return BL_ERR_NULL;
  uint32_t err = 0;
  if (bl::chain_error(*plan, &err, stream) != hipSuccess) return BL_ERR_HIP;
  return err ? BL_ERR_TIMEOUT : BL_OK;
}

}  // extern "C"

extern "C" {

int bitlinear_rmsnorm_swish_gate(const void *o, const void *g, const void *w, int dtype,
                                 int64_t M, int64_t K, float eps, void *z, hipStream_t stream) {
  if (!dtype_ok(dtype)) return BL_ERR_DTYPE;
  if (!m_ok(M) || K < 128 || K % 128 != 0) return BL_ERR_SHAPE;
  if (K > bl::kGateMaxK) return BL_ERR_UNSUPPORTED;
  if (!eps_ok(eps)) return BL_ERR_EPS;
  if (M == 0) return BL_OK;
  if (!o || !g || !w || !z) return BL_ERR_NULL;
  if (!aligned16(o) || !aligned16(g) || !aligned16(w) || !aligned16(z)) return BL_ERR_ALIGN;
  bl::GateArgs a{};
  a.o = o;
  a.g = g;
  a.w = w;
  a.gate_eps = eps;
  a.dtype = dtype;
  a.M = M;
  a.K = K;
  a.z = z;
  return hip_status(BL_LAUNCH(bl::launch_gate(a, stream)));
}

namespace {
bool mlgru_shape_ok(int64_t B, int64_t T, int64_t D) {
  return B >= 0 && T >= 0 && D >= 0 && D % 8 == 0 && B <= bl::kMlgruMaxB && D <= bl::kMlgruMaxD &&
         T <= bl::kMlgruMaxT;
}
}  // namespace

size_t bitlinear_mlgru_workspace_bytes(int64_t B, int64_t T, int64_t D) {
  if (!mlgru_shape_ok(B, T, D)) return 0;
  return bl::mlgru_workspace_bytes(B, T, D);
}

int bitlinear_mlgru_scan(const void *i, const void *f, int dtype, int64_t B, int64_t T, int64_t D,
                         const float *h0, void *h, float *hT, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (!dtype_ok(dtype)) return BL_ERR_DTYPE;
  if (!mlgru_shape_ok(B, T, D)) return BL_ERR_SHAPE;
  if (B == 0 || T == 0 || D == 0) return BL_OK;
  if (!i || !f || !h) return BL_ERR_NULL;
  if (!aligned16(i) || !aligned16(f) || !aligned16(h)) return BL_ERR_ALIGN;
  const size_t need = bl::mlgru_workspace_bytes(B, T, D);
  if (need > 0 && (!ws || ws_bytes < need)) return BL_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return BL_ERR_ALIGN;
  bl::MlgruArgs a{};
  a.i = i;
  a.f = f;
  a.dtype = dtype;
  a.B = B;
  a.T = T;
  a.D = D;
  a.h0 = h0;
  a.h = h;
  a.hT = hT;
  a.ws = ws;
  return hip_status(BL_LAUNCH(bl::launch_mlgru_scan(a, stream)));
}

int bitlinear_forward_gated(const void *o, const void *g, const void *gate_w, float gate_eps,
                            int x_dtype, int64_t M, int64_t K, const void *gain,
                            const void *packed, const float *beta, int64_t N, void *y,
                            int y_dtype, float eps, void *ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return BL_ERR_DTYPE;
  if (!nk_ok(N, K) || !m_ok(M)) return BL_ERR_SHAPE;
  if (K > bl::kGateMaxK) return BL_ERR_UNSUPPORTED;
  if (!eps_ok(eps) || !eps_ok(gate_eps)) return BL_ERR_EPS;
  if (M == 0) return BL_OK;
  if (!o || !g || !gate_w || !gain || !packed || !beta || !y) return BL_ERR_NULL;
  if (!ws || ws_bytes < fwd_ws_bytes(M, K)) return BL_ERR_WORKSPACE;
  if (!aligned16(o) || !aligned16(g) || !aligned16(gate_w) || !aligned16(gain) ||
      !aligned16(packed) || !aligned16(y) || !aligned16(ws) ||
      (reinterpret_cast<uintptr_t>(beta) & 3u))
    return BL_ERR_ALIGN;
  if (bl::decode_gated_fits(M, K, x_dtype)) {
    // one launch: the decode kernel's row mode with the gate in front
    bl::DecodeGateArgs d{};
    d.o = o;
    d.g = g;
    d.gate_w = gate_w;
    d.gate_eps = gate_eps;
    d.x_dtype = x_dtype;
    d.M = M;
    d.N = N;
    d.K = K;
    d.gain = gain;
    d.eps = eps;
    d.packed = packed;
    d.beta = beta;
    d.out = y;
    d.out_kind = y_dtype;
    return hip_status(BL_LAUNCH(bl::launch_decode_gated(d, stream)));
  }
  const FwdWs w = carve(ws, M, K);
  bl::GateArgs a{};
  a.o = o;
  a.g = g;
  a.w = gate_w;
  a.gate_eps = gate_eps;
  a.dtype = x_dtype;
  a.M = M;
  a.K = K;
  a.gain = gain;
  a.eps = eps;
  a.xq = w.xq;
  a.s = w.s;
  a.rowsum = w.rowsum;
  if (BL_LAUNCH(bl::launch_gate(a, stream)) != hipSuccess) return BL_ERR_HIP;
  if (M <= bl::kSkinnyMaxM)
    return hip_status(BL_LAUNCH(bl::launch_skinny(
        pre_call(w.xq, w.s, w.rowsum, packed, beta, M, N, K, y, y_dtype), stream)));
  return hip_status(BL_LAUNCH(bl::launch_gemm_mfma(w.xq, w.rowsum, w.s, packed, beta, M, N, K, y,
                                                   y_dtype, false, stream)));
}

}  // extern "C"
