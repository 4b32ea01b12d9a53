// Host side of the C ABI declared in include/rrs.h: argument validation,
// buffer carving and kernel launches. Validation happens before any HIP call,
// so a rejected call touches neither the device nor the runtime.

#include "rrs.h"
#include "rrs_internal.h"

#include <algorithm>

#define RRS_API extern "C" __attribute__((visibility("default")))

namespace {

using rrs::align256;

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) { return 31 - __builtin_clz(static_cast<unsigned>(x)); }

// K: a power of two in [64, 8192], or m 2^k with m in {12, 20, 28} (the
// Kronecker rotation; see rrs::kron_split)
bool valid_K(int K) {
  if (K <= 0) return false;
  if (pow2(K)) return ilog2(K) >= rrs::kMinLog2K && ilog2(K) <= rrs::kMaxLog2K;
  int m = 0, ln = 0;
  return rrs::kron_split(K, &m, &ln);
}
bool valid_G(int G, int K) { return pow2(G) && G >= rrs::kMinG && G <= K && K % G == 0; }

// every device pointer argument is read or written with 16-byte accesses
bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
template <typename... P>
bool all_a16(const P*... p) { return (a16(p) && ...); }

size_t sync_bytes(int K, int G) {
  // 64-bit tagged group maxima per workgroup of the one-launch front end
  return align256(sizeof(uint32_t) * (rrs::kSyncPartials + 2 * static_cast<size_t>(rrs::kMaxFusedWG) * (K / G)));
}

struct WsLayout {
  size_t sync, xq, dx, S, rows, rows_bytes, total;
};

// sync | xq | dx | S | rows; the row area (the rotated, reordered fp32 rows
// the Kronecker front end keeps between its stats and quantise passes) is
// there only for K = m 2^k
WsLayout ws_layout(int M, int K, int G) {
  WsLayout l{};
  l.sync = 0;
  l.xq = sync_bytes(K, G);
  l.dx = l.xq + align256(rrs::codes_bytes(static_cast<size_t>(M), K));
  l.S = l.dx + align256(sizeof(float) * static_cast<size_t>(M));
  l.rows = l.S + align256(sizeof(float) * static_cast<size_t>(K / G));
  l.rows_bytes = pow2(K) ? 0 : align256(sizeof(float) * static_cast<size_t>(M) * K);
  l.total = l.rows + l.rows_bytes;
  return l;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

int hip_status(hipError_t e) { return e == hipSuccess ? RRS_OK : RRS_EHIP; }

}  // namespace

RRS_API const char* rrs_status_string(int status) {
  switch (status) {
    case RRS_OK: return "RRS_OK";
    case RRS_EINVAL: return "RRS_EINVAL: invalid argument";
    case RRS_EUNSUPPORTED: return "RRS_EUNSUPPORTED: unsupported configuration";
    case RRS_EHIP: return "RRS_EHIP: HIP runtime or launch failure";
    case RRS_ETOOBIG: return "RRS_ETOOBIG: request exceeds the fixed scratch of rrs_linear_noalloc";
    default: return "RRS: unknown status";
  }
}

RRS_API const char* rrs_version(void) { return "rrs-gfx950 1.0"; }

RRS_API size_t rrs_weight_bytes(int K, int N) {
  if (!valid_K(K) || N < 1) return 0;
  return align256(rrs::codes_bytes(static_cast<size_t>(N), K)) + align256(sizeof(float) * static_cast<size_t>(N));
}

RRS_API size_t rrs_codes_bytes(int M, int K) {
  if (M < 0 || !valid_K(K)) return 0;
  return rrs::codes_bytes(static_cast<size_t>(M), K);
}

RRS_API size_t rrs_sync_bytes(int K, int G) {
  if (!valid_K(K) || !valid_G(G, K)) return 0;
  return sync_bytes(K, G);
}

RRS_API size_t rrs_workspace_bytes(int M, int K, int G) {
  if (M < 0 || !valid_K(K) || !valid_G(G, K)) return 0;
  return ws_layout(M, K, G).total;
}

RRS_API size_t rrs_calibrate_workspace_bytes(int K) {
  if (!valid_K(K)) return 0;
  return align256(sizeof(uint32_t) * static_cast<size_t>(K));
}

RRS_API int rrs_workspace_init(void* ws, size_t ws_bytes, hipStream_t s) {
  if (ws == nullptr || ws_bytes < 256 || ws_bytes % 4 || !a16(ws)) return RRS_EINVAL;
  // all of it: the tagged maxima of the one-launch front end must not hold
  // a stale tag from memory that was never initialised
  const size_t n = ws_bytes / sizeof(uint32_t);
  return hip_status(rrs::launch_zero_u32(static_cast<uint32_t*>(ws), n, s));
}

namespace {

constexpr int kFrontendFlags = RRS_FLAG_NO_ROTATE | RRS_FLAG_NO_SMOOTH | RRS_FLAG_TWO_PASS | RRS_FLAG_TEST_GIVE_UP;
static_assert(RRS_FLAG_NO_ROTATE == rrs::kFlagNoRotate && RRS_FLAG_NO_SMOOTH == rrs::kFlagNoSmooth &&
                  RRS_FLAG_TWO_PASS == rrs::kFlagTwoPass && RRS_FLAG_TEST_GIVE_UP == rrs::kFlagGiveUp,
              "public and internal flag values agree");

int calibrate_impl(const void* X_cal_fp16, int T, int K, const uint32_t* dsign, int flags, int32_t* perm,
                   void* ws, size_t ws_bytes, hipStream_t s) {
  if (X_cal_fp16 == nullptr || perm == nullptr || ws == nullptr) return RRS_EINVAL;
  if (T < 1 || !valid_K(K)) return RRS_EINVAL;
  if (flags & ~RRS_FLAG_NO_ROTATE) return RRS_EINVAL;
  if (dsign != nullptr && (flags & RRS_FLAG_NO_ROTATE)) return RRS_EINVAL;  // the signs belong to the rotation
  if (ws_bytes < rrs_calibrate_workspace_bytes(K)) return RRS_EINVAL;
  if (!all_a16(X_cal_fp16, perm, ws, dsign)) return RRS_EINVAL;
  return hip_status(rrs::launch_calibrate(static_cast<const uint16_t*>(X_cal_fp16), T, K, dsign, perm,
                                          static_cast<uint32_t*>(ws), s, !(flags & RRS_FLAG_NO_ROTATE)));
}

int prepare_impl(const void* W_fp16, int K, int N, const int32_t* perm, const uint32_t* dsign, int flags,
                 void* wq, hipStream_t s) {
  if (W_fp16 == nullptr || perm == nullptr || wq == nullptr) return RRS_EINVAL;
  if (!valid_K(K) || N < 1) return RRS_EINVAL;
  if (flags & ~RRS_FLAG_NO_ROTATE) return RRS_EINVAL;
  if (dsign != nullptr && (flags & RRS_FLAG_NO_ROTATE)) return RRS_EINVAL;
  if (!all_a16(W_fp16, perm, wq, dsign)) return RRS_EINVAL;
  uint8_t* codes = static_cast<uint8_t*>(wq);
  float* dw = reinterpret_cast<float*>(codes + align256(rrs::codes_bytes(static_cast<size_t>(N), K)));
  return hip_status(rrs::launch_weight_prep(static_cast<const uint16_t*>(W_fp16), K, N, perm, dsign,
                                            codes, dw, s, !(flags & RRS_FLAG_NO_ROTATE)));
}

int frontend_impl(const void* X_fp16, int M, int K, int G, const int32_t* perm, const uint32_t* dsign,
                  uint8_t* xq, float* dx, float* S, void* ws, size_t ws_bytes, int flags, hipStream_t s) {
  if (M < 0 || !valid_K(K) || !valid_G(G, K)) return RRS_EINVAL;
  if (flags & ~kFrontendFlags) return RRS_EINVAL;
  if (dsign != nullptr && (flags & RRS_FLAG_NO_ROTATE)) return RRS_EINVAL;  // the signs belong to the rotation
  if (perm == nullptr || S == nullptr || ws == nullptr) return RRS_EINVAL;
  if (M > 0 && (X_fp16 == nullptr || xq == nullptr || dx == nullptr)) return RRS_EINVAL;
  if (ws_bytes < sync_bytes(K, G)) return RRS_EINVAL;
  if (!all_a16(X_fp16, perm, xq, dx, S, ws, dsign)) return RRS_EINVAL;
  if (M == 0) return RRS_OK;
  // a workspace of rrs_linear's size: the Kronecker front end keeps its rows
  // in the row area, unless another argument lies there
  float* zrows = nullptr;
  const WsLayout l = ws_layout(M, K, G);
  if (l.rows_bytes && ws_bytes >= l.total) {
    uint8_t* r = static_cast<uint8_t*>(ws) + l.rows;
    const size_t mk = static_cast<size_t>(M) * K;
    if (!overlap(r, l.rows_bytes, X_fp16, 2 * mk) && !overlap(r, l.rows_bytes, xq, rrs::codes_bytes(static_cast<size_t>(M), K)) &&
        !overlap(r, l.rows_bytes, dx, 4 * static_cast<size_t>(M)) &&
        !overlap(r, l.rows_bytes, S, 4 * static_cast<size_t>(K / G)) &&
        !overlap(r, l.rows_bytes, perm, 4 * static_cast<size_t>(K)) &&
        (dsign == nullptr || !overlap(r, l.rows_bytes, dsign, static_cast<size_t>(K / 8))))
      zrows = reinterpret_cast<float*>(r);
  }
  return hip_status(rrs::launch_frontend(static_cast<const uint16_t*>(X_fp16), M, K, G, perm, dsign, xq,
                                         dx, S, static_cast<uint32_t*>(ws), flags, s, zrows));
}

// Largest weight stream the front end prefetches (a quarter of MI355X's
// 256 MB memory-side cache).
constexpr size_t kPrefetchMaxBytes = size_t(64) << 20;
// Share of each wave's run of weight codes the front end reads ahead, in
// quarters (the rounds the GEMM's waves fetch first).
constexpr int kPrefetchQuarters = 3;

int linear_impl(const void* X_fp16, int M, int K, int N, int G, const int32_t* perm, const uint32_t* dsign,
                int flags, const void* wq, float* Y, void* ws, size_t ws_bytes, hipStream_t s) {
  if (M < 0 || N < 1 || !valid_K(K) || !valid_G(G, K)) return RRS_EINVAL;
  if (flags & ~kFrontendFlags) return RRS_EINVAL;
  if (dsign != nullptr && (flags & RRS_FLAG_NO_ROTATE)) return RRS_EINVAL;
  if (perm == nullptr || wq == nullptr || ws == nullptr) return RRS_EINVAL;
  if (M > 0 && (X_fp16 == nullptr || Y == nullptr)) return RRS_EINVAL;
  const WsLayout l = ws_layout(M, K, G);
  if (ws_bytes < l.total) return RRS_EINVAL;
  if (!all_a16(X_fp16, perm, wq, Y, ws, dsign)) return RRS_EINVAL;
  if (M == 0) return RRS_OK;
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* xq = base + l.xq;
  float* dx = reinterpret_cast<float*>(base + l.dx);
  float* S = reinterpret_cast<float*>(base + l.S);
  float* zrows = l.rows_bytes ? reinterpret_cast<float*>(base + l.rows) : nullptr;
  uint32_t* sync = reinterpret_cast<uint32_t*>(base + l.sync);
  const uint8_t* codes = static_cast<const uint8_t*>(wq);
  // The front end reads the GEMM's weight codes ahead into the memory-side
  // cache where its launch can (it decides by its form). The few-token GEMM
  // streams the weights once: its waves each stream a run of K / waves codes
  // of a row pair (K / waves bytes of the stored layout) from its start, so
  // the first rounds of every run are read. Before the tiled GEMM, all of
  // them (period = keep).
  const size_t wbytes = rrs::codes_bytes(static_cast<size_t>(N), K);
  const bool small = rrs::gemm_small_applies(M, K, N, G);
  const bool pf = wbytes <= kPrefetchMaxBytes;
  const int period = !pf ? 0 : small ? K / rrs::small_waves(K) : 16;
  const int keep = !pf ? 0 : small ? std::max(128, period * kPrefetchQuarters / 4 / 128 * 128) : 16;
  hipError_t e = rrs::launch_frontend(static_cast<const uint16_t*>(X_fp16), M, K, G, perm, dsign, xq, dx,
                                      S, sync, flags, s, zrows, pf ? codes : nullptr, pf ? wbytes : 0, period, keep);
  if (e != hipSuccess) return RRS_EHIP;
  const float* dw = reinterpret_cast<const float*>(codes + align256(rrs::codes_bytes(static_cast<size_t>(N), K)));
  // the GEMM reads the workspace's error word: a front end whose grid-wide
  // wait gave up (now or in an earlier call on this workspace) makes Y NaN
  const rrs::GemmCall gc{xq, dx, S, M, K, N, G, codes, dw, Y, nullptr, 0, 0, 0, 0,
                         !(flags & RRS_FLAG_NO_ROTATE), sync + rrs::kSyncError};
  return hip_status(rrs::launch_gemm(gc, s));
}

}  // namespace

RRS_API int rrs_calibrate_perm(const void* X_cal_fp16, int T, int K, int32_t* perm, void* ws,
                               size_t ws_bytes, hipStream_t s) {
  return calibrate_impl(X_cal_fp16, T, K, nullptr, 0, perm, ws, ws_bytes, s);
}

RRS_API int rrs_calibrate_perm_signed(const void* X_cal_fp16, int T, int K, const uint32_t* dsign, int32_t* perm,
                                      void* ws, size_t ws_bytes, hipStream_t s) {
  if (dsign == nullptr) return RRS_EINVAL;
  return calibrate_impl(X_cal_fp16, T, K, dsign, 0, perm, ws, ws_bytes, s);
}

RRS_API int rrs_calibrate_perm_ex(const void* X_cal_fp16, int T, int K, const uint32_t* dsign, int flags,
                                  int32_t* perm, void* ws, size_t ws_bytes, hipStream_t s) {
  return calibrate_impl(X_cal_fp16, T, K, dsign, flags, perm, ws, ws_bytes, s);
}

RRS_API int rrs_prepare_weights(const void* W_fp16, int K, int N, const int32_t* perm, void* wq,
                                hipStream_t s) {
  return prepare_impl(W_fp16, K, N, perm, nullptr, 0, wq, s);
}

RRS_API int rrs_prepare_weights_signed(const void* W_fp16, int K, int N, const int32_t* perm,
                                       const uint32_t* dsign, void* wq, hipStream_t s) {
  if (dsign == nullptr) return RRS_EINVAL;
  return prepare_impl(W_fp16, K, N, perm, dsign, 0, wq, s);
}

RRS_API int rrs_prepare_weights_ex(const void* W_fp16, int K, int N, const int32_t* perm, const uint32_t* dsign,
                                   int flags, void* wq, hipStream_t s) {
  return prepare_impl(W_fp16, K, N, perm, dsign, flags, wq, s);
}

RRS_API int rrs_frontend(const void* X_fp16, int M, int K, int G, const int32_t* perm, uint8_t* xq,
                         float* dx, float* S, void* ws, size_t ws_bytes, int flags, hipStream_t s) {
  return frontend_impl(X_fp16, M, K, G, perm, nullptr, xq, dx, S, ws, ws_bytes, flags, s);
}

RRS_API int rrs_frontend_signed(const void* X_fp16, int M, int K, int G, const int32_t* perm,
                                const uint32_t* dsign, uint8_t* xq, float* dx, float* S, void* ws,
                                size_t ws_bytes, int flags, hipStream_t s) {
  if (dsign == nullptr) return RRS_EINVAL;
  return frontend_impl(X_fp16, M, K, G, perm, dsign, xq, dx, S, ws, ws_bytes, flags, s);
}

RRS_API int rrs_frontend_passes(int M, int K, int flags) {
  if (M < 1 || !valid_K(K)) return RRS_EINVAL;
  if (flags & ~kFrontendFlags) return RRS_EINVAL;
  const int n = rrs::frontend_launches(M, K, flags);
  return n > 0 ? n : RRS_EHIP;
}

RRS_API int rrs_gemm(const uint8_t* xq, const float* dx, const float* S, int M, int K, int N, int G,
                     const void* wq, float* Y, hipStream_t s) {
  if (M < 0 || N < 1 || !valid_K(K) || !valid_G(G, K)) return RRS_EINVAL;
  if (S == nullptr || wq == nullptr) return RRS_EINVAL;
  if (M > 0 && (xq == nullptr || dx == nullptr || Y == nullptr)) return RRS_EINVAL;
  if (!all_a16(xq, dx, S, wq, Y)) return RRS_EINVAL;
  if (M == 0) return RRS_OK;
  const uint8_t* codes = static_cast<const uint8_t*>(wq);
  const float* dw = reinterpret_cast<const float*>(codes + align256(rrs::codes_bytes(static_cast<size_t>(N), K)));
  const rrs::GemmCall gc{xq, dx, S, M, K, N, G, codes, dw, Y, nullptr, 0, 0, 0, 0, true, nullptr};
  return hip_status(rrs::launch_gemm(gc, s));
}

RRS_API int rrs_gemm_form(int M, int K, int N, int G) {
  if (M < 1 || N < 1 || !valid_K(K) || !valid_G(G, K)) return RRS_EINVAL;
  return rrs::gemm_small_applies(M, K, N, G) ? RRS_GEMM_FEW_TOKENS : RRS_GEMM_TILED;
}

RRS_API int rrs_gemm_partials(const uint8_t* xq, int M, int K, int N, int G, const void* wq, int m0,
                              int m1, int n0, int n1, int32_t* P, hipStream_t s) {
  if (M < 1 || N < 1 || !valid_K(K) || !valid_G(G, K)) return RRS_EINVAL;
  if (xq == nullptr || wq == nullptr || P == nullptr) return RRS_EINVAL;
  if (m0 < 0 || m1 > M || m0 >= m1 || n0 < 0 || n1 > N || n0 >= n1) return RRS_EINVAL;
  if (!all_a16(xq, wq, P)) return RRS_EINVAL;
  const uint8_t* codes = static_cast<const uint8_t*>(wq);
  const float* dw = reinterpret_cast<const float*>(codes + align256(rrs::codes_bytes(static_cast<size_t>(N), K)));
  const rrs::GemmCall gc{xq, nullptr, nullptr, M, K, N, G, codes, dw, nullptr, P, m0, m1, n0, n1, true, nullptr};
  return hip_status(rrs::launch_gemm(gc, s));
}

RRS_API int rrs_linear(const void* X_fp16, int M, int K, int N, int G, const int32_t* perm,
                       const void* wq, float* Y, void* ws, size_t ws_bytes, hipStream_t s) {
  return linear_impl(X_fp16, M, K, N, G, perm, nullptr, 0, wq, Y, ws, ws_bytes, s);
}

RRS_API int rrs_linear_signed(const void* X_fp16, int M, int K, int N, int G, const int32_t* perm,
                              const uint32_t* dsign, const void* wq, float* Y, void* ws, size_t ws_bytes,
                              hipStream_t s) {
  if (dsign == nullptr) return RRS_EINVAL;
  return linear_impl(X_fp16, M, K, N, G, perm, dsign, 0, wq, Y, ws, ws_bytes, s);
}

RRS_API int rrs_linear_ex(const void* X_fp16, int M, int K, int N, int G, const int32_t* perm,
                          const uint32_t* dsign, int flags, const void* wq, float* Y, void* ws, size_t ws_bytes,
                          hipStream_t s) {
  return linear_impl(X_fp16, M, K, N, G, perm, dsign, flags, wq, Y, ws, ws_bytes, s);
}
