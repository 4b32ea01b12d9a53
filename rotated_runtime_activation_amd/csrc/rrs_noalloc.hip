// rrs_linear_noalloc: the RRS A4W4 linear layer for callers that cannot
// allocate (code under stream capture, tight serving loops, harnesses that
// forbid hipMalloc). The workspace that rrs_linear takes from the caller
// (synchronisation block, packed activation codes, token and group scales)
// lives here in a file-scope device array of a fixed size instead; the
// kernels are rrs_linear's.
//
// In host code `scratch` is only a stand-in for the device array: the
// array's device address, one per GPU, comes from hipGetSymbolAddress the
// first time a call runs on that GPU and is what every launch receives.

#include <mutex>

#include "rrs.h"
#include "rrs_internal.h"

#define RRS_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = size_t(24) << 20;
static_assert(kScratchBytes == RRS_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");

// Zero when the code object loads (the synchronisation block must start
// zeroed; its one-launch epoch then makes clearing between calls
// unnecessary).
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
uint8_t* g_ptr[kMaxDevices] = {};

// Device address of this GPU's copy of the array (nullptr on failure).
uint8_t* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_ptr[dev] = static_cast<uint8_t*>(p);
  }
  return g_ptr[dev];
}

}  // namespace

RRS_API int rrs_linear_noalloc(const void* X_fp16, int M, int K, int N, int G, const int32_t* perm,
                               const void* wq, float* Y, hipStream_t s) {
  // the same shape checks as rrs_linear, then the scratch capacity
  if (M < 0 || N < 1) return RRS_EINVAL;
  const size_t sync = rrs_sync_bytes(K, G);  // 0 for an invalid K or G
  if (sync == 0) return RRS_EINVAL;
  if (perm == nullptr || wq == nullptr) return RRS_EINVAL;
  if (M > 0 && (X_fp16 == nullptr || Y == nullptr)) return RRS_EINVAL;
  const uintptr_t mis = (reinterpret_cast<uintptr_t>(X_fp16) | reinterpret_cast<uintptr_t>(perm) |
                         reinterpret_cast<uintptr_t>(wq) | reinterpret_cast<uintptr_t>(Y)) & 15;
  if (mis) return RRS_EINVAL;
  if (M == 0) return RRS_OK;
  // sync | xq | dx | S, as rrs_linear's workspace (no Kronecker row area:
  // for K = m 2^k the three-launch front end rotates every row twice)
  const size_t xq_off = sync;
  const size_t dx_off = xq_off + rrs::align256(rrs::codes_bytes(static_cast<size_t>(M), K));
  const size_t S_off = dx_off + rrs::align256(sizeof(float) * static_cast<size_t>(M));
  const size_t total = S_off + rrs::align256(sizeof(float) * static_cast<size_t>(K / G));
  if (total > kScratchBytes) return RRS_ETOOBIG;
  uint8_t* base = scratch_on_current_device();
  if (base == nullptr) return RRS_EHIP;
  uint8_t* xq = base + xq_off;
  float* dx = reinterpret_cast<float*>(base + dx_off);
  float* S = reinterpret_cast<float*>(base + S_off);
  uint32_t* sw = reinterpret_cast<uint32_t*>(base);
  if (rrs::launch_frontend(static_cast<const uint16_t*>(X_fp16), M, K, G, perm, nullptr, xq, dx, S, sw, 0, s,
                           nullptr) != hipSuccess)
    return RRS_EHIP;
  const uint8_t* codes = static_cast<const uint8_t*>(wq);
  const float* dw = reinterpret_cast<const float*>(codes + rrs::align256(rrs::codes_bytes(static_cast<size_t>(N), K)));
  const rrs::GemmCall gc{xq, dx, S, M, K, N, G, codes, dw, Y, nullptr, 0, 0, 0, 0, true, sw + rrs::kSyncError};
  return rrs::launch_gemm(gc, s) == hipSuccess ? RRS_OK : RRS_EHIP;
}
