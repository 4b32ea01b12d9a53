// Internal declarations shared by the HIP translation units of librrs.
// Not part of the public ABI (that is include/rrs.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rrs {

// Largest and smallest supported Hadamard sizes / group sizes.
constexpr int kMinLog2K = 6;
constexpr int kMaxLog2K = 13;
constexpr int kMinG = 32;

// Layout of the synchronisation block at the start of a workspace (uint32
// words unless noted):
//   [2]    error word: nonzero once a bounded wait gave up (only
//          rrs_workspace_init clears it)
//   [3]    epoch of the one-launch front end (calls so far, mod 2^32)
//   [17408, 17408 + 2 * 512 K/G) one-launch group maxima: one row of K/G
//          64-bit words per workgroup, this call's epoch in the high half
//          and the maximum's float bits in the low half (never needs
//          clearing)
// Every other word below 17408 is reserved and stays zero.
// rrs_workspace_init zeroes the whole block.
constexpr int kSyncError = 2;
constexpr int kSyncEpoch = 3;
constexpr int kMaxFusedWG = 512;
constexpr int kSyncPartials = 17408;
// Bounded spin of the one-launch forms' grid-wide wait: after this many
// polls (seconds of polling) a workgroup gives up: it raises the error word,
// marks its own outputs (NaN token scales, and NaN group scales from the
// workgroup that writes them) and runs to its end, so every wave exits
// whatever happens to the other workgroups. A limit of 0 (the failure-path
// test flag) gives up after the first poll in every workgroup.
constexpr uint32_t kSpinLimit = 1u << 22;

// Front-end flags (the public ones of rrs.h, plus the test flag)
constexpr int kFlagNoRotate = 1;
constexpr int kFlagNoSmooth = 2;
constexpr int kFlagTwoPass = 4;
constexpr int kFlagGiveUp = 8;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Stored layout of a matrix of packed codes (the activation codes xq and the
// prepared weight codes): rows in pairs, each row's K/2 bytes cut into
// 64-byte pieces (128 codes, one tiled-GEMM stage), piece c of rows 2p and
// 2p + 1 side by side in one 128-byte line. Byte b of row r lies at
//   (r / 2) * 2 rs + (b / 64) * 128 + (r % 2) * 64 + b % 64,
// with rs = K/2 rounded up to 64 (K = 64 uses 32 bytes of each piece). A
// stage of a tile's rows then reads whole lines; with one row per line half
// of every line it fetched went unused until the next stage.
__host__ __device__ constexpr size_t codes_row_stride(int K) { return (static_cast<size_t>(K / 2) + 63) & ~size_t(63); }
__host__ __device__ constexpr size_t codes_bytes(size_t rows, int K) {
  return ((rows + 1) / 2) * 2 * codes_row_stride(K);
}
__host__ __device__ inline size_t codes_offset(size_t r, size_t b, size_t rs) {
  return (r >> 1) * 2 * rs + ((b >> 6) << 7) + ((r & 1) << 6) + (b & 63);
}

// Front end (activation rows): one launch when its workgroups all fit on
// the device at once, else a stats pass, a reduce and a quantise pass.
//   flags: bit0 = skip rotation, bit1 = skip smoothing (S = 1),
//          bit2 = always use the three launches.
//   dsign: signed rotation x D H, K-bit mask (bit j set: channel j negated),
//          or nullptr for the plain rotation.
//   zrows: Kronecker K only: room for the M x K fp32 rotated, reordered rows
//          (the quantise pass then streams them instead of rotating again),
//          or nullptr.
//   kFlagGiveUp (bit3): the one-launch forms' wait gives up at once (tests
//          of the failure path; every kernel still ends normally).
//   prefetch / prefetch_bytes: device memory the caller reads next (the
//          layer's weight codes); where the front end leaves most of the
//          device idle (the one-row-per-workgroup form) extra workgroups of
//          the same launch read the first prefetch_keep bytes of every
//          prefetch_period bytes of it once (both multiples of 16), so that
//          they sit in the memory-side cache when the next kernel starts.
//          nullptr: none.
hipError_t launch_frontend(const uint16_t* X, int M, int K, int G, const int32_t* perm,
                           const uint32_t* dsign, uint8_t* xq, float* dx, float* S_out, uint32_t* sync,
                           int flags, hipStream_t s, float* zrows = nullptr, const void* prefetch = nullptr,
                           size_t prefetch_bytes = 0, int prefetch_period = 0, int prefetch_keep = 0);

// Compute units of the current device (cached per device).
int device_cus();

// Waves per workgroup of the few-token GEMM at K (0: not served); each wave
// runs K / waves consecutive codes of every row.
int small_waves(int K);

// Launches the front end would use for M rows on the current device (1 or
// 3), -1 for an unsupported K.
int frontend_launches(int M, int K, int flags);

// Offline weight preparation: W [K, N] row-major fp16 -> wq [N][K/2] + dw [N]
// (H D W with a sign mask, H W without; W itself, reordered, with
// rotate = false).
hipError_t launch_weight_prep(const uint16_t* W, int K, int N, const int32_t* perm,
                              const uint32_t* dsign, uint8_t* wq, float* dw, hipStream_t s,
                              bool rotate = true);

// Calibration permutation: per-channel |max| of the rotated rows (the raw
// rows with rotate = false), then a stable descending rank. ws holds K uint32.
hipError_t launch_calibrate(const uint16_t* Xc, int T, int K, const uint32_t* dsign, int32_t* perm,
                            uint32_t* ws, hipStream_t s, bool rotate = true);

// Zero n uint32 words (fill kernel; used instead of hipMemsetAsync).
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t s);

// Grouped INT4 GEMM: Y = c dx dw sum_g S_g P_g with c = 1/K for codes of
// rotated rows (the Hadamard pair's two 1/sqrt(K)) and c = 1 without the
// rotation (rotated = false). If P != nullptr the kernel that would write Y
// (the same instantiation, with the accumulator cleared where it would be
// rescaled) instead writes the int32 partials of the window [m0,m1) x
// [n0,n1). err: a device word (the workspace's error word) that, when
// nonzero as the kernel runs, makes it write NaN to every output; nullptr
// for none.
struct GemmCall {
  const uint8_t* xq;
  const float* dx;
  const float* S;
  int M, K, N, G;
  const uint8_t* wq;
  const float* dw;
  float* Y;
  int32_t* P;
  int m0, m1, n0, n1;
  bool rotated;
  const uint32_t* err;
};
hipError_t launch_gemm(const GemmCall& c, hipStream_t s);

// Few-token form of the same product: whether it serves (M, K, N, G), and
// its launch. launch_gemm dispatches to it by itself.
bool gemm_small_applies(int M, int K, int N, int G);
hipError_t launch_gemm_small(const GemmCall& c, hipStream_t s);

// Kronecker rotation H_m (x) H_n for K = m n, m in {12, 20, 28}, n = 2^k
// (64 <= n, K <= kMaxKronK; n <= 1024 for m = 12, n <= 512 otherwise).
constexpr int kMaxKronK = 16384;
bool kron_split(int K, int* m, int* log2n);
// Launches of the Kronecker front end for M rows (1 or 3; queries the
// device's occupancy).
int kron_frontend_launches(int M, int K, int flags);
// S_g = max over `nrows` rows of K/G group maxima (float bits) at `part`,
// 1 where every row holds 0 (the stats passes' reduce).
hipError_t launch_group_max(const uint32_t* part, int nrows, int ngroups, float* S_out, hipStream_t s);

hipError_t launch_frontend_kron(const uint16_t* X, int M, int K, int G, const int32_t* perm, const uint32_t* dsign,
                                uint8_t* xq, float* dx, float* S_out, uint32_t* sync, int flags, hipStream_t s,
                                float* zrows);
hipError_t launch_weight_prep_kron(const uint16_t* W, int K, int N, const int32_t* perm, const uint32_t* dsign,
                                   uint8_t* wq, float* dw, hipStream_t s, bool rotate);
hipError_t launch_colmax_kron(const uint16_t* Xc, int T, int K, const uint32_t* dsign, uint32_t* colmax,
                              hipStream_t s, bool rotate);

}  // namespace rrs
