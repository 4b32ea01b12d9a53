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
// polls (seconds of polling) a workgroup raises the error word and runs to
// its end, so every wave exits whatever happens to the other workgroups.
constexpr uint32_t kSpinLimit = 1u << 22;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Front end (activation rows): one launch when its workgroups all fit on
// the device at once, else a stats pass, a reduce and a quantise pass.
//   flags: bit0 = skip rotation, bit1 = skip smoothing (S = 1),
//          bit2 = always use the three launches.
//   dsign: signed rotation x D H, K-bit mask (bit j set: channel j negated),
//          or nullptr for the plain rotation.
//   zrows: Kronecker K only: room for the M x K fp32 rotated, reordered rows
//          (the quantise pass then streams them instead of rotating again),
//          or nullptr.
hipError_t launch_frontend(const uint16_t* X, int M, int K, int G, const int32_t* perm,
                           const uint32_t* dsign, uint8_t* xq, float* dx, float* S_out, uint32_t* sync,
                           int flags, hipStream_t s, float* zrows = nullptr);

// Launches the front end would use for M rows on the current device (1 or
// 3), -1 for an unsupported K.
int frontend_launches(int M, int K, int flags);

// Offline weight preparation: W [K, N] row-major fp16 -> wq [N][K/2] + dw [N]
// (H D W with a sign mask, H W without).
hipError_t launch_weight_prep(const uint16_t* W, int K, int N, const int32_t* perm,
                              const uint32_t* dsign, uint8_t* wq, float* dw, hipStream_t s);

// Calibration permutation: per-channel |max| of the rotated rows, then a
// stable descending rank. ws holds K uint32.
hipError_t launch_calibrate(const uint16_t* Xc, int T, int K, const uint32_t* dsign, int32_t* perm,
                            uint32_t* ws, hipStream_t s);

// Zero n uint32 words (fill kernel; used instead of hipMemsetAsync).
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t s);

// Grouped INT4 GEMM. Y = (1/K) dx dw sum_g S_g P_g. If P != nullptr the
// kernel instead writes the int32 partials of the window [m0,m1) x [n0,n1).
hipError_t launch_gemm(const uint8_t* xq, const float* dx, const float* S, int M, int K,
                       int N, int G, const uint8_t* wq, const float* dw, float* Y, int32_t* P,
                       int m0, int m1, int n0, int n1, hipStream_t s);

// Few-token form of the same product (Y only): whether it serves
// (M, K, N, G), and its launch. launch_gemm dispatches to it by itself.
bool gemm_small_applies(int M, int K, int N, int G);
hipError_t launch_gemm_small(const uint8_t* xq, const float* dx, const float* S, int M, int K, int N, int G,
                             const uint8_t* wq, const float* dw, float* Y, hipStream_t s);

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
                                   uint8_t* wq, float* dw, hipStream_t s);
hipError_t launch_colmax_kron(const uint16_t* Xc, int T, int K, const uint32_t* dsign, uint32_t* colmax,
                              hipStream_t s);

}  // namespace rrs
