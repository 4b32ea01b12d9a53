// Grouped INT4 x INT4 GEMM of the RRS A4W4 linear for few tokens
// (decode-shaped calls), on gfx950.
//
// Same arithmetic as the tiled kernel (Y[t, n] = (1/K) dx[t] dw[n]
// sum_g S[g] P_g[t, n], group scales applied to each group's exact integer
// partial before fp32 accumulation; RRS summary page, atlas.scime.ai,
// "Approach"; RRS rebuttal page, paperhub.cn, "Novelty"), shaped for the
// case where the packed weights are the only large operand and the run time
// is the time to stream them from HBM once.
//
// One workgroup owns 32 output channels and a slice of up to 64 tokens
// (grid y walks the slices; one 32 x 32 accumulator block per 32 tokens,
// v_mfma_f32_32x32x64_f8f6f4 on codes
// widened to exact fp8 subnormals as in the tiled kernel). Its 8 waves
// split K into equal runs of k-steps (64 codes); each wave rescales its
// accumulator when it enters a new group, makes its sum absolute at the end
// (times the scale of its last group), and the 8 sums are added in LDS in a
// fixed order. Runs and groups are powers of two, so either every run holds
// whole groups or every group holds whole runs; in the second case the
// runs' sums are exact integer pieces of one group partial, which are added
// exactly before the group's scale is applied once.
//
// Loads: a wave reads its operands a round (4 k-steps, one 128-byte line of
// every row) at a time with whole-line coalesced loads into registers, two
// rounds ahead; at its turn a round goes through a wave-private LDS buffer
// (row-major, 16-byte chunks XOR-swizzled by row) that turns it into MFMA
// fragments. With N / 32 workgroups per token slice (256 at N = 8192) every
// CU streams its own slice of the weights; further token slices stream them
// again (from the Infinity Cache when they fit there).

#include <atomic>
#include <type_traits>

#include "rrs_internal.h"

namespace rrs {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Waves per workgroup: 8 when K is a multiple of 2048; otherwise the
// largest of 7, 6, 5, 4 that splits K into whole rounds (see small_waves).
// More than 8 (three waves per SIMD) would cap a wave below the registers
// the main loop needs.
constexpr int kMaxWaves = 8;
constexpr int kTN = 32;      // output channels per workgroup
constexpr int kSmallMaxTokens = 512;  // token count past which the tiled kernel always serves
constexpr int kRound = 4;    // k-steps per round (128 bytes of a row)
constexpr int kRows = 128;   // bytes of a row per round
constexpr int kPairRound = 2 * kRows;  // stored bytes of a row pair per round (two stage lines)
constexpr float kUnit = 262144.0f;  // 2^18: one integer product in accumulator units

struct SmallArgs {
  const uint8_t* xq;
  const float* dx;
  const float* S;
  const uint8_t* wq;
  const float* dw;
  float* Y;
  int32_t* P;           // partials window (partials variant), zeroed before the launch
  const uint32_t* err;  // nonzero word: write NaN to every output (nullptr: none)
  float ybase;          // 2^18 / K for rotated codes, 2^18 without the rotation
  int M, N, K, log2G;
  int pm0, pm1, pn0, pn1;
};

// a-codes (even) and b-codes (odd) of a packed word as e4m3 subnormals
__device__ __forceinline__ uint32_t ecodes(uint32_t w) { return w & 0x87878787u; }
__device__ __forceinline__ uint32_t ocodes(uint32_t w) { return __builtin_amdgcn_alignbit(w, w, 4) & 0x87878787u; }
// A weight stream much larger than the caches is read once per call: with
// WSTREAM its loads are non-temporal, so they do not push the activation
// codes (read by every workgroup of an XCD) out of L2.
template <bool WSTREAM>
__device__ __forceinline__ v4u wload(const v4u* p) {
  if constexpr (WSTREAM)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}
__device__ __forceinline__ v8i widen(v4u w) {
  return v8i{(int)ecodes(w.x), (int)ocodes(w.x), (int)ecodes(w.y), (int)ocodes(w.y),
             (int)ecodes(w.z), (int)ocodes(w.z), (int)ecodes(w.w), (int)ocodes(w.w)};
}

// byte offset of 16-byte chunk c of row r in a wave's round buffer
__device__ __forceinline__ int swz(int r, int c) { return r * kRows + ((c ^ (r & 7)) << 4); }

// The partials variant: add an exact integer piece of group g's partial
// (accumulator units 2^-18; the sum of the NA accumulators given), held by
// this wave, into P for the window's outputs. Register e of lane l in block
// j holds token t0 + 32 j + l % 32, channel n0 + 8 (e / 4) + 4 (l / 32) +
// e % 4.
template <int TJ>
__device__ __forceinline__ void dump_piece(const SmallArgs& a, const v16f (&acc)[TJ], const v16f (&acc2)[TJ],
                                           bool both, int t0, int n0, int lane, int g, int ngroups) {
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int t = t0 + 32 * j + (lane & 31);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int n = n0 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (t >= a.pm0 && t < a.pm1 && n >= a.pn0 && n < a.pn1) {
        const size_t o = (static_cast<size_t>(t - a.pm0) * (a.pn1 - a.pn0) + (n - a.pn0)) * ngroups + g;
        const float v = both ? acc[j][e] + acc2[j][e] : acc[j][e];
        atomicAdd(&a.P[o], static_cast<int32_t>(v * kUnit));
      }
    }
  }
}

// TJ: 32-token blocks per slice (1 for M <= 32, else 2); NR: rounds of loads
// in flight (1 or 2; divides the wave's round count); KS: min(k-steps per
// group, kRound), the spacing of possible group starts inside a round, or 0
// for G = 32 (two groups in every k-step); WV: waves per workgroup.
// A VALU read of a 16-pass MFMA's last result registers needs at least 20
// issue slots after it on gfx950, and the compiler's own padding has been
// found one short where a rescale read the MFMA issued just before it (or
// one block's MFMA before it, at G = 64). So no rescale does: with one
// token block (TJ = 1), and at G = 64 (a rescale at every k-step), the wave
// keeps two accumulators per block, for G >= 64 one for the even and one
// for the odd k-steps, for G = 32 one for each group of a k-step's two,
// each rescaled right before its own next MFMA from the group it last
// took; otherwise (two blocks, G = 32 or G >= 128) the other block's MFMA
// lies between (at G = 32 every block's first-group MFMA is issued before
// any block's rescale into the second group).
// PARTIALS: the same main loop with the accumulators multiplied by 0 where
// they would be rescaled, and every wave's integer piece of a group added
// into P where the group (or the wave's run) ends; no Y.
template <int TJ, int NR, int KS, int WV, bool PARTIALS, bool WSTREAM>
__global__ void __launch_bounds__(WV * 64) gemm_small_kernel(SmallArgs a) {
  constexpr int kWaves = WV, kThreads = WV * 64;
  static_assert(WV <= kMaxWaves && 64 + kTN + 3 * WV <= kThreads, "one thread per scale preloaded");
  constexpr int kWL = 4;            // W loads per lane per round (32 rows / 8)
  constexpr int kXL = 4 * TJ;       // X loads per lane per round
  constexpr int kBuf = (32 + 32 * TJ) * kRows;  // round buffer bytes per wave
  static_assert(TJ * 16 * 64 * 4 <= kBuf, "a wave's sums fit its round buffer");
  static_assert(kMaxKronK >= (1 << kMaxLog2K), "group ratio table sized by the largest K");
  __shared__ float s_rat[kMaxKronK / 32];   // S[g-1] / S[g]
  __shared__ float s_rat2[kMaxKronK / 32];  // S[g-2] / S[g] (G <= 64)
  __shared__ float s_dx[64];         // dx[t] 2^18 / K (0 past M)
  __shared__ float s_dw[kTN];        // dw of the workgroup's channels (0 past N)
  __shared__ float s_last[kWaves];   // scale of the group of each wave's last code
  __shared__ float s_lastp[2 * kWaves];  // scale of the last group of each wave's two accumulators
  __shared__ float s_out[64 * (kTN + 1)];  // the summed tile, token-major, rows padded by one word
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[kWaves][kBuf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * kTN;
  // this workgroup's token slice: rows t0 .. t0 + Mt - 1 of xq, dx and Y
  const int t0 = blockIdx.y * 64;
  const int Mt = min(64, a.M - t0);
  const size_t rs = codes_row_stride(a.K);  // stored layout: row pairs, 64-byte pieces side by side
  const uint8_t* xq = a.xq + static_cast<size_t>(t0) * rs;  // t0 is even
  const float* dx = a.dx + t0;
  float* Y = a.Y + static_cast<size_t>(t0) * a.N;
  const int ngroups = a.K >> a.log2G;
  // k-steps per group for G >= 64 (KS = 0 is G = 32: two groups per k-step)
  const int log2spg = KS == 0 ? 0 : a.log2G - 6;
  const int kspg = 1 << log2spg;
  const int kpw = (a.K >> 6) / kWaves;  // k-steps per wave (a multiple of kRound)
  const int ks0 = wave * kpw;
  const int rounds = kpw / kRound;

  // coalesced load i of a round: row 8 i + lane / 8, chunk lane % 8 (rows
  // clamped to the matrix; clamped rows feed outputs that are never stored).
  // In the stored layout a row pair's round is 256 contiguous bytes (the
  // pair's two stage lines), so each load moves four whole 256-byte runs.
  const int lr = lane >> 3, lc = lane & 7;
  // (a wave-uniform base per operand plus a 32-bit offset per lane and
  // load: one register per load stream instead of a 64-bit pointer)
  // the wave's first k-step ks0 starts piece ks0 / 2 of every row (ks0 is
  // a multiple of a round, so even)
  const uint8_t* wbase = a.wq + static_cast<size_t>(n0) * rs + (ks0 / 2) * 128;  // n0 is even
  const uint8_t* xbase = xq + (ks0 / 2) * 128;
  uint32_t woff[kWL], xoff[kXL];
#pragma unroll
  for (int i = 0; i < kWL; ++i)
    woff[i] = static_cast<uint32_t>(codes_offset(min(n0 + 8 * i + lr, a.N - 1) - n0, lc * 16, rs));
#pragma unroll
  for (int i = 0; i < kXL; ++i) xoff[i] = static_cast<uint32_t>(codes_offset(min(8 * i + lr, Mt - 1), lc * 16, rs));

  uint8_t* buf = s_buf[wave];
  v4u rw[NR][kWL], rx[NR][kXL];
  constexpr int NA = (TJ == 1 || KS == 1) ? 2 : 1;  // accumulators per token block
  v16f acc[NA][TJ];
#pragma unroll
  for (int p = 0; p < NA; ++p)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[p][j][e] = 0.f;

  // The scale operands the loop and the epilogue need are loaded into
  // registers before the first rounds (clamped indices: every thread loads,
  // each keeps what its slot below needs). Loads complete in order, so
  // scales loaded after the rounds would hold the first round until the
  // second had landed too; loaded first, they are in by the time round 0
  // is. A set error word (a front end whose grid-wide wait gave up) makes
  // every output NaN.
  uint32_t r_err = 0u;
  float r_s0 = 1.f, r_s1 = 1.f, r_s2 = 1.f, r_dx = 0.f, r_dw = 0.f, r_last = 1.f;
  if (!PARTIALS) {
    if (a.err != nullptr) r_err = *a.err;
    const int g0 = min(tid, ngroups - 1);
    r_s0 = a.S[g0];
    r_s1 = a.S[max(g0 - 1, 0)];
    r_s2 = a.S[max(g0 - 2, 0)];
    r_dx = dx[min(tid, Mt - 1)];
    r_dw = a.dw[min(n0 + max(tid - 64, 0), a.N - 1)];
    int last = 0;  // code whose group scale this thread's s_last / s_lastp slot takes
    if (tid >= 64 + kTN && tid < 64 + kTN + kWaves) {
      const int w = tid - 64 - kTN;
      last = (w + 1) * kpw * 64 - 1;  // the wave's last code
    } else if (tid >= 64 + kTN + kWaves && tid < 64 + kTN + 3 * kWaves) {
      // last code of accumulator q of wave w: G = 32, codes 32 q .. 32 q + 31
      // of the wave's last k-step; else the last k-step of parity q
      const int i = tid - 64 - kTN - kWaves, w = i >> 1, q = i & 1;
      last = KS == 0 ? ((w + 1) * kpw - 1) * 64 + 32 * q + 31 : ((w + 1) * kpw - 2 + q) * 64 + 63;
    }
    r_last = a.S[last >> a.log2G];
  }
#pragma unroll
  for (int s = 0; s < NR; ++s) {
    const int off = min(s, rounds - 1) * kPairRound;
#pragma unroll
    for (int i = 0; i < kWL; ++i) rw[s][i] = wload<WSTREAM>(reinterpret_cast<const v4u*>(wbase + off + woff[i]));
#pragma unroll
    for (int i = 0; i < kXL; ++i) rx[s][i] = *reinterpret_cast<const v4u*>(xbase + off + xoff[i]);
    // round s's loads all go out before round s + 1's: loads complete in
    // order, so interleaved they would hold round s until s + 1 had landed
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!PARTIALS) {
    const float base = r_err != 0u ? __builtin_nanf("") : a.ybase;
    if (tid < ngroups) {
      s_rat[tid] = tid > 0 ? r_s1 / r_s0 : 1.f;
      if (a.log2G <= 6) s_rat2[tid] = tid > 1 ? r_s2 / r_s0 : 1.f;
    }
    for (int g = tid + kThreads; g < ngroups; g += kThreads) {  // more groups than threads
      s_rat[g] = a.S[g - 1] / a.S[g];
      if (a.log2G <= 6) s_rat2[g] = a.S[g - 2] / a.S[g];
    }
    if (tid < 64) {
      s_dx[tid] = tid < Mt ? r_dx * base : 0.f;
    } else if (tid < 64 + kTN) {
      s_dw[tid - 64] = n0 + tid - 64 < a.N ? r_dw : 0.f;
    } else if (tid < 64 + kTN + kWaves) {
      s_last[tid - 64 - kTN] = r_last;
    } else if (tid < 64 + kTN + 3 * kWaves) {
      s_lastp[tid - 64 - kTN - kWaves] = r_last;
    }
  }
  __syncthreads();

  // Rounds NR ahead are fetched into the slot just emptied. For G >= 64 the
  // last NR rounds run as a second pass of the loop that fetches nothing
  // (at K = N = 8192 these would be a third of a wave's loads). At G = 32
  // every iteration refills (past the end with the last round again), which
  // keeps that instantiation's schedule unchanged.
  constexpr bool kPeel = KS > 0;
  for (int pass = 0; pass < (kPeel ? 2 : 1); ++pass) {
  const int rbeg = pass == 0 ? 0 : rounds - NR;
  const int rend = (kPeel && pass == 0) ? rounds - NR : rounds;
  for (int r0 = rbeg; r0 < rend; r0 += NR) {
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      const int r = r0 + s;
      // round -> LDS: W rows 0..31, then X rows 32.. (in-order LDS within
      // the wave: these writes land after the previous round's fragment
      // reads)
#pragma unroll
      for (int i = 0; i < kWL; ++i) *reinterpret_cast<v4u*>(buf + swz(8 * i + lr, lc)) = rw[s][i];
#pragma unroll
      for (int i = 0; i < kXL; ++i) *reinterpret_cast<v4u*>(buf + swz(32 + 8 * i + lr, lc)) = rx[s][i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // refill the slot with the round NR ahead
      if (!kPeel || pass == 0) {
        const int off = min(r + NR, rounds - 1) * kPairRound;
#pragma unroll
        for (int i = 0; i < kWL; ++i) rw[s][i] = wload<WSTREAM>(reinterpret_cast<const v4u*>(wbase + off + woff[i]));
#pragma unroll
        for (int i = 0; i < kXL; ++i) rx[s][i] = *reinterpret_cast<const v4u*>(xbase + off + xoff[i]);
      }
#pragma unroll
      for (int u = 0; u < kRound; ++u) {
        const int ks = r * kRound + u;
        const int c = 2 * u + (lane >> 5);
        const v8i fw = widen(*reinterpret_cast<const v4u*>(buf + swz(lane & 31, c)));
        const int kg = ks0 + ks;
        if constexpr (KS == 0) {
          // G = 32: lanes 0-31 carry codes 0-31 of the k-step (group 2 kg)
          // and lanes 32-63 codes 32-63 (group 2 kg + 1), for both operands.
          // Two MFMAs per block, each with the other lane half of the
          // weights zeroed.
          const bool lo = lane < 32;
          const v8i z = {0, 0, 0, 0, 0, 0, 0, 0};
          const v8i fw0 = lo ? fw : z, fw1 = lo ? z : fw;
          if constexpr (NA == 2 && TJ == 1) {
            // acc[0] takes the even groups, acc[1] the odd ones; each moves
            // from the group two back to its current one (S_{g-2} / S_g)
            const float f0 = ks > 0 ? (PARTIALS ? 0.f : s_rat2[2 * kg]) : 1.f;
            const float f1 = ks > 0 ? (PARTIALS ? 0.f : s_rat2[2 * kg + 1]) : 1.f;
            const v8i fx = widen(*reinterpret_cast<const v4u*>(buf + swz(32 + (lane & 31), c)));
            acc[0][0] *= f0;
            acc[0][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw0, fx, acc[0][0], 0, 0, 0, 0, 0, 0);
            acc[NA - 1][0] *= f1;
            acc[NA - 1][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw1, fx, acc[NA - 1][0], 0, 0, 0, 0, 0, 0);
            if constexpr (PARTIALS) {
              dump_piece<TJ>(a, acc[0], acc[0], false, t0, n0, lane, 2 * kg, ngroups);
              dump_piece<TJ>(a, acc[NA - 1], acc[0], false, t0, n0, lane, 2 * kg + 1, ngroups);
            }
          } else {
            // one accumulator per block, moved from group 2 kg - 1 to 2 kg
            // and then to 2 kg + 1; every block's first MFMA goes out before
            // any block's second rescale
            const float f0 = ks > 0 ? (PARTIALS ? 0.f : s_rat[2 * kg]) : 1.f;
            const float f1 = PARTIALS ? 0.f : s_rat[2 * kg + 1];
            v8i fx[TJ];
#pragma unroll
            for (int j = 0; j < TJ; ++j) fx[j] = widen(*reinterpret_cast<const v4u*>(buf + swz(32 + 32 * j + (lane & 31), c)));
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
              acc[0][j] *= f0;
              acc[0][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw0, fx[j], acc[0][j], 0, 0, 0, 0, 0, 0);
            }
            if constexpr (PARTIALS) dump_piece<TJ>(a, acc[0], acc[0], false, t0, n0, lane, 2 * kg, ngroups);
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
              acc[0][j] *= f1;
              acc[0][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw1, fx[j], acc[0][j], 0, 0, 0, 0, 0, 0);
            }
            if constexpr (PARTIALS) dump_piece<TJ>(a, acc[0], acc[0], false, t0, n0, lane, 2 * kg + 1, ngroups);
          }
        } else if constexpr (NA == 2) {
          // acc[q] (q = k-step parity, fixed by the unrolled u: a round is 4
          // k-steps) last took k-step kg - 2. G = 64: one group per k-step,
          // so that was two groups back (S_{g-2} / S_g); G >= 128: one group
          // back in the first two k-steps of a group, else the same group.
          // Group starts fall on k-steps with u % KS == 0, so the multiply
          // is compiled in only where one can apply (by 1 where none does).
          const int q = (u & 1) * (NA - 1);
          if (KS == 1 || u % KS < 2) {
            float f = 1.f;
            if (ks >= 2) {
              if (kspg == 1)
                f = PARTIALS ? 0.f : s_rat2[kg];
              else if ((kg & (kspg - 1)) < 2)
                f = PARTIALS ? 0.f : s_rat[kg >> log2spg];
            }
#pragma unroll
            for (int j = 0; j < TJ; ++j) acc[q][j] *= f;
          }
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const v8i fx = widen(*reinterpret_cast<const v4u*>(buf + swz(32 + 32 * j + (lane & 31), c)));
            acc[q][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw, fx, acc[q][j], 0, 0, 0, 0, 0, 0);
          }
          // the group ends here, or the wave's run ends inside it (a piece):
          // at G = 64 the group is acc[q] alone, else both accumulators
          // hold pieces of it
          if (PARTIALS && (((kg + 1) & (kspg - 1)) == 0 || ks == kpw - 1))
            dump_piece<TJ>(a, acc[q], acc[(NA - 1) - q], kspg > 1, t0, n0, lane, kg >> log2spg, ngroups);
        } else {
          // entering a new group: the accumulator goes from units of S_{g-1}
          // to units of S_g. Group starts fall only on k-steps with
          // u % KS == 0; the multiply there is unconditional (by 1 when no
          // group starts, and at the wave's first k-step, whose sum so far
          // is empty).
          if (u % KS == 0) {
            const float rg = PARTIALS ? 0.f : s_rat[kg >> log2spg];
            const float f = (ks > 0 && (kg & (kspg - 1)) == 0) ? rg : 1.f;
#pragma unroll
            for (int j = 0; j < TJ; ++j) acc[0][j] *= f;
          }
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const v8i fx = widen(*reinterpret_cast<const v4u*>(buf + swz(32 + 32 * j + (lane & 31), c)));
            acc[0][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw, fx, acc[0][j], 0, 0, 0, 0, 0, 0);
          }
          // the group ends here, or the wave's run ends inside it (a piece)
          if (PARTIALS && (((kg + 1) & (kspg - 1)) == 0 || ks == kpw - 1))
            dump_piece<TJ>(a, acc[0], acc[0], false, t0, n0, lane, kg >> log2spg, ngroups);
        }
      }
    }
  }
  }

  if constexpr (PARTIALS) return;

  // When a group spans several waves (kpw < kspg), each wave's run lies in
  // one group and its sum is an exact integer piece of that group's
  // partial: the pieces are added exactly first and the group's scale is
  // applied once. Otherwise every wave holds whole groups: its sum is made
  // absolute with the scale of its last group.
  const bool pieces = kpw < kspg;
  const int wpg = pieces ? kspg / kpw : 1;  // waves per group
  float* part = reinterpret_cast<float*>(buf);
  if constexpr (NA == 2) {
    const float sl0 = pieces ? 1.f : s_lastp[2 * wave], sl1 = pieces ? 1.f : s_lastp[2 * wave + 1];
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        part[(j * 16 + e) * 64 + lane] = acc[0][j][e] * sl0 + acc[NA - 1][j][e] * sl1;
  } else {
    const float sl = pieces ? 1.f : s_last[wave];
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) part[(j * 16 + e) * 64 + lane] = acc[0][j][e] * sl;
  }
  __syncthreads();

  // Sum of the 8 waves' sums in their storage order (consecutive threads
  // on consecutive words: a token-major walk here would put one token's
  // channels 64 words apart, all in one LDS bank), into a token-major tile.
  // Register e of lane l in block j holds token 32 j + l % 32, channel
  // 8 (e / 4) + 4 (l / 32) + e % 4.
  for (int idx = tid; idx < TJ * 16 * 64; idx += kThreads) {
    float pv[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) pv[w] = reinterpret_cast<const float*>(s_buf[w])[idx];
    float v = 0.f;
    if (!pieces) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += pv[w];
    } else {
      // p collects one group's exact partial from its waves' pieces
      float p = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        p += pv[w];
        if (((w + 1) & (wpg - 1)) == 0) {
          v += p * s_last[w + 1 - wpg];
          p = 0.f;
        }
      }
    }
    const int j = idx >> 10, e = (idx >> 6) & 15, l = idx & 63;
    const int t = 32 * j + (l & 31);
    const int nl = 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
    s_out[t * (kTN + 1) + nl] = v;
  }
  __syncthreads();
  // Y[t, n0 .. n0 + 31]: 128-byte rows
  for (int id = tid; id < TJ * 32 * kTN; id += kThreads) {
    const int t = id / kTN, nl = id % kTN;
    const int n = n0 + nl;
    if (t >= Mt || n >= a.N) continue;
    Y[static_cast<size_t>(t) * a.N + n] = s_out[t * (kTN + 1) + nl] * s_dx[t] * s_dw[nl];
  }
}

}  // namespace

// Waves per workgroup for K (0: not served): every wave gets the same whole
// number of rounds (256 codes each). K a multiple of 2048 takes 8 waves;
// other K (m 2^k, or 1024) the largest of 7, 6, 5, 4 waves that divides its
// round count.
int small_waves(int K) {
  if (K % 2048 == 0) return 8;
  if (K % 256 != 0) return 0;
  const int rounds = K / 256;
  for (int w : {7, 6, 5, 4})
    if (rounds % w == 0) return w;
  return 0;
}

// Compute units of the current device (cached per device; 256 if the
// device cannot be queried).
int device_cus() {
  constexpr int kDevs = 64;
  static std::atomic<int> cache[kDevs];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 256;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cache[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// A wave's run and the group must nest (one a multiple of the other), so
// that no group is cut part-way into a wave. Up to 64 tokens this kernel
// then always serves. Past that it serves while it needs
// fewer rounds of resident workgroups (one per CU) than the tiled
// kernel, weighted by what one round of each costs at this K (measured with
// both kernels alone at M = 65 .. 512: a tiled round costs about 4.8 times
// a few-token round at K = 8192, 3.6 times at K = 4096; 3 is assumed at
// K = 2048).
bool gemm_small_applies(int M, int K, int N, int G) {
  if (M < 1 || N < 1 || G < 32 || (G & (G - 1)) != 0 || K > kMaxKronK || K % G != 0) return false;
  const int wv = small_waves(K);
  if (wv == 0) return false;
  const int kpw = K / 64 / wv, kspg = G >= 64 ? G / 64 : 1;  // k-steps per wave, per group
  if (kpw % kspg != 0 && kspg % kpw != 0) return false;
  if (M <= 64) return true;
  if (M > kSmallMaxTokens) return false;
  const long cus = device_cus();
  const long ws = static_cast<long>((N + kTN - 1) / kTN) * ((M + 63) / 64);
  const long wt = static_cast<long>((N + 255) / 256) * ((M + 127) / 128);
  const long rs = (ws + cus - 1) / cus, rt = (wt + cus - 1) / cus;
  const long ratio10 = K >= 8192 ? 48 : K >= 4096 ? 36 : 30;  // tenths
  return rs * 10 < rt * ratio10;
}

hipError_t launch_gemm_small(const GemmCall& gc, hipStream_t s) {
  const int M = gc.M, K = gc.K, N = gc.N, G = gc.G;
  if (!gemm_small_applies(M, K, N, G)) return hipErrorInvalidValue;
  SmallArgs a{};
  a.xq = gc.xq;
  a.dx = gc.dx;
  a.S = gc.S;
  a.wq = gc.wq;
  a.dw = gc.dw;
  a.Y = gc.Y;
  a.P = gc.P;
  a.err = gc.err;
  a.ybase = gc.rotated ? kUnit / static_cast<float>(K) : kUnit;
  a.M = M;
  a.N = N;
  a.K = K;
  a.log2G = __builtin_ctz(static_cast<unsigned>(G));
  a.pm0 = gc.m0; a.pm1 = gc.m1; a.pn0 = gc.n0; a.pn1 = gc.n1;
  const bool partials = gc.P != nullptr;
  if (partials) {
    // the pieces are added into P: clear the window first
    const size_t words = static_cast<size_t>(gc.m1 - gc.m0) * (gc.n1 - gc.n0) * (K / G);
    const hipError_t e = launch_zero_u32(reinterpret_cast<uint32_t*>(gc.P), words, s);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((N + kTN - 1) / kTN, (M + 63) / 64);
  // one 64-token slice (the weights are read once) and more weight codes than
  // half the L2s hold (each XCD streams an eighth of them through its 4 MiB)
  const bool wstream = !partials && grid.y == 1 && static_cast<size_t>(K) * N / 2 > (size_t(16) << 20);
  const int wv = small_waves(K);
  const int rounds = (a.K >> 6) / wv / kRound;  // per wave: 1, 2, 4 for K = 2048, 4096, 8192; 7 for 14336
  const int spg = G >> 6;
  const int ks = G == 32 ? 0 : spg < kRound ? spg : kRound;
  // instantiations: TJ in {1, 2}, NR in {1, 2}, KS in {0 (G = 32), 1, 2, 4},
  // WV in {4, 5, 6, 7, 8}, each with and without the partials dump, and
  // without the dump also with streaming weight loads
  auto go2 = [&](auto tj, auto nr, auto w, auto pt, auto ws) {
    constexpr int TJ = decltype(tj)::value, NR = decltype(nr)::value, WV = decltype(w)::value;
    constexpr bool PT = decltype(pt)::value, WS = decltype(ws)::value;
    const dim3 block(WV * 64);
    switch (ks) {
      case 0: hipLaunchKernelGGL((gemm_small_kernel<TJ, NR, 0, WV, PT, WS>), grid, block, 0, s, a); break;
      case 1: hipLaunchKernelGGL((gemm_small_kernel<TJ, NR, 1, WV, PT, WS>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((gemm_small_kernel<TJ, NR, 2, WV, PT, WS>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((gemm_small_kernel<TJ, NR, kRound, WV, PT, WS>), grid, block, 0, s, a); break;
    }
  };
  auto go = [&](auto tj, auto nr, auto w) {
    using T = std::integral_constant<bool, true>;
    using F = std::integral_constant<bool, false>;
    if (partials)
      go2(tj, nr, w, T{}, F{});
    else if (wstream)
      go2(tj, nr, w, F{}, T{});
    else
      go2(tj, nr, w, F{}, F{});
  };
  auto by_waves = [&](auto tj, auto nr) {
    switch (wv) {
      case 4: go(tj, nr, std::integral_constant<int, 4>{}); break;
      case 5: go(tj, nr, std::integral_constant<int, 5>{}); break;
      case 6: go(tj, nr, std::integral_constant<int, 6>{}); break;
      case 7: go(tj, nr, std::integral_constant<int, 7>{}); break;
      default: go(tj, nr, std::integral_constant<int, 8>{}); break;
    }
  };
  auto by_rounds = [&](auto tj) {
    if (rounds % 2 != 0)  // NR divides the round count
      by_waves(tj, std::integral_constant<int, 1>{});
    else
      by_waves(tj, std::integral_constant<int, 2>{});
  };
  if (M <= 32)
    by_rounds(std::integral_constant<int, 1>{});
  else
    by_rounds(std::integral_constant<int, 2>{});
  return hipGetLastError();
}

}  // namespace rrs
