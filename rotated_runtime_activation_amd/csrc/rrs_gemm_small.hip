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
constexpr float kUnit = 262144.0f;  // 2^18: one integer product in accumulator units

struct SmallArgs {
  const uint8_t* xq;
  const float* dx;
  const float* S;
  const uint8_t* wq;
  const float* dw;
  float* Y;
  int M, N, K, log2G;
};

// a-codes (even) and b-codes (odd) of a packed word as e4m3 subnormals
__device__ __forceinline__ uint32_t ecodes(uint32_t w) { return w & 0x87878787u; }
__device__ __forceinline__ uint32_t ocodes(uint32_t w) { return __builtin_amdgcn_alignbit(w, w, 4) & 0x87878787u; }
__device__ __forceinline__ v8i widen(v4u w) {
  return v8i{(int)ecodes(w.x), (int)ocodes(w.x), (int)ecodes(w.y), (int)ocodes(w.y),
             (int)ecodes(w.z), (int)ocodes(w.z), (int)ecodes(w.w), (int)ocodes(w.w)};
}

// byte offset of 16-byte chunk c of row r in a wave's round buffer
__device__ __forceinline__ int swz(int r, int c) { return r * kRows + ((c ^ (r & 7)) << 4); }

// TJ: 32-token blocks per slice (1 for M <= 32, else 2); NR: rounds of loads
// in flight (1 or 2; divides the wave's round count); KS: min(k-steps per
// group, kRound), the spacing of possible group starts inside a round, or 0
// for G = 32 (two groups in every k-step); WV: waves per workgroup.
template <int TJ, int NR, int KS, int WV>
__global__ void __launch_bounds__(WV * 64) gemm_small_kernel(SmallArgs a) {
  constexpr int kWaves = WV, kThreads = WV * 64;
  static_assert(WV <= kMaxWaves && 64 + kTN + WV <= kThreads, "one thread per scale preloaded");
  constexpr int kWL = 4;            // W loads per lane per round (32 rows / 8)
  constexpr int kXL = 4 * TJ;       // X loads per lane per round
  constexpr int kBuf = (32 + 32 * TJ) * kRows;  // round buffer bytes per wave
  static_assert(TJ * 16 * 64 * 4 <= kBuf, "a wave's sums fit its round buffer");
  static_assert(kMaxKronK >= (1 << kMaxLog2K), "group ratio table sized by the largest K");
  __shared__ float s_rat[kMaxKronK / 32];
  __shared__ float s_dx[64];         // dx[t] 2^18 / K (0 past M)
  __shared__ float s_dw[kTN];        // dw of the workgroup's channels (0 past N)
  __shared__ float s_last[kWaves];   // scale of each wave's last group
  __shared__ float s_out[64 * (kTN + 1)];  // the summed tile, token-major, rows padded by one word
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[kWaves][kBuf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * kTN;
  const int Kb = a.K / 2;
  // this workgroup's token slice: rows t0 .. t0 + Mt - 1 of xq, dx and Y
  const int t0 = blockIdx.y * 64;
  const int Mt = min(64, a.M - t0);
  const uint8_t* xq = a.xq + static_cast<size_t>(t0) * Kb;
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
  // clamped to the matrix; clamped rows feed outputs that are never stored)
  const int lr = lane >> 3, lc = lane & 7;
  const uint8_t* wsrc[kWL];
  const uint8_t* xsrc[kXL];
#pragma unroll
  for (int i = 0; i < kWL; ++i)
    wsrc[i] = a.wq + static_cast<size_t>(min(n0 + 8 * i + lr, a.N - 1)) * Kb + ks0 * 32 + lc * 16;
#pragma unroll
  for (int i = 0; i < kXL; ++i)
    xsrc[i] = xq + static_cast<size_t>(min(8 * i + lr, Mt - 1)) * Kb + ks0 * 32 + lc * 16;

  uint8_t* buf = s_buf[wave];
  v4u rw[NR][kWL], rx[NR][kXL];
  v16f acc[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

#pragma unroll
  for (int s = 0; s < NR; ++s) {
    const int off = min(s, rounds - 1) * kRows;
#pragma unroll
    for (int i = 0; i < kWL; ++i) rw[s][i] = *reinterpret_cast<const v4u*>(wsrc[i] + off);
#pragma unroll
    for (int i = 0; i < kXL; ++i) rx[s][i] = *reinterpret_cast<const v4u*>(xsrc[i] + off);
  }
  // the scales the loop and the epilogue need, read up front after the
  // first rounds' loads: their latency then overlaps those loads instead of
  // ending the kernel (as plain loads at the end they cost several
  // microseconds per call)
  const float base = kUnit / static_cast<float>(a.K);
  for (int g = tid; g < ngroups; g += kThreads) s_rat[g] = g > 0 ? a.S[g - 1] / a.S[g] : 1.f;
  if (tid < 64) {
    s_dx[tid] = tid < Mt ? dx[tid] * base : 0.f;
  } else if (tid < 64 + kTN) {
    const int n = n0 + tid - 64;
    s_dw[tid - 64] = n < a.N ? a.dw[n] : 0.f;
  } else if (tid < 64 + kTN + kWaves) {
    const int w = tid - 64 - kTN;
    s_last[w] = a.S[(((w + 1) * kpw) * 64 - 1) >> a.log2G];  // group of the wave's last code
  }
  __syncthreads();

  for (int r0 = 0; r0 < rounds; r0 += NR) {
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
      // refill the slot with the round NR ahead (past the end: the last
      // round again, so every iteration issues the same loads)
      const int off = min(r + NR, rounds - 1) * kRows;
#pragma unroll
      for (int i = 0; i < kWL; ++i) rw[s][i] = *reinterpret_cast<const v4u*>(wsrc[i] + off);
#pragma unroll
      for (int i = 0; i < kXL; ++i) rx[s][i] = *reinterpret_cast<const v4u*>(xsrc[i] + off);
#pragma unroll
      for (int u = 0; u < kRound; ++u) {
        const int ks = r * kRound + u;
        // entering a new group: the accumulator goes from units of S_{g-1}
        // to units of S_g. Group starts fall only on k-steps with
        // u % KS == 0; the multiply there is unconditional (by 1 when no
        // group starts, and at the wave's first k-step, whose sum so far is
        // empty).
        const int c = 2 * u + (lane >> 5);
        const v8i fw = widen(*reinterpret_cast<const v4u*>(buf + swz(lane & 31, c)));
        if constexpr (KS == 0) {
          // G = 32: lanes 0-31 carry codes 0-31 of the k-step (group 2 kg)
          // and lanes 32-63 codes 32-63 (group 2 kg + 1), for both operands.
          // Two MFMAs, each with the other lane half of the weights zeroed,
          // and the rescale into the second group between them.
          const int kg = ks0 + ks;
          const float f0 = ks > 0 ? s_rat[2 * kg] : 1.f, f1 = s_rat[2 * kg + 1];
          const bool lo = lane < 32;
          const v8i z = {0, 0, 0, 0, 0, 0, 0, 0};
          const v8i fw0 = lo ? fw : z, fw1 = lo ? z : fw;
          v8i fx[TJ];
#pragma unroll
          for (int j = 0; j < TJ; ++j) fx[j] = widen(*reinterpret_cast<const v4u*>(buf + swz(32 + 32 * j + (lane & 31), c)));
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            acc[j] *= f0;
            acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw0, fx[j], acc[j], 0, 0, 0, 0, 0, 0);
            acc[j] *= f1;
            acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw1, fx[j], acc[j], 0, 0, 0, 0, 0, 0);
          }
        } else {
          if (u % KS == 0) {
            const int kg = ks0 + ks;
            const float rg = s_rat[kg >> log2spg];
            const float f = (ks > 0 && (kg & (kspg - 1)) == 0) ? rg : 1.f;
#pragma unroll
            for (int j = 0; j < TJ; ++j) acc[j] *= f;
          }
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const v8i fx = widen(*reinterpret_cast<const v4u*>(buf + swz(32 + 32 * j + (lane & 31), c)));
            acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw, fx, acc[j], 0, 0, 0, 0, 0, 0);
          }
        }
      }
    }
  }

  // When a group spans several waves (kpw < kspg), each wave's run lies in
  // one group and its sum is an exact integer piece of that group's
  // partial: the pieces are added exactly first and the group's scale is
  // applied once. Otherwise every wave holds whole groups: its sum is made
  // absolute with the scale of its last group.
  const bool pieces = kpw < kspg;
  const int wpg = pieces ? kspg / kpw : 1;  // waves per group
  const float sl = pieces ? 1.f : s_last[wave];
  float* part = reinterpret_cast<float*>(buf);
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) part[(j * 16 + e) * 64 + lane] = acc[j][e] * sl;
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

// A wave's run and the group must nest (one a multiple of the other), so
// that no group is cut part-way into a wave. Up to 64 tokens this kernel
// then always serves. Past that it serves while it needs
// fewer rounds of resident workgroups (one per CU, 256 CUs) than the tiled
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
  constexpr long kCUs = 256;
  const long ws = static_cast<long>((N + kTN - 1) / kTN) * ((M + 63) / 64);
  const long wt = static_cast<long>((N + 255) / 256) * ((M + 127) / 128);
  const long rs = (ws + kCUs - 1) / kCUs, rt = (wt + kCUs - 1) / kCUs;
  const long ratio10 = K >= 8192 ? 48 : K >= 4096 ? 36 : 30;  // tenths
  return rs * 10 < rt * ratio10;
}

hipError_t launch_gemm_small(const uint8_t* xq, const float* dx, const float* S, int M, int K, int N, int G,
                             const uint8_t* wq, const float* dw, float* Y, hipStream_t s) {
  if (!gemm_small_applies(M, K, N, G)) return hipErrorInvalidValue;
  SmallArgs a{};
  a.xq = xq;
  a.dx = dx;
  a.S = S;
  a.wq = wq;
  a.dw = dw;
  a.Y = Y;
  a.M = M;
  a.N = N;
  a.K = K;
  a.log2G = __builtin_ctz(static_cast<unsigned>(G));
  const dim3 grid((N + kTN - 1) / kTN, (M + 63) / 64);
  const int wv = small_waves(K);
  const int rounds = (a.K >> 6) / wv / kRound;  // per wave: 1, 2, 4 for K = 2048, 4096, 8192; 7 for 14336
  const int spg = G >> 6;
  const int ks = G == 32 ? 0 : spg < kRound ? spg : kRound;
  // instantiations: TJ in {1, 2}, NR in {1, 2}, KS in {0 (G = 32), 1, 2, 4},
  // WV in {4, 5, 6, 7, 8}
  auto go = [&](auto tj, auto nr, auto w) {
    constexpr int TJ = decltype(tj)::value, NR = decltype(nr)::value, WV = decltype(w)::value;
    const dim3 block(WV * 64);
    switch (ks) {
      case 0: hipLaunchKernelGGL((gemm_small_kernel<TJ, NR, 0, WV>), grid, block, 0, s, a); break;
      case 1: hipLaunchKernelGGL((gemm_small_kernel<TJ, NR, 1, WV>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((gemm_small_kernel<TJ, NR, 2, WV>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((gemm_small_kernel<TJ, NR, kRound, WV>), grid, block, 0, s, a); break;
    }
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
