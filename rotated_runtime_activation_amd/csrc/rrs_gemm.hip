// Grouped INT4 x INT4 GEMM of the RRS A4W4 linear on gfx950.
//
// Y[t, n] = (1/K) dx[t] dw[n] sum_g S[g] P_g[t, n],
// P_g[t, n] = sum_{j in group g} q[t, j] qw[n, j]    (exact int32)
//
// The group scale multiplies each group's integer partial before the fp32
// accumulation: the smoothing is not migrated into the weights (RRS summary
// page, atlas.scime.ai, "Approach"), and grouping the scales along K keeps
// the contraction in wide integer tiles (RRS rebuttal page, paperhub.cn,
// "Novelty": per-channel scales do not fit the hardware's tiled scheme).
//
// gfx950 has no 4-bit integer matrix instruction, so codes are widened to
// int8 on their way into LDS and multiplied with v_mfma_i32_16x16x64_i8
// (v_mfma_i32_16x16x32_i8 when G = 32). The widening keeps each code in the
// high nibble of its byte (16 q, one AND per four codes), so every product
// carries a factor 256 that the epilogue removes exactly.
//
// Both operands are K-contiguous ("NT"): xq [M][K/2], wq [N][K/2]. Within a
// packed 32-bit word the widening emits the even codes then the odd codes;
// A and B are widened the same way, so the contraction pairs equal K
// indices and each 16-byte chunk stays inside one group (G >= 32).

#include "rrs_internal.h"

namespace rrs {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kThreads = 256;

struct GemmArgs {
  const uint8_t* xq;
  const float* dx;
  const float* S;
  const uint8_t* wq;
  const float* dw;
  float* Y;
  int32_t* P;       // partials window (null: normal output)
  int M, N, K, log2G;
  int pm0, pm1, pn0, pn1;
  float out_scale;  // 1 / (256 K)
};

// 16 packed bytes (32 codes) -> 32 int8 bytes holding 16 * code.
__device__ __forceinline__ void widen16(const uint4 p, uint32_t (&o)[8]) {
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = (w[i] << 4) & 0xf0f0f0f0u;   // even codes
    o[2 * i + 1] = w[i] & 0xf0f0f0f0u;      // odd codes
  }
}

template <int KS>
struct Step;
template <>
struct Step<64> {  // 16x16x64 i8: 16 bytes of K per lane
  static constexpr int kPackedRowBytes = 32;
  typedef v4i frag;
  __device__ static v4i mma(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
};
template <>
struct Step<32> {  // 16x16x32 i8: 8 bytes of K per lane
  static constexpr int kPackedRowBytes = 16;
  typedef long frag;
  __device__ static v4i mma(long a, long b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, c, 0, 0, 0);
  }
};

template <int KS>
__global__ void __launch_bounds__(kThreads) gemm_kernel(GemmArgs a) {
  using St = Step<KS>;
  constexpr int ROWB = KS + 16;  // LDS row stride (bytes): widened step + pad
  constexpr int PRB = St::kPackedRowBytes;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kBM * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][kBN * ROWB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kBM;
  const int n0 = blockIdx.x * kBN;
  const int Kb = a.K / 2;  // packed bytes per row
  const int nsteps = a.K / KS;
  const int steps_per_group = (1 << a.log2G) / KS;

  // global -> register staging: each thread moves PRB/2 packed bytes of one
  // A row and of one B row per step (KS=64: 16 B; KS=32: 8 B)
  const int ld_row = tid >> 1;
  const int ld_off = (tid & 1) * (PRB / 2);
  const bool a_ok = m0 + ld_row < a.M;
  const bool b_ok = n0 + ld_row < a.N;
  const uint8_t* gA = a.xq + static_cast<size_t>(m0 + ld_row) * Kb + ld_off;
  const uint8_t* gB = a.wq + static_cast<size_t>(n0 + ld_row) * Kb + ld_off;

  auto load = [&](int step, uint4& ra, uint4& rb) {
    ra = make_uint4(0, 0, 0, 0);
    rb = make_uint4(0, 0, 0, 0);
    const int kb = step * PRB;
    if constexpr (KS == 64) {
      if (a_ok) ra = *reinterpret_cast<const uint4*>(gA + kb);
      if (b_ok) rb = *reinterpret_cast<const uint4*>(gB + kb);
    } else {
      if (a_ok) { const uint2 t = *reinterpret_cast<const uint2*>(gA + kb); ra.x = t.x; ra.y = t.y; }
      if (b_ok) { const uint2 t = *reinterpret_cast<const uint2*>(gB + kb); rb.x = t.x; rb.y = t.y; }
    }
  };
  auto store = [&](int buf, const uint4& ra, const uint4& rb) {
    uint32_t oa[8], ob[8];
    widen16(ra, oa);
    widen16(rb, ob);
    uint8_t* pa = &sA[buf][ld_row * ROWB + ld_off * 2];
    uint8_t* pb = &sB[buf][ld_row * ROWB + ld_off * 2];
    if constexpr (KS == 64) {
      reinterpret_cast<uint4*>(pa)[0] = make_uint4(oa[0], oa[1], oa[2], oa[3]);
      reinterpret_cast<uint4*>(pa)[1] = make_uint4(oa[4], oa[5], oa[6], oa[7]);
      reinterpret_cast<uint4*>(pb)[0] = make_uint4(ob[0], ob[1], ob[2], ob[3]);
      reinterpret_cast<uint4*>(pb)[1] = make_uint4(ob[4], ob[5], ob[6], ob[7]);
    } else {
      reinterpret_cast<uint4*>(pa)[0] = make_uint4(oa[0], oa[1], oa[2], oa[3]);
      reinterpret_cast<uint4*>(pb)[0] = make_uint4(ob[0], ob[1], ob[2], ob[3]);
    }
  };

  v4i acc[4][4];
  float accf[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) accf[i][j][e] = 0.f;
    }

  uint4 ra, rb;
  load(0, ra, rb);
  store(0, ra, rb);
  __syncthreads();

  // MFMA operand addresses: lane -> row/col (lane & 15), K bytes
  // (lane >> 4) * (KS / 4)
  const int fr = lane & 15;
  const int fk = (lane >> 4) * (KS / 4);

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) load(step + 1, ra, rb);

    typename St::frag fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i] = *reinterpret_cast<const typename St::frag*>(&sA[buf][(wm * 64 + i * 16 + fr) * ROWB + fk]);
      fb[i] = *reinterpret_cast<const typename St::frag*>(&sB[buf][(wn * 64 + i * 16 + fr) * ROWB + fk]);
    }
    const int gs = step % steps_per_group;
    if (gs == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = St::mma(fa[i], fb[j], v4i{0, 0, 0, 0});
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = St::mma(fa[i], fb[j], acc[i][j]);
    }

    if (gs == steps_per_group - 1) {
      const int g = step / steps_per_group;
      if (a.P == nullptr) {
        const float sg = a.S[g];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) accf[i][j][e] = fmaf(sg, static_cast<float>(acc[i][j][e]), accf[i][j][e]);
      } else {
        const int ng = a.K >> a.log2G;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
              const int col = n0 + wn * 64 + j * 16 + (lane & 15);
              if (row >= a.pm0 && row < a.pm1 && col >= a.pn0 && col < a.pn1) {
                const size_t o = (static_cast<size_t>(row - a.pm0) * (a.pn1 - a.pn0) + (col - a.pn0)) * ng + g;
                a.P[o] = acc[i][j][e] >> 8;
              }
            }
      }
    }

    if (more) store(buf ^ 1, ra, rb);
    __syncthreads();
  }

  if (a.P != nullptr) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
      if (row >= a.M) continue;
      const float rs = a.dx[row] * a.out_scale;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + (lane & 15);
        if (col < a.N) a.Y[static_cast<size_t>(row) * a.N + col] = accf[i][j][e] * rs * a.dw[col];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* xq, const float* dx, const float* S, int M, int log2K,
                       int N, int G, const uint8_t* wq, const float* dw, float* Y, int32_t* P,
                       int m0, int m1, int n0, int n1, hipStream_t s) {
  GemmArgs a{};
  a.xq = xq;
  a.dx = dx;
  a.S = S;
  a.wq = wq;
  a.dw = dw;
  a.Y = Y;
  a.P = P;
  a.M = M;
  a.N = N;
  a.K = 1 << log2K;
  a.log2G = __builtin_ctz(static_cast<unsigned>(G));
  a.pm0 = m0; a.pm1 = m1; a.pn0 = n0; a.pn1 = n1;
  a.out_scale = 1.0f / (256.0f * static_cast<float>(a.K));
  if (M == 0 || N == 0) return hipSuccess;
  dim3 grid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM);
  if (P != nullptr) {
    // only the tiles that cover the window
    grid = dim3((n1 - 1) / kBN + 1, (m1 - 1) / kBM + 1);
  }
  if (G == 32)
    hipLaunchKernelGGL(gemm_kernel<32>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace rrs
