// Front end of the RRS A4W4 linear on gfx950: online Hadamard rotation,
// fixed channel reorder, runtime group-wise smoothing, per-token symmetric
// INT4 quantisation and nibble packing. The same row machinery also serves
// the offline weight preparation (per-output-channel INT4 of H W) and the
// calibration reorder (channel |max| after rotation).
//
// Method: RRS summary page (atlas.scime.ai), "Approach"; RRS rebuttal page
// (paperhub.cn), "Novelty" and reorder answers; per-token quantiser and its
// scale max|row| / (2^(b-1) - 1) from the AGC-OR page (paperpeel.com),
// Sec. 3.1 and App. B.1.
//
// Data movement (one wavefront owns one "block" of B = max(K, 4096)
// contiguous elements, i.e. one row, or 4096/K whole rows when K < 4096):
//   * load: lane L takes 16-byte chunks, element f = 8L + 512i + e of the
//     block sits in register 8i + e (coalesced 1 KiB per load instruction);
//   * rotation phase 1: butterflies over the in-register index bits
//     (f bits 0-2 and 9..);
//   * transpose through LDS so f bits 3-8 become register bits (lane
//     l = (f & 7) | ((f >> 9) & 7) << 3, register (f >> 3) & 63 | (f >> 12) << 6);
//   * rotation phase 2: butterflies over f bits 3-8;
//   * reorder: registers go back to LDS (conflict-free b128) and every lane
//     gathers its E = B/64 consecutive reordered positions through a
//     per-workgroup address table built from perm.
// The Sylvester transform is unnormalised (sums and differences only); the
// exact 1/K of the normalised pair is applied once in the GEMM epilogue and
// cancels out of the codes.

#include "rrs_internal.h"

namespace rrs {
namespace {

constexpr int kWave = 64;
// Adding 1.5 * 2^23 to 0 <= x < 2^22 rounds x to the nearest integer (ties
// to even, the default mode) and leaves it in the low mantissa bits: for a
// code magnitude (<= 7) the low 3 bits of the result are the magnitude.
constexpr float kMagic = 12582912.0f;

enum Mode { kStats = 0, kQuant = 1, kWeight = 2, kColmax = 3 };

template <int LOG2K>
struct Cfg {
  static constexpr int kLog2B = LOG2K > 12 ? LOG2K : 12;  // block = max(K, 4096)
  static constexpr int kB = 1 << kLog2B;
  static constexpr int kE = kB / kWave;                   // elements per lane
  static constexpr int kLog2E = kLog2B - 6;
  static constexpr int kChunks = kE / 8;                  // 16-byte loads per lane
  static constexpr int kRows = kB >> LOG2K;               // rows per block
  // LDS: one transpose/gather buffer per wave plus a shared table.
  static constexpr int kWaves = kLog2B == 12 ? 8 : 3;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kBufFloats = kB + kB / 64;         // + transpose padding
};

struct FeArgs {
  const uint16_t* src;  // X [M][K] (activations) or W [K][ldw] (weights), fp16 bits
  int rows;             // tokens, or output channels for weights
  int ldw;              // weights: row stride of W
  int log2G;
  int smooth;           // 0: S = 1 (rotation-only ablation, and weights)
  const int32_t* perm;
  uint32_t* sync;       // synchronisation block (stats / quant)
  uint8_t* codes;       // [rows][K/2]
  float* scale;         // [rows]
  float* S_out;         // [K/G]
  uint32_t* colmax;     // [K] (calibration)
};

__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// Transpose-buffer address of block element f: 8 floats of padding after
// every 512 make both the phase-1 writes and the phase-2 reads
// lane-base + immediate-offset and spread the phase-2 reads over all banks.
__device__ __forceinline__ constexpr int tpos(int f) { return f + 8 * (f >> 9); }

// Gather-buffer address of (lane, register): four consecutive registers of
// a lane are one 16-byte word, lanes side by side (conflict-free b128).
__device__ __forceinline__ constexpr int gpos(int lane, int r) {
  return ((r >> 2) << 8) | (lane << 2) | (r & 3);
}

template <int E>
__device__ __forceinline__ void butterfly(float (&v)[E], int h) {
#pragma unroll
  for (int r = 0; r < E; ++r) {
    if (!(r & h)) {
      const float a = v[r], b = v[r + h];
      v[r] = a + b;
      v[r + h] = a - b;
    }
  }
}

// Byte 0 (resp. byte 3) of four words, gathered into one word.
__device__ __forceinline__ uint32_t gather_b0(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
  const uint32_t t01 = __builtin_amdgcn_perm(x1, x0, 0x0c0c0400u);
  const uint32_t t23 = __builtin_amdgcn_perm(x3, x2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(t23, t01, 0x05040100u);
}
__device__ __forceinline__ uint32_t gather_b3(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
  const uint32_t t01 = __builtin_amdgcn_perm(x1, x0, 0x0c0c0703u);
  const uint32_t t23 = __builtin_amdgcn_perm(x3, x2, 0x0c0c0703u);
  return __builtin_amdgcn_perm(t23, t01, 0x05040100u);
}

// Eight codes -> one packed word. mag[i] holds |code i| in its low 3 bits,
// sgn[i] the float whose sign is the sign of code i. Layout (8 codes per
// little-endian word, a_j = code 2j, b_j = code 2j+1): byte j carries |a_j|
// in bits 0-2, |b_j| in bits 4-6 and sign(a_j) in bit 7; bit 3 of byte
// (j+1) mod 4 carries sign(b_j). With it, w & 0x87878787 and
// rotr(w, 4) & 0x87878787 are the a- and b-codes as fp8 e4m3 subnormals.
__device__ __forceinline__ uint32_t pack8(const uint32_t* mag, const uint32_t* sgn) {
  const uint32_t ma = gather_b0(mag[0], mag[2], mag[4], mag[6]);
  const uint32_t mb = gather_b0(mag[1], mag[3], mag[5], mag[7]);
  const uint32_t sa = gather_b3(sgn[0], sgn[2], sgn[4], sgn[6]);
  const uint32_t sb = gather_b3(sgn[7], sgn[1], sgn[3], sgn[5]);
  return ma | (mb << 4) | (sa & 0x80808080u) | ((sb >> 4) & 0x08080808u);
}

template <int LOG2K, int MODE, bool ROTATE>
__global__ void __launch_bounds__(Cfg<LOG2K>::kThreads)
frontend_kernel(FeArgs a) {
  using C = Cfg<LOG2K>;
  constexpr int K = 1 << LOG2K;
  constexpr int B = C::kB, E = C::kE, WAVES = C::kWaves;
  constexpr int NS = E / 32;  // 32-wide sub-segments per lane (G >= 32)

  __shared__ float s_buf[WAVES][C::kBufFloats];
  __shared__ uint32_t s_tab[B];                 // gather table, or channel max
  __shared__ float s_grp[K / 32];               // group max (stats) / 1/S (quant)

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int G = 1 << a.log2G;
  const int ngroups = K >> a.log2G;

  // ---- per-workgroup set-up -------------------------------------------
  if constexpr (MODE == kColmax) {
    for (int k = tid; k < K; k += C::kThreads) s_tab[k] = 0u;
  } else {
    // s_tab[gpos(l, r)] = gather-buffer address of the element that lane l,
    // register r needs: position p = E*l + r of the block, row p / K,
    // reordered column p % K, source channel perm[p % K].
    for (int idx = tid; idx < B; idx += C::kThreads) {
      const int c4 = idx >> 8, l = (idx >> 2) & 63, rr = idx & 3;
      const int p = E * l + (c4 << 2) + rr;
      const int f = ((p >> LOG2K) << LOG2K) | a.perm[p & (K - 1)];
      int sl, sr;
      if (ROTATE) {
        sl = (f & 7) | (((f >> 9) & 7) << 3);
        sr = ((f >> 3) & 63) | ((f >> 12) << 6);
      } else {
        sl = (f >> 3) & 63;
        sr = (f & 7) | ((f >> 9) << 3);
      }
      s_tab[idx] = static_cast<uint32_t>(gpos(sl, sr));
    }
    if constexpr (MODE == kStats) {
      for (int g = tid; g < ngroups; g += C::kThreads) s_grp[g] = 0.f;
    } else if constexpr (MODE == kQuant) {
      for (int g = tid; g < ngroups; g += C::kThreads) {
        float sg = 1.f;
        if (a.smooth) {
          sg = __uint_as_float(a.sync[kSyncGroups + g]);
          if (!(sg > 0.f)) sg = 1.f;  // all-zero group over every token
        }
        s_grp[g] = 1.f / sg;
      }
    }
  }
  __syncthreads();

  const int blk = blockIdx.x * WAVES + wave;
  const int row0 = blk * C::kRows;
  if (row0 < a.rows) {
    // ---- load ------------------------------------------------------------
    float v[E];
#pragma unroll
    for (int i = 0; i < C::kChunks; ++i) {
      const int f0 = 8 * lane + 512 * i;
      const int row = row0 + (f0 >> LOG2K);
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (row < a.rows) {
        if constexpr (MODE == kWeight) {
          // column `row` of W [K][ldw], channels k0..k0+7
          const int k0 = f0 & (K - 1);
          const uint16_t* p = a.src + static_cast<size_t>(k0) * a.ldw + row;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = static_cast<uint32_t>(p[(2 * e) * static_cast<size_t>(a.ldw)]) |
                   (static_cast<uint32_t>(p[(2 * e + 1) * static_cast<size_t>(a.ldw)]) << 16);
        } else {
          const uint4 q = *reinterpret_cast<const uint4*>(a.src + static_cast<size_t>(row0) * K + f0);
          w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * i + 2 * e] = h2f(w[e] & 0xffffu);
        v[8 * i + 2 * e + 1] = h2f(w[e] >> 16);
      }
    }

    float* wb = s_buf[wave];
    if constexpr (ROTATE) {
      // ---- rotation, phase 1: register bits <-> f bits 0-2, 9.. --------
#pragma unroll
      for (int rb = 0; rb < C::kLog2E; ++rb) {
        const int fb = rb < 3 ? rb : rb + 6;
        if (fb < LOG2K) butterfly<E>(v, 1 << rb);
      }
      // ---- transpose ---------------------------------------------------
#pragma unroll
      for (int i = 0; i < C::kChunks; ++i) {
        const int t = tpos(8 * lane + 512 * i);
        *reinterpret_cast<float4*>(wb + t) = make_float4(v[8 * i], v[8 * i + 1], v[8 * i + 2], v[8 * i + 3]);
        *reinterpret_cast<float4*>(wb + t + 4) = make_float4(v[8 * i + 4], v[8 * i + 5], v[8 * i + 6], v[8 * i + 7]);
      }
      lds_fence();
      {
        const int base = (lane & 7) + (lane >> 3) * (512 + 8);
#pragma unroll
        for (int r = 0; r < E; ++r) v[r] = wb[base + 8 * (r & 63) + (4096 + 64) * (r >> 6)];
      }
      lds_fence();
      // ---- rotation, phase 2: f bits 3-8 -------------------------------
#pragma unroll
      for (int rb = 0; rb < 6; ++rb) {
        if (rb + 3 < LOG2K) butterfly<E>(v, 1 << rb);
      }
    }

    if constexpr (MODE == kColmax) {
      // channel |max| over the block's rows (LDS), folded into global below
#pragma unroll
      for (int r = 0; r < E; ++r) {
        const int f = (lane & 7) | ((r & 63) << 3) | ((lane >> 3) << 9) | ((r >> 6) << 12);
        if (row0 + (f >> LOG2K) < a.rows)
          atomicMax(&s_tab[f & (K - 1)], __float_as_uint(fabsf(v[r])));
      }
    } else {
      // ---- reorder: scatter registers, gather reordered positions ------
#pragma unroll
      for (int c = 0; c < E / 4; ++c)
        *reinterpret_cast<float4*>(wb + gpos(lane, 4 * c)) = make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
      lds_fence();
#pragma unroll
      for (int c = 0; c < E / 4; ++c) {
        const uint4 ad = reinterpret_cast<const uint4*>(s_tab)[c * 64 + lane];
        v[4 * c] = wb[ad.x];
        v[4 * c + 1] = wb[ad.y];
        v[4 * c + 2] = wb[ad.z];
        v[4 * c + 3] = wb[ad.w];
      }
      lds_fence();

      // v[r] = Zp of block position p = E*lane + r: row rl, column j0 + r
      const int rl = (E * lane) >> LOG2K;
      const int j0 = (E * lane) & (K - 1);
      const bool row_ok = row0 + rl < a.rows;

      // ---- per-row group |max| -----------------------------------------
      float m[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float x = fabsf(v[32 * s]);
#pragma unroll
        for (int r = 1; r < 32; ++r) x = fmaxf(x, fabsf(v[32 * s + r]));
        m[s] = x;
      }
      // merge sub-segments of the same group inside the lane
#pragma unroll
      for (int st = 1; st < NS; st <<= 1) {
        if (G > 32 * st) {
          float t[NS];
#pragma unroll
          for (int s = 0; s < NS; ++s) t[s] = fmaxf(m[s], m[s ^ st]);
#pragma unroll
          for (int s = 0; s < NS; ++s) m[s] = t[s];
        }
      }
      // and across the G / E lanes of a group
      for (int d = 1; d * E < G; d <<= 1) {
#pragma unroll
        for (int s = 0; s < NS; ++s) m[s] = fmaxf(m[s], __shfl_xor(m[s], d));
      }

      if constexpr (MODE == kStats) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int j = j0 + 32 * s;
          if (row_ok && (j & (G - 1)) == 0 && m[s] > 0.f)
            atomicMax(reinterpret_cast<uint32_t*>(&s_grp[j >> a.log2G]), __float_as_uint(m[s]));
        }
      } else {
        // ---- per-token scale, codes, pack ------------------------------
        float inv[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) inv[s] = (MODE == kQuant) ? s_grp[(j0 + 32 * s) >> a.log2G] : 1.f;
        float rmax = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) rmax = fmaxf(rmax, m[s] * inv[s]);
        for (int d = 1; d * E < K; d <<= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, d));
        const float k7 = rmax > 0.f ? 7.f / rmax : 0.f;
        uint32_t packed[E / 8];
#pragma unroll
        for (int o = 0; o < E / 8; ++o) {
          uint32_t mag[8], sgn[8];
          const float ks = inv[(8 * o) / 32] * k7;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            mag[e] = __float_as_uint(fmaf(fabsf(v[8 * o + e]), ks, kMagic));
            sgn[e] = __float_as_uint(v[8 * o + e]);
          }
          packed[o] = pack8(mag, sgn);
        }
        if (row_ok) {
          uint8_t* dst = a.codes + static_cast<size_t>(row0 + rl) * (K / 2) + j0 / 2;
#pragma unroll
          for (int o = 0; o < E / 32; ++o)
            reinterpret_cast<uint4*>(dst)[o] = make_uint4(packed[4 * o], packed[4 * o + 1], packed[4 * o + 2], packed[4 * o + 3]);
          if (j0 == 0) a.scale[row0 + rl] = rmax / 7.f;
        }
      }
    }
  }

  // ---- fold the workgroup's partial maxima into global memory ----------
  if constexpr (MODE == kStats) {
    __syncthreads();
    for (int g = tid; g < ngroups; g += C::kThreads) {
      const uint32_t bits = __float_as_uint(s_grp[g]);
      if (bits) atomicMax(&a.sync[kSyncGroups + g], bits);
    }
  } else if constexpr (MODE == kColmax) {
    __syncthreads();
    for (int k = tid; k < K; k += C::kThreads) {
      const uint32_t bits = s_tab[k];
      if (bits) atomicMax(&a.colmax[k], bits);
    }
  } else if constexpr (MODE == kQuant) {
    // The last workgroup to finish reading the running maxima publishes the
    // guarded scales and re-zeroes the synchronisation block for the next
    // call (every workgroup copied its scales to LDS before arriving here).
    __shared__ int s_last;
    __syncthreads();
    if (tid == 0) {
      __threadfence();
      const uint32_t done = atomicAdd(&a.sync[kSyncCounter], 1u);
      s_last = done == gridDim.x - 1;
    }
    __syncthreads();
    if (s_last) {
      __threadfence();
      for (int g = tid; g < ngroups; g += C::kThreads) {
        const float sg = __uint_as_float(a.sync[kSyncGroups + g]);
        a.S_out[g] = (a.smooth && sg > 0.f) ? sg : 1.f;
        a.sync[kSyncGroups + g] = 0u;
      }
      if (tid == 0) a.sync[kSyncCounter] = 0u;
    }
  }
}

// Stable descending rank: perm[rank(j)] = j with rank(j) = #{i : c_i > c_j}
// + #{i < j : c_i == c_j} (values compared as non-negative float bits).
__global__ void __launch_bounds__(1024) rank_kernel(const uint32_t* c, int K, int32_t* perm) {
  __shared__ uint32_t s_c[1 << kMaxLog2K];
  for (int k = threadIdx.x; k < K; k += blockDim.x) s_c[k] = c[k];
  __syncthreads();
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < K; j += gridDim.x * blockDim.x) {
    const uint32_t cj = s_c[j];
    int rank = 0;
    for (int i = 0; i < K; ++i) {
      const uint32_t ci = s_c[i];
      rank += (ci > cj) || (ci == cj && i < j);
    }
    perm[rank] = j;
  }
}

__global__ void zero_u32_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

template <int LOG2K, int MODE, bool ROTATE>
hipError_t launch_mode(const FeArgs& a, hipStream_t s) {
  using C = Cfg<LOG2K>;
  const int nblk = (a.rows + C::kRows - 1) / C::kRows;
  const int grid = (nblk + C::kWaves - 1) / C::kWaves;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((frontend_kernel<LOG2K, MODE, ROTATE>), dim3(grid), dim3(C::kThreads), 0, s, a);
  return hipGetLastError();
}

template <int MODE, bool ROTATE>
hipError_t dispatch_k(int log2K, const FeArgs& a, hipStream_t s) {
  switch (log2K) {
    case 6: return launch_mode<6, MODE, ROTATE>(a, s);
    case 7: return launch_mode<7, MODE, ROTATE>(a, s);
    case 8: return launch_mode<8, MODE, ROTATE>(a, s);
    case 9: return launch_mode<9, MODE, ROTATE>(a, s);
    case 10: return launch_mode<10, MODE, ROTATE>(a, s);
    case 11: return launch_mode<11, MODE, ROTATE>(a, s);
    case 12: return launch_mode<12, MODE, ROTATE>(a, s);
    case 13: return launch_mode<13, MODE, ROTATE>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_frontend(const uint16_t* X, int M, int log2K, int G, const int32_t* perm,
                           uint8_t* xq, float* dx, float* S_out, uint32_t* sync, int flags,
                           hipStream_t s) {
  FeArgs a{};
  a.src = X;
  a.rows = M;
  a.log2G = __builtin_ctz(static_cast<unsigned>(G));
  a.smooth = (flags & 2) ? 0 : 1;
  a.perm = perm;
  a.sync = sync;
  a.codes = xq;
  a.scale = dx;
  a.S_out = S_out;
  const bool rotate = !(flags & 1);
  hipError_t e;
  if (a.smooth) {
    e = rotate ? dispatch_k<kStats, true>(log2K, a, s) : dispatch_k<kStats, false>(log2K, a, s);
    if (e != hipSuccess) return e;
  }
  return rotate ? dispatch_k<kQuant, true>(log2K, a, s) : dispatch_k<kQuant, false>(log2K, a, s);
}

hipError_t launch_weight_prep(const uint16_t* W, int log2K, int N, const int32_t* perm,
                              uint8_t* wq, float* dw, hipStream_t s) {
  FeArgs a{};
  a.src = W;
  a.rows = N;
  a.ldw = N;
  a.log2G = log2K;
  a.smooth = 0;
  a.perm = perm;
  a.codes = wq;
  a.scale = dw;
  return dispatch_k<kWeight, true>(log2K, a, s);
}

hipError_t launch_calibrate(const uint16_t* Xc, int T, int log2K, int32_t* perm, uint32_t* ws,
                            hipStream_t s) {
  const int K = 1 << log2K;
  hipError_t e = launch_zero_u32(ws, static_cast<size_t>(K), s);
  if (e != hipSuccess) return e;
  FeArgs a{};
  a.src = Xc;
  a.rows = T;
  a.log2G = log2K;
  a.colmax = ws;
  e = dispatch_k<kColmax, true>(log2K, a, s);
  if (e != hipSuccess) return e;
  const int grid = (K + 1023) / 1024;
  hipLaunchKernelGGL(rank_kernel, dim3(grid), dim3(1024), 0, s, ws, K, perm);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 1024 ? blocks : 1024);
  hipLaunchKernelGGL(zero_u32_kernel, dim3(grid), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace rrs
