// Front end of the RRS A4W4 linear for K = m 2^k, m in {12, 20, 28} (no
// power of two; e.g. K = 14336 = 28 * 512): the rotation is the Kronecker
// product H_K = H_m (x) H_n, n = 2^k, with H_m from Paley's constructions
// and Sylvester H_n; element f = i n + j of a row (i < m, j < n).
//
// Method as in rrs_frontend.hip (RRS summary page, atlas.scime.ai,
// "Approach"; RRS rebuttal page, paperhub.cn, "Novelty"; per-token scale of
// the AGC-OR page, paperpeel.com, Sec. 3.1 and App. B.1; signed rotation,
// AGC-OR Sec. 4.1 and 4.6). Hadamard matrices of order 12, 20 and 28 are not
// Sylvester matrices; QuaRot-style rotations use such Kronecker products for
// hidden sizes like 14336.
//
// One workgroup of 512 threads rotates one row at a time (loading its next
// row meanwhile): H_m runs first on the matrix cores (fp16 32 x 32 x 16
// MFMA against +-1 H_m^T: exact products, fp32 sums), its operands loaded
// from memory straight into the matrix-core layout; then H_n runs as
// butterfly levels, the lowest in registers where a lane holds adjacent
// columns and the rest as two radix-16 passes over the fp32 row in LDS
// (two radix-8 passes at n = 64). The two factors commute
// (H_m (x) H_n = (H_m (x) I)(I (x) H_n)). Then the row is
// gathered in reordered order through perm, eight positions (one packed
// word) per thread and step.
//
// The group scales need every token first, so the smoothed front end is
// three launches: stats (each row's group maxima into its own row of a
// scratch area, the codes buffer, which the quantise pass overwrites later;
// no atomics), reduce (S = max over those rows), quantise. Given a row area
// of 4 M K bytes, the stats pass also stores each rotated, reordered fp32
// row and the quantise pass streams them back (one workgroup per row);
// without one it rotates every row again. Both give the same bits: the
// quantise arithmetic is the same and the rows are those the stats pass
// reduced.
// Weight preparation and calibration use the same rotation.

#include "rrs_codes.h"
#include "rrs_internal.h"

#include <atomic>

namespace rrs {
namespace {

constexpr int kKT = 512;  // threads per workgroup

enum KronMode { kKStats = 0, kKQuant = 1, kKWeight = 2, kKColmax = 3, kKFused = 4 };

// ---- Paley Hadamard matrices H_m[i][a], built at compile time -------------
constexpr int legendre(int a, int q) {
  a %= q;
  if (a < 0) a += q;
  if (a == 0) return 0;
  int r = 1, b = a, e = (q - 1) / 2;
  while (e) {
    if (e & 1) r = r * b % q;
    b = b * b % q;
    e >>= 1;
  }
  return r == 1 ? 1 : -1;
}

// m = 12, 20: construction I with q = m - 1 (q = 3 mod 4), H = I + S,
// S = [[0, 1^T], [-1, Q]], Q[i][j] = chi(j - i). m = 28: construction II with
// q = 13 (q = 1 mod 4), C = [[0, 1^T], [1, Q]], H = [[C + I, C - I],
// [C - I, -C - I]].
constexpr int paley(int m, int i, int a) {
  if (m == 12 || m == 20) {
    if (i == a || i == 0) return 1;
    if (a == 0) return -1;
    return legendre(a - i, m - 1);
  }
  const int br = i / 14, bc = a / 14, r = i % 14, c = a % 14;
  const int C = (r == c) ? 0 : (r == 0 || c == 0) ? 1 : legendre(c - r, 13);
  const int e = r == c ? 1 : 0;
  if (br == 0 && bc == 0) return C + e;
  if (br == 1 && bc == 1) return -C - e;
  return C - e;
}

template <int M>
struct PaleyNeg {  // bit i of neg[a]: H_M[i][a] = -1
  uint32_t neg[M];
  constexpr PaleyNeg() : neg() {
    for (int a = 0; a < M; ++a) {
      uint32_t w = 0;
      for (int i = 0; i < M; ++i)
        if (paley(M, i, a) < 0) w |= 1u << i;
      neg[a] = w;
    }
  }
};

constexpr int popcount32(uint32_t x) {
  int n = 0;
  for (; x; x &= x - 1) ++n;
  return n;
}

// H^T H = M I: any two distinct columns differ in exactly M / 2 signs
template <int M>
constexpr bool paley_orthogonal() {
  constexpr PaleyNeg<M> P{};
  for (int a = 0; a < M; ++a)
    for (int b = a + 1; b < M; ++b)
      if (2 * popcount32(P.neg[a] ^ P.neg[b]) != M) return false;
  return true;
}
static_assert(paley_orthogonal<12>() && paley_orthogonal<20>() && paley_orthogonal<28>(),
              "Paley matrices are Hadamard");

struct KronArgs {
  const uint16_t* src;  // X [rows][K], or W [K][ldw] (weights)
  int rows;
  int ldw;
  int log2G;
  int smooth;
  int rotate;
  const int32_t* perm;
  const uint8_t* dsign;  // K-bit sign mask or nullptr
  const float* S_in;     // quant: group scales from the reduce pass
  uint32_t* part;        // stats: [gridDim.x][K/G] partial maxima (float bits)
  uint8_t* codes;        // [rows][K/2]
  float* scale;          // [rows]
  float* S_out;          // [K/G] (quant without smoothing: 1)
  uint32_t* colmax;      // [K] (calibration)
  float* zrows;          // stats: [rows][K] rotated, reordered rows, or nullptr
  uint32_t* sync;        // one launch: the synchronisation block (epoch, error word, tagged rows)
  uint32_t spin_limit;   // polls before the one-launch wait gives up (0: after the first)
};

__device__ __forceinline__ void bfly(float& x, float& y) {
  const float a = x, b = y;
  x = a + b;
  y = a - b;
}

// Row buffer index of element f: four floats of padding after every 64, so
// that the strided accesses of the passes, the matrix-core stores and the
// gather spread over the LDS banks, and every run of 8 elements starting at
// a multiple of 8 stays one aligned 32-byte piece (two 16-byte accesses).
__device__ __forceinline__ constexpr int rpad(int f) { return f + 4 * (f >> 6); }
template <int K>
constexpr int kRowFloats = K + K / 16;

// Butterflies over R bits of f starting at bit B, in LDS (every run of n = 2^LOG2N).
template <int K, int B, int R>
__device__ __forceinline__ void lds_pass(float* row, int tid) {
  constexpr int P = 1 << R;
  for (int t = tid; t < (K >> R); t += kKT) {
    const int lo = t & ((1 << B) - 1), hi = t >> B;
    const int base = (hi << (B + R)) | lo;
    float v[P];
#pragma unroll
    for (int u = 0; u < P; ++u) v[u] = row[rpad(base + (u << B))];
#pragma unroll
    for (int h = 1; h < P; h <<= 1)
#pragma unroll
      for (int u = 0; u < P; ++u)
        if (!(u & h)) bfly(v[u], v[u + h]);
#pragma unroll
    for (int u = 0; u < P; ++u) row[rpad(base + (u << B))] = v[u];
  }
  __syncthreads();
}

// The first pass (f bits 0-2): each thread's 8 elements are consecutive,
// read and written as two 16-byte words (as eight scalar accesses, lanes 8
// floats apart share LDS banks eight ways).
template <int K>
__device__ __forceinline__ void lds_pass_low3(float* row, int tid) {
  for (int t = tid; t < K / 8; t += kKT) {
    float4* p = reinterpret_cast<float4*>(row + rpad(8 * t));
    const float4 lo = p[0], hi = p[1];
    float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (!(u & h)) bfly(v[u], v[u + h]);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
  __syncthreads();
}

// A first pass over f bits 0-3: each thread's 16 elements are consecutive,
// read and written as four 16-byte words.
template <int K>
__device__ __forceinline__ void lds_pass_low4(float* row, int tid) {
  for (int t = tid; t < K / 16; t += kKT) {
    float4* p = reinterpret_cast<float4*>(row + rpad(16 * t));
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 w = p[q];
      v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
    }
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (!(u & h)) bfly(v[u], v[u + h]);
#pragma unroll
    for (int q = 0; q < 4; ++q) p[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
  __syncthreads();
}

// Later passes (B >= 2): f bits 0-1 take no part, so each thread carries 4
// adjacent elements (one 16-byte word) through its R levels, 2^R words
// 2^B apart.
template <int K, int B, int R>
__device__ __forceinline__ void lds_pass_vec(float* row, int tid) {
  static_assert(B >= 2, "bits 0-1 stay inside a 16-byte word");
  constexpr int P = 1 << R;
  for (int t = tid; t < (K >> (R + 2)); t += kKT) {
    const int lo = t & ((1 << (B - 2)) - 1), hi = t >> (B - 2);
    const int base = (hi << (B + R)) | (lo << 2);
    float4 v[P];
#pragma unroll
    for (int u = 0; u < P; ++u) v[u] = *reinterpret_cast<const float4*>(row + rpad(base + (u << B)));
#pragma unroll
    for (int h = 1; h < P; h <<= 1)
#pragma unroll
      for (int u = 0; u < P; ++u)
        if (!(u & h)) {
          bfly(v[u].x, v[u + h].x);
          bfly(v[u].y, v[u + h].y);
          bfly(v[u].z, v[u + h].z);
          bfly(v[u].w, v[u + h].w);
        }
#pragma unroll
    for (int u = 0; u < P; ++u) *reinterpret_cast<float4*>(row + rpad(base + (u << B))) = v[u];
  }
  __syncthreads();
}

// Passes with B >= 1 whose items are pairs: f bit 0 takes no part, so each
// thread carries 2 adjacent elements (one 8-byte word) through its R
// levels, 2^R words 2^B apart (32 floats per item at R = 4).
template <int K, int B, int R>
__device__ __forceinline__ void lds_pass_pair(float* row, int tid) {
  static_assert(B >= 1, "bit 0 stays inside an 8-byte word");
  constexpr int P = 1 << R;
  for (int t = tid; t < (K >> (R + 1)); t += kKT) {
    const int lo = t & ((1 << (B - 1)) - 1), hi = t >> (B - 1);
    const int base = (hi << (B + R)) | (lo << 1);
    float2 v[P];
#pragma unroll
    for (int u = 0; u < P; ++u) v[u] = *reinterpret_cast<const float2*>(row + rpad(base + (u << B)));
#pragma unroll
    for (int h = 1; h < P; h <<= 1)
#pragma unroll
      for (int u = 0; u < P; ++u)
        if (!(u & h)) {
          bfly(v[u].x, v[u + h].x);
          bfly(v[u].y, v[u + h].y);
        }
#pragma unroll
    for (int u = 0; u < P; ++u) *reinterpret_cast<float2*>(row + rpad(base + (u << B))) = v[u];
  }
  __syncthreads();
}

template <int K, int B, int LOG2N>
__device__ __forceinline__ void lds_passes(float* row, int tid) {
  if constexpr (B < LOG2N) {
    constexpr int R = (LOG2N - B) < 3 ? (LOG2N - B) : 3;
    if constexpr (B == 0 && R == 3)
      lds_pass_low3<K>(row, tid);
    else if constexpr (B >= 2)
      lds_pass_vec<K, B, R>(row, tid);
    else
      lds_pass<K, B, R>(row, tid);
    lds_passes<K, B + R, LOG2N>(row, tid);
  }
}

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// H_m on the matrix cores, on the raw fp16 row: Z1[a][j] = sum_i H_m[i][a]
// x[i][j] is a 32 x 32 x MP product per tile of 32 columns j, A = H_m^T
// (+-1, zero-padded to MP = 16 or 32 rows and columns), B = the row read
// at stride n from the fp16 buffer (8 halves of consecutive i per lane,
// consecutive lanes on consecutive j). Products are exact, sums fp32. Rows
// a >= m of a tile are padding and not written.
template <int M>
struct HmFrag {
  static constexpr int MP = M <= 16 ? 16 : 32;
  static constexpr int KS = MP / 16;  // 16-deep k-steps
  v4u a[KS];
};

template <int M>
__device__ __forceinline__ HmFrag<M> hm_frags(int lane) {
  constexpr PaleyNeg<M> P{};
  HmFrag<M> h;
  const int ar = lane & 31;
#pragma unroll
  for (int ks = 0; ks < HmFrag<M>::KS; ++ks) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t w = 0;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int k = 16 * ks + 8 * (lane >> 5) + 2 * d + t;  // i
        uint32_t v = 0;
        if (k < M && ar < M) v = ((P.neg[ar] >> k) & 1u) ? 0xbc00u : 0x3c00u;
        w |= v << (16 * t);
      }
      h.a[ks][d] = w;
    }
  }
  return h;
}

// The row as the matrix cores take it. Wave w owns columns
// w * 32 * CP .. (w + 1) * 32 * CP - 1 (CP = N / 256 columns per lane, at
// least 1; at N < 256 only N / 32 waves hold columns). Lane l loads, for
// each 16-deep k-step ks and e = 0 .. 7, the CP adjacent halves
// x[i][j0 .. j0 + CP - 1], i = 16 ks + 8 (l / 32) + e, j0 = w 32 CP +
// CP (l % 32): consecutive lanes read consecutive 2 CP-byte pieces of a run
// (whole lines for CP >= 2), and no fp16 copy of the row goes through LDS.
// Tile c (c < CP) of the wave is the 32 columns j0 + c of its lanes: its B
// operand holds x[i][j0 + c] for the lane's eight i, two halves per dword,
// put together from the loaded pieces with byte permutes. Rows i >= m read
// as 0.
template <int M, int LOG2N>
struct HmRow {
  static constexpr int N = 1 << LOG2N;
  static constexpr int CP = N >= 1024 ? 4 : N >= 512 ? 2 : 1;
  static constexpr int CW = CP == 4 ? 2 : 1;   // dwords per loaded piece
  static constexpr int NW = N / (32 * CP);     // waves that hold columns (<= 8)
  static constexpr int KS = HmFrag<M>::KS;
  static_assert(NW >= 1 && NW <= kKT / 64, "columns per wave");
  uint32_t v[KS][8][CW];
};

// Column j0 of this lane (first of CP), and whether its wave holds columns.
template <int M, int LOG2N>
__device__ __forceinline__ int hm_col(int tid) {
  using R = HmRow<M, LOG2N>;
  return (tid >> 6) * 32 * R::CP + R::CP * (tid & 31);
}

// Element f = i n + j of row `row`, fp16 bits: X [rows][K], or column `row`
// of W [K][ldw] (weights).
template <int MODE, int K>
__device__ __forceinline__ uint32_t load_half(const KronArgs& a, int row, int f) {
  if constexpr (MODE == kKWeight)
    return static_cast<uint32_t>(a.src[static_cast<size_t>(f) * a.ldw + row]);
  else
    return static_cast<uint32_t>(a.src[static_cast<size_t>(row) * K + f]);
}

template <int M, int LOG2N, int MODE>
__device__ __forceinline__ void hm_load(HmRow<M, LOG2N>& r, const KronArgs& a, int row, int tid) {
  using R = HmRow<M, LOG2N>;
  constexpr int N = R::N, K = M * N;
  const int lane = tid & 63;
  const int j0 = hm_col<M, LOG2N>(tid);
  const bool cols = (tid >> 6) < R::NW;
#pragma unroll
  for (int ks = 0; ks < R::KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 16 * ks + 8 * (lane >> 5) + e;
      const int f = i * N + j0;
      const bool ok = cols && i < M;
      if constexpr (MODE == kKWeight) {
        uint32_t h[R::CP];
#pragma unroll
        for (int c = 0; c < R::CP; ++c) h[c] = ok ? load_half<MODE, K>(a, row, f + c) : 0u;
#pragma unroll
        for (int d = 0; d < R::CW; ++d)
          r.v[ks][e][d] = R::CP == 1 ? h[0] : (h[2 * d] | (h[2 * d + 1] << 16));
      } else {
        const uint16_t* p = a.src + static_cast<size_t>(row) * K + f;
        if constexpr (R::CP == 1) {
          r.v[ks][e][0] = ok ? static_cast<uint32_t>(*p) : 0u;
        } else if constexpr (R::CP == 2) {
          r.v[ks][e][0] = ok ? *reinterpret_cast<const uint32_t*>(p) : 0u;
        } else {
          const uint2 q = ok ? *reinterpret_cast<const uint2*>(p) : make_uint2(0u, 0u);
          r.v[ks][e][0] = q.x;
          r.v[ks][e][1] = q.y;
        }
      }
    }
}

// Sign-mask bits of the lane's loaded elements, bit (ks 8 + e) CP + c for
// x[i][j0 + c]; at most 32 (KS 8 CP <= 32 for every instantiated m, n).
template <int M, int LOG2N>
__device__ __forceinline__ uint32_t hm_sign_bits(const uint8_t* dsign, int tid) {
  using R = HmRow<M, LOG2N>;
  static_assert(R::KS * 8 * R::CP <= 32, "sign bits per lane");
  if (!dsign || (tid >> 6) >= R::NW) return 0u;
  const int lane = tid & 63;
  const int j0 = hm_col<M, LOG2N>(tid);
  uint32_t bits = 0u;
#pragma unroll
  for (int ks = 0; ks < R::KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 16 * ks + 8 * (lane >> 5) + e;
      if (i < M) {
#pragma unroll
        for (int c = 0; c < R::CP; ++c) {
          const int f = i * R::N + j0 + c;
          bits |= ((static_cast<uint32_t>(dsign[f >> 3]) >> (f & 7)) & 1u) << ((ks * 8 + e) * R::CP + c);
        }
      }
    }
  return bits;
}

// Flip the fp16 sign bits the mask selects (the signed rotation x D).
template <int M, int LOG2N>
__device__ __forceinline__ void hm_apply_signs(HmRow<M, LOG2N>& r, uint32_t bits) {
  using R = HmRow<M, LOG2N>;
#pragma unroll
  for (int ks = 0; ks < R::KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t b = bits >> ((ks * 8 + e) * R::CP);
#pragma unroll
      for (int d = 0; d < R::CW; ++d) {
        const uint32_t bd = R::CP == 1 ? (b & 1u) : (b >> (2 * d)) & 3u;
        r.v[ks][e][d] ^= ((bd & 1u) << 15) | ((bd & 2u) << 30);
      }
    }
}

// H_m on the matrix cores from the loaded pieces: Z1[a][j] = sum_i H_m[i][a]
// x[i][j], written to the fp32 row buffer (rows a >= m are padding, not
// written). Products are exact, sums fp32.
template <int M, int LOG2N>
__device__ __forceinline__ void hm_mfma(const HmRow<M, LOG2N>& r, float* row, const HmFrag<M>& h, int tid) {
  using R = HmRow<M, LOG2N>;
  if ((tid >> 6) >= R::NW) return;  // wave-uniform
  const int lane = tid & 63;
  const int j0 = hm_col<M, LOG2N>(tid);
  v16f acc[R::CP];
#pragma unroll
  for (int c = 0; c < R::CP; ++c) {
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < R::KS; ++ks) {
      // halves (i0 + 2d, i0 + 2d + 1) of column j0 + c: half c % 2 of dword
      // c / 2 of each piece
      constexpr uint32_t kSel[2] = {0x05040100u, 0x07060302u};
      v4u b;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = r.v[ks][2 * d][c / 2], hi = r.v[ks][2 * d + 1][c / 2];
        b[d] = R::CP == 1 ? (lo | (hi << 16)) : __builtin_amdgcn_perm(hi, lo, kSel[c & 1]);
      }
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, h.a[ks]), __builtin_bit_cast(v8h, b),
                                                      acc[c], 0, 0, 0);
    }
  }
  // register q of lane l: row a = 8 (q / 4) + 4 (l / 32) + q % 4, column j0 + c
  if constexpr (R::CP == 2) {
    // columns j0 and j0 + 1 (j0 even) differ in f bit 0: H_n's first level
    // here, and each pair goes to the row buffer as one 8-byte word
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int ar = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
      float x = acc[0][q], y = acc[1][q];
      bfly(x, y);
      if (ar < M) *reinterpret_cast<float2*>(row + rpad(ar * R::N + j0)) = make_float2(x, y);
    }
  } else if constexpr (R::CP == 4) {
    // columns j0 .. j0 + 3 (j0 a multiple of 4) span f bits 0 and 1: both
    // levels here, in that order, and each quad goes out as one 16-byte word
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int ar = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
      float x0 = acc[0][q], x1 = acc[1][q], x2 = acc[2][q], x3 = acc[3][q];
      bfly(x0, x1);
      bfly(x2, x3);
      bfly(x0, x2);
      bfly(x1, x3);
      if (ar < M) *reinterpret_cast<float4*>(row + rpad(ar * R::N + j0)) = make_float4(x0, x1, x2, x3);
    }
  } else {
#pragma unroll
    for (int c = 0; c < R::CP; ++c)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int ar = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (ar < M) row[rpad(ar * R::N + j0 + c)] = acc[c][q];
      }
  }
}

// H_n along every run of the row buffer, levels in the order of the bits.
// With two or four columns per lane (n = 512, 1024) hm_mfma ran the first
// one or two levels; the remaining eight bits take two radix-16 passes over
// pairs. At n = 256 and 128 a radix-16 pass over 16 consecutive elements
// comes first, then one pass over pairs; n = 64 keeps two radix-8 passes.
template <int M, int LOG2N>
__device__ __forceinline__ void hn_passes(float* row, int tid) {
  constexpr int K = M << LOG2N;
  constexpr int CP = HmRow<M, LOG2N>::CP;
  if constexpr (CP == 2 && LOG2N == 9) {
    lds_pass_pair<K, 1, 4>(row, tid);
    lds_pass_pair<K, 5, 4>(row, tid);
  } else if constexpr (CP == 4 && LOG2N == 10) {
    lds_pass_pair<K, 2, 4>(row, tid);
    lds_pass_pair<K, 6, 4>(row, tid);
  } else if constexpr (CP == 1 && (LOG2N == 8 || LOG2N == 7)) {
    lds_pass_low4<K>(row, tid);
    lds_pass_pair<K, 4, LOG2N - 4>(row, tid);
  } else {
    static_assert(CP == 1, "in-register levels only where the passes above expect them");
    lds_passes<K, 0, LOG2N>(row, tid);
  }
}

// Without the rotation: the loaded elements widened into the row buffer.
template <int M, int LOG2N>
__device__ __forceinline__ void hm_store_plain(const HmRow<M, LOG2N>& r, float* row, int tid) {
  using R = HmRow<M, LOG2N>;
  if ((tid >> 6) >= R::NW) return;
  const int lane = tid & 63;
  const int j0 = hm_col<M, LOG2N>(tid);
#pragma unroll
  for (int ks = 0; ks < R::KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 16 * ks + 8 * (lane >> 5) + e;
      if (i < M) {
#pragma unroll
        for (int c = 0; c < R::CP; ++c) {
          const uint32_t w = r.v[ks][e][c / 2];
          row[rpad(i * R::N + j0 + c)] = h2f(R::CP == 1 || (c & 1) == 0 ? (w & 0xffffu) : (w >> 16));
        }
      }
    }
}

__device__ __forceinline__ float block_max(float v, float* s_red, int tid) {
  v = lanes_max(v, 64);  // v >= 0
  if ((tid & 63) == 0) s_red[tid >> 6] = v;
  __syncthreads();
  float m = s_red[0];
#pragma unroll
  for (int w = 1; w < kKT / 64; ++w) m = fmaxf(m, s_red[w]);
  __syncthreads();
  return m;
}

template <int M, int LOG2N, int MODE>
__global__ void __launch_bounds__(kKT) kron_kernel(KronArgs a) {
  constexpr int N = 1 << LOG2N, K = M * N;
  constexpr int W8 = K / 8;                      // 16-byte chunks = packed words (8 positions) per row
  constexpr int SW = (W8 + kKT - 1) / kKT;       // chunks / words per thread
  __shared__ __attribute__((aligned(16))) float s_row[kRowFloats<K>];
  __shared__ float s_grp[K / 32];                // group maxima, or inverse scales
  __shared__ float s_red[kKT / 64];
  const int tid = threadIdx.x;
  const int ngroups = K >> a.log2G;
  const HmFrag<M> hf = hm_frags<M>(tid & 63);

  if constexpr (MODE == kKStats || MODE == kKFused) {
    for (int g = tid; g < ngroups; g += kKT) s_grp[g] = 0.f;
  } else if constexpr (MODE == kKQuant) {
    for (int g = tid; g < ngroups; g += kKT) s_grp[g] = a.smooth ? 1.f / a.S_in[g] : 1.f;
    if (!a.smooth && blockIdx.x == 0)
      for (int g = tid; g < ngroups; g += kKT) a.S_out[g] = 1.f;
  } else if constexpr (MODE == kKWeight) {
    for (int g = tid; g < ngroups; g += kKT) s_grp[g] = 1.f;
  }

  // the permutation is the same for every row: its row buffer indices stay
  // in registers; the sign bits of the lane's elements likewise
  int pp[SW][8];
  const uint32_t sbits = hm_sign_bits<M, LOG2N>(a.dsign, tid);
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    const int w = tid + s * kKT;
    if constexpr (MODE != kKColmax) {
      if (w < W8) {
        const int4 p0 = *reinterpret_cast<const int4*>(a.perm + 8 * w);
        const int4 p1 = *reinterpret_cast<const int4*>(a.perm + 8 * w + 4);
        pp[s][0] = rpad(p0.x); pp[s][1] = rpad(p0.y); pp[s][2] = rpad(p0.z); pp[s][3] = rpad(p0.w);
        pp[s][4] = rpad(p1.x); pp[s][5] = rpad(p1.y); pp[s][6] = rpad(p1.z); pp[s][7] = rpad(p1.w);
      }
    }
  }
  __syncthreads();

  // one launch: every workgroup reads the epoch before it publishes its row,
  // so none can see the next call's value
  uint32_t epoch = 0, spin_limit = a.spin_limit;
  if constexpr (MODE == kKFused) {
    epoch = __hip_atomic_load(&a.sync[kSyncEpoch], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    // a workspace whose wait failed before gives up at once
    if (__hip_atomic_load(&a.sync[kSyncError], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) spin_limit = 0u;
  }

  // rows blockIdx.x, + gridDim.x, ...: the next row's pieces load while this
  // one is processed (one launch: one row per workgroup)
  // (the offline weight preparation reads columns of W in 2-byte loads, one
  // address each: it loads its row at the top of the loop instead, which
  // keeps those addresses out of the live set)
  constexpr bool kAhead = MODE != kKWeight;
  HmRow<M, LOG2N> nxt;
  if (kAhead && blockIdx.x < a.rows) hm_load<M, LOG2N, MODE>(nxt, a, blockIdx.x, tid);
  for (int row = blockIdx.x; row < a.rows; row += gridDim.x) {
    bool gave_up = false;  // the one-launch wait gave up (the outputs are marked)
    HmRow<M, LOG2N> cur;
    if constexpr (kAhead) {
      cur = nxt;
      const int nrow = row + gridDim.x;
      if (nrow < a.rows) hm_load<M, LOG2N, MODE>(nxt, a, nrow, tid);
    } else {
      hm_load<M, LOG2N, MODE>(cur, a, row, tid);
    }
    // ---- signs (fp16 sign bits), then H_m on the matrix cores into the row
    // buffer (or the plain row without the rotation)
    if (a.dsign) hm_apply_signs<M, LOG2N>(cur, sbits);
    if (a.rotate) {
      hm_mfma<M, LOG2N>(cur, s_row, hf, tid);  // H_m across the runs
      __syncthreads();
      hn_passes<M, LOG2N>(s_row, tid);           // H_n along each run
    } else {
      hm_store_plain<M, LOG2N>(cur, s_row, tid);
      __syncthreads();
    }

    if constexpr (MODE == kKColmax) {
      // channel |max| of the rotated rows (calibration; before any reorder)
      for (int k = tid; k < K; k += kKT) {
        const uint32_t bits = __float_as_uint(fabsf(s_row[rpad(k)]));
        if (bits) atomicMax(&a.colmax[k], bits);
      }
    } else {
      // ---- gather eight reordered positions per word
      float z[SW][8];
#pragma unroll
      for (int s = 0; s < SW; ++s) {
        const int w = tid + s * kKT;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[s][e] = (w < W8) ? s_row[pp[s][e]] : 0.f;
      }
      if constexpr (MODE == kKStats || MODE == kKFused) {
        if (MODE == kKStats && a.zrows) {
          float4* zr = reinterpret_cast<float4*>(a.zrows + static_cast<size_t>(row) * K);
#pragma unroll
          for (int s = 0; s < SW; ++s) {
            const int w = tid + s * kKT;
            if (w < W8) {
              zr[2 * w] = make_float4(z[s][0], z[s][1], z[s][2], z[s][3]);
              zr[2 * w + 1] = make_float4(z[s][4], z[s][5], z[s][6], z[s][7]);
            }
          }
        }
#pragma unroll
        for (int s = 0; s < SW; ++s) {
          const int w = tid + s * kKT;
          if (w < W8) {
            float m = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(z[s][e]));
            if (m > 0.f) atomicMax(reinterpret_cast<uint32_t*>(&s_grp[(8 * w) >> a.log2G]), __float_as_uint(m));
          }
        }
      }
      if constexpr (MODE == kKFused) {
        // publish this row's group maxima as 64-bit words tagged with the
        // epoch (single-copy atomic stores), poll every row until all carry
        // it, reduce them here; the reordered row stays in registers
        __syncthreads();
        // the only workgroup (one row) already holds every token's maxima:
        // it skips the exchange (a round trip) (the error word was read at
        // the start); it still advances the epoch, so the count of
        // one-launch calls stays exact
        const bool alone = gridDim.x == 1;
        uint64_t* part = reinterpret_cast<uint64_t*>(a.sync + kSyncPartials);
        const uint64_t tag = static_cast<uint64_t>(epoch) << 32;
        if (alone) {
          gave_up = spin_limit == 0u;  // the error word was read at the start
        } else {
          for (int g = tid; g < ngroups; g += kKT)
            __hip_atomic_store(&part[static_cast<size_t>(row) * ngroups + g], tag | __float_as_uint(s_grp[g]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __syncthreads();
          for (int g = tid; g < ngroups; g += kKT) s_grp[g] = 0.f;
          __syncthreads();
          {
            constexpr int kBatch = 8;
            const int n = static_cast<int>(gridDim.x) * ngroups;
            for (int base = tid; base < n; base += kKT * kBatch) {
              uint64_t b[kBatch];
              uint32_t it = 0;
              for (;;) {
  #pragma unroll
                for (int k = 0; k < kBatch; ++k) {
                  const int idx = base + k * kKT;
                  b[k] = idx < n ? __hip_atomic_load(&part[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : tag;
                }
                bool all = spin_limit > 0;
  #pragma unroll
                for (int k = 0; k < kBatch; ++k) all &= (b[k] >> 32) == epoch;
                if (all) break;
                if (++it >= spin_limit) {
                  gave_up = true;
                  break;
                }
                __builtin_amdgcn_s_sleep(2);
              }
  #pragma unroll
              for (int k = 0; k < kBatch; ++k) {
                const uint32_t bits = static_cast<uint32_t>(b[k]);
                if (bits) atomicMax(reinterpret_cast<uint32_t*>(&s_grp[(base + k * kKT) % ngroups]), bits);
              }
            }
          }
        }
        // a workgroup that gave up raises the error word and marks its outputs
        gave_up = __syncthreads_or(gave_up);
        if (gave_up && tid == 0) atomicOr(&a.sync[kSyncError], 1u);
        // every workgroup has read the old epoch (it tagged its row with old + 1);
        // a failed call leaves it
        if (row == 0 && tid == 0 && !gave_up)
          __hip_atomic_store(&a.sync[kSyncEpoch], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int g = tid; g < ngroups; g += kKT) {
          float sg = s_grp[g];
          if (!(sg > 0.f)) sg = 1.f;  // all-zero group over every token
          if (row == 0) a.S_out[g] = gave_up ? __builtin_nanf("") : sg;
          s_grp[g] = 1.f / sg;
        }
        __syncthreads();
      }
      if constexpr (MODE != kKStats) {
        // per-token (or per-output-channel) scale of the smoothed row
        float r = 0.f;
#pragma unroll
        for (int s = 0; s < SW; ++s) {
          const int w = tid + s * kKT;
          if (w < W8) {
            const float inv = s_grp[(8 * w) >> a.log2G];
#pragma unroll
            for (int e = 0; e < 8; ++e) r = fmaxf(r, fabsf(z[s][e]) * inv);
          }
        }
        r = block_max(r, s_red, tid);
        const float k7 = r > 0.f ? 7.f / r : 0.f;
        constexpr size_t rs = codes_row_stride(K);
#pragma unroll
        for (int s = 0; s < SW; ++s) {
          const int w = tid + s * kKT;
          if (w < W8) {
            const float ks = s_grp[(8 * w) >> a.log2G] * k7;
            uint32_t mag[8], sgn[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              mag[e] = __float_as_uint(fmaf(fabsf(z[s][e]), ks, kMagic));
              sgn[e] = __float_as_uint(z[s][e]);
            }
            *reinterpret_cast<uint32_t*>(a.codes + codes_offset(row, 4 * w, rs)) = pack8(mag, sgn);
          }
        }
        if (tid == 0) a.scale[row] = gave_up ? __builtin_nanf("") : r / 7.f;
      }
    }
    __syncthreads();  // the row buffers are reused by the next row
  }

  if constexpr (MODE == kKStats) {
    // this workgroup's maxima over its rows into its own partial row
    for (int g = tid; g < ngroups; g += kKT) a.part[blockIdx.x * ngroups + g] = __float_as_uint(s_grp[g]);
  }
}

// Quantise pass over stored rows: one workgroup per row streams the row the
// stats pass stored and runs the quantise pass's arithmetic on it (smooth,
// per-token scale, round, pack). SW = packed words per thread.
template <int SW>
__global__ void __launch_bounds__(kKT) kron_quant_rows_kernel(KronArgs a, int K) {
  __shared__ float s_grp[kMaxKronK / 32];  // inverse group scales
  __shared__ float s_red[kKT / 64];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int W8 = K / 8;
  const int ngroups = K >> a.log2G;
  const float4* zr = reinterpret_cast<const float4*>(a.zrows + static_cast<size_t>(row) * K);
  float z[SW][8];
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    const int w = tid + s * kKT;
    float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
    if (w < W8) {
      lo = zr[2 * w];
      hi = zr[2 * w + 1];
    }
    z[s][0] = lo.x; z[s][1] = lo.y; z[s][2] = lo.z; z[s][3] = lo.w;
    z[s][4] = hi.x; z[s][5] = hi.y; z[s][6] = hi.z; z[s][7] = hi.w;
  }
  for (int g = tid; g < ngroups; g += kKT) s_grp[g] = 1.f / a.S_in[g];
  __syncthreads();

  float r = 0.f;
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    const int w = tid + s * kKT;
    if (w < W8) {
      const float inv = s_grp[(8 * w) >> a.log2G];
#pragma unroll
      for (int e = 0; e < 8; ++e) r = fmaxf(r, fabsf(z[s][e]) * inv);
    }
  }
  r = block_max(r, s_red, tid);
  const float k7 = r > 0.f ? 7.f / r : 0.f;
  const size_t rs = codes_row_stride(K);
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    const int w = tid + s * kKT;
    if (w < W8) {
      const float ks = s_grp[(8 * w) >> a.log2G] * k7;
      uint32_t mag[8], sgn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mag[e] = __float_as_uint(fmaf(fabsf(z[s][e]), ks, kMagic));
        sgn[e] = __float_as_uint(z[s][e]);
      }
      *reinterpret_cast<uint32_t*>(a.codes + codes_offset(row, 4 * w, rs)) = pack8(mag, sgn);
    }
  }
  if (tid == 0) a.scale[row] = r / 7.f;
}

hipError_t launch_quant_rows(const KronArgs& a, int K, hipStream_t s) {
  const int sw = (K / 8 + kKT - 1) / kKT;
  switch (sw) {
    case 1: hipLaunchKernelGGL(kron_quant_rows_kernel<1>, dim3(a.rows), dim3(kKT), 0, s, a, K); break;
    case 2: hipLaunchKernelGGL(kron_quant_rows_kernel<2>, dim3(a.rows), dim3(kKT), 0, s, a, K); break;
    case 3: hipLaunchKernelGGL(kron_quant_rows_kernel<3>, dim3(a.rows), dim3(kKT), 0, s, a, K); break;
    case 4: hipLaunchKernelGGL(kron_quant_rows_kernel<4>, dim3(a.rows), dim3(kKT), 0, s, a, K); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int M, int LOG2N, int MODE>
hipError_t launch_kron_mode(const KronArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((kron_kernel<M, LOG2N, MODE>), dim3(grid), dim3(kKT), 0, s, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch_kron(int m, int log2n, const KronArgs& a, int grid, hipStream_t s) {
#define RRS_KCASE(MM, LN) \
  if (m == MM && log2n == LN) return launch_kron_mode<MM, LN, MODE>(a, grid, s);
  RRS_KCASE(12, 6) RRS_KCASE(12, 7) RRS_KCASE(12, 8) RRS_KCASE(12, 9) RRS_KCASE(12, 10)
  RRS_KCASE(20, 6) RRS_KCASE(20, 7) RRS_KCASE(20, 8) RRS_KCASE(20, 9)
  RRS_KCASE(28, 6) RRS_KCASE(28, 7) RRS_KCASE(28, 8) RRS_KCASE(28, 9)
#undef RRS_KCASE
  return hipErrorInvalidValue;
}

constexpr int kKronRowsWG = 256;  // workgroups of the row loops (one per CU; each prefetches its next row)

// Workgroups of the one-launch kron_kernel<M, LOG2N, kKFused> the current
// device holds at once (occupancy per CU x CUs), cached per device; -1 if
// unknown.
template <int M, int LOG2N>
int fused_capacity_mn() {
  constexpr int kDevices = 64;
  static std::atomic<int> cache[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return -1;
  int cap = cache[dev].load(std::memory_order_relaxed);
  if (cap == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kron_kernel<M, LOG2N, kKFused>, kKT, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu <= 0 ||
        cus <= 0) {
      cap = -1;
    } else {
      cap = per_cu * cus;
    }
    cache[dev].store(cap, std::memory_order_relaxed);
  }
  return cap;
}

int kron_fused_capacity(int m, int log2n) {
#define RRS_KCAP(MM, LN) \
  if (m == MM && log2n == LN) return fused_capacity_mn<MM, LN>();
  RRS_KCAP(12, 6) RRS_KCAP(12, 7) RRS_KCAP(12, 8) RRS_KCAP(12, 9) RRS_KCAP(12, 10)
  RRS_KCAP(20, 6) RRS_KCAP(20, 7) RRS_KCAP(20, 8) RRS_KCAP(20, 9)
  RRS_KCAP(28, 6) RRS_KCAP(28, 7) RRS_KCAP(28, 8) RRS_KCAP(28, 9)
#undef RRS_KCAP
  return -1;
}

// The smoothed front end fits one launch when every row gets a workgroup
// and all of them are resident together (they wait for each other).
bool kron_fused_fits(int M, int m, int log2n) {
  if (M < 1 || M > kKronRowsWG || M > kMaxFusedWG) return false;
  const int cap = kron_fused_capacity(m, log2n);
  return cap > 0 && M <= cap;
}

}  // namespace

bool kron_split(int K, int* m, int* log2n) {
  for (int mm : {12, 20, 28}) {
    if (K % mm) continue;
    const int n = K / mm;
    if (n < 64 || (n & (n - 1))) continue;
    const int ln = 31 - __builtin_clz(static_cast<unsigned>(n));
    if (mm * n > kMaxKronK || (mm == 12 && ln > 10) || (mm != 12 && ln > 9)) continue;
    *m = mm;
    *log2n = ln;
    return true;
  }
  return false;
}

int kron_frontend_launches(int M, int K, int flags) {
  if (flags & 2) return 1;  // no smoothing: the quantise pass alone
  int m = 0, log2n = 0;
  if (!kron_split(K, &m, &log2n)) return -1;
  return (!(flags & 4) && kron_fused_fits(M, m, log2n)) ? 1 : 3;
}

hipError_t launch_frontend_kron(const uint16_t* X, int M, int K, int G, const int32_t* perm, const uint32_t* dsign,
                                uint8_t* xq, float* dx, float* S_out, uint32_t* sync, int flags,
                                hipStream_t s, float* zrows) {
  int m = 0, log2n = 0;
  if (!kron_split(K, &m, &log2n)) return hipErrorInvalidValue;
  KronArgs a{};
  a.src = X;
  a.rows = M;
  a.log2G = __builtin_ctz(static_cast<unsigned>(G));
  a.smooth = (flags & 2) ? 0 : 1;
  a.rotate = (flags & 1) ? 0 : 1;
  a.perm = perm;
  a.dsign = reinterpret_cast<const uint8_t*>(dsign);
  a.codes = xq;
  a.scale = dx;
  a.S_out = S_out;
  a.S_in = S_out;
  a.spin_limit = (flags & kFlagGiveUp) ? 0u : kSpinLimit;
  // the stats pass's partial rows (one per workgroup, K/G words; at most M
  // of them) fit the codes buffer (K/2 bytes per token, G >= 32), which the
  // quantise pass overwrites afterwards
  a.part = reinterpret_cast<uint32_t*>(xq);
  const int ngroups = K / G;
  if (a.smooth && !(flags & 4) && kron_fused_fits(M, m, log2n)) {
    // few rows: one launch, one row per workgroup, grid-wide wait on the
    // group maxima in the synchronisation block
    a.sync = sync;
    return dispatch_kron<kKFused>(m, log2n, a, M, s);
  }
  if (a.smooth) {
    // rows kept only when the rotation runs (without it the quantise pass
    // reads X itself, as cheap as the stored rows)
    a.zrows = a.rotate ? zrows : nullptr;
    const int gs = M < kKronRowsWG ? M : kKronRowsWG;
    hipError_t e = dispatch_kron<kKStats>(m, log2n, a, gs, s);
    if (e != hipSuccess) return e;
    e = launch_group_max(a.part, gs, ngroups, S_out, s);
    if (e != hipSuccess) return e;
    if (a.zrows) return launch_quant_rows(a, K, s);
  }
  return dispatch_kron<kKQuant>(m, log2n, a, M < kKronRowsWG ? M : kKronRowsWG, s);
}

hipError_t launch_weight_prep_kron(const uint16_t* W, int K, int N, const int32_t* perm, const uint32_t* dsign,
                                   uint8_t* wq, float* dw, hipStream_t s, bool rotate) {
  int m = 0, log2n = 0;
  if (!kron_split(K, &m, &log2n)) return hipErrorInvalidValue;
  KronArgs a{};
  a.src = W;
  a.rows = N;
  a.ldw = N;
  a.log2G = __builtin_ctz(static_cast<unsigned>(K & -K));  // one group: no smoothing
  a.smooth = 0;
  a.rotate = rotate ? 1 : 0;
  a.perm = perm;
  a.dsign = reinterpret_cast<const uint8_t*>(dsign);
  a.codes = wq;
  a.scale = dw;
  return dispatch_kron<kKWeight>(m, log2n, a, N < kKronRowsWG ? N : kKronRowsWG, s);
}

hipError_t launch_colmax_kron(const uint16_t* Xc, int T, int K, const uint32_t* dsign, uint32_t* colmax,
                              hipStream_t s, bool rotate) {
  int m = 0, log2n = 0;
  if (!kron_split(K, &m, &log2n)) return hipErrorInvalidValue;
  KronArgs a{};
  a.src = Xc;
  a.rows = T;
  a.log2G = 5;
  a.rotate = rotate ? 1 : 0;
  a.dsign = reinterpret_cast<const uint8_t*>(dsign);
  a.colmax = colmax;
  return dispatch_kron<kKColmax>(m, log2n, a, T < 1024 ? T : 1024, s);
}

}  // namespace rrs
