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
//   * rotation, K = 4096 and 8192: the load layout is the A operand of the
//     fp16 32 x 32 x 16 MFMA, so one 64-point factor of the Sylvester
//     transform runs on the matrix cores against a +-1 fragment and the
//     other in registers (plus one lane-half level); see rotate_block_mfma;
//   * rotation, K <= 2048: phase 1 butterflies over the in-register index
//     bits (f bits 0-2 and 9..), a transpose through LDS so f bits 3-8
//     become register bits (lane l = (f & 7) | ((f >> 9) & 7) << 3,
//     register (f >> 3) & 63 | (f >> 12) << 6), phase 2 over f bits 3-8;
//   * reorder: registers go back to LDS (conflict-free b128) and every lane
//     gathers its E = B/64 consecutive reordered positions through a
//     per-workgroup address table built from perm.
// The Sylvester transform is unnormalised (sums and differences only); the
// exact 1/K of the normalised pair is applied once in the GEMM epilogue and
// cancels out of the codes.
//
// The group scales need every token of the call before any token can be
// quantised. The one-launch form (fused_kernel) keeps each wave's rotated,
// reordered rows in registers across one grid-wide wait on the group
// maxima, so X is read from memory once; it is used whenever all its
// workgroups fit on the device together. For few tokens at K = 1024 ..
// 8192 (up to 256 rows) rowsplit_kernel gives each row a whole workgroup
// instead (one launch as well); called from rrs_linear its launch can also
// carry workgroups that read the GEMM's weight codes ahead, on the compute
// units the rows leave idle. Otherwise a stats launch (per-workgroup
// maxima rows), a reduce launch and a quantise launch; the stats and
// quantise launches each rotate the rows (X is read twice).

#include "rrs_internal.h"
#include "rrs_codes.h"

#include <atomic>

namespace rrs {
namespace {

constexpr int kWave = 64;

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
  uint32_t* sync;       // synchronisation block (one-launch form)
  uint32_t* part;       // stats pass: one row of K/G group maxima per workgroup
  uint8_t* codes;       // [rows][K/2]
  float* scale;         // [rows]
  float* S_out;         // [K/G]
  uint32_t* colmax;     // [K] (calibration)
  const uint8_t* dsign; // signed rotation: K-bit mask, bit j set -> channel j negated (nullptr: none)
  uint32_t spin_limit;  // polls before the one-launch wait gives up (0: after the first)
  const uint4* pf;      // one-row-per-workgroup launch: memory for the extra workgroups to read
  size_t pf_words;      // its 16-byte words
  int pf_period;        // ... read as the first pf_keep words of every pf_period
  int pf_keep;
  int pf_wg;            // extra workgroups (blockIdx.x >= rows)
  uint32_t* pf_sink;    // nullptr: keeps the reads from being dropped, never written
};

__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }


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

// ---- matrix-core form of the rotation for K = 4096 -----------------------
// H_4096 factors over any split of the 12 index bits of f into two sets,
// H_4096 = H_64(f bits 0-2, 8-10) (x) H_64(f bits 3-7, 11). The load
// layout (element f = 8L + 512i + e in half e of chunk i of lane L) already
// is the A operand of v_mfma_f32_32x32x16_f16 with row = f bits 3-7 (lane %
// 32), k = f bits 0-2 (half e), 8 (lane / 32) and 9-10 (k-step = i % 4), and
// a second tile for f bit 11 (i / 4): so the first factor is 16 fp16 MFMAs
// against a +-1 matrix (exact products of the fp16 inputs, fp32 sums), with
// no widening. The accumulators hold column n = f bits (0-2, 8-10) in lane
// % 32 and the tile index, row bits f3, f4, f6, f7 in the register and f5
// in lane / 32 (32 x 32 accumulator layout); the second factor is five
// in-register butterfly levels and one level across the lane halves with
// v_permlane32_swap, which trades register bit 0 (f3) and lane bit 5 (f5).
// Element f then sits in lane m12_lane(f), register m12_reg(f).
__device__ __forceinline__ constexpr int m12_lane(int f) {
  return (f & 7) | (((f >> 8) & 1) << 3) | (((f >> 9) & 1) << 4) | (((f >> 3) & 1) << 5);
}
__device__ __forceinline__ constexpr int m12_reg(int f) {
  return ((f >> 5) & 1) | (((f >> 4) & 1) << 1) | (((f >> 6) & 1) << 2) | (((f >> 7) & 1) << 3) |
         (((f >> 10) & 1) << 4) | (((f >> 11) & 1) << 5);
}
__device__ __forceinline__ constexpr int m12_elem(int lane, int r) {
  return (lane & 7) | (((lane >> 5) & 1) << 3) | (((r >> 1) & 1) << 4) | ((r & 1) << 5) |
         (((r >> 2) & 1) << 6) | (((r >> 3) & 1) << 7) | (((lane >> 3) & 1) << 8) |
         (((lane >> 4) & 1) << 9) | (((r >> 4) & 1) << 10) | (((r >> 5) & 1) << 11);
}
constexpr bool m12_bijective() {
  for (int f = 0; f < 4096; ++f) {
    const int l = m12_lane(f), r = m12_reg(f);
    if (l < 0 || l > 63 || r < 0 || r > 63 || m12_elem(l, r) != f) return false;
  }
  return true;
}
static_assert(m12_bijective(), "lane/register layout of the matrix-core rotation is a bijection");

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// B operand of k-step ks, column tile tj: lane l, half e holds H_64[k][n]
// with k = e + 8 (l / 32) + 16 ks and n = l % 32 + 32 tj, read as 6-bit
// labels of f bits (0, 1, 2, 8, 9, 10); sign = parity of popcount(k & n)
// = parity(e & l % 8) xor (l / 32 & l bit 3) xor parity(ks & (l bit 4 |
// tj << 1)).
struct HFrags {
  v4u b[2][4];  // [tj][ks]
};

__device__ __forceinline__ HFrags h64_frags(int lane) {
  const uint32_t a = lane & 7;
  v4u base;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t s0 = __builtin_popcount((2 * d) & a) & 1u;
    const uint32_t s1 = __builtin_popcount((2 * d + 1) & a) & 1u;
    base[d] = 0x3c003c00u | (s0 << 15) | (s1 << 31);
  }
  const uint32_t hn3 = ((lane >> 5) & (lane >> 3)) & 1u;
  const uint32_t n4 = (lane >> 4) & 1u;
  HFrags h;
#pragma unroll
  for (int tj = 0; tj < 2; ++tj)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t c = hn3 ^ (__builtin_popcount(static_cast<uint32_t>(ks) & (n4 | (tj << 1))) & 1u);
      h.b[tj][ks] = base ^ ((0u - c) & 0x80008000u);
    }
  return h;
}

// Rotate the 4096 elements in chunks w[C0 .. C0+7] into v[V0 .. V0+63]
// (layout m12_lane / m12_reg).
template <int C0, int V0, int NC, int NV>
__device__ __forceinline__ void rotate4096_mfma(float (&v)[NV], const uint4 (&w)[NC], const HFrags& h) {
  v16f acc[2][2];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[ti][tj][e] = 0.f;
#pragma unroll
  for (int tj = 0; tj < 2; ++tj) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const uint4 c = w[C0 + 4 * ti + ks];
        const v4u x = {c.x, c.y, c.z, c.w};
        acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, x),
                                                             __builtin_bit_cast(v8h, h.b[tj][ks]), acc[ti][tj], 0, 0, 0);
      }
    }
  }
  // v[V0 + 32 ti + 16 tj + r] = accumulator register r of tile (ti, tj):
  // register bits f3, f4, f6, f7, then f10 (tj), f11 (ti)
  float u[64];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int r = 0; r < 16; ++r) u[32 * ti + 16 * tj + r] = acc[ti][tj][r];
  butterfly<64>(u, 1);   // f3
  butterfly<64>(u, 2);   // f4
  butterfly<64>(u, 4);   // f6
  butterfly<64>(u, 8);   // f7
  butterfly<64>(u, 32);  // f11
  // f5 across the lane halves: after the swap, u[R] holds (lanes 0-31)
  // register R and (lanes 32-63) register R + 1 of the lower half, u[R + 1]
  // the same of the upper half; one butterfly finishes the level
#pragma unroll
  for (int R = 0; R < 64; R += 2) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(u[R]), __float_as_uint(u[R + 1]), false, false);
    const float x = __uint_as_float(sw[0]), y = __uint_as_float(sw[1]);
    v[V0 + R] = x + y;
    v[V0 + R + 1] = x - y;
  }
}

// Whole-block rotation on the matrix cores for K = 4096 and 8192 (two
// 4096 halves, then one butterfly level over f bit 12 = register bit 6).
template <int LOG2K>
__device__ __forceinline__ void rotate_block_mfma(float (&v)[Cfg<LOG2K>::kE], const uint4 (&w)[Cfg<LOG2K>::kChunks],
                                                  int lane) {
  static_assert(LOG2K == 12 || LOG2K == 13, "matrix-core rotation: K = 4096 or 8192");
  constexpr int E = Cfg<LOG2K>::kE, NC = Cfg<LOG2K>::kChunks;
  const HFrags h = h64_frags(lane);
  rotate4096_mfma<0, 0, NC, E>(v, w, h);
  if constexpr (LOG2K == 13) {
    rotate4096_mfma<8, 64, NC, E>(v, w, h);
    butterfly<E>(v, 64);
  }
}

// (lane, register) of element f after rotate_block_mfma, and back
template <int LOG2K>
__device__ __forceinline__ constexpr int mfma_lane(int f) { return m12_lane(f & 4095); }
template <int LOG2K>
__device__ __forceinline__ constexpr int mfma_reg(int f) { return m12_reg(f & 4095) | ((f >> 12) << 6); }
template <int LOG2K>
__device__ __forceinline__ constexpr int mfma_elem(int lane, int r) { return m12_elem(lane, r & 63) | ((r >> 6) << 12); }
constexpr bool mfma13_bijective() {
  for (int f = 0; f < 8192; ++f)
    if (mfma_elem<13>(mfma_lane<13>(f), mfma_reg<13>(f)) != f || mfma_reg<13>(f) > 127) return false;
  return true;
}
static_assert(mfma13_bijective(), "lane/register layout of the K = 8192 matrix-core rotation is a bijection");

// ---------------------------------------------------------------- row steps
// The steps below work on one wavefront's block of B = max(K, 4096)
// elements: lane L holds E = B/64 values in v[].

// s_tab[gpos(l, r)] = gather-buffer address of the element that lane l,
// register r needs after the reorder: position p = E*l + r of the block, row
// p / K, reordered column p % K, source channel perm[p % K].
// The table is built in two parts so that a kernel can issue the perm
// loads first, then its activation loads, and fill the table while the
// activations are in flight. Entries 4j .. 4j+3 share lane and chunk and
// take four consecutive positions, so their channels are one 16-byte load.
typedef int v4i __attribute__((ext_vector_type(4)));

template <int LOG2K>
struct TableLoads {
  static constexpr int kQuads = Cfg<LOG2K>::kB / 4;
  static constexpr int kIt = (kQuads + Cfg<LOG2K>::kThreads - 1) / Cfg<LOG2K>::kThreads;
  v4i pv[kIt];
};

template <int LOG2K>
__device__ __forceinline__ constexpr int table_pos(int idx) {  // position p of entry idx (rr = 0)
  return Cfg<LOG2K>::kE * ((idx >> 2) & 63) + ((idx >> 8) << 2);
}

template <int LOG2K>
__device__ __forceinline__ void table_loads(TableLoads<LOG2K>& t, const int32_t* perm, int tid) {
  using T = TableLoads<LOG2K>;
  constexpr int K = 1 << LOG2K;
#pragma unroll
  for (int it = 0; it < T::kIt; ++it) {
    const int j = tid + it * Cfg<LOG2K>::kThreads;
    if (j < T::kQuads) t.pv[it] = *reinterpret_cast<const v4i*>(perm + (table_pos<LOG2K>(4 * j) & (K - 1)));
  }
}

template <int LOG2K, bool ROTATE>
__device__ __forceinline__ void table_fill(uint32_t* s_tab, const TableLoads<LOG2K>& t, int tid) {
  using T = TableLoads<LOG2K>;
  constexpr int K = 1 << LOG2K;
#pragma unroll
  for (int it = 0; it < T::kIt; ++it) {
    const int j = tid + it * Cfg<LOG2K>::kThreads;
    if (j < T::kQuads) {
      const int idx = 4 * j;
      const int p = table_pos<LOG2K>(idx);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int f = ((p >> LOG2K) << LOG2K) | t.pv[it][rr];
        int sl, sr;
        if (ROTATE && LOG2K >= 12) {
          sl = mfma_lane<LOG2K>(f);
          sr = mfma_reg<LOG2K>(f);
        } else if (ROTATE) {
          sl = (f & 7) | (((f >> 9) & 7) << 3);
          sr = ((f >> 3) & 63) | ((f >> 12) << 6);
        } else {
          sl = (f >> 3) & 63;
          sr = (f & 7) | ((f >> 9) << 3);
        }
        s_tab[idx + rr] = static_cast<uint32_t>(gpos(sl, sr));
      }
    }
  }
}

// fp16 words of a block of activation rows X [rows][K]: element
// f = 8L + 512i + e of the block lands in word w[i], half e. Rows past the
// last read the last row instead (every load is unconditional, so wait
// counts stay exact); no result of such a row is ever stored or reduced.
template <int LOG2K>
__device__ __forceinline__ void load_block(uint4 (&w)[Cfg<LOG2K>::kChunks], const uint16_t* src, int rows,
                                           int row0, int lane) {
  constexpr int K = 1 << LOG2K;
#pragma unroll
  for (int i = 0; i < Cfg<LOG2K>::kChunks; ++i) {
    const int f0 = 8 * lane + 512 * i;
    const int row = min(row0 + (f0 >> LOG2K), rows - 1);
    w[i] = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(row) * K + (f0 & (K - 1)));
  }
}

// Signed rotation (x D H, D = diag(+-1)): the mask byte of the 8 channels
// of each 16-byte chunk, loaded with the block; flipping an fp16 sign bit
// is exact. Rows of the block share the channels of their column offset.
template <int LOG2K>
struct SignLoads {
  uint32_t b[Cfg<LOG2K>::kChunks];
};

template <int LOG2K>
__device__ __forceinline__ void sign_loads(SignLoads<LOG2K>& sl, const uint8_t* dsign, int lane) {
  constexpr int K = 1 << LOG2K;
#pragma unroll
  for (int i = 0; i < Cfg<LOG2K>::kChunks; ++i)
    sl.b[i] = dsign ? static_cast<uint32_t>(dsign[((8 * lane + 512 * i) & (K - 1)) >> 3]) : 0u;
}

template <int LOG2K>
__device__ __forceinline__ void apply_signs(uint4 (&w)[Cfg<LOG2K>::kChunks], const SignLoads<LOG2K>& sl) {
#pragma unroll
  for (int i = 0; i < Cfg<LOG2K>::kChunks; ++i) {
    const uint32_t b = sl.b[i];  // bit e: half e of the chunk
    w[i].x ^= ((b & 1u) << 15) | ((b & 2u) << 30);
    w[i].y ^= ((b & 4u) << 13) | ((b & 8u) << 28);
    w[i].z ^= ((b & 16u) << 11) | ((b & 32u) << 26);
    w[i].w ^= ((b & 64u) << 9) | ((b & 128u) << 24);
  }
}

template <int LOG2K>
__device__ __forceinline__ void widen_block(float (&v)[Cfg<LOG2K>::kE], const uint4 (&w)[Cfg<LOG2K>::kChunks]) {
#pragma unroll
  for (int i = 0; i < Cfg<LOG2K>::kChunks; ++i) {
    const uint32_t q[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * i + 2 * e] = h2f(q[e] & 0xffffu);
      v[8 * i + 2 * e + 1] = h2f(q[e] >> 16);
    }
  }
}

// Sylvester rotation of every row of the block (unnormalised): phase 1 over
// the register-index bits of f (bits 0-2 and 9..), a padded LDS transpose,
// phase 2 over f bits 3-8. Leaves element f in lane (f & 7) | ((f >> 9) & 7)
// << 3, register ((f >> 3) & 63) | (f >> 12) << 6.
template <int LOG2K>
__device__ __forceinline__ void rotate_block(float (&v)[Cfg<LOG2K>::kE], float* wb, int lane) {
  using C = Cfg<LOG2K>;
  constexpr int E = C::kE;
#pragma unroll
  for (int rb = 0; rb < C::kLog2E; ++rb) {
    const int fb = rb < 3 ? rb : rb + 6;
    if (fb < LOG2K) butterfly<E>(v, 1 << rb);
  }
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
#pragma unroll
  for (int rb = 0; rb < 6; ++rb) {
    if (rb + 3 < LOG2K) butterfly<E>(v, 1 << rb);
  }
}

// Reorder: scatter the registers to LDS, gather the reordered positions
// through the table. Afterwards v[r] is position p = E*lane + r of the block.
template <int LOG2K>
__device__ __forceinline__ void reorder_block(float (&v)[Cfg<LOG2K>::kE], float* wb, const uint32_t* s_tab,
                                              int lane) {
  constexpr int E = Cfg<LOG2K>::kE;
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
}

// Per-lane |max| of each 32-wide sub-segment, merged so that m[s] is the
// max over the whole group (of the lane's row) the sub-segment belongs to.
template <int LOG2K>
__device__ __forceinline__ void group_max(const float (&v)[Cfg<LOG2K>::kE], float (&m)[Cfg<LOG2K>::kE / 32],
                                          int G) {
  constexpr int E = Cfg<LOG2K>::kE, NS = E / 32;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float x = fabsf(v[32 * s]);
#pragma unroll
    for (int r = 1; r < 32; ++r) x = fmaxf(x, fabsf(v[32 * s + r]));
    m[s] = x;
  }
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
  if (G > E) {  // a group spans G / E lanes (at most 64)
#pragma unroll
    for (int s = 0; s < NS; ++s) m[s] = lanes_max(m[s], min(G / E, 64));
  }
}

// Fold the block's per-row group maxima into the workgroup's LDS maxima.
template <int LOG2K>
__device__ __forceinline__ void fold_group_max(const float (&m)[Cfg<LOG2K>::kE / 32], float* s_grp, int log2G,
                                               int rows, int row0, int lane) {
  constexpr int K = 1 << LOG2K, E = Cfg<LOG2K>::kE;
  const int rl = (E * lane) >> LOG2K;
  const int j0 = (E * lane) & (K - 1);
  const int G = 1 << log2G;
#pragma unroll
  for (int s = 0; s < E / 32; ++s) {
    const int j = j0 + 32 * s;
    if (row0 + rl < rows && (j & (G - 1)) == 0 && m[s] > 0.f)
      atomicMax(reinterpret_cast<uint32_t*>(&s_grp[j >> log2G]), __float_as_uint(m[s]));
  }
}

// Per-token scale, codes and packing of one block. s_inv[g] = 1 / S_g (or
// 1 without smoothing). Writes codes [rows][K/2] and scale[row] = r / 7.
template <int LOG2K>
__device__ __forceinline__ void quantise_block(const float (&v)[Cfg<LOG2K>::kE],
                                               const float (&m)[Cfg<LOG2K>::kE / 32], const float* s_inv,
                                               int log2G, uint8_t* codes, float* scale, int rows, int row0,
                                               int lane, bool bad = false) {
  constexpr int K = 1 << LOG2K, E = Cfg<LOG2K>::kE, NS = E / 32;
  const int rl = (E * lane) >> LOG2K;
  const int j0 = (E * lane) & (K - 1);
  float inv[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) inv[s] = s_inv[(j0 + 32 * s) >> log2G];
  float rmax = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) rmax = fmaxf(rmax, m[s] * inv[s]);
  if (K > E) rmax = lanes_max(rmax, min(K / E, 64));  // a row spans K / E lanes
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
  if (row0 + rl < rows) {
    uint8_t* dst = codes + codes_offset(row0 + rl, j0 / 2, codes_row_stride(K));  // E / 2 bytes in one piece
#pragma unroll
    for (int o = 0; o < E / 32; ++o)
      reinterpret_cast<uint4*>(dst)[o] = make_uint4(packed[4 * o], packed[4 * o + 1], packed[4 * o + 2], packed[4 * o + 3]);
    // a workgroup whose wait gave up marks its rows' scales
    if (j0 == 0) scale[row0 + rl] = bad ? __builtin_nanf("") : rmax / 7.f;
  }
}

// ----------------------------------------------------------- one-pass kernels
// Stats and quantise passes of the three-launch front end, the offline weight
// preparation (columns of W as rows) and the calibration channel maxima.
// Each wave owns the blocks blockIdx.x * WAVES + wave + i * gridDim.x * WAVES:
// the stats and quantise passes launch at most as many workgroups as the
// device holds at once, so a workgroup builds its gather table once and
// each wave loads its next block while it processes the current one (the
// other modes launch one block per wave).
template <int LOG2K, int MODE, bool ROTATE>
__global__ void __launch_bounds__(Cfg<LOG2K>::kThreads)
frontend_kernel(FeArgs a) {
  using C = Cfg<LOG2K>;
  constexpr int K = 1 << LOG2K;
  constexpr int E = C::kE, WAVES = C::kWaves;
  constexpr bool kLoop = MODE == kStats || MODE == kQuant;

  __shared__ float s_buf[WAVES][C::kBufFloats];
  __shared__ uint32_t s_tab[C::kB];             // gather table, or channel max
  __shared__ float s_grp[K / 32];               // group max (stats) / 1/S (quant)

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int ngroups = K >> a.log2G;
  const int stride = gridDim.x * WAVES;
  int blk = blockIdx.x * WAVES + wave;

  // table loads, then the activation rows, both before the set-up
  TableLoads<LOG2K> tl;
  if constexpr (MODE != kColmax) table_loads<LOG2K>(tl, a.perm, tid);
  uint4 w[C::kChunks];
  if constexpr (MODE != kWeight) load_block<LOG2K>(w, a.src, a.rows, blk * C::kRows, lane);
  SignLoads<LOG2K> sg;
  if constexpr (ROTATE) sign_loads<LOG2K>(sg, a.dsign, lane);
  __builtin_amdgcn_sched_barrier(0);

  // ---- per-workgroup set-up -------------------------------------------
  if constexpr (MODE == kColmax) {
    for (int k = tid; k < K; k += C::kThreads) s_tab[k] = 0u;
  } else {
    table_fill<LOG2K, ROTATE>(s_tab, tl, tid);
    if constexpr (MODE == kStats) {
      for (int g = tid; g < ngroups; g += C::kThreads) s_grp[g] = 0.f;
    } else if constexpr (MODE == kQuant) {
      for (int g = tid; g < ngroups; g += C::kThreads) {
        float sg = 1.f;
        if (a.smooth) {
          sg = a.S_out[g];            // from the reduce launch
          if (!(sg > 0.f)) sg = 1.f;  // all-zero group over every token
        }
        s_grp[g] = 1.f / sg;
      }
    } else {
      for (int g = tid; g < ngroups; g += C::kThreads) s_grp[g] = 1.f;
    }
  }
  __syncthreads();

  for (; blk * C::kRows < a.rows; blk += stride) {
    const int row0 = blk * C::kRows;
    // the wave's next block loads while this one is processed
    uint4 wn[kLoop ? C::kChunks : 1];
    const bool more = kLoop && (blk + stride) * C::kRows < a.rows;
    if constexpr (kLoop) {
      if (more) load_block<LOG2K>(wn, a.src, a.rows, (blk + stride) * C::kRows, lane);
    }
    if constexpr (MODE == kWeight) {
      // column `row` of W [K][ldw], channels k0..k0+7
#pragma unroll
      for (int i = 0; i < C::kChunks; ++i) {
        const int f0 = 8 * lane + 512 * i;
        const int row = row0 + (f0 >> LOG2K);
        uint32_t q[4] = {0u, 0u, 0u, 0u};
        if (row < a.rows) {
          const int k0 = f0 & (K - 1);
          const uint16_t* p = a.src + static_cast<size_t>(k0) * a.ldw + row;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            q[e] = static_cast<uint32_t>(p[(2 * e) * static_cast<size_t>(a.ldw)]) |
                   (static_cast<uint32_t>(p[(2 * e + 1) * static_cast<size_t>(a.ldw)]) << 16);
        }
        w[i] = make_uint4(q[0], q[1], q[2], q[3]);
      }
    }
    float v[E];
    float* wb = s_buf[wave];
    if constexpr (ROTATE) {
      if (a.dsign) apply_signs<LOG2K>(w, sg);
    }
    if constexpr (ROTATE && LOG2K >= 12) {
      rotate_block_mfma<LOG2K>(v, w, lane);
    } else {
      widen_block<LOG2K>(v, w);
      if constexpr (ROTATE) rotate_block<LOG2K>(v, wb, lane);
    }

    if constexpr (MODE == kColmax) {
      // channel |max| over the block's rows (LDS), folded into global below
#pragma unroll
      for (int r = 0; r < E; ++r) {
        // block element in register r of this lane: the rotations' output
        // layouts, or the load layout (f = 8 lane + 512 i + e in register
        // 8 i + e) without the rotation
        const int f = !ROTATE        ? (r & 7) | (lane << 3) | ((r >> 3) << 9)
                      : LOG2K >= 12 ? mfma_elem<LOG2K>(lane, r)
                                    : (lane & 7) | ((r & 63) << 3) | ((lane >> 3) << 9) | ((r >> 6) << 12);
        if (row0 + (f >> LOG2K) < a.rows)
          atomicMax(&s_tab[f & (K - 1)], __float_as_uint(fabsf(v[r])));
      }
    } else {
      reorder_block<LOG2K>(v, wb, s_tab, lane);
      float m[E / 32];
      group_max<LOG2K>(v, m, 1 << a.log2G);
      if constexpr (MODE == kStats)
        fold_group_max<LOG2K>(m, s_grp, a.log2G, a.rows, row0, lane);
      else
        quantise_block<LOG2K>(v, m, s_grp, a.log2G, a.codes, a.scale, a.rows, row0, lane);
    }
    if constexpr (kLoop) {
      if (!more) break;
#pragma unroll
      for (int i = 0; i < C::kChunks; ++i) w[i] = wn[i];
    } else {
      break;
    }
  }

  // ---- the workgroup's partial maxima, the channel maxima ---------------
  if constexpr (MODE == kStats) {
    // its own row of the partial area: plain stores (same-address atomics
    // from every workgroup would serialise)
    __syncthreads();
    for (int g = tid; g < ngroups; g += C::kThreads)
      a.part[static_cast<size_t>(blockIdx.x) * ngroups + g] = __float_as_uint(s_grp[g]);
  } else if constexpr (MODE == kColmax) {
    __syncthreads();
    for (int k = tid; k < K; k += C::kThreads) {
      const uint32_t bits = s_tab[k];
      if (bits) atomicMax(&a.colmax[k], bits);
    }
  } else if constexpr (MODE == kQuant) {
    // with smoothing the reduce launch wrote S; without it S = 1
    if (!a.smooth && blockIdx.x == 0)
      for (int g = tid; g < ngroups; g += C::kThreads) a.S_out[g] = 1.f;
  }
}

// S_g = max over `nrows` partial rows of group maxima (float bits), 1 where
// every row holds 0: one workgroup per group, threads over rows.
__global__ void __launch_bounds__(256) group_max_kernel(const uint32_t* part, int nrows, int ngroups,
                                                        float* S_out) {
  __shared__ uint32_t s_m[4];
  const int g = blockIdx.x, tid = threadIdx.x;
  uint32_t m = 0u;
  for (int r = tid; r < nrows; r += 256) m = max(m, part[static_cast<size_t>(r) * ngroups + g]);
  m = lanes_max_u32(m, 64);
  if ((tid & 63) == 0) s_m[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    m = max(max(s_m[0], s_m[1]), max(s_m[2], s_m[3]));
    const float v = __uint_as_float(m);
    S_out[g] = v > 0.f ? v : 1.f;
  }
}

// ------------------------------------------------------------- fused kernel
// The whole activation front end in one launch: each wave rotates, reorders
// and reduces R blocks and keeps them in registers; each workgroup stores
// its group maxima in its own row of the synchronisation block and raises
// its arrival flag to this call's epoch; once every flag shows the epoch,
// each workgroup reduces all rows itself and smooths, quantises and packs
// its blocks from its registers. X is read once, and no two workgroups ever
// update the same word (same-address atomics from every XCD serialise).
// All workgroups must be resident at once; the launcher checks the grid
// against the device's occupancy.
// Weight codes a thread of the one-launch form reads ahead for the tiled
// GEMM, in 16-byte loads: 256 workgroups of 512 threads cover 8 MiB.
constexpr int kFusedPrefetchLoads = 4;

template <int LOG2K, bool ROTATE, int R>
__global__ void __launch_bounds__(Cfg<LOG2K>::kThreads)
fused_kernel(FeArgs a) {
  using C = Cfg<LOG2K>;
  constexpr int K = 1 << LOG2K;
  constexpr int E = C::kE, WAVES = C::kWaves;

  __shared__ float s_buf[WAVES][C::kBufFloats];
  __shared__ uint32_t s_tab[C::kB];
  __shared__ float s_grp[K / 32];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int ngroups = K >> a.log2G;
  const int nwg = gridDim.x;
  int row0[R];
#pragma unroll
  for (int q = 0; q < R; ++q) row0[q] = ((blockIdx.x * R + q) * WAVES + wave) * C::kRows;

  TableLoads<LOG2K> tl;
  table_loads<LOG2K>(tl, a.perm, tid);
  uint4 w[R][C::kChunks];
#pragma unroll
  for (int q = 0; q < R; ++q) load_block<LOG2K>(w[q], a.src, a.rows, row0[q], lane);
  SignLoads<LOG2K> sg;
  if constexpr (ROTATE) sign_loads<LOG2K>(sg, a.dsign, lane);
  // every load is issued before the table is filled: waiting for the perm
  // loads then leaves the activation loads in flight
  __builtin_amdgcn_sched_barrier(0);
  // every workgroup reads the epoch before raising its flag, so none can
  // see the next call's value
  const uint32_t epoch =
      __hip_atomic_load(&a.sync[kSyncEpoch], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  // Weight read-ahead (rrs_linear before the tiled GEMM, one block per
  // wave): this workgroup's share of the weight codes, issued once the row
  // is rotated (HBM is idle from there to the wait; issued with the row's
  // own loads they competed with them, 0.7 us slower at M = 2048) and
  // consumed before the maxima are published, so none of the front end's
  // other waits includes them; the lines sit in the memory-side cache when
  // the GEMM starts. The loads are unconditional (without a read-ahead
  // every thread reads the first 16 bytes of the synchronisation block, and
  // an index past the end reads the last word): the compiler counts loads
  // in flight per path, and a conditional load made the waits for the
  // rows' own loads also wait for the read-ahead.
  uint4 pfv[kFusedPrefetchLoads];

  table_fill<LOG2K, ROTATE>(s_tab, tl, tid);
  for (int g = tid; g < ngroups; g += C::kThreads) s_grp[g] = 0.f;
  __syncthreads();

  // ---- rotate, reorder, group maxima; the blocks stay in registers --------
  float v[R][E];
  float m[R][E / 32];
  float* wb = s_buf[wave];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    if constexpr (ROTATE) {
      if (a.dsign) apply_signs<LOG2K>(w[q], sg);
    }
    if constexpr (ROTATE && LOG2K >= 12) {
      rotate_block_mfma<LOG2K>(v[q], w[q], lane);
    } else {
      widen_block<LOG2K>(v[q], w[q]);
      if constexpr (ROTATE) rotate_block<LOG2K>(v[q], wb, lane);
    }
    if constexpr (R == 1) {
      const uint4* src = a.pf ? a.pf : reinterpret_cast<const uint4*>(a.sync);
      const size_t words = a.pf ? a.pf_words : 1;
      const size_t per = (words + nwg - 1) / nwg;
      const size_t b = static_cast<size_t>(blockIdx.x) * per;
#pragma unroll
      for (int u = 0; u < kFusedPrefetchLoads; ++u)
        pfv[u] = src[min(b + tid + static_cast<size_t>(u) * C::kThreads, words - 1)];
    }
    reorder_block<LOG2K>(v[q], wb, s_tab, lane);
    group_max<LOG2K>(v[q], m[q], 1 << a.log2G);
    fold_group_max<LOG2K>(m[q], s_grp, a.log2G, a.rows, row0[q], lane);
  }
  if constexpr (R == 1) {  // the read-ahead's values only feed an XOR stored when pf_sink is set (never)
    uint32_t x = 0u;
#pragma unroll
    for (int u = 0; u < kFusedPrefetchLoads; ++u) x ^= pfv[u].x ^ pfv[u].y ^ pfv[u].z ^ pfv[u].w;
    if (a.pf_sink) a.pf_sink[tid] = x;
  }
  __syncthreads();

  // ---- publish this workgroup's maxima, read everyone's ---------------------
  // Each workgroup stores its group maxima in its own row of 64-bit words
  // tagged with this call's epoch in the high half (single-copy atomic
  // stores); the readers poll the rows themselves until every word carries
  // the epoch, so the data and the arrival need one round trip, not two.
  // Every cross-workgroup word is written and read with relaxed agent-scope
  // atomics, which go to the device-coherent level directly (no L2
  // write-back or invalidate, which acquire/release would add per access).
  // A grid of one workgroup already holds every token's maxima: it skips
  // the exchange (a round trip) and reads the error word alone; it still
  // advances the epoch, so the count of one-launch calls stays exact.
  const bool alone = nwg == 1;
  bool gave_up = false;
  uint64_t* part = reinterpret_cast<uint64_t*>(a.sync + kSyncPartials);
  const uint64_t tag = static_cast<uint64_t>(epoch) << 32;
  if (alone) {
    gave_up = __hip_atomic_load(&a.sync[kSyncError], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
              a.spin_limit == 0u;
  } else {
    for (int g = tid; g < ngroups; g += C::kThreads)
      __hip_atomic_store(&part[blockIdx.x * ngroups + g], tag | __float_as_uint(s_grp[g]), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    for (int g = tid; g < ngroups; g += C::kThreads) s_grp[g] = 0.f;
    __syncthreads();

    // ---- S_g = max over the workgroups' rows (all loads of a poll in flight) --
    // a workspace whose wait failed before (error word set until it is
    // initialised again) holds tags of no use: give up at once. Read here,
    // with the first poll: read at the start, its value (uniform, moved to a
    // scalar register at once) made the workgroup wait for every load issued
    // before it, the rows' own included.
    const uint32_t spin_limit =
        __hip_atomic_load(&a.sync[kSyncError], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ? 0u : a.spin_limit;
    {
      constexpr int kBatch = 16;
      const int n = nwg * ngroups;
      const bool same_group = C::kThreads % ngroups == 0;  // thread always on group tid % ngroups
      uint32_t mx = 0u;
      for (int base = tid; base < n; base += C::kThreads * kBatch) {
        uint64_t b[kBatch];
        uint32_t it = 0;
        for (;;) {
  #pragma unroll
          for (int k = 0; k < kBatch; ++k) {
            const int idx = base + k * C::kThreads;
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
          const uint32_t v = static_cast<uint32_t>(b[k]);
          if (same_group) {
            mx = max(mx, v);
          } else if (v) {
            atomicMax(reinterpret_cast<uint32_t*>(&s_grp[(base + k * C::kThreads) % ngroups]), v);
          }
        }
      }
      if (same_group && mx) atomicMax(reinterpret_cast<uint32_t*>(&s_grp[tid % ngroups]), mx);
    }
  }
  // a workgroup that gave up raises the error word and marks its outputs
  gave_up = __syncthreads_or(gave_up);
  if (gave_up && tid == 0) atomicOr(&a.sync[kSyncError], 1u);
  // every workgroup has read the old epoch (it tagged its row with old + 1);
  // a failed call leaves it
  if (blockIdx.x == 0 && tid == 0 && !gave_up)
    __hip_atomic_store(&a.sync[kSyncEpoch], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  for (int g = tid; g < ngroups; g += C::kThreads) {
    float sg = s_grp[g];
    if (!(sg > 0.f)) sg = 1.f;  // all-zero group over every token
    if (blockIdx.x == 0) a.S_out[g] = gave_up ? __builtin_nanf("") : sg;
    s_grp[g] = 1.f / sg;
  }
  __syncthreads();

  // ---- smooth, quantise, pack ------------------------------------------------
#pragma unroll
  for (int q = 0; q < R; ++q)
    quantise_block<LOG2K>(v[q], m[q], s_grp, a.log2G, a.codes, a.scale, a.rows, row0[q], lane, gave_up);
}

// Stable descending rank: perm[rank(j)] = j with rank(j) = #{i : c_i > c_j}
// + #{i < j : c_i == c_j} (values compared as non-negative float bits).
__global__ void __launch_bounds__(1024) rank_kernel(const uint32_t* c, int K, int32_t* perm) {
  __shared__ uint32_t s_c[kMaxKronK];  // K <= kMaxKronK (>= 2^kMaxLog2K)
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

// Workgroups of a one-pass launch over `rows` rows of length 2^log2K
// (blocks of max(K, 4096) elements, Cfg's waves per workgroup).
constexpr int pass_grid(int log2K, int rows) {
  const int log2B = log2K > 12 ? log2K : 12;
  const int per_block = 1 << (log2B - log2K);
  const int waves = log2B == 12 ? 8 : 3;
  return ((rows + per_block - 1) / per_block + waves - 1) / waves;
}

constexpr int kMaxDevices = 64;

// Workgroups of frontend_kernel<LOG2K, MODE, ROTATE> the current device
// holds at once (occupancy per CU x CUs), cached per device; -1 if unknown.
template <int LOG2K, int MODE, bool ROTATE>
int pass_capacity() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  int cap = cache[dev].load(std::memory_order_relaxed);
  if (cap == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, frontend_kernel<LOG2K, MODE, ROTATE>,
                                                     Cfg<LOG2K>::kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        per_cu <= 0 || cus <= 0) {
      cap = -1;
    } else {
      cap = per_cu * cus;
    }
    cache[dev].store(cap, std::memory_order_relaxed);
  }
  return cap;
}

// One pass over `a.rows` rows; the stats and quantise passes take at most
// one workgroup per resident slot (each wave then loops over its blocks).
// *grid_out (if given) receives the launched grid.
template <int LOG2K, int MODE, bool ROTATE>
hipError_t launch_mode(const FeArgs& a, hipStream_t s, int* grid_out) {
  using C = Cfg<LOG2K>;
  static_assert(pass_grid(LOG2K, 1000) == ((1000 + C::kRows - 1) / C::kRows + C::kWaves - 1) / C::kWaves,
                "pass_grid follows Cfg");
  int grid = pass_grid(LOG2K, a.rows);
  if constexpr (MODE == kStats || MODE == kQuant) {
    const int cap = pass_capacity<LOG2K, MODE, ROTATE>();
    if (cap > 0 && grid > cap) grid = cap;
  }
  if (grid_out) *grid_out = grid;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((frontend_kernel<LOG2K, MODE, ROTATE>), dim3(grid), dim3(C::kThreads), 0, s, a);
  return hipGetLastError();
}

template <int MODE, bool ROTATE>
hipError_t dispatch_k(int log2K, const FeArgs& a, hipStream_t s, int* grid_out = nullptr) {
  switch (log2K) {
    case 6: return launch_mode<6, MODE, ROTATE>(a, s, grid_out);
    case 7: return launch_mode<7, MODE, ROTATE>(a, s, grid_out);
    case 8: return launch_mode<8, MODE, ROTATE>(a, s, grid_out);
    case 9: return launch_mode<9, MODE, ROTATE>(a, s, grid_out);
    case 10: return launch_mode<10, MODE, ROTATE>(a, s, grid_out);
    case 11: return launch_mode<11, MODE, ROTATE>(a, s, grid_out);
    case 12: return launch_mode<12, MODE, ROTATE>(a, s, grid_out);
    case 13: return launch_mode<13, MODE, ROTATE>(a, s, grid_out);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------- one row per workgroup
// Few tokens (decode-shaped calls, K = 1024 .. 8192): the one-wave-per-row
// kernel above leaves most of the chip idle and runs each row's whole chain
// on one wave. Here a workgroup of K / 8 threads (512 at K = 8192) owns one
// row: thread t holds elements E t .. E t + E - 1 (E = 8, or 16 at
// K = 8192), runs the butterflies over the E-index bits in registers, then
// three passes over the padded row in LDS cover the other bits (radix 8;
// the last pass takes the 2 or 1 bits left at K = 2048 or 1024). The reorder reads each output
// position's source channel straight from the row buffer through perm.
// Group maxima, the grid-wide wait (same epoch-tagged rows as fused_kernel,
// one row per workgroup), the per-token scale and the packing follow the
// kernels above with the same arithmetic.
constexpr int kRowThreads = 512;  // the most threads of a row workgroup (K = 4096, 8192)
// Threads of a row workgroup: K / 8 (eight elements each) up to K = 4096,
// 512 at K = 8192 (sixteen each).
template <int LOG2K>
constexpr int row_threads() {
  return LOG2K >= 12 ? kRowThreads : (1 << LOG2K) / 8;
}
// Weight read-ahead: loads a thread keeps in flight (its whole share in one
// batch), and how long a prefetch workgroup sleeps first (s_sleep 32 is
// about 2048 cycles, 0.85 us at 2.4 GHz) so that the rows' own loads go
// out ahead of it.
constexpr int kPrefetchLoads = 24;
constexpr int kPrefetchSleeps = 1;
// Workgroup `wg` of `nwg` reads its contiguous share of the first `keep`
// 16-byte words of every `period` words of p[0, words) once (one batch of
// loads per thread when the share is at most kPrefetchLoads words per
// thread). Each load's address takes a 64-bit division, which spreads a
// thread's loads over a few microseconds; computed incrementally (one
// division per thread) they went out back to back and the row workgroups'
// latency-bound chain queued behind the burst: M = 1, K = N = 8192
// 16.9 -> 19.0 us, M = 16, K = N = 4096 14.3 -> 16.5 us. The values only
// feed an XOR that is stored when `sink` is set (never): the reads exist to
// bring the memory into the memory-side cache for the kernel that follows.
__device__ __forceinline__ void prefetch_share(const uint4* p, size_t words, int period, int keep, int wg, int nwg,
                                               int tid, int T, uint32_t* sink) {
  constexpr int kU = kPrefetchLoads;
  for (int d = 0; d < kPrefetchSleeps; ++d) __builtin_amdgcn_s_sleep(32);
  const size_t kept = words / period * keep;
  const size_t per = (kept + nwg - 1) / nwg;
  const size_t b = static_cast<size_t>(wg) * per;
  const size_t e = min(kept, b + per);
  uint32_t x = 0u;
  for (size_t i = b + tid; i < e; i += static_cast<size_t>(T) * kU) {
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t j = i + static_cast<size_t>(u) * T;
      v[u] = j < e ? p[j / keep * period + j % keep] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (sink) sink[tid] = x;
}

// rowsplit_kernel modes: the one-launch front end (one row per workgroup,
// grid-wide wait), and the stats and quantise passes of the three launches
// (rows looped over the grid).
enum RowMode { kRowOne = 0, kRowStats = 1, kRowQuant = 2 };

__device__ __forceinline__ constexpr int rowpad(int f) { return f + 4 * (f >> 6); }

template <int LOG2K, int B>
__device__ __forceinline__ void row_pass8(float* row, int tid) {
  constexpr int K = 1 << LOG2K, T = row_threads<LOG2K>();
  constexpr int R = LOG2K - B < 3 ? LOG2K - B : 3;  // bits of this pass (the last may take fewer)
  constexpr int P = 1 << R;
  for (int t = tid; t < (K >> R); t += T) {
    const int lo = t & ((1 << B) - 1), hi = t >> B;
    const int base = (hi << (B + R)) | lo;
    float v[P];
#pragma unroll
    for (int u = 0; u < P; ++u) v[u] = row[rowpad(base + (u << B))];
#pragma unroll
    for (int h = 1; h < P; h <<= 1) butterfly<P>(v, h);
#pragma unroll
    for (int u = 0; u < P; ++u) row[rowpad(base + (u << B))] = v[u];
  }
  __syncthreads();
}

// The same pass with items of two adjacent elements (f bit 0 is done in
// registers), moved as one 8-byte LDS word: at K = 8192 (16 elements per
// thread) faster than 4-byte words (decode front end 7.46 -> 7.22 us, the
// three-launch passes at M = 1024 25.4 -> 23.1 us), at K = 4096 slower.
template <int LOG2K, int B>
__device__ __forceinline__ void row_pass8_pairs(float* row, int tid) {
  constexpr int K = 1 << LOG2K, T = row_threads<LOG2K>();
  constexpr int R = LOG2K - B < 3 ? LOG2K - B : 3;
  constexpr int P = 1 << R;
  for (int t = tid; t < (K >> (R + 1)); t += T) {
    const int lo = t & ((1 << (B - 1)) - 1), hi = t >> (B - 1);
    const int base = (hi << (B + R)) | (lo << 1);
    float v0[P], v1[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const float2 q = *reinterpret_cast<const float2*>(row + rowpad(base + (u << B)));
      v0[u] = q.x;
      v1[u] = q.y;
    }
#pragma unroll
    for (int h = 1; h < P; h <<= 1) {
      butterfly<P>(v0, h);
      butterfly<P>(v1, h);
    }
#pragma unroll
    for (int u = 0; u < P; ++u) *reinterpret_cast<float2*>(row + rowpad(base + (u << B))) = make_float2(v0[u], v1[u]);
  }
  __syncthreads();
}

template <int LOG2K, bool ROTATE, int RM>
__global__ void __launch_bounds__(row_threads<LOG2K>()) rowsplit_kernel(FeArgs a) {
  constexpr int K = 1 << LOG2K;
  constexpr int T = row_threads<LOG2K>();
  constexpr int E = K / T;  // 8, or 16 at K = 8192
  constexpr int LOG2E = E == 16 ? 4 : 3;
  static_assert(E == 8 || E == 16, "K = 1024 .. 8192");
  __shared__ __attribute__((aligned(16))) float s_row[K + K / 16];
  __shared__ float s_grp[K / 32];
  __shared__ float s_red[T / 64];

  const int tid = threadIdx.x;
  if (RM == kRowOne && static_cast<int>(blockIdx.x) >= a.rows) {  // a prefetch workgroup
    prefetch_share(a.pf, a.pf_words, a.pf_period, a.pf_keep, static_cast<int>(blockIdx.x) - a.rows, a.pf_wg, tid, T,
                   a.pf_sink);
    return;
  }
  const int lane = tid & 63;
  const int ngroups = K >> a.log2G;
  const int G = 1 << a.log2G;
  const int p0 = E * tid;  // this thread's first element / output position

  // ---- loads: perm of the outputs, then the activations (and signs)
  int src[E];
#pragma unroll
  for (int c = 0; c < E / 4; ++c) {
    const int4 q = *reinterpret_cast<const int4*>(a.perm + p0 + 4 * c);
    src[4 * c] = rowpad(q.x);
    src[4 * c + 1] = rowpad(q.y);
    src[4 * c + 2] = rowpad(q.z);
    src[4 * c + 3] = rowpad(q.w);
  }
  // one launch: one row per workgroup, whose epoch is read after the row's
  // loads are issued (its value goes to a scalar register at once, and the
  // wait for it covers every load issued before it); passes: rows
  // blockIdx.x, + gridDim.x, ...
  uint32_t epoch = 0u;
  if constexpr (RM == kRowQuant) {
    // S from the reduce launch; without smoothing S = 1 (written here)
    for (int g = tid; g < ngroups; g += T) {
      float sg = a.smooth ? a.S_out[g] : 1.f;
      if (!(sg > 0.f)) sg = 1.f;  // all-zero group over every token
      if (!a.smooth && blockIdx.x == 0) a.S_out[g] = 1.f;
      s_grp[g] = 1.f / sg;
    }
  } else {
    for (int g = tid; g < ngroups; g += T) s_grp[g] = 0.f;
  }
  for (int row = blockIdx.x; row < a.rows; row += gridDim.x) {
  bool gave_up = false;  // the one-launch wait gave up (the outputs are marked)
  uint4 w[E / 8];
#pragma unroll
  for (int i = 0; i < E / 8; ++i)
    w[i] = *reinterpret_cast<const uint4*>(a.src + static_cast<size_t>(row) * K + p0 + 8 * i);
  if (ROTATE && a.dsign) {
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      const uint32_t b = a.dsign[(p0 >> 3) + i];
      w[i].x ^= ((b & 1u) << 15) | ((b & 2u) << 30);
      w[i].y ^= ((b & 4u) << 13) | ((b & 8u) << 28);
      w[i].z ^= ((b & 16u) << 11) | ((b & 32u) << 26);
      w[i].w ^= ((b & 64u) << 9) | ((b & 128u) << 24);
    }
  }
  // (a lone row workgroup, which exchanges nothing, reads the error word
  // here too: its wait covers the same loads)
  uint32_t err_alone = 0u;
  if (RM == kRowOne && a.smooth) {
    epoch = __hip_atomic_load(&a.sync[kSyncEpoch], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    if (a.rows == 1)
      err_alone = __hip_atomic_load(&a.sync[kSyncError], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- rotate: E-index bits in registers, the other nine bits in LDS
  float v[E];
#pragma unroll
  for (int i = 0; i < E / 8; ++i) {
    const uint32_t q[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * i + 2 * e] = h2f(q[e] & 0xffffu);
      v[8 * i + 2 * e + 1] = h2f(q[e] >> 16);
    }
  }
  if (ROTATE) {
#pragma unroll
    for (int h = 1; h < E; h <<= 1) butterfly<E>(v, h);
  }
#pragma unroll
  for (int c = 0; c < E / 4; ++c)
    *reinterpret_cast<float4*>(s_row + rowpad(p0 + 4 * c)) = make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
  __syncthreads();
  if (ROTATE) {
    if constexpr (LOG2K == 13) {
      row_pass8_pairs<LOG2K, LOG2E>(s_row, tid);
      row_pass8_pairs<LOG2K, LOG2E + 3>(s_row, tid);
      row_pass8_pairs<LOG2K, LOG2E + 6>(s_row, tid);
    } else {
      row_pass8<LOG2K, LOG2E>(s_row, tid);
      row_pass8<LOG2K, LOG2E + 3>(s_row, tid);
      row_pass8<LOG2K, LOG2E + 6>(s_row, tid);
    }
  }

  // ---- reorder, then the group maximum of this row (all E in one group)
#pragma unroll
  for (int r = 0; r < E; ++r) v[r] = s_row[src[r]];
  float m = fabsf(v[0]);
#pragma unroll
  for (int r = 1; r < E; ++r) m = fmaxf(m, fabsf(v[r]));
  const int g0 = p0 >> a.log2G;
  if (RM == kRowStats || (RM == kRowOne && a.smooth)) {
    float mg = m;
    if (G > E) mg = lanes_max(mg, min(G / E, 64));
    if ((p0 & (G - 1)) == 0 || (lane == 0)) {
      if (mg > 0.f) atomicMax(reinterpret_cast<uint32_t*>(&s_grp[g0]), __float_as_uint(mg));
    }
  }
  if constexpr (RM == kRowStats) {
    __syncthreads();  // the row buffer is reused by the next row
    continue;
  }
  if (RM == kRowOne && a.smooth) {
    __syncthreads();

    // ---- publish this row's maxima, read every row's (as fused_kernel);
    // the only row workgroup already holds every token's maxima: it skips
    // the exchange (a round trip) and reads the error word alone; it still
    // advances the epoch, so the count of one-launch calls stays exact
    const bool alone = a.rows == 1;
    uint64_t* part = reinterpret_cast<uint64_t*>(a.sync + kSyncPartials);
    const uint64_t tag = static_cast<uint64_t>(epoch) << 32;
    if (alone) {
      gave_up = err_alone != 0u || a.spin_limit == 0u;
    } else {
      for (int g = tid; g < ngroups; g += T)
        __hip_atomic_store(&part[static_cast<size_t>(row) * ngroups + g], tag | __float_as_uint(s_grp[g]),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      for (int g = tid; g < ngroups; g += T) s_grp[g] = 0.f;
      __syncthreads();
      {
        // a workspace whose wait failed before gives up at once (as
        // fused_kernel; read here with the first poll for the same reason)
        const uint32_t spin_limit =
            __hip_atomic_load(&a.sync[kSyncError], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ? 0u : a.spin_limit;
        constexpr int kBatch = 8;
        const int n = a.rows * ngroups;  // the row workgroups (prefetch ones publish nothing)
        for (int base = tid; base < n; base += T * kBatch) {
          uint64_t b[kBatch];
          uint32_t it = 0;
          for (;;) {
  #pragma unroll
            for (int k = 0; k < kBatch; ++k) {
              const int idx = base + k * T;
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
            if (bits) atomicMax(reinterpret_cast<uint32_t*>(&s_grp[(base + k * T) % ngroups]), bits);
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
    for (int g = tid; g < ngroups; g += T) {
      float sg = s_grp[g];
      if (!(sg > 0.f)) sg = 1.f;  // all-zero group over every token
      if (row == 0) a.S_out[g] = gave_up ? __builtin_nanf("") : sg;
      s_grp[g] = 1.f / sg;
    }
  } else if (RM == kRowOne) {
    for (int g = tid; g < ngroups; g += T) {
      if (row == 0) a.S_out[g] = 1.f;
      s_grp[g] = 1.f;
    }
  }
  __syncthreads();

  // ---- per-token scale (max over the row of |Zp| / S_g), codes, packing
  const float inv = s_grp[g0];
  float rmax = m * inv;
  rmax = lanes_max(rmax, 64);
  if (lane == 0) s_red[tid >> 6] = rmax;
  __syncthreads();
  rmax = s_red[0];
#pragma unroll
  for (int k = 1; k < T / 64; ++k) rmax = fmaxf(rmax, s_red[k]);
  const float k7 = rmax > 0.f ? 7.f / rmax : 0.f;
  const float ks = inv * k7;
  uint32_t packed[E / 8];
#pragma unroll
  for (int o = 0; o < E / 8; ++o) {
    uint32_t mag[8], sgn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mag[e] = __float_as_uint(fmaf(fabsf(v[8 * o + e]), ks, kMagic));
      sgn[e] = __float_as_uint(v[8 * o + e]);
    }
    packed[o] = pack8(mag, sgn);
  }
  uint8_t* dst = a.codes + codes_offset(row, p0 / 2, codes_row_stride(K));  // E / 2 bytes in one piece
  if constexpr (E == 16)
    *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
  else
    *reinterpret_cast<uint32_t*>(dst) = packed[0];
  if (tid == 0) a.scale[row] = gave_up ? __builtin_nanf("") : rmax / 7.f;
  if constexpr (RM == kRowOne) break;  // one row: no loop
  __syncthreads();                     // s_row and s_red are reused by the next row
  }

  if constexpr (RM == kRowStats) {
    // this workgroup's maxima over its rows into its own partial row
    __syncthreads();
    for (int g = tid; g < ngroups; g += T)
      a.part[static_cast<size_t>(blockIdx.x) * ngroups + g] = __float_as_uint(s_grp[g]);
  }
}

// Workgroups of fused_kernel<LOG2K, ROTATE, R> that the current device holds
// at once (occupancy per CU x CUs), cached per device; -1 if unknown.
template <int LOG2K, bool ROTATE, int R>
int fused_capacity() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  int cap = cache[dev].load(std::memory_order_relaxed);
  if (cap == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_kernel<LOG2K, ROTATE, R>,
                                                     Cfg<LOG2K>::kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        per_cu <= 0 || cus <= 0) {
      cap = -1;
    } else {
      cap = per_cu * cus;
    }
    cache[dev].store(cap, std::memory_order_relaxed);
  }
  return cap;
}

// Launch the fused front end with R blocks per wave if its grid fits on the
// device at once; returns false (nothing launched) otherwise.
template <int LOG2K, bool ROTATE, int R>
bool try_fused(const FeArgs& a, hipStream_t s, hipError_t* err) {
  using C = Cfg<LOG2K>;
  const int nblk = (a.rows + C::kRows - 1) / C::kRows;
  const int grid = (nblk + C::kWaves * R - 1) / (C::kWaves * R);
  const int cap = fused_capacity<LOG2K, ROTATE, R>();
  if (cap <= 0 || grid > cap || grid > kMaxFusedWG) return false;
  FeArgs b = a;
  // the read-ahead rides along only where one batch of loads per thread
  // covers all of it (and with one block per wave)
  if (R != 1 || b.pf_period != b.pf_keep ||
      b.pf_words > static_cast<size_t>(grid) * C::kThreads * kFusedPrefetchLoads)
    b.pf = nullptr;
  hipLaunchKernelGGL((fused_kernel<LOG2K, ROTATE, R>), dim3(grid), dim3(C::kThreads), 0, s, b);
  *err = hipGetLastError();
  return true;
}

// Blocks per wave of the one-launch form for `rows` rows (1 or 2), or 0
// when its grid does not fit on the current device at once.
template <int LOG2K, bool ROTATE>
int fused_blocks_per_wave(int rows) {
  using C = Cfg<LOG2K>;
  const int nblk = (rows + C::kRows - 1) / C::kRows;
  const int g1 = (nblk + C::kWaves - 1) / C::kWaves;
  int cap = fused_capacity<LOG2K, ROTATE, 1>();
  if (cap > 0 && g1 <= cap && g1 <= kMaxFusedWG) return 1;
  if constexpr (LOG2K <= 12) {
    const int g2 = (nblk + 2 * C::kWaves - 1) / (2 * C::kWaves);
    cap = fused_capacity<LOG2K, ROTATE, 2>();
    if (cap > 0 && g2 <= cap && g2 <= kMaxFusedWG) return 2;
  }
  return 0;
}

template <int LOG2K, bool ROTATE>
bool launch_fused(const FeArgs& a, hipStream_t s, hipError_t* err) {
  if (try_fused<LOG2K, ROTATE, 1>(a, s, err)) return true;
  if constexpr (LOG2K <= 12) {
    if (try_fused<LOG2K, ROTATE, 2>(a, s, err)) return true;
  }
  return false;
}

// Workgroups of rowsplit_kernel the device holds at once (cached per device).
template <int LOG2K, bool ROTATE, int RM>
int rowsplit_capacity() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  int cap = cache[dev].load(std::memory_order_relaxed);
  if (cap == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, rowsplit_kernel<LOG2K, ROTATE, RM>, row_threads<LOG2K>(),
                                                     0) !=
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

// Token counts up to which one row per workgroup beats one row per wave
// (measured at K = 4096 and 8192).
constexpr int kRowSplitMaxRows = 256;

template <int LOG2K, bool ROTATE>
bool rowsplit_fits(int rows) {
  if (rows < 1 || rows > kRowSplitMaxRows || rows > kMaxFusedWG) return false;
  const int cap = rowsplit_capacity<LOG2K, ROTATE, kRowOne>();
  return cap > 0 && rows <= cap;
}

bool rowsplit_applies(int log2K, bool rotate, int rows) {
  if (log2K == 10) return rotate ? rowsplit_fits<10, true>(rows) : rowsplit_fits<10, false>(rows);
  if (log2K == 11) return rotate ? rowsplit_fits<11, true>(rows) : rowsplit_fits<11, false>(rows);
  if (log2K == 12) return rotate ? rowsplit_fits<12, true>(rows) : rowsplit_fits<12, false>(rows);
  if (log2K == 13) return rotate ? rowsplit_fits<13, true>(rows) : rowsplit_fits<13, false>(rows);
  return false;
}

// Extra workgroups of a one-row-per-workgroup launch that prefetch: the
// compute units the rows leave idle (0: fewer than 64).
int prefetch_workgroups(int rows) {
  const int idle = device_cus() - rows;
  return idle >= 64 ? idle : 0;
}

template <int LOG2K, bool ROTATE>
hipError_t launch_rowsplit(const FeArgs& a, hipStream_t s) {
  const int grid = a.rows + (a.pf ? a.pf_wg : 0);
  hipLaunchKernelGGL((rowsplit_kernel<LOG2K, ROTATE, kRowOne>), dim3(grid), dim3(row_threads<LOG2K>()), 0, s, a);
  return hipGetLastError();
}

// A stats or quantise pass of the three launches on the row kernel (used at
// K = 8192): at most one workgroup per resident slot, each looping over its
// rows. *grid_out receives the launched grid.
template <int LOG2K, bool ROTATE, int RM>
hipError_t launch_row_pass(const FeArgs& a, hipStream_t s, int* grid_out) {
  const int cap = rowsplit_capacity<LOG2K, ROTATE, RM>();
  const int grid = cap > 0 && a.rows > cap ? cap : a.rows;
  if (grid_out) *grid_out = grid;
  hipLaunchKernelGGL((rowsplit_kernel<LOG2K, ROTATE, RM>), dim3(grid), dim3(row_threads<LOG2K>()), 0, s, a);
  return hipGetLastError();
}

template <int RM>
hipError_t row_pass_k(int log2K, bool rotate, const FeArgs& a, hipStream_t s, int* grid_out = nullptr) {
  if (log2K != 13) return hipErrorInvalidValue;
  return rotate ? launch_row_pass<13, true, RM>(a, s, grid_out) : launch_row_pass<13, false, RM>(a, s, grid_out);
}

hipError_t rowsplit_k(int log2K, bool rotate, const FeArgs& a, hipStream_t s) {
  if (log2K == 10) return rotate ? launch_rowsplit<10, true>(a, s) : launch_rowsplit<10, false>(a, s);
  if (log2K == 11) return rotate ? launch_rowsplit<11, true>(a, s) : launch_rowsplit<11, false>(a, s);
  if (log2K == 12) return rotate ? launch_rowsplit<12, true>(a, s) : launch_rowsplit<12, false>(a, s);
  return rotate ? launch_rowsplit<13, true>(a, s) : launch_rowsplit<13, false>(a, s);
}

template <bool ROTATE>
bool fused_k(int log2K, const FeArgs& a, hipStream_t s, hipError_t* err) {
  switch (log2K) {
    case 6: return launch_fused<6, ROTATE>(a, s, err);
    case 7: return launch_fused<7, ROTATE>(a, s, err);
    case 8: return launch_fused<8, ROTATE>(a, s, err);
    case 9: return launch_fused<9, ROTATE>(a, s, err);
    case 10: return launch_fused<10, ROTATE>(a, s, err);
    case 11: return launch_fused<11, ROTATE>(a, s, err);
    case 12: return launch_fused<12, ROTATE>(a, s, err);
    case 13: return launch_fused<13, ROTATE>(a, s, err);
    default: return false;
  }
}

}  // namespace

hipError_t launch_group_max(const uint32_t* part, int nrows, int ngroups, float* S_out, hipStream_t s) {
  if (ngroups <= 0) return hipSuccess;
  hipLaunchKernelGGL(group_max_kernel, dim3(ngroups), dim3(256), 0, s, part, nrows, ngroups, S_out);
  return hipGetLastError();
}

hipError_t launch_frontend(const uint16_t* X, int M, int K, int G, const int32_t* perm,
                           const uint32_t* dsign, uint8_t* xq, float* dx, float* S_out, uint32_t* sync,
                           int flags, hipStream_t s, float* zrows, const void* prefetch, size_t prefetch_bytes,
                           int prefetch_period, int prefetch_keep) {
  if (K & (K - 1)) return launch_frontend_kron(X, M, K, G, perm, dsign, xq, dx, S_out, sync, flags, s, zrows);
  const int log2K = __builtin_ctz(static_cast<unsigned>(K));
  FeArgs a{};
  a.dsign = reinterpret_cast<const uint8_t*>(dsign);
  a.src = X;
  a.rows = M;
  a.log2G = __builtin_ctz(static_cast<unsigned>(G));
  a.smooth = (flags & 2) ? 0 : 1;
  a.perm = perm;
  a.sync = sync;
  a.codes = xq;
  a.scale = dx;
  a.S_out = S_out;
  a.spin_limit = (flags & kFlagGiveUp) ? 0u : kSpinLimit;
  const bool rotate = !(flags & 1);
  hipError_t e = hipSuccess;
  // few tokens at K = 4096 / 8192: one row per workgroup, one launch
  const bool pf_ok = prefetch && prefetch_period >= 16 && prefetch_period % 16 == 0 && prefetch_keep >= 16 &&
                     prefetch_keep % 16 == 0 && prefetch_keep <= prefetch_period &&
                     prefetch_bytes >= size_t(prefetch_period);
  if (pf_ok) {
    a.pf = static_cast<const uint4*>(prefetch);
    a.pf_words = prefetch_bytes / 16;
    a.pf_period = prefetch_period / 16;
    a.pf_keep = prefetch_keep / 16;
  }
  if (!(flags & 4) && rowsplit_applies(log2K, rotate, M)) {
    if (pf_ok) {
      a.pf_wg = prefetch_workgroups(M);
      // only where one batch of loads per thread covers it: a longer
      // prefetch would outlast the rows and delay the kernel that follows
      const int threads = log2K >= 12 ? kRowThreads : (1 << log2K) / 8;
      const size_t kept = a.pf_words / a.pf_period * a.pf_keep;
      if (a.pf_wg == 0 || kept > static_cast<size_t>(a.pf_wg) * threads * kPrefetchLoads) a.pf = nullptr;
    }
    return rowsplit_k(log2K, rotate, a, s);
  }
  if (a.smooth) {
    // one launch when every workgroup fits on the device at once
    if (!(flags & 4) && (rotate ? fused_k<true>(log2K, a, s, &e) : fused_k<false>(log2K, a, s, &e))) return e;
    a.pf = nullptr;  // the passes carry no read-ahead
    // else stats, reduce, quantise. The stats rows (one per workgroup) sit
    // in the codes buffer, which the quantise pass overwrites after the
    // reduce has read them: at most pass_grid(log2K, M) rows of K/G words
    // take at most M K / 32 bytes of its M K / 2 (K/G <= K/32 words, and a
    // workgroup covers at least 3 rows, or 8 blocks of 4096/K rows when
    // K < 4096).
    const int ngroups = K / G;
    if (static_cast<size_t>(pass_grid(log2K, M)) * ngroups * 4 > static_cast<size_t>(M) * (K / 2))
      return hipErrorInvalidValue;
    a.part = reinterpret_cast<uint32_t*>(xq);
    int nrows = 0;
    // K = 8192: the row kernel's passes (24 waves per CU) beat the block
    // kernel's (3 waves per CU); at K = 4096 the block kernel's passes, with
    // the rotation on the matrix cores and 8 waves, are faster
    if (log2K == 13)
      e = row_pass_k<kRowStats>(log2K, rotate, a, s, &nrows);
    else
      e = rotate ? dispatch_k<kStats, true>(log2K, a, s, &nrows) : dispatch_k<kStats, false>(log2K, a, s, &nrows);
    if (e != hipSuccess) return e;
    e = launch_group_max(a.part, nrows, ngroups, S_out, s);
    if (e != hipSuccess) return e;
  }
  if (log2K == 13) return row_pass_k<kRowQuant>(log2K, rotate, a, s);
  return rotate ? dispatch_k<kQuant, true>(log2K, a, s) : dispatch_k<kQuant, false>(log2K, a, s);
}

int frontend_launches(int M, int K, int flags) {
  if (K & (K - 1)) {
    int m = 0, ln = 0;
    return kron_split(K, &m, &ln) ? kron_frontend_launches(M, K, flags) : -1;
  }
  const int log2K = __builtin_ctz(static_cast<unsigned>(K));
  if (flags & 2) return 1;
  if (flags & 4) return 3;
  const bool rotate = !(flags & 1);
  if (rowsplit_applies(log2K, rotate, M)) return 1;
  int r = 0;
  switch (log2K) {
#define RRS_CASE(L) case L: r = rotate ? fused_blocks_per_wave<L, true>(M) : fused_blocks_per_wave<L, false>(M); break;
    RRS_CASE(6) RRS_CASE(7) RRS_CASE(8) RRS_CASE(9) RRS_CASE(10) RRS_CASE(11) RRS_CASE(12) RRS_CASE(13)
#undef RRS_CASE
    default: return -1;
  }
  return r > 0 ? 1 : 3;
}

hipError_t launch_weight_prep(const uint16_t* W, int K, int N, const int32_t* perm,
                              const uint32_t* dsign, uint8_t* wq, float* dw, hipStream_t s, bool rotate) {
  if (K & (K - 1)) return launch_weight_prep_kron(W, K, N, perm, dsign, wq, dw, s, rotate);
  const int log2K = __builtin_ctz(static_cast<unsigned>(K));
  FeArgs a{};
  a.dsign = reinterpret_cast<const uint8_t*>(dsign);
  a.src = W;
  a.rows = N;
  a.ldw = N;
  a.log2G = log2K;
  a.smooth = 0;
  a.perm = perm;
  a.codes = wq;
  a.scale = dw;
  return rotate ? dispatch_k<kWeight, true>(log2K, a, s) : dispatch_k<kWeight, false>(log2K, a, s);
}

hipError_t launch_calibrate(const uint16_t* Xc, int T, int K, const uint32_t* dsign, int32_t* perm,
                            uint32_t* ws, hipStream_t s, bool rotate) {
  hipError_t e = launch_zero_u32(ws, static_cast<size_t>(K), s);
  if (e != hipSuccess) return e;
  if (K & (K - 1)) {
    e = launch_colmax_kron(Xc, T, K, dsign, ws, s, rotate);
  } else {
    const int log2K = __builtin_ctz(static_cast<unsigned>(K));
    FeArgs a{};
    a.src = Xc;
    a.rows = T;
    a.log2G = log2K;
    a.colmax = ws;
    a.dsign = reinterpret_cast<const uint8_t*>(dsign);
    e = rotate ? dispatch_k<kColmax, true>(log2K, a, s) : dispatch_k<kColmax, false>(log2K, a, s);
  }
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
