// Grouped INT4 x INT4 GEMM of the RRS A4W4 linear on gfx950.
//
// Y[t, n] = (1/K) dx[t] dw[n] sum_g S[g] P_g[t, n],
// P_g[t, n] = sum_{j in group g} q[t, j] qw[n, j]    (exact integers)
//
// The group scale multiplies each group's integer partial before the fp32
// accumulation: the smoothing is not migrated into the weights (RRS summary
// page, atlas.scime.ai, "Approach"), and grouping the scales along K keeps
// the contraction in wide tiles (RRS rebuttal page, paperhub.cn, "Novelty":
// per-channel scales do not fit the hardware's tiled scheme).
//
// gfx950 has no 4-bit integer matrix instruction. Each 4-bit code widens to
// an fp8 e4m3 subnormal, +-|q| * 2^-9, which the matrix core multiplies
// exactly; products (+-|q_a q_b| * 2^-18) and group sums (< 2^24 units) are
// exact in the fp32 accumulator, so the group partials are the exact
// integers scaled by 2^-18. The packing puts each code's sign and magnitude
// where one AND (even codes) or a rotate and an AND (odd codes) yields the
// e4m3 byte: 3 VALU operations per 8 codes.
//
// The group rescale runs inside the accumulator: after group g the MFMA
// accumulator holds (sum_{g' <= g} S_g' P_g') / S_g, so entering group g+1
// costs one multiply by S_g / S_{g+1} per output and the products of the
// next group accumulate on top. No separate integer accumulator is kept.
//
// Tiles: 256 output channels x 128 tokens per workgroup, 4 waves of
// 128 x 64. The MFMA A operand is the weight tile (rows n), the B operand the
// activation tile (rows t), so runs of four accumulator registers are four
// consecutive output channels of one token. A tile inside Y goes out
// through the idle rings: set 0 writes the finished tile there as token
// rows, and all eight waves store whole 1-KiB rows of Y with streaming
// (non-temporal) stores (a ragged tile stores its 16-byte runs directly).
// K advances in stages of 128 codes (64 packed bytes per row): direct
// global -> LDS loads into 3-slot rings (two stages in flight), then
// per-wave widening of the packed fragments -> MFMA. Two sets of 4 waves
// split K and add their partial sums at the end.
// v_mfma_f32_32x32x64_f8f6f4 serves G >= 64 (one instruction never crosses
// a group boundary), v_mfma_f32_16x16x32_fp8_fp8 G = 32. The 32 x 32 shape
// is chosen for its length: an MFMA hides only a few VALU issue slots of the
// widening and rescale that go with it, and a 64-cycle 32 x 32 x 64 MFMA
// hides about three times as many as a 32-cycle 16 x 16 x 128 one for the
// same products.

#include "rrs_internal.h"

namespace rrs {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kTN = 256;       // output channels per workgroup tile
constexpr int kTT = 128;       // tokens per workgroup tile
constexpr int kThreads = 256;  // 4 waves: 2 (n) x 2 (t), each 128 x 64
constexpr int kRowB = 64;      // packed bytes per row per stage (128 codes)
constexpr int kLineB = 128;    // stored bytes per row pair per stage (both rows' pieces)
constexpr int kWB = kTN * kRowB;
constexpr int kXB = kTT * kRowB;
constexpr int kStageB = kWB + kXB;
constexpr float kUnit = 262144.0f;  // 2^18: one integer product in accumulator units

struct GemmArgs {
  const uint8_t* xq;
  const float* dx;
  const float* S;
  const uint8_t* wq;
  const float* dw;
  float* Y;
  int32_t* P;  // partials window (partials variant)
  const uint32_t* err;  // nonzero word: write NaN to every output (nullptr: none)
  float ybase;          // 2^18 / K for rotated codes, 2^18 without the rotation
  int M, N, K, log2G;
  int pm0, pm1, pn0, pn1;
  int tiles_t, tiles_n;
};

// a-codes (even) and b-codes (odd) of a packed word as e4m3 subnormals
__device__ __forceinline__ uint32_t ecodes(uint32_t w) { return w & 0x87878787u; }
__device__ __forceinline__ uint32_t ocodes(uint32_t w) {
  return __builtin_amdgcn_alignbit(w, w, 4) & 0x87878787u;
}

// MFMA shapes. KM: codes of K per instruction; BR: rows (and columns) of an
// accumulator block; NQ: runs of four consecutive output channels per lane
// in a block. Lane l's fragment holds row l % BR of a block; its codes sit
// at logical 16-byte chunk chunk(ks, l) of the stage row plus byte inner(l).
template <int KM>
struct Mma;

template <>
struct Mma<64> {  // 32 x 32 x 64: 32 codes (16 packed bytes) per lane
  typedef v8i frag;
  typedef v16f acc_t;
  static constexpr int BR = 32, NQ = 4, kSteps = 2, kLog2K = 6;
  __device__ static int chunk(int ks, int l) { return ks * 2 + (l >> 5); }
  __device__ static int inner(int) { return 0; }
  // register r of lane l: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
  __device__ static int qrow(int q, int l) { return 8 * q + 4 * (l >> 5); }
  __device__ static frag load(const uint8_t* p) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    return v8i{(int)ecodes(w.x), (int)ocodes(w.x), (int)ecodes(w.y), (int)ocodes(w.y),
               (int)ecodes(w.z), (int)ocodes(w.z), (int)ecodes(w.w), (int)ocodes(w.w)};
  }
  __device__ static acc_t mma(frag a, frag b, acc_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
  __device__ static acc_t zero() {
    acc_t z;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = 0.f;
    return z;
  }
  __device__ static v4f quad(const acc_t& c, int q) { return v4f{c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]}; }
  __device__ static void set_quad(acc_t& c, int q, v4f v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c[4 * q + e] = v[e];
  }
};

template <>
struct Mma<32> {  // 16 x 16 x 32: 8 codes (4 packed bytes) per lane
  typedef long frag;
  typedef v4f acc_t;
  static constexpr int BR = 16, NQ = 1, kSteps = 4, kLog2K = 5;
  __device__ static int chunk(int ks, int) { return ks; }
  __device__ static int inner(int l) { return (l >> 4) * 4; }
  // register r of lane l: row 4 (l / 16) + r, column l % 16
  __device__ static int qrow(int, int l) { return 4 * (l >> 4); }
  __device__ static frag load(const uint8_t* p) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    return static_cast<long>(static_cast<uint64_t>(ecodes(w)) | (static_cast<uint64_t>(ocodes(w)) << 32));
  }
  __device__ static acc_t mma(frag a, frag b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
  }
  __device__ static acc_t zero() { return v4f{0.f, 0.f, 0.f, 0.f}; }
  __device__ static v4f quad(const acc_t& c, int) { return c; }
  __device__ static void set_quad(acc_t& c, int, v4f v) { c = v; }
};

// Split K: the workgroup is two sets of 4 waves over the same output tile;
// set 0 runs the first half of K, set 1 the second, and their partial sums
// meet in LDS at the end. Two waves per SIMD let one wave's widening and
// rescale overlap the other's matrix instructions.
constexpr int kSets = 2;
constexpr int kThreadsWG = kSets * kThreads;

// LDS rings, one per set, three slots each (two stages in flight). Separate
// arrays let the compiler tell which direct-to-LDS load a fragment read
// depends on (with one array it would wait for every load in flight).
constexpr int kRing = 3;
constexpr uint32_t kBarSpinLimit = 1u << 22;  // polls before a set barrier gives up
__shared__ __attribute__((aligned(1024))) uint8_t s_r00[kStageB];
__shared__ __attribute__((aligned(1024))) uint8_t s_r01[kStageB];
__shared__ __attribute__((aligned(1024))) uint8_t s_r02[kStageB];
__shared__ __attribute__((aligned(1024))) uint8_t s_r10[kStageB];
__shared__ __attribute__((aligned(1024))) uint8_t s_r11[kStageB];
__shared__ __attribute__((aligned(1024))) uint8_t s_r12[kStageB];

template <int SET, int SLOT>
__device__ __forceinline__ uint8_t* ring() {
  if (SET == 0) return SLOT == 0 ? s_r00 : SLOT == 1 ? s_r01 : s_r02;
  return SLOT == 0 ? s_r10 : SLOT == 1 ? s_r11 : s_r12;
}

// 1-KiB chunk c (0 <= c < 144) of the six ring buffers, used to park the
// second set's partial sums once the rings are idle. c is wave-uniform.
// The compiler places the six arrays back to back in declaration order;
// the address arithmetic then needs no branch (the test folds to a
// constant, the switch only stands in if the layout ever differs).
__device__ __forceinline__ float* park_chunk(int c) {
  uint8_t* b0 = s_r00;
  if (s_r01 == b0 + kStageB && s_r02 == b0 + 2 * kStageB && s_r10 == b0 + 3 * kStageB &&
      s_r11 == b0 + 4 * kStageB && s_r12 == b0 + 5 * kStageB)
    return reinterpret_cast<float*>(b0 + c * 1024);
  uint8_t* b;
  switch (c / 24) {
    case 0: b = s_r00; break;
    case 1: b = s_r01; break;
    case 2: b = s_r02; break;
    case 3: b = s_r10; break;
    case 4: b = s_r11; break;
    default: b = s_r12; break;
  }
  return reinterpret_cast<float*>(b + (c % 24) * 1024);
}

// vmcnt(n) and lgkmcnt(0), expcnt unconstrained (gfx9 s_waitcnt encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] in bits 15:14). The
// barrier that follows then also publishes this wave's LDS stores.
#define RRS_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0070)

template <int KM, bool PARTIALS, int SPG>
struct GemmCtx {
  using Mm = Mma<KM>;
  static constexpr int kDmaPerWave = (kStageB / 1024) / (kThreads / 64);  // 6

  const GemmArgs& a;
  int lane, wn, wt, n0, t0, Kb, nstage, log2spg, ngroups;
  int st0, st1;                      // this set's stage range [st0, st1)
  const uint8_t* wbase;               // uniform: weight row n0 of the tile
  const uint8_t* xbase;               // uniform: activation row t0 of the tile
  uint32_t voff[kDmaPerWave];         // this lane's offset from its block's base: row and 16-byte piece
  uint32_t lblk[kDmaPerWave];         // uniform: LDS offset of each block in a stage
  int wave6;                          // uniform: first DMA block of this wave
  static constexpr int TI = 128 / Mm::BR;  // accumulator blocks per wave along n
  static constexpr int TJ = 64 / Mm::BR;   // and along t
  int fW, fX, swz;
  typename Mm::acc_t acc[TI][TJ];
  const float* rat;
  uint32_t* sbar;   // this set's arrival counter (LDS)
  uint32_t* sbar2;   // both sets' counters, set 0's first (LDS)
  int setid;         // this wave's set
  uint32_t nbar = 0;

  __device__ GemmCtx(const GemmArgs& args, const float* s_rat) : a(args), rat(s_rat) {}

  // DMA block d of stage st into ring slot `base`: the scalar base (block
  // row plus stage) and the lane's fixed offset form the address, so a
  // stage's loads cost no vector instructions. The load is written in
  // assembly so that the compiler does not track it: its wait insertion
  // loses the ring slots' alias scopes across the loop's back edge and then
  // drains every load in flight (the next stage's included) before a
  // stage's first fragment read, which leaves one stage of prefetch instead
  // of two. The kernel orders these loads itself: each wave waits for its
  // own loads of a stage, then the set barrier, before any fragment read of
  // it. The instruction writes no register (its data goes to LDS at M0 plus
  // 16 bytes per lane), so nothing the compiler allocates is overwritten
  // while it is in flight; M0 is set here for every load (nothing else in
  // this file uses it).
  __device__ __forceinline__ void issue_one(uint8_t* base, int st, int d) {
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    // both scalar operands are uniform; readfirstlane keeps them in scalar
    // registers where the compiler cannot prove it (a no-op elsewhere). Its
    // result is a signed int: widen through uint32_t, never directly.
    const uint32_t lds = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
        static_cast<int>(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)base)) + lblk[d])));
    const uint64_t ra = reinterpret_cast<uint64_t>((wave6 + d < 16 ? wbase : xbase) + st * kLineB);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(ra))));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(ra >> 32))));
    const uint8_t* rows = reinterpret_cast<const uint8_t*>(static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff[d]), "s"(rows), "s"(lds)
                 : "memory");  // M0 is reserved: the compiler keeps no value of its own there
  }

  __device__ __forceinline__ void issue(uint8_t* base, int st) {
#pragma unroll
    for (int d = 0; d < kDmaPerWave; ++d) issue_one(base, st, d);
  }

  // One stage of products; the DMA of stage nst into slot NSLOT is issued
  // one block after each of the first rows of products, so the address
  // unit's work for it spreads over the stage instead of stalling every
  // wave right after the barrier.
  __device__ __forceinline__ void compute(const uint8_t* stage, uint8_t* next, int st, int nst) {
#pragma unroll
    for (int ks = 0; ks < Mm::kSteps; ++ks) {
      const int step = st * Mm::kSteps + ks;
      if (step << Mm::kLog2K >= a.K) break;  // K = 64: half a stage
      const int gs = step & ((1 << log2spg) - 1);
      // logical chunk of this k-step, stored at chunk position logical ^ swizzle
      const int koff = ((Mm::chunk(ks, lane) * 16) ^ swz) + Mm::inner(lane);
      typename Mm::frag fx[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j) fx[j] = Mm::load(stage + fX + j * Mm::BR * kRowB + koff);
      // Entering a new group rescales the accumulator by S_{g-1} / S_g (the
      // partials dump multiplies it by 0 instead: the same instructions).
      // With SPG (MFMA k-steps per group) known at compile time, each block
      // is multiplied just before its first product of the group: its
      // previous product was issued a full row of blocks earlier and has
      // retired, so neither the multiplies nor the matrix core wait on each
      // other. When a group is one stage (two k-steps), that would put all
      // of the rescale in the first k-step (200 vector instructions against
      // 72 in the second, for 8 matrix instructions each), so the first
      // half of the rows is rescaled at the end of the previous group
      // instead, two rows after its last product (same value, same
      // rounding). Otherwise (G > 128, one group over several stages) the
      // whole accumulator is scaled at the group's first k-step.
      if constexpr (SPG == 2 && Mm::kSteps == 2 && !PARTIALS) {
        if (ks == 0) {
          const float r = step > st0 * Mm::kSteps ? rat[step >> log2spg] : 1.f;
          products<kLateHalf>(stage, next, koff, fx, r, ks, nst);
        } else {  // the next group's ratio, if the next stage is this set's
          const float r = st + 1 < st1 ? rat[(step + 1) >> log2spg] : 1.f;
          products<kEarlyHalf>(stage, next, koff, fx, r, ks, nst);
        }
      } else if constexpr (SPG > 0) {
        if (ks % SPG == 0) {  // folds: ks is an unrolled index
          const float r = step > st0 * Mm::kSteps ? (PARTIALS ? 0.f : rat[step >> log2spg]) : 1.f;
          products<kAll>(stage, next, koff, fx, r, ks, nst);
        } else {
          products<kNone>(stage, next, koff, fx, 1.f, ks, nst);
        }
      } else {
        if (gs == 0 && step > st0 * Mm::kSteps) {
          // the previous k-step's last products were issued just before:
          // two more issue slots keep the multiplies past their results
          // (the compiler's own padding can fall one short across the
          // branch into this block)
          __builtin_amdgcn_sched_barrier(0);
          asm volatile("s_nop 1");
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) acc[i][j] = PARTIALS ? Mm::zero() : acc[i][j] * rat[step >> log2spg];
        }
        products<kNone>(stage, next, koff, fx, 1.f, ks, nst);
      }
      // a group that ends inside this set (with one group over all of K the
      // two sets' integer halves are added first; the epilogue dumps them)
      if (PARTIALS && ngroups > 1 && gs == (1 << log2spg) - 1) dump(step >> log2spg);
    }
  }

  // Where a k-step multiplies accumulator blocks by r: kNone nowhere; kAll
  // every block right before its product; kLateHalf the second half of the
  // rows right before their products; kEarlyHalf the first half of the
  // rows, row i - TI/2 after the products of row i (its own products were
  // issued two rows earlier and have retired).
  enum Rescale { kNone, kAll, kLateHalf, kEarlyHalf };

  // The products of one k-step. One DMA block of the next stage goes out
  // after each row of products.
  template <int RS>
  __device__ __forceinline__ void products(const uint8_t* stage, uint8_t* next, int koff,
                                           const typename Mm::frag (&fx)[TJ], float r, int ks, int nst) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const typename Mm::frag fw = Mm::load(stage + fW + i * Mm::BR * kRowB + koff);
      const bool pre = RS == kAll || (RS == kLateHalf && i >= TI / 2);
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = Mm::mma(fw, fx[j], pre ? acc[i][j] * r : acc[i][j]);
      if (RS == kEarlyHalf && i >= TI / 2) {
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i - TI / 2][j] = acc[i - TI / 2][j] * r;
      }
      const int d = ks * TI + i;
      if (d < kDmaPerWave) issue_one(next, nst, d);
    }
  }

  __device__ void dump(int g) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int t = t0 + wt * 64 + j * Mm::BR + (lane % Mm::BR);
#pragma unroll
        for (int q = 0; q < Mm::NQ; ++q) {
          const v4f v = Mm::quad(acc[i][j], q);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int n = n0 + wn * 128 + i * Mm::BR + Mm::qrow(q, lane) + e;
            if (t >= a.pm0 && t < a.pm1 && n >= a.pn0 && n < a.pn1) {
              const size_t o = (static_cast<size_t>(t - a.pm0) * (a.pn1 - a.pn0) + (n - a.pn0)) * ngroups + g;
              a.P[o] = static_cast<int32_t>(v[e] * kUnit);
            }
          }
        }
      }
  }

  // Barrier of the set's four waves only: an LDS arrival counter that every
  // wave bumps once per stage, then polls until all four have (bounded
  // poll; the count only grows within a launch). The caller has waited for
  // its own loads and LDS accesses, so after the wait every block of the
  // stage is in LDS and every read of the slot about to be refilled is
  // done. The two sets of a workgroup never wait for each other, so they
  // drift apart and one set's waits overlap the other's matrix work.
  // The counter is accessed in inline assembly that waits for its own
  // result: as plain LDS accesses the compiler cannot tell them apart from
  // the direct-to-LDS loads in flight and would drain all of them first.
  __device__ __forceinline__ void set_barrier() {
    nbar += 4;
    typedef __attribute__((address_space(3))) uint32_t lds_u32;
    const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u32*)sbar));
    const uint32_t one = 1u;
    if (lane == 0) asm volatile("ds_add_u32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(addr), "v"(one) : "memory");
    // each poll reads both sets' counters (adjacent words) at once: this
    // set's decides the wait, the other set's the priority below
    const uint32_t both_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u32*)sbar2));
    uint32_t no = 0u;
    for (uint32_t it = 0; it < kBarSpinLimit; ++it) {
      uint64_t both;
      asm volatile("ds_read2_b32 %0, %1 offset1:1\n\ts_waitcnt lgkmcnt(0)" : "=v"(both) : "v"(both_addr) : "memory");
      const uint32_t c0 = static_cast<uint32_t>(both), c1 = static_cast<uint32_t>(both >> 32);
      const uint32_t n = __builtin_amdgcn_readfirstlane(setid ? c1 : c0);
      no = __builtin_amdgcn_readfirstlane(setid ? c0 : c1);
      if (n >= nbar) break;
      __builtin_amdgcn_s_sleep(0);
    }
    // Balance the sets: wave w of each set shares a SIMD, and with equal
    // priorities the older wave (set 0) wins every issue conflict, so set 1
    // would finish its half of K several microseconds late. A wave whose set
    // is a stage or more behind the other set raises its priority.
    if (no > nbar)
      __builtin_amdgcn_s_setprio(2);
    else
      __builtin_amdgcn_s_setprio(0);
  }

  // One stage: stage st is read from slot `cur`, stage st + 2 is fetched
  // into `next`, the slot stage st - 1 just released. Every step issues the
  // same number of loads (past the set's last stage it re-reads that stage
  // into the released slot, which is never read again), so the wait is
  // constant.
  __device__ __forceinline__ void step(const uint8_t* cur, uint8_t* next, int st) {
    // this stage's blocks have landed once at most one newer stage of this
    // wave is in flight; the barrier publishes the set's blocks and frees
    // the slot of stage st - 1
    RRS_WAIT_VM(kDmaPerWave);
    set_barrier();
    const int nst = min(st + kRing - 1, st1 - 1);
    if (st < st1)
      compute(cur, next, st, nst);
    else
      issue(next, st);
  }

  // Steps s .. s + n - 1 (n <= 3) of the set, the ring slots passed as
  // distinct restrict pointers: inlined, they give every direct-to-LDS load
  // and every fragment read an alias scope, from which the compiler's wait
  // insertion tells which loads in flight a read depends on. Without scopes
  // it makes each fragment read wait for every load in flight, the one
  // fetched two stages ahead included.
  __device__ __forceinline__ void revolution(int s, int n, uint8_t* __restrict__ r0, uint8_t* __restrict__ r1,
                                             uint8_t* __restrict__ r2) {
    step(r0, r2, st0 + s);
    if (n > 1) step(r1, r0, st0 + s + 1);
    if (n > 2) step(r2, r1, st0 + s + 2);
  }

  template <int SET>
  __device__ void prologue() {  // the set's first two stages in flight
    issue(ring<SET, 0>(), st0);
    issue(ring<SET, 1>(), min(st0 + 1, st1 - 1));
  }

  template <int SET>
  __device__ void run(int nsteps) {
    uint8_t* r0 = ring<SET, 0>();
    uint8_t* r1 = ring<SET, 1>();
    uint8_t* r2 = ring<SET, 2>();
    int s = 0;
    for (; s + kRing <= nsteps; s += kRing) revolution(s, kRing, r0, r1, r2);
    if (s < nsteps) revolution(s, nsteps - s, r0, r1, r2);
    RRS_WAIT_VM(0);
  }
};

// SPG: MFMA k-steps per group when a group is a whole number of k-steps
// that divides a stage (the rescale then folds into the product loop), else 0
template <int KM, bool PARTIALS, int SPG>
__global__ void __launch_bounds__(kThreadsWG) gemm_kernel(GemmArgs a) {
  __shared__ float s_rat[kMaxKronK / kMinG];  // one per group (K <= kMaxKronK)
  __shared__ uint32_t s_bar[kSets];
  __shared__ float s_rs[kTT];       // dx[t] 2^18 / K of the tile's tokens
  __shared__ float s_dw[kTN];       // dw[n] of the tile's output channels
  __shared__ float s_send[kSets];   // each set's last group scale
  GemmCtx<KM, PARTIALS, SPG> c(a, s_rat);
  const int tid = threadIdx.x;
  const int set = __builtin_amdgcn_readfirstlane(tid / kThreads);  // uniform: stage bounds stay scalar
  const int stid = tid % kThreads;
  c.lane = stid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(stid >> 6);  // uniform, for scalar addressing
  c.wn = wave >> 1;
  c.wt = wave & 1;

  // XCD-aware tile order: consecutive workgroup ids land on different XCDs,
  // so give each XCD a contiguous run of the tile sequence; inside bands of
  // 4 output tiles the token tile runs fastest (neighbours share weights).
  // At M = 2048, N = 4096 an XCD's 32 tiles are then 4 weight tiles x 8
  // token tiles (4 MiB of codes, its L2's size) rather than 8 x 4 (5 MiB).
  const int ntiles = a.tiles_t * a.tiles_n;
  int wg = blockIdx.x;
  if ((ntiles & 7) == 0) wg = (wg & 7) * (ntiles >> 3) + (wg >> 3);
  const int band = 4 * a.tiles_t;
  const int bi = wg / band, bo = wg % band;
  const int bn = min(4, a.tiles_n - bi * 4);
  c.n0 = (bi * 4 + bo % bn) * kTN;
  c.t0 = (bo / bn) * kTT;

  c.Kb = a.K / 2;
  c.nstage = (a.K + 127) / 128;
  c.log2spg = a.log2G - Mma<KM>::kLog2K;  // MFMA k-steps per group
  c.ngroups = a.K >> a.log2G;
  // K halves. With two or more groups the halves meet on a group boundary:
  // half of the groups when a group spans whole stages (G >= 128; an odd
  // group count, possible for K = m 2^k, leaves the larger share to set 1),
  // else half of the stages. The partials dump splits K the same way.
  int half = (c.nstage + 1) / 2;
  if (c.ngroups > 1 && a.log2G >= 7) half = (c.ngroups / 2) << (a.log2G - 7);
  c.st0 = set == 0 ? 0 : half;
  c.st1 = set == 0 ? half : c.nstage;
  const int nsteps = max(half, c.nstage - half);  // both sets step in lockstep

  // DMA blocks of a stage: 1 KiB = 16 rows x 64 B; blocks 0..15 hold the
  // weight rows, 16..23 the activation rows; wave w moves blocks 6w..6w+5.
  // Lane i fills 16-byte slot i of the block: row 16b + i / 4 of the
  // matrix (clamped to it; clamped rows only feed outputs that are never
  // stored), 16-byte chunk (i & 3) ^ ((i >> 3) & 3) of that row's stage
  // piece. The XOR swizzle spreads the eight rows a fragment read serves at
  // once over all 32 LDS banks (rows 64 bytes apart would otherwise hit the
  // same banks every two rows). In the stored layout the stage pieces of
  // rows 2p and 2p + 1 form one 128-byte line, so the eight lanes of a row
  // pair load a whole line, and a stage advances by a line. With K = 64
  // (one stage of 32 bytes per row) the chunks past the row's codes re-read
  // its first bytes: in bounds, and never multiplied (only K codes are
  // used). Every other K is a multiple of 128. The tile's first rows
  // (n0 < N, t0 < M; both even) are the scalar bases; a lane's offset from
  // them stays below 256 rows, so 32 bits hold it.
  const size_t rs = codes_row_stride(a.K);  // tile bases: n0 and t0 are even rows
  c.wbase = a.wq + static_cast<size_t>(c.n0) * rs;
  c.xbase = a.xq + static_cast<size_t>(c.t0) * rs;
  c.wave6 = wave * GemmCtx<KM, PARTIALS, SPG>::kDmaPerWave;
#pragma unroll
  for (int d = 0; d < GemmCtx<KM, PARTIALS, SPG>::kDmaPerWave; ++d) {
    const int blk = c.wave6 + d;
    const bool wrows = blk < 16;
    const int base_row = wrows ? c.n0 : c.t0;
    const int row = min(base_row + (blk & 15) * 16 + (c.lane >> 2), (wrows ? a.N : a.M) - 1);
    int goff = ((c.lane & 3) ^ ((c.lane >> 3) & 3)) * 16;
    if (goff >= c.Kb) goff &= 15;
    const int rt = row - base_row;  // stored layout: row pairs share each stage's 128-byte line
    c.voff[d] = static_cast<uint32_t>(codes_offset(rt, goff, rs));
    c.lblk[d] = blk * 1024;
  }

  if (!PARTIALS) {
    // s_rat[g] = S[g-1] / S[g]: entering group g rescales the accumulator
    for (int g = tid; g < c.ngroups; g += kThreadsWG) s_rat[g] = g > 0 ? a.S[g - 1] / a.S[g] : 1.f;
    // epilogue operands, read now so their latency hides behind the main
    // loop (zero past the matrix edge; those outputs are never stored).
    // A set error word (a front end whose grid-wide wait gave up) makes
    // every output NaN.
    const bool poison = a.err != nullptr && *a.err != 0u;
    const float base = poison ? __builtin_nanf("") : a.ybase;
    if (tid < kTT) {
      const int t = c.t0 + tid;
      s_rs[tid] = t < a.M ? a.dx[t] * base : 0.f;
    } else if (tid < kTT + kTN) {
      const int n = c.n0 + tid - kTT;
      s_dw[tid - kTT] = n < a.N ? a.dw[n] : 0.f;
    } else if (tid < kTT + kTN + kSets) {
      const int st_end = tid - kTT - kTN == 0 ? half : c.nstage;  // end stage of set 0 / set 1
      s_send[tid - kTT - kTN] = a.S[((st_end * 128 > a.K ? a.K : st_end * 128) - 1) >> a.log2G];
    }
  }

  // the first stages' loads go out after the tables' reads above: loads
  // complete in order, so tables read after them would hold the first step
  // until the second stage has landed too
  if (set == 0) {
    c.template prologue<0>();
  } else if (c.st1 > c.st0) {
    c.template prologue<1>();
  }

  // fragment rows: row lane % BR of each BR-row block; the swizzle of the
  // row's 16-row DMA block is ((row & 15) >> 1) & 3
  constexpr int BR = Mma<KM>::BR;
  c.swz = (((c.lane & 15) >> 1) & 3) * 16;
  c.fW = (c.wn * 128 + (c.lane % BR)) * kRowB;
  c.fX = kWB + (c.wt * 64 + (c.lane % BR)) * kRowB;
  constexpr int TI = GemmCtx<KM, PARTIALS, SPG>::TI, TJ = GemmCtx<KM, PARTIALS, SPG>::TJ, NQ = Mma<KM>::NQ;

#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) c.acc[i][j] = Mma<KM>::zero();

  if (tid < kSets) s_bar[tid] = 0u;
  c.sbar = &s_bar[set];
  c.sbar2 = &s_bar[0];
  c.setid = set;
  __syncthreads();  // tables and counters published
  if (set == 0) {
    c.template run<0>(nsteps);
  } else if (c.st1 > c.st0) {
    c.template run<1>(nsteps);
  }  // else: no second half (K <= 128)
  const bool one_group = c.ngroups == 1;
  if (PARTIALS && !one_group) return;  // every group was dumped by its set

  // ---- combine the halves ------------------------------------------------
  // With two or more groups the halves meet on a group boundary (K / 2 is a
  // multiple of G), so each half is a finished sum over whole groups: set 1
  // parks its sum made absolute (times its last group's scale) and set 0
  // adds its own. With one group (G = K) the two halves are integer parts of
  // the same group partial: they are added exactly first and scaled once,
  // so a partial that cancels to zero stays exactly zero.
  const float s_end = PARTIALS ? 1.f : s_send[set];
  // park chunk of run q of block (i, j) of this wave (32 chunks of 1 KiB)
  auto chunk_of = [&](int i, int j, int q) { return wave * 32 + (i * TJ + j) * NQ + q; };
  __syncthreads();  // all rings idle: park set 1's 4 x 32 tiles of 1 KiB there
  if (set == 1) {
    // no second half (K <= 128): park zeros
    const float m1 = c.st1 > c.st0 ? (one_group ? 1.f : s_end) : 0.f;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          reinterpret_cast<v4f*>(park_chunk(chunk_of(i, j, q)))[c.lane] = Mma<KM>::quad(c.acc[i][j], q) * m1;
  }
  __syncthreads();
  // whole tile in range: Y leaves through the idle rings as token rows
  const bool rings = s_r01 == s_r00 + kStageB && s_r02 == s_r00 + 2 * kStageB && s_r10 == s_r00 + 3 * kStageB &&
                     s_r11 == s_r00 + 4 * kStageB && s_r12 == s_r00 + 5 * kStageB;  // back to back
  const bool full = rings && c.t0 + kTT <= a.M && c.n0 + kTN <= a.N && (a.N & 3) == 0;  // uniform
  if (set == 1 && (PARTIALS || !full)) return;
  const float m0 = one_group ? 1.f : s_end;  // set 0's own last group
  const float fin = one_group ? s_end : 1.f;
  if constexpr (PARTIALS) {
    // one group: the exact sum of the two integer halves is the partial
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          Mma<KM>::set_quad(c.acc[i][j], q, Mma<KM>::quad(c.acc[i][j], q) +
                                                reinterpret_cast<const v4f*>(park_chunk(chunk_of(i, j, q)))[c.lane]);
    c.dump(0);
    return;
  }

  // ---- epilogue: Y[t, n..n+3] = (both halves, absolute) 2^18 / K dx[t] dw[n]
  if (full) {
    // row t of the tile at t * kYRow bytes of the rings (16 bytes of
    // padding per row: a 16-lane group's rows fall in distinct banks)
    constexpr int kYRow = kTN * 4 + 16;
    static_assert(kTT * kYRow <= 6 * kStageB, "Y tile exceeds the rings");
    uint8_t* yl = s_r00;
    if (set == 0) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int tl = c.wt * 64 + j * BR + (c.lane % BR);
          const float rs = fin * s_rs[tl];
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const int nl = c.wn * 128 + i * BR + Mma<KM>::qrow(q, c.lane);
            const v4f dwv = *reinterpret_cast<const v4f*>(s_dw + nl);
            const v4f v = (Mma<KM>::quad(c.acc[i][j], q) * m0 +
                           reinterpret_cast<const v4f*>(park_chunk(chunk_of(i, j, q)))[c.lane]) * rs;
            Mma<KM>::set_quad(c.acc[i][j], q, v * dwv);
          }
        }
    }
    __syncthreads();  // every parked sum read before the rows overwrite them
    if (set == 0) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int tl = c.wt * 64 + j * BR + (c.lane % BR);
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const int nl = c.wn * 128 + i * BR + Mma<KM>::qrow(q, c.lane);
            *reinterpret_cast<v4f*>(yl + tl * kYRow + nl * 4) = Mma<KM>::quad(c.acc[i][j], q);
          }
        }
    }
    __syncthreads();
    // eight waves, one token row (1 KiB) per store
    const int gw = set * (kThreads / 64) + wave;
    // all of a wave's rows read first, then stored; the stores stream
    // (non-temporal): Y is not read back here, and 32 MiB of dirty lines
    // left in the caches would be written back under the next kernel
    constexpr int kWaves = kSets * (kThreads / 64);
    v4f rows[kTT / kWaves];
#pragma unroll
    for (int k = 0; k < kTT / kWaves; ++k)
      rows[k] = *reinterpret_cast<const v4f*>(yl + (gw + k * kWaves) * kYRow + c.lane * 16);
#pragma unroll
    for (int k = 0; k < kTT / kWaves; ++k)
      __builtin_nontemporal_store(rows[k], reinterpret_cast<v4f*>(a.Y + static_cast<size_t>(c.t0 + gw + k * kWaves) * a.N +
                                                                  c.n0 + c.lane * 4));
    return;
  }
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int tl = c.wt * 64 + j * BR + (c.lane % BR);  // token in the tile
      const int t = c.t0 + tl;
      const float rs = fin * s_rs[tl];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int nl = c.wn * 128 + i * BR + Mma<KM>::qrow(q, c.lane);  // first of 4 channels
        const int n = c.n0 + nl;
        const float4 dwv = *reinterpret_cast<const float4*>(s_dw + nl);
        const v4f v = (Mma<KM>::quad(c.acc[i][j], q) * m0 +
                       reinterpret_cast<const v4f*>(park_chunk(chunk_of(i, j, q)))[c.lane]) * rs;
        if (full) {
          *reinterpret_cast<float4*>(a.Y + static_cast<size_t>(t) * a.N + n) =
              make_float4(v[0] * dwv.x, v[1] * dwv.y, v[2] * dwv.z, v[3] * dwv.w);
        } else if (t < a.M && n < a.N) {
          float* y = a.Y + static_cast<size_t>(t) * a.N + n;
          y[0] = v[0] * dwv.x;
          if (n + 1 < a.N) y[1] = v[1] * dwv.y;
          if (n + 2 < a.N) y[2] = v[2] * dwv.z;
          if (n + 3 < a.N) y[3] = v[3] * dwv.w;
        }
      }
    }
}

template <int KM, int SPG>
hipError_t launch_km(const GemmArgs& a, bool partials, hipStream_t s) {
  const dim3 grid(a.tiles_t * a.tiles_n);
  if (partials)
    hipLaunchKernelGGL((gemm_kernel<KM, true, SPG>), grid, dim3(kThreadsWG), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<KM, false, SPG>), grid, dim3(kThreadsWG), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmCall& gc, hipStream_t s) {
  const int M = gc.M, N = gc.N, K = gc.K, G = gc.G;
  if (M == 0 || N == 0) return hipSuccess;
  // the partials come from the kernel that would write Y for this shape
  if (gemm_small_applies(M, K, N, G)) return launch_gemm_small(gc, s);
  GemmArgs a{};
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
  a.tiles_t = (M + kTT - 1) / kTT;
  a.tiles_n = (N + kTN - 1) / kTN;
  switch (G) {
    case 32: return launch_km<32, 1>(a, partials, s);
    case 64: return launch_km<64, 1>(a, partials, s);
    case 128: return launch_km<64, 2>(a, partials, s);
    default: return launch_km<64, 0>(a, partials, s);
  }
}

}  // namespace rrs
