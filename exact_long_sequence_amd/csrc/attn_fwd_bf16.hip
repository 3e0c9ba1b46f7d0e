// Fused, streamed exact attention forward for bf16 on gfx950 (CDNA4).
//
// Schedule (the memory-centric pipeline of "From Attention Graph to
// FlashAttention - A Memory-Centric Compilation Approach in AICF", section 3:
// load a Q tile, stream K/V tiles, partial scores, online softmax update,
// accumulate; no score / probability tensor ever leaves the chip):
//
//   one workgroup = one (batch, head, query tile of BM = 32 * WAVES rows)
//   Q tile:   HBM -> VGPR once, held as MFMA operands for the whole key loop
//   K/V tile: HBM/L2 -> LDS by direct-to-LDS loads into an LDS ring; later
//             tiles are in flight while the current one is computed
//   per wave (32 query rows), per K/V tile of BN keys:
//     S^T = K Q^T            bf16 MFMA 32x32x16, fp32 accumulate
//     online softmax          fp32; one v_exp_f32 per score, per-lane row stats
//     O^T += V^T P^T          bf16 MFMA 32x32x16, V fed by LDS transpose reads
//   epilogue: O = O^T / l, rounded to bf16 once.
//
// Computing the transposed score block S^T (keys down the MFMA rows, the
// wave's 32 queries across the 32 lanes) makes every softmax statistic
// lane-local: each lane owns one query, its 16 values per 32x32 block are that
// query's scores for 16 keys, and the other 16 keys of the block sit in the
// lane 32 apart.  The row max therefore needs one permlane32 swap per tile,
// and the rescale of the output accumulator is one multiply by a per-lane
// scalar.  The row sum is either lane-local too (two-element dot products,
// merged across the lane pair in the epilogue) or, at d = 128, formed on the
// matrix core (a 0/1 selection operand times P, next to the P x V MFMAs),
// which leaves two VALU operations per score (fma, exp) and one conversion
// per pair.  The accumulator O^T has the same
// lane = query layout, and the probabilities come out of the score MFMA
// already in the B-operand layout of the P x V MFMA.  This is the "parallel
// execution pattern for efficient softmax" of "I/O Analysis is All You Need:
// An I/O Analysis for Long-Sequence Attention" (abstract, optimisation 3)
// mapped onto 64-wide wavefronts.
//
// The shift of the exponentials is lazy.  Any shift gives the same softmax
// (it cancels between numerator and denominator), so the shift is taken from
// the first key tile's row maxima and moved again only when a tile's row sum
// shows a probability above 2^16 (by that sum's power of two, rescaling the
// running output and row sum).  The per-tile row maximum is not needed on the
// common path.  A VALU row sum is tested before the tile's P x V (the tile is
// recomputed after moving the shift).  A matrix-core row sum is known one
// MFMA phase after its P, so the test comes after the tile's P x V; if that
// sum exceeds 2^64 (a probability that large times |V| could have overflowed
// the fp32 accumulator) or is not finite (an exp2 overflowed), the workgroup
// computes its rows again with the shift checked before every tile.
//
// Two loop forms share the per-tile building blocks (selected per head size
// at the bottom of this file):
//  * ping-pong (default): eight waves in two groups of four, one wave of each
//    group per SIMD; barriers offset the groups by half a tile, so on every
//    SIMD one group issues its MFMA stream while the other runs the softmax;
//  * sequential: four waves, each running S, softmax, O per tile in turn over
//    an N-stage LDS ring; the overlap of MFMA with VALU then comes only from
//    the other workgroup's waves on the same SIMD.
// Both realise the three-level overlap of the I/O analysis (optimisation 2):
// HBM/L2 -> LDS by DMA of later tiles, LDS -> VGPR operand reads ahead of the
// MFMAs that use them, and MFMA under the VALU softmax.

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace attnio {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTauLog2 = 8.0f;        // shift moves when a row maximum exceeds it by 2^8
constexpr float kLazySumMax = 65536.f;  // a tile row sum above this moves the shift
// A matrix-core row sum is tested after the tile's P x V is already in the
// fp32 accumulator.  Every partial sum of that product is bounded by
// (tile row sum) * max|V|, so a tile whose row sum stays at or below 2^64
// cannot have overflowed it while max|V| < 2^63; a larger sum (finite or not)
// sends the workgroup to the safe pass.  Testing only for a non-finite sum
// would miss probabilities up to 2^128, finite in bf16 and fp32, whose
// products with |V| > 1 overflow.
constexpr float kSafeSumMax = 0x1p64f;

// Where the row sums of P are formed is a property of each compiled tiling
// (Tiling::rowsum_mfma below): on the matrix core (a 0/1 selection operand
// times P, next to the P x V MFMAs, one tile late) or on the VALU (two-element
// dot products, in the softmax).  The matrix-core form takes half a VALU
// operation per score off the softmax but needs 4 + 4 QB more registers.

// Shape of one compiled tiling.  QB: 32-row query blocks per wave (a wave
// owns 32 QB queries; each K or V operand read from LDS feeds QB MFMAs).
template <int D, int BN, int WAVES, int NSTAGES, int QB = 1>
struct Cfg {
  static constexpr int BM = 32 * WAVES * QB;              // query rows per workgroup
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CHUNKS = ROW_BYTES / 16;          // 16-byte chunks per row
  static constexpr int ROWS_PER_256 = 256 / ROW_BYTES;   // rows sharing one 256 B bank line
  static constexpr int TILE_BYTES = BN * ROW_BYTES;      // one K or one V tile
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;     // K + V
  static constexpr int STAGES = NSTAGES;                 // (K, V) tile pairs in the LDS ring
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  // the epilogue stages every output row of the workgroup in LDS
  static constexpr int OUT_BYTES = BM * ROW_BYTES;
  static constexpr int LDS_ALLOC = LDS_BYTES > OUT_BYTES ? LDS_BYTES : OUT_BYTES;
  static_assert(BN % 32 == 0 && D % 32 == 0, "MFMA blocking");
  static_assert(LDS_ALLOC + 16 <= 160 * 1024, "gfx950 LDS is 160 KiB per CU");
};

// XOR swizzles of the 16-byte chunk index inside an LDS row.  K rows are read
// 16 bytes per lane by 32 consecutive rows; V rows are read 8 bytes per lane by
// the transpose read, 4 rows x 4 chunks per 32 lanes.  Both keep every group of
// lanes that the LDS serves together on distinct banks (measured: no bank
// conflicts).
template <class C>
__device__ __forceinline__ int swz_k(int row) {
  return (row / C::ROWS_PER_256) % C::CHUNKS;
}
template <class C>
__device__ __forceinline__ int swz_v(int row) {
  return (4 * ((row / C::ROWS_PER_256) % 4)) % C::CHUNKS;
}

// v_permlane32_swap with both operands = x: lanes 0-31 get (own, lane+32),
// lanes 32-63 get (lane-32, own).  Either way the pair is {own, partner}.
__device__ __forceinline__ u32x2 swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  u32x2 out = {r[0], r[1]};
  return out;
}

// One direct-to-LDS load of 16 bytes per lane: lane i of the wave writes LDS
// bytes [lds + 16 i, lds + 16 i + 16) with the 16 bytes at gbase + voff.  It is
// issued as inline assembly so that the compiler does not treat it as an LDS
// store it must wait for before every LDS read of the other stages: completion
// is awaited explicitly (s_waitcnt vmcnt) before the workgroup barrier that
// hands a stage over.  M0 carries the wave-uniform LDS address.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(gbase) : "memory");
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Debug build (ATTNIO_DEBUG_POISON=1): every K/V buffer of the LDS ring is
// filled with bf16 NaNs as soon as the ring protocol lets it be overwritten,
// before the DMA that refills it, so that a wave reading a buffer outside the
// half steps the protocol gives it turns the output into NaNs.  Off in the
// product build.
#ifndef ATTNIO_DEBUG_POISON
#define ATTNIO_DEBUG_POISON 0
#endif
constexpr bool kPoison = ATTNIO_DEBUG_POISON != 0;

// NaN-fill `bytes` of LDS from byte address `lds` by `nthreads` threads
// (thread index `t` among them), then wait for the writes to land so that a
// DMA issued next by the same wave cannot be overtaken by them.
__device__ __forceinline__ void poison_lds(uint32_t lds, int bytes, int nthreads, int t) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  for (int o = t * 16; o < bytes; o += nthreads * 16)
    *(u32x4_t __attribute__((address_space(3)))*)(uintptr_t)(lds + (uint32_t)o) = nan4;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// wait until at most N tile DMAs of this wave are still in flight
template <int N>
__device__ __forceinline__ void wait_dma_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ----------------------------------------------------------------------------
// Per-tile building blocks, for one wave and its 32 query rows (lane (h, c)
// owns query c).  They are force-inlined so that each loop form can place
// them freely.
// ----------------------------------------------------------------------------

// LDS operands are read this many MFMAs ahead of their use.  One wave per SIMD
// issues the whole MFMA chain of a phase, so the LDS latency must be covered by
// its own earlier MFMAs; measured on MI355X, a distance of 2 or more keeps a
// lone 32x32x16 chain at its full rate of one MFMA per 32 cycles even with
// 1 KiB of LDS reads per MFMA, while reading 1-2 ahead (what the compiler
// schedules on its own) costs about 40%.
// Read-ahead distance in operand reads: 4 MFMAs at QB = 1; at QB = 2 each read
// feeds two MFMAs, so 2 reads cover the same distance.
template <int QB>
constexpr int read_ahead() { return QB == 1 ? 4 : 2; }

// One MFMA phase as a single stream of MFMAs, for the wave's QB query blocks:
//   DO_PV: O^T (D x 32 queries) += V_tile^T P^T   ((BN/16) x (D/32) V operands)
//          and, with DO_RS, the tile's row sums of P (BN/16 MFMAs, 16x16x32)
//   DO_QK: S^T (BN keys x 32 queries) = K_tile Q^T ((D/16) x (BN/32) K operands)
// in that order.  Each operand read from LDS feeds QB MFMAs (one per query
// block, different B operands).  Each group of QB * D/32 (resp. QB * BN/32)
// consecutive MFMAs writes independent accumulators.
//
// Row sums on the matrix core.  The 16x16x32 instruction reads a B operand of
// 32 k x 16 columns with lane 16g + j holding k = 8g .. 8g + 7 of column j, so
// the P operand of one 16-key step (lane 32h + c: keys 8h .. 8h + 7 of query
// c) is, to it, column j = c % 16 with lane groups g = 2h + c / 16.  The
// selection operand `sel` has rows 0 and 8 equal to 1 on the groups of even g
// (query j) and rows 4 and 12 equal to 1 on the groups of odd g (query
// j + 16), all else 0.  Output row 4g' of column j lands in lane 16g' + j, so
// element 0 of every lane's 4-float result is the sum of its own query's 16
// probabilities of the step, over both halves of the wave.  These are the same
// bf16-rounded values that multiply V, so l matches the numerator exactly in
// what it sums.
//
// The V operand uses the transpose read: lane 16g + 4j + q supplies V row
// (16 st + 8u + 4h + j), columns 32 db + 16 (g % 2) + 4 q .. +3, and lane
// 16g + i receives column 32 db + 16 (g % 2) + i of those four rows, which is
// the A-operand layout (d down the rows, keys along k).  The key order inside
// each 16-key step matches the order in which the S^T accumulator holds the
// same keys, so P needs no register shuffle.  The K operand is one 16-byte
// read of row kb*32 + c.  A scheduling barrier after every operand's MFMAs
// pins the read-ahead distance (counted in operand reads).
template <class C, int D, int BN, int QB, int R, bool DO_PV, bool DO_QK, bool DO_RS>
__device__ __forceinline__ void mfma_stream(const char LDS_AS* vl, const bf16x8 (&pb)[QB][BN / 16],
                                            f32x16 (&acc)[QB][D / 32], const bf16x8& sel,
                                            f32x4 (&lsum)[QB], const char LDS_AS* kl,
                                            const bf16x8 (&qf)[QB][D / 16], f32x16 (&s)[QB][BN / 32],
                                            int lane) {
  const int half = lane / 32, col = lane % 32;
  const int g = lane / 16;
  const int jr = (lane % 16) / 4;
  const int qq = lane % 4;
  constexpr int NPV = DO_PV ? (BN / 16) * (D / 32) : 0;
  constexpr int NQK = DO_QK ? (D / 16) * (BN / 32) : 0;
  constexpr int NM = NPV + NQK;
  // Every operand address is the lane's base address of this tile XOR a
  // compile-time constant, plus an immediate row offset.  The swizzles are
  // XORs on the chunk index with a period that divides the row steps, and the
  // tile bases are multiples of the tile size, so
  //   K: row kb*32 + col, chunk (2 ks + half) ^ swz_k(col)
  //      = (kbase ^ 32 ks) + kb * 32 rows,
  //   V: row st*16 + u*8 + 4 half + jr, chunk (2 db + ...) ^ swz_v(4 half + jr)
  //      = (vbase ^ 64 db) + (st*16 + u*8) rows.
  // Only the two bases are live across the phase: the empty asm hides their
  // value, so the compiler forms each offset where it is used instead of
  // keeping one register per distinct offset for the whole key loop.
  static_assert(32 % (C::ROWS_PER_256 * C::CHUNKS) == 0 && 8 % (4 * C::ROWS_PER_256) == 0,
                "swizzle periods must divide the operand row steps");
  uint32_t kbase =
      (uint32_t)(uintptr_t)kl + (uint32_t)(col * C::ROW_BYTES + ((half ^ swz_k<C>(col)) * 16));
  const int vrow = half * 4 + jr;
  uint32_t vbase = (uint32_t)(uintptr_t)vl +
                         (uint32_t)(vrow * C::ROW_BYTES + ((((g % 2) * 2 + qq / 2) ^ swz_v<C>(vrow)) * 16) +
                                    (qq % 2) * 8);
  asm volatile("" : "+v"(kbase), "+v"(vbase));
  auto read = [&](int m) __attribute__((always_inline)) {
    bf16x8 a;
    if (m < NPV) {
      const int st = m / (D / 32), db = m % (D / 32);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t addr = (vbase ^ (uint32_t)(db * 64)) + (uint32_t)((st * 16 + u * 8) * C::ROW_BYTES);
        const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS*)(uintptr_t)addr);
        const bf16x4 vb = __builtin_bit_cast(bf16x4, v4);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[u * 4 + e] = vb[e];
      }
    } else {
      const int mq = m - NPV;
      const int ks = mq / (BN / 32), kb = mq % (BN / 32);
      const uint32_t addr = (kbase ^ (uint32_t)(ks * 32)) + (uint32_t)(kb * 32 * C::ROW_BYTES);
      a = *(const bf16x8 LDS_AS*)(uintptr_t)addr;
    }
    return a;
  };
  bf16x8 ring[R + 1];
#pragma unroll
  for (int m = 0; m < R && m < NM; ++m) ring[m] = read(m);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    if (m + R < NM) ring[(m + R) % (R + 1)] = read(m + R);
    const bf16x8 a = ring[m % (R + 1)];
    if (m < NPV) {
      const int st = m / (D / 32), db = m % (D / 32);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb][st], acc[qb][db], 0, 0, 0);
      if (DO_RS && db == D / 32 - 1) {
        const f32x4 zero4 = {};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          lsum[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb[qb][st], st == 0 ? zero4 : lsum[qb],
                                                             0, 0, 0);
      }
    } else {
      const int mq = m - NPV;
      const int ks = mq / (BN / 32), kb = mq % (BN / 32);
      const f32x16 zero = {};
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ks], ks == 0 ? zero : s[qb][kb], 0,
                                                            0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The MFMA phase of the split form (two query blocks per wave, ping-pong, row
// sums on the matrix core): S^T(t) of both blocks first (each K operand read
// feeds two MFMAs), then the row-sum MFMAs of P(t-1) for both blocks, then
// the P x V MFMAs of tile t-1 with valu(mp) called after the two MFMAs of V
// operand mp.  The MFMA wave runs its block-0 softmax of tile t there: VALU
// work between a wave's own MFMAs runs under them, while the same work in the
// softmax wave of the SIMD would lengthen the half step.  Operand addressing
// and read-ahead as in mfma_stream.
template <class C, int D, int BN, int R, class VALU>
__device__ __forceinline__ void mfma_stream_split(const char LDS_AS* vl, const bf16x8 (&pb)[2][BN / 16],
                                                  f32x16 (&acc)[2][D / 32], const bf16x8& sel,
                                                  f32x4 (&lsum)[2], const char LDS_AS* kl,
                                                  const bf16x8 (&qf)[2][D / 16], f32x16 (&s)[2][BN / 32],
                                                  int lane, VALU&& valu) {
  const int half = lane / 32, col = lane % 32;
  const int g = lane / 16;
  const int jr = (lane % 16) / 4;
  const int qq = lane % 4;
  constexpr int NQK = (D / 16) * (BN / 32);
  constexpr int NPV = (BN / 16) * (D / 32);
  constexpr int NM = NQK + NPV;
  uint32_t kbase =
      (uint32_t)(uintptr_t)kl + (uint32_t)(col * C::ROW_BYTES + ((half ^ swz_k<C>(col)) * 16));
  const int vrow = half * 4 + jr;
  uint32_t vbase = (uint32_t)(uintptr_t)vl +
                   (uint32_t)(vrow * C::ROW_BYTES + ((((g % 2) * 2 + qq / 2) ^ swz_v<C>(vrow)) * 16) +
                              (qq % 2) * 8);
  asm volatile("" : "+v"(kbase), "+v"(vbase));
  auto read = [&](int m) __attribute__((always_inline)) {
    bf16x8 a;
    if (m < NQK) {
      const int ks = m / (BN / 32), kb = m % (BN / 32);
      const uint32_t addr = (kbase ^ (uint32_t)(ks * 32)) + (uint32_t)(kb * 32 * C::ROW_BYTES);
      a = *(const bf16x8 LDS_AS*)(uintptr_t)addr;
    } else {
      const int mp = m - NQK, st = mp / (D / 32), db = mp % (D / 32);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t addr = (vbase ^ (uint32_t)(db * 64)) + (uint32_t)((st * 16 + u * 8) * C::ROW_BYTES);
        const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS*)(uintptr_t)addr);
        const bf16x4 vb = __builtin_bit_cast(bf16x4, v4);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[u * 4 + e] = vb[e];
      }
    }
    return a;
  };
  bf16x8 ring[R + 1];
#pragma unroll
  for (int m = 0; m < R && m < NM; ++m) ring[m] = read(m);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    if (m + R < NM) ring[(m + R) % (R + 1)] = read(m + R);
    const bf16x8 a = ring[m % (R + 1)];
    if (m < NQK) {
      const int ks = m / (BN / 32), kb = m % (BN / 32);
      const f32x16 zero = {};
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ks], ks == 0 ? zero : s[qb][kb], 0, 0, 0);
      if (m == NQK - 1) {
        const f32x4 zero4 = {};
#pragma unroll
        for (int st = 0; st < BN / 16; ++st)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            lsum[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb[qb][st], st == 0 ? zero4 : lsum[qb],
                                                               0, 0, 0);
      }
    } else {
      const int mp = m - NQK, st = mp / (D / 32), db = mp % (D / 32);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb][st], acc[qb][db], 0, 0, 0);
      valu(mp);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Masked scores become -inf (or +inf when the scale is negative, so that they
// still map to exp2(-inf) = 0).  Only diagonal and padding tiles call this.
template <int BN, bool CAUSAL, bool NEG>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[BN / 32], int j0, int L, int qrow, int half) {
#pragma unroll
  for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + kb * 32 + (r / 4) * 8 + half * 4 + (r % 4);
      bool ok = key < L;
      if (CAUSAL) ok = ok && (key <= qrow);
      s[kb][r] = ok ? s[kb][r] : (NEG ? INFINITY : -INFINITY);
    }
}

// Row extreme of the raw scores (max, or min for a negative scale), over the
// lane's 16 values per block and the partner lane 32 apart.  Four independent
// chains: a single chain of dependent max operations is bound by VALU latency.
template <int BN, bool NEG>
__device__ __forceinline__ float row_extreme(const f32x16 (&s)[BN / 32]) {
  float m4[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) m4[k] = s[0][k];
#pragma unroll
  for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
    for (int r = (kb == 0 ? 4 : 0); r < 16; ++r)
      m4[r % 4] = NEG ? fminf(m4[r % 4], s[kb][r]) : fmaxf(m4[r % 4], s[kb][r]);
  const float mx = NEG ? fminf(fminf(m4[0], m4[1]), fminf(m4[2], m4[3]))
                       : fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
  const u32x2 pr = swap_halves(mx);
  return NEG ? fminf(__uint_as_float(pr[0]), __uint_as_float(pr[1]))
             : fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

// P = exp2(S*c - m) rounded to bf16 and packed as the B operands of the P x V
// MFMA (operand i covers keys 16 i .. 16 i + 15 of the tile).  Two VALU
// operations per score (fma, exp) plus one conversion per pair.  With
// VALU_SUM, also returns this lane's sum of the rounded values over the tile
// (its 16 keys of each 32; four independent chains of two-element dot
// products); otherwise the row sums are formed on the matrix core in the next
// MFMA phase and 0 is returned.
template <int BN, bool VALU_SUM>
__device__ __forceinline__ float softmax_p(const f32x16 (&s)[BN / 32], float c, float m_use,
                                           bf16x8 (&pb)[BN / 16]) {
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      bf16x8 p;
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8)
        p[t8] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][sp * 8 + t8], c, -m_use));
      if (VALU_SUM) {
#pragma unroll
        for (int t2 = 0; t2 < 4; ++t2) {
          const bf16x2 pp = {p[2 * t2], p[2 * t2 + 1]};
          l4[t2] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l4[t2], false);
        }
      }
      pb[kb * 2 + sp] = p;
    }
  return (l4[0] + l4[1]) + (l4[2] + l4[3]);
}

// ----------------------------------------------------------------------------
// The kernel.
// ----------------------------------------------------------------------------

// One compiled tiling: head size, keys per K/V tile, waves per workgroup,
// 32-row query blocks per wave, LDS stages of the sequential form, loop form,
// workgroups resident per CU (the residency the register budget and the
// causal key order assume), causal key snake, row sums on the matrix core.
template <int D_, int BN_, int WAVES_, int QB_, int STAGES_, bool PINGPONG_, int WG_PER_CU_, bool SNAKE_,
          bool RS_MFMA_, bool RS_IN_STREAM_ = false, bool SPLIT_ = false, bool MF16_ = false>
struct Variant {
  static constexpr int D = D_, BN = BN_, WAVES = WAVES_, QB = QB_;
  // every product on the 16x16x32 MFMA (attn_fwd_bf16_mf16_kernel below)
  static constexpr bool MF16 = MF16_;
  // split softmax: with two query blocks per wave in the ping-pong form, the
  // MFMA wave computes its block-0 softmax inside its own MFMA phase (see
  // mfma_stream_split) and the softmax half step keeps block 1
  static constexpr bool SPLIT = SPLIT_ && PINGPONG_ && QB_ == 2 && RS_MFMA_ && RS_IN_STREAM_;
  static constexpr int STAGES = PINGPONG_ ? 2 : STAGES_;
  static constexpr bool PINGPONG = PINGPONG_, KEYS_SNAKE = SNAKE_, RS_MFMA = RS_MFMA_;
  // where the matrix-core row sums are issued in the ping-pong form: by the
  // MFMA wave, next to the P x V MFMAs of its phase, or (false) by the
  // softmax wave at the start of its half step, in the window where the MFMA
  // wave waits for its first LDS operands (the sequential form always puts
  // them in the P x V stream)
  static constexpr bool RS_IN_STREAM = RS_MFMA_ && (RS_IN_STREAM_ || !PINGPONG_);
  static constexpr int WG_PER_CU = WG_PER_CU_;
  using C = Cfg<D, BN, WAVES, STAGES, QB>;
};

template <class VT, bool CAUSAL, bool NEG_SCALE>
__global__ __launch_bounds__(64 * VT::WAVES, (VT::WAVES / 4) * VT::WG_PER_CU)
void attn_fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                          const __bf16* __restrict__ V, __bf16* __restrict__ O,
                          const int32_t* __restrict__ kv_len, float* __restrict__ lse, int H,
                          int N, float c, int n_qtiles) {
  constexpr int D = VT::D, BN = VT::BN, WAVES = VT::WAVES, QB = VT::QB, WG_PER_CU = VT::WG_PER_CU;
  constexpr bool PINGPONG = VT::PINGPONG, KEYS_SNAKE = VT::KEYS_SNAKE, RS_MFMA = VT::RS_MFMA;
  constexpr int R = read_ahead<QB>();
  using C = typename VT::C;
  static_assert(!PINGPONG || WAVES % 2 == 0, "ping-pong needs two equal wave groups");
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform
  const int lane = tid % 64;
  const int half = lane / 32;   // h
  const int col = lane % 32;    // c: the query of each block this lane owns

  // ---- XCD-aware work assignment: (batch*head, query tile) ----
  // Workgroups are dispatched round-robin over the 8 XCDs (block x runs on
  // XCD x % 8).  Every query tile of a head is given to one XCD, so the head's
  // K and V stream through that XCD's L2 once per resident generation of query
  // tiles.  When B*H is a multiple of 8, heads are dealt to XCDs round-robin
  // (head j to XCD j % 8), which also mixes the batches (and so the key-padding
  // lengths) evenly over the XCDs; otherwise each XCD takes a contiguous range.
  const int G = gridDim.x;
  const int x = blockIdx.x;
  const int xcd = x % 8, idx = x / 8;
  int bh, qt;
  if ((G / n_qtiles) % 8 == 0) {
    bh = xcd + 8 * (idx / n_qtiles);
    qt = idx % n_qtiles;
  } else {
    const int per = G / 8, rem = G % 8;
    const int logical = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    bh = logical / n_qtiles;
    qt = logical % n_qtiles;
  }
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest query tiles first
  const int b = bh / H;

  int L = N;
  if (kv_len != nullptr) {
    L = kv_len[b];
    L = L < 0 ? 0 : (L > N ? N : L);
  }
  L = __builtin_amdgcn_readfirstlane(L);
  const int q0 = qt * C::BM;
  int kend = L;
  if (CAUSAL) kend = min(kend, min(N, q0 + C::BM));
  kend = __builtin_amdgcn_readfirstlane(kend);
  const int ntiles = (kend + BN - 1) / BN;
  // Key order (online softmax does not depend on it).  Causal query tiles of
  // a head run on one XCD longest first, RESIDENT at a time; call each such
  // group a generation.  With KEYS_SNAKE, even generations walk their keys up
  // from key 0 and odd ones down from the diagonal, so each generation starts
  // on the keys the previous one ended on, which are still in L2; otherwise
  // all walk up.
  constexpr int RESIDENT = 32 * WG_PER_CU;  // workgroups resident on one XCD
  const bool keys_down = CAUSAL && KEYS_SNAKE && (((n_qtiles - 1 - qt) / RESIDENT) & 1);
  auto ktile = [&](int t) __attribute__((always_inline)) { return keys_down ? ntiles - 1 - t : t; };

  const size_t slice = (size_t)bh * N * D;
  const __bf16* Qs = Q + slice;
  const char* Kg = (const char*)(K + slice);
  const char* Vg = (const char*)(V + slice);
  __bf16* Os = O + slice;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

  // DMA of K or V tile t into LDS byte offset `dst` of the ring, by NW waves
  // starting at wave W0 (each issues TILE_BYTES / (1 KiB * NW) loads).  Load i
  // of a lane fills LDS bytes pos = (i*64*NW + 64*(wave-W0) + lane)*16 of the
  // tile, i.e. row pos / ROW_BYTES and physical chunk (pos % ROW_BYTES) / 16;
  // the lane fetches the logical chunk that the swizzle stores there.  Load i
  // covers the rows of load 0 moved down by i * RSTEP, a multiple of the
  // swizzle period, so its global offset is load 0's plus i * 16 * 64 * NW:
  // on full tiles that step goes into the scalar base and one VGPR offset per
  // lane serves every load.  A tail tile clamps rows >= kend to kend - 1
  // (masked keys: they only need to be finite memory inside the tensor; keys
  // >= kv_len are never read).
  auto issue = [&](auto nw_tag, int w0, const char* gsrc, bool is_v, int t, uint32_t dst)
      __attribute__((always_inline)) {
    constexpr int NW = decltype(nw_tag)::value;
    constexpr int TH = 64 * NW;
    constexpr int NLOADS = C::TILE_BYTES / 16 / TH;
    constexpr int RSTEP = TH * 16 / C::ROW_BYTES;  // rows between loads i and i + 1
    static_assert(C::TILE_BYTES % (16 * TH) == 0, "tile must split evenly over the issuing waves");
    static_assert((TH * 16) % C::ROW_BYTES == 0 && RSTEP % 16 == 0,
                  "loads must step by whole rows and whole swizzle periods");
    const int j0 = ktile(t) * BN;
    const char* gt = gsrc + (size_t)j0 * C::ROW_BYTES;
    int last = kend - 1 - j0;  // last valid row of this tile
    const int wl = wave - w0;
    const int pos0 = (wl * 64 + lane) * 16;
    const int row0 = pos0 / C::ROW_BYTES;
    const int lch = ((pos0 % C::ROW_BYTES) / 16) ^ (is_v ? swz_v<C>(row0) : swz_k<C>(row0));
    const uint32_t l0 = lds_base + dst + (uint32_t)(wl * 64 * 16);
    if (last >= BN - 1) {
      uint32_t o = (uint32_t)(row0 * C::ROW_BYTES + lch * 16);
      asm volatile("" : "+v"(o));  // one live offset; each load adds its step
#pragma unroll
      for (int i = 0; i < NLOADS; ++i)
        dma16(gt, o + (uint32_t)(i * TH * 16), __builtin_amdgcn_readfirstlane(l0 + (uint32_t)(i * TH * 16)));
    } else {
      // hide `last` (loop-invariant for the one tail tile) and the lane's row
      // and chunk so that the clamped offsets are formed here rather than
      // kept live across the key loop
      last = __builtin_amdgcn_readfirstlane(last);
      int r0 = row0, c16 = lch * 16;
      asm volatile("" : "+s"(last), "+v"(r0), "+v"(c16));
#pragma unroll
      for (int i = 0; i < NLOADS; ++i) {
        // min(row0 + i*RSTEP, last) = min(row0, last - i*RSTEP) + i*RSTEP
        const int lim = last - i * RSTEP;
        const int grow = r0 < lim ? r0 : lim;
        const uint32_t o = (uint32_t)(grow * C::ROW_BYTES + c16) + (uint32_t)(i * TH * 16);
        dma16(gt, o, __builtin_amdgcn_readfirstlane(l0 + (uint32_t)(i * TH * 16)));
      }
    }
  };
  const int qw0 = q0 + wave * 32 * QB;  // first query row of this wave; block qb: qw0 + 32 qb + col
  auto need_mask = [&](int t) __attribute__((always_inline)) {
    const int j0 = ktile(t) * BN;
    return (j0 + BN > L) || (CAUSAL && (j0 + BN - 1 > qw0));
  };

  // ---- Q fragments (B operand of S^T = K Q^T): lane (h, c) holds
  //      Q[qw0 + 32 qb + c][16*ks + 8*h .. +7] for every qb, ks ----
  // Q is read once, so its loads are non-temporal: they do not push out of L2
  // the K/V tiles that the other query tiles of the head on this XCD are about
  // to read.  O, written once, leaves the same way from the epilogue (in whole
  // lines: a non-temporal store of 8-byte pieces would leave L2 unable to
  // merge them, measured at 4.8x the bytes written).
  bf16x8 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = qw0 + 32 * qb + col;
    const int qrow_c = qrow < N ? qrow : N - 1;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[qb][ks] = __builtin_nontemporal_load((const bf16x8*)(Qs + (size_t)qrow_c * D + ks * 16 + half * 8));
  }
  // Q operands must have arrived before the key loop: an empty asm that reads
  // them makes the compiler wait for their loads here, so that no wait for a
  // load of its own lands inside the loop, where the only vector-memory
  // operations are the tile DMAs (awaited explicitly before each barrier).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(qf[qb][ks]));

  // Selection operand of the row-sum MFMA (see mfma_stream): lane 16g + i
  // holds row i, k-group g of a 16 x 32 matrix that is 1 on rows 0 and 8 for
  // even g and on rows 4 and 12 for odd g.
  bf16x8 sel;
  {
    const int i = lane % 16, g = lane / 16;
    const bool one = (g % 2 == 0) ? (i == 0 || i == 8) : (i == 4 || i == 12);
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[e] = (__bf16)(one ? 1.f : 0.f);
  }

  // Row sums on the matrix core are issued either in the P x V stream of the
  // MFMA phase or, in the ping-pong form, by the softmax wave at the start of
  // its half step, while the MFMA wave of the SIMD waits for the first LDS
  // operands of the freshly published tiles (the matrix pipe is otherwise
  // idle there, as long as that wait outlasts the row-sum MFMAs).
  constexpr bool RS_STREAM = VT::RS_IN_STREAM;
  f32x16 acc[QB][D / 32];
  float m_run[QB];   // running shift per query block, exp2 domain (scores * c)
  float l_run[QB];   // row sum of this lane's query: whole (RS_MFMA), else its 16 keys of each 32
  f32x4 lsum[QB];    // element 0: this query's sum of the last tile's P (matrix core)
  bool bad;          // a tile's row sum exceeded the bound the accumulator can take

  f32x16 s0[QB][BN / 32];
  bf16x8 pb[QB][BN / 16];

  // Move the shift of query block qb to the current row extremes of s0 where
  // a row's extreme exceeds it by more than 2^TAU, rescaling acc and l.  The
  // rescales here and in fold_sum are per-lane branches (executed under the
  // lane mask, skipped when no lane needs them): as wave-uniform branches the
  // compiler gave the two paths different accumulator registers and copied
  // all of them on the common path of every tile.
  auto update_shift = [&](int qb) __attribute__((always_inline)) {
    const float m_tile = row_extreme<BN, NEG_SCALE>(s0[qb]) * c;
    if (m_tile > m_run[qb] + kTauLog2) {
      const float m_new = fmaxf(m_run[qb], m_tile);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
      l_run[qb] *= alpha;
    }
  };
  // Row sums of the P held in pb (16x16x32 MFMAs with the selection operand).
  auto rowsum_mfma = [&]() __attribute__((always_inline)) {
    const f32x4 zero4 = {};
#pragma unroll
    for (int st = 0; st < BN / 16; ++st)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        lsum[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb[qb][st], st == 0 ? zero4 : lsum[qb], 0, 0, 0);
  };
  // Fold in the row sums of the previous tile (formed after its P x V).  The
  // shift is lazy: it is taken from the first tile that shows a row a visible
  // key and afterwards moved only when a tile's row sum shows a probability
  // above 2^16, by the integer part of that sum's log2 (an exact power-of-two
  // rescale of acc and l).  Any shift gives the same softmax (it cancels
  // between numerator and denominator), so the result is exact up to
  // rounding.  The test comes one tile late, after the tile's P x V: a sum
  // above kSafeSumMax (or not finite: some exp2 overflowed) means the
  // accumulator may already hold an overflowed product, and the workgroup then
  // recomputes its rows with the shift checked before every tile (the safe
  // pass below).
  auto fold_one = [&](int qb) __attribute__((always_inline)) {
    const float rs = lsum[qb][0];
    bad = bad || !(rs <= kSafeSumMax);
    l_run[qb] += rs;
    if (rs > kLazySumMax && rs <= kSafeSumMax) {
      const float mv = floorf(__builtin_amdgcn_logf(rs));
      const float alpha = __builtin_amdgcn_exp2f(-mv);
      m_run[qb] += mv;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
      l_run[qb] *= alpha;
    }
  };
  auto fold_sum = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) fold_one(qb);
  };
  // VALU part of tile t: fold the previous tile's row sums, mask, shift (first
  // visible tile, or every tile in the safe pass), P(t).
  // With the VALU row sum the test needs no deferral: the tile's sum is known
  // before its P x V, and a tile whose sum exceeds 2^16 (or is not finite) is
  // recomputed after moving the shift to the tile's row maxima.
  auto softmax_tile = [&](int t, auto safe_tag) __attribute__((always_inline)) {
    constexpr bool SAFE = decltype(safe_tag)::value;
    if (RS_MFMA) fold_sum();
    const bool msk = need_mask(t);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (msk) mask_tile<BN, CAUSAL, NEG_SCALE>(s0[qb], ktile(t) * BN, L, qw0 + 32 * qb + col, half);
      if (RS_MFMA) {
        // per lane: the two lanes of a query (c, c + 32) share m_run, so the
        // permlane32 swap in row_extreme only pairs active lanes
        if (SAFE || m_run[qb] == -INFINITY) update_shift(qb);
        softmax_p<BN, false>(s0[qb], c, m_run[qb] == -INFINITY ? 0.f : m_run[qb], pb[qb]);
      } else {
        float lt = softmax_p<BN, true>(s0[qb], c, m_run[qb] == -INFINITY ? 0.f : m_run[qb], pb[qb]);
        if (__builtin_amdgcn_ballot_w64(!(lt <= kLazySumMax) || m_run[qb] == -INFINITY) != 0) {
          update_shift(qb);
          lt = softmax_p<BN, true>(s0[qb], c, m_run[qb] == -INFINITY ? 0.f : m_run[qb], pb[qb]);
        }
        l_run[qb] += lt;
      }
    }
  };

  // Split form, block 0 inside the MFMA phase of tile t: the fold of tile
  // t-1's row sums and the shift decisions of tile t, as in fold_one and
  // update_shift, except that acc[0] is still accumulating P(t-1) V(t-1)
  // there, so its rescale is recorded (a0, r0) and applied after the phase;
  // l and the shift change at once.
  auto split_head0 = [&](int t, auto safe_tag, float& a0, bool& r0) __attribute__((always_inline)) {
    constexpr bool SAFE = decltype(safe_tag)::value;
    const float rs = lsum[0][0];
    bad = bad || !(rs <= kSafeSumMax);
    l_run[0] += rs;
    if (rs > kLazySumMax && rs <= kSafeSumMax) {
      const float mv = floorf(__builtin_amdgcn_logf(rs));
      const float alpha = __builtin_amdgcn_exp2f(-mv);
      m_run[0] += mv;
      l_run[0] *= alpha;
      a0 *= alpha;
      r0 = true;
    }
    if (need_mask(t)) mask_tile<BN, CAUSAL, NEG_SCALE>(s0[0], ktile(t) * BN, L, qw0 + col, half);
    if (SAFE || m_run[0] == -INFINITY) {
      const float m_tile = row_extreme<BN, NEG_SCALE>(s0[0]) * c;
      if (m_tile > m_run[0] + kTauLog2) {
        const float m_new = fmaxf(m_run[0], m_tile);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[0] - m_new);
        m_run[0] = m_new;
        l_run[0] *= alpha;
        a0 *= alpha;
        r0 = true;
      }
    }
  };
  // P operand i of block 0 (keys 16 i .. 16 i + 15), as softmax_p packs it
  auto split_pack0 = [&](int i, bf16x8 (&pbn)[BN / 16]) __attribute__((always_inline)) {
    const float m0 = m_run[0] == -INFINITY ? 0.f : m_run[0];
    const int kb = i / 2, sp = i % 2;
    bf16x8 p;
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8)
      p[t8] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s0[0][kb][sp * 8 + t8], c, -m0));
    pbn[i] = p;
  };
  // the softmax half step of the split form: block 1 only
  auto softmax_block1 = [&](int t, auto safe_tag) __attribute__((always_inline)) {
    constexpr bool SAFE = decltype(safe_tag)::value;
    fold_one(1);
    if (need_mask(t)) mask_tile<BN, CAUSAL, NEG_SCALE>(s0[1], ktile(t) * BN, L, qw0 + 32 + col, half);
    if (SAFE || m_run[1] == -INFINITY) update_shift(1);
    softmax_p<BN, false>(s0[1], c, m_run[1] == -INFINITY ? 0.f : m_run[1], pb[1]);
  };

  // One pass over the keys.  The safe pass is a second, straight-line copy
  // (a loop around one copy would carry every accumulator across its back
  // edge and push the register count past the two-waves-per-SIMD limit).
  auto run_pass = [&](auto safe_tag) __attribute__((always_inline)) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][db][r] = 0.f;
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) lsum[qb][r] = 0.f;
  }
  bad = false;

  if constexpr (PINGPONG) {
    // Ping-pong.  The waves split into two groups of WAVES/2; waves w and
    // w + WAVES/2 share a SIMD.  Every wave runs the same straight loop
    // MFMA(t), barrier, VALU(t), barrier, with
    //   MFMA(t) = O += V(t-1)^T P(t-1)^T (t >= 1), then S(t) = K(t) Q^T (t < ntiles)
    //   VALU(t) = [row sums of P(t-1) on the matrix core,] softmax of tile t;
    // group 1 passes one extra barrier first, which shifts it half a tile
    // behind group 0 (a barrier counts arrivals, not program locations), so on
    // each SIMD one group's MFMA stream runs under the other's softmax.  The
    // MFMA phase runs at raised wave priority.  K and V tiles have two LDS
    // buffers each.  Global half-step h = 2t starts group 0's MFMA(t) and
    // group 1's VALU(t-1); there group 1 issues the DMA of K(t+1) and waits
    // for it at the end of h = 2t + 1.  Group 0 issues the DMA of V(t) at the
    // start of its VALU(t) (h = 2t + 1: V(t-2)'s buffer was last read in
    // h = 2t - 1) and waits for it at the end of that half step.  The DMAs are
    // issued by softmax waves only (a wave stalls while the CU's load path
    // drains its DMAs, which the MFMA stream cannot absorb), and split over
    // both groups so that each softmax half step carries half of them.
    const int grp = wave / (WAVES / 2);  // wave-uniform
    auto kd = [&](int t) __attribute__((always_inline)) { return (uint32_t)((t & 1) * C::TILE_BYTES); };
    auto vd = [&](int t) __attribute__((always_inline)) { return (uint32_t)((2 + (t & 1)) * C::TILE_BYTES); };
    std::integral_constant<int, WAVES / 2> half_tag;
    std::integral_constant<int, WAVES> all_tag;
    // group 1's DMA at its VALU(t - 1): K(t + 1)
    auto issue_step = [&](int t) __attribute__((always_inline)) {
      if (t + 1 < ntiles) issue(half_tag, WAVES / 2, Kg, false, t + 1, kd(t + 1));
    };
    // one half-step pair of tile t; `mf` is the MFMA phase
    auto step = [&](int t, auto&& mf, auto&& vf) __attribute__((always_inline)) {
      __builtin_amdgcn_s_setprio(2);
      mf();
      __builtin_amdgcn_s_setprio(0);
      if (grp == 1) wait_dma();
      __syncthreads();
      if (RS_MFMA && !RS_STREAM && t > 0) rowsum_mfma();  // P(t - 1), still in pb
      if (kPoison && grp == 1) {
        // group 1, softmax(t): V(t - 1) was last read in the previous half step
        // (group 1's P x V of it) and its buffer is refilled with V(t + 1)
        // next half step; K(t)'s buffer gets K(t + 2) now
        const int gt = tid - 64 * (WAVES / 2);
        if (t >= 1) poison_lds(lds_base + vd(t + 1), C::TILE_BYTES, 64 * (WAVES / 2), gt);
        if (t + 2 < ntiles) poison_lds(lds_base + kd(t + 2), C::TILE_BYTES, 64 * (WAVES / 2), gt);
      }
      if (grp == 1) issue_step(t + 1);
      else issue(half_tag, 0, Vg, true, t, vd(t));
      vf();
      // keep the softmax in this half step: without these uses the compiler
      // sinks the exponentials past the barrier, next to the P x V MFMAs
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int i = 0; i < BN / 16; ++i) asm volatile("" ::"v"(pb[qb][i]));
        asm volatile("" ::"v"(l_run[qb]));
      }
      if (grp == 0) wait_dma();
      __syncthreads();
    };
    if (ntiles > 0) {
      // K(0) by every wave, or by group 0 when the tile is smaller than one
      // 16-byte load per thread of the workgroup
      if constexpr (C::TILE_BYTES % (16 * C::THREADS) == 0) issue(all_tag, 0, Kg, false, 0, kd(0));
      else if (grp == 0) issue(half_tag, 0, Kg, false, 0, kd(0));
      wait_dma();
      __syncthreads();
      if (grp == 1) {
        issue_step(0);
        __syncthreads();
      }
      step(0, [&]() __attribute__((always_inline)) {
        mfma_stream<C, D, BN, QB, R, false, true, false>(smem, pb, acc, sel, lsum, smem + kd(0), qf, s0, lane);
      }, [&]() __attribute__((always_inline)) { softmax_tile(0, safe_tag); });
      if constexpr (VT::SPLIT && !decltype(safe_tag)::value) {
        // the P x V operands of block 0: P(t-1) in pb[0] (read by this
        // phase's MFMAs), P(t) built in pbn and moved to pb[0] after them.
        // (The safe pass, rare, takes the plain form below: the split form's
        // extra live values there pushed the kernel past the register file.)
        bf16x8 pbn[BN / 16];
        constexpr int NPV = (BN / 16) * (D / 32), KP = NPV / (BN / 16);
        for (int t = 1; t < ntiles; ++t)
          step(t, [&]() __attribute__((always_inline)) {
            float a0 = 1.f;
            bool r0 = false;
            mfma_stream_split<C, D, BN, R>(smem + vd(t - 1), pb, acc, sel, lsum, smem + kd(t), qf, s0, lane,
                                           [&](int mp) __attribute__((always_inline)) {
                                             if (mp == 0) split_head0(t, safe_tag, a0, r0);
                                             if (mp % KP == KP - 1) split_pack0(mp / KP, pbn);
                                           });
            if (r0) {
#pragma unroll
              for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[0][db][r] *= a0;
            }
#pragma unroll
            for (int i = 0; i < BN / 16; ++i) pb[0][i] = pbn[i];
          }, [&]() __attribute__((always_inline)) { softmax_block1(t, safe_tag); });
      } else {
        for (int t = 1; t < ntiles; ++t)
          step(t, [&]() __attribute__((always_inline)) {
            mfma_stream<C, D, BN, QB, R, true, true, RS_STREAM>(smem + vd(t - 1), pb, acc, sel, lsum,
                                                                smem + kd(t), qf, s0, lane);
          }, [&]() __attribute__((always_inline)) { softmax_tile(t, safe_tag); });
      }
      __builtin_amdgcn_s_setprio(2);
      mfma_stream<C, D, BN, QB, R, true, false, RS_STREAM>(smem + vd(ntiles - 1), pb, acc, sel, lsum, smem,
                                                           qf, s0, lane);
      __builtin_amdgcn_s_setprio(0);
      if (RS_MFMA) {
        if (!RS_STREAM) rowsum_mfma();
        fold_sum();
      }
      if (grp == 0) __syncthreads();  // group 1's last VALU barrier
    }
  } else {
    // Sequential form over an LDS ring of STAGES (K, V) tile pairs: the DMAs of
    // tile t + STAGES - 1 are in flight while tile t is computed.
    constexpr int AHEAD = C::STAGES - 1;
    static_assert(C::TILE_BYTES % (16 * C::THREADS) == 0, "tile must split evenly over the threads");
    constexpr int LOADS = C::TILE_BYTES / 16 / C::THREADS;  // 16 B loads per thread per tile
    std::integral_constant<int, WAVES> all_tag;
    auto sk = [&](int t) __attribute__((always_inline)) { return (uint32_t)((t % C::STAGES) * C::STAGE_BYTES); };
    auto sv = [&](int t) __attribute__((always_inline)) { return sk(t) + (uint32_t)C::TILE_BYTES; };
#pragma unroll
    for (int i = 0; i < AHEAD; ++i)
      if (i < ntiles) {
        issue(all_tag, 0, Kg, false, i, sk(i));
        issue(all_tag, 0, Vg, true, i, sv(i));
      }
    wait_dma();
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const bool more = t + AHEAD < ntiles;
      // tile t - 1's slot: last read before the barrier that ended step t - 1
      if (kPoison && more) poison_lds(lds_base + sk(t + AHEAD), C::STAGE_BYTES, C::THREADS, tid);
      if (more) {
        issue(all_tag, 0, Kg, false, t + AHEAD, sk(t + AHEAD));
        issue(all_tag, 0, Vg, true, t + AHEAD, sv(t + AHEAD));
      }
      mfma_stream<C, D, BN, QB, R, false, true, false>(smem, pb, acc, sel, lsum, smem + sk(t), qf, s0, lane);
      softmax_tile(t, safe_tag);
      mfma_stream<C, D, BN, QB, R, true, false, RS_STREAM>(smem + sv(t), pb, acc, sel, lsum, smem, qf, s0,
                                                           lane);
      // tile t + 1 must have landed; the DMAs of tiles t + 2 .. t + AHEAD may
      // stay in flight (2 * LOADS instructions per tile and wave)
      if (more) wait_dma_n<(AHEAD - 1) * 2 * LOADS>();
      else wait_dma();
      __syncthreads();
    }
    if (RS_MFMA) fold_sum();
  }
  };
  // The fast pass; then a workgroup vote.  Every wave has finished the pass
  // (no DMA is in flight and no LDS tile is read after the barrier), so the
  // safe pass can reuse the ring.
  int LDS_AS* vote = (int LDS_AS*)(smem + C::LDS_ALLOC);
  if (tid == 0) *vote = 0;
  run_pass(std::false_type{});
  if (RS_MFMA) {  // the VALU row sum tests every tile before its P x V
    if (bad) *vote = 1;
    __syncthreads();
    if (*vote != 0) run_pass(std::true_type{});
  }

  // ---------------- epilogue: O = O^T / l ----------------
  // O leaves through LDS so that it can be written in whole lines with
  // non-temporal stores (streamed past L2, where the K/V tiles of the head's
  // other query tiles stay).  Lane (h, c) holds 4-element pieces of row c of
  // each block; it writes them into the block's 32 x ROW_BYTES slice of the
  // (now idle) LDS, 16-byte chunks XOR-swizzled by the row (spreads the 32
  // rows' equal columns over the banks); then each store instruction of the
  // wave writes 1 KiB of whole rows, 16 contiguous bytes per lane.
  __syncthreads();  // every wave is past its last read of the K/V ring
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l_tot = l_run[qb];
    if (!RS_MFMA) {
      const u32x2 lp = swap_halves(l_run[qb]);
      l_tot = __uint_as_float(lp[0]) + __uint_as_float(lp[1]);
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int qrow = qw0 + 32 * qb + col;
    // log-sum-exp: sum_j 2^(c s_j) = 2^m_run * l, so ln(sum_j e^(scale s_j)) = (m_run + log2 l) ln 2
    // (one 128-byte line per block: the 32 lanes of half 0 write consecutive rows)
    if (lse != nullptr && half == 0 && qrow < N)
      __builtin_nontemporal_store(l_tot > 0.f ? (m_run[qb] + log2f(l_tot)) * kLn2 : -INFINITY,
                                  lse + (size_t)bh * N + qrow);
    char LDS_AS* ost = smem + (wave * QB + qb) * 32 * C::ROW_BYTES;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[qb][db][a4 * 4 + e] * inv);
        const int byte = (db * 32 + a4 * 8 + half * 4) * 2;  // within row c
        const int ch = (byte / 16) ^ (col % C::CHUNKS);
        *(bf16x4 LDS_AS*)(ost + col * C::ROW_BYTES + ch * 16 + byte % 16) = o;
      }
  }
  constexpr int ROWS_PER_STORE = 64 / C::CHUNKS;  // rows one 64-lane store covers
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const char LDS_AS* ost = smem + (wave * QB + qb) * 32 * C::ROW_BYTES;
    const int q_b = qw0 + 32 * qb;  // first query row of this block
#pragma unroll
    for (int i = 0; i < 32 / ROWS_PER_STORE; ++i) {
      const int row = i * ROWS_PER_STORE + lane / C::CHUNKS;
      const int chunk = lane % C::CHUNKS;
      const u32x4 v = *(const u32x4 LDS_AS*)(ost + row * C::ROW_BYTES + ((chunk ^ (row % C::CHUNKS)) * 16));
      if (q_b + row < N)
        __builtin_nontemporal_store(v, (u32x4*)(Os + (size_t)(q_b + row) * D + chunk * 8));
    }
  }
}

// ----------------------------------------------------------------------------
// The 16x16x32 form of the ping-pong kernel (d = 128).
// ----------------------------------------------------------------------------
// Same schedule, tiles, LDS ring, hand-over and lazy shift as the kernel
// above, with every product on v_mfma_f32_16x16x32_bf16.  On MI355X a long
// all-CU MFMA stream on random operands is power limited, and the smaller
// shape, which reads and writes half the accumulator data per multiply-add,
// delivered 0.83 of the bf16 nameplate against 0.70 for 32x32x16 (measured).
//
// A wave's 32 queries form two blocks of 16 (h = 0, 1); lane l = 16 g + n
// owns query n of each block.  Per 16-key block kb, S^T (16 keys x 16
// queries) has lane (g, n) holding keys 16 kb + 4g .. +3 of query n.  P^T of
// a 32-key step st (the B operand of P x V: 32 keys x 16 queries) takes, in
// lane (g, n), the keys 32 st + 16 u + 4 g + e of blocks 2 st + u (u = 0, 1,
// e = 0..3) as reduction index k = 8 g + 4 u + e: built lane-locally from
// two S^T blocks.  The V operand (A: 16 d-rows x 32 keys) is read in the same
// key order by two transpose reads of four key rows.  O^T (16 d x 16 queries
// per block) has lane (g, n) holding d = 16 db + 4 g .. +3 of query n.  Row
// sums: an all-ones A operand times P^T gives every output row the column
// sums, so each lane receives its own query's sum over the step.  Row maxima
// (first visible tile, safe pass) reduce over the four lanes n, n + 16,
// n + 32, n + 48 of a query (two lane swaps).

// Chunk swizzle of V rows for the transpose reads of this form: the four
// rows of one read and the two 16-lane groups of a half-wave (rows 4 apart)
// land on distinct 16-byte chunks, 512 bytes over all banks.  Period 8 rows.
template <class C>
__device__ __forceinline__ int swz_v16(int row) {
  static_assert(C::CHUNKS == 16, "d = 128 rows");
  return 2 * ((row % 4) + 4 * ((row / 4) % 2));
}

// v_permlane16_swap with both operands = x: the pair is {own, lane ^ 16}.
__device__ __forceinline__ u32x2 swap_rows16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  u32x2 out = {r[0], r[1]};
  return out;
}

// One MFMA phase (as mfma_stream): DO_PV, O^T += V^T P^T over the tile's
// (BN/32) x (D/16) V operands (and, with DO_RS, the row sums of each 32-key
// step); DO_QK, S^T = K Q^T over (D/32) x (BN/16) K operands.  Each operand
// feeds two MFMAs (query blocks h = 0, 1).  Operand addresses as in
// mfma_stream: a lane base XOR a compile-time constant plus an immediate
// row offset:
//   K: row 16 kb + n, chunk (4 ks + g) ^ n = (kbase ^ 64 ks) + 16 kb rows,
//   V: row 32 st + 16 u + 4 g + j, chunk (2 db + q / 2) ^ swz_v16
//      = (vbase ^ 32 db) + (32 st + 16 u) rows   (lane n = 4 j + q).
template <class C, int D, int BN, int R, bool DO_PV, bool DO_QK, bool DO_RS>
__device__ __forceinline__ void mfma_stream16(const char LDS_AS* vl, const bf16x8 (&pb)[2][BN / 32],
                                              f32x4 (&acc)[2][D / 16], const bf16x8& ones, f32x4 (&lsum)[2],
                                              const char LDS_AS* kl, const bf16x8 (&qf)[2][D / 32],
                                              f32x4 (&s)[2][BN / 16], int lane) {
  const int g = lane / 16, n = lane % 16;
  const int j = n / 4, q = n % 4;
  constexpr int NPV = DO_PV ? (BN / 32) * (D / 16) : 0;
  constexpr int NQK = DO_QK ? (D / 32) * (BN / 16) : 0;
  constexpr int NM = NPV + NQK;
  static_assert(D == 128 && C::ROWS_PER_256 == 1, "16x16x32 form: d = 128");
  uint32_t kbase = (uint32_t)(uintptr_t)kl + (uint32_t)(n * C::ROW_BYTES + ((g ^ swz_k<C>(n)) * 16));
  const int vrow = 4 * g + j;
  uint32_t vbase = (uint32_t)(uintptr_t)vl +
                   (uint32_t)(vrow * C::ROW_BYTES + (((q / 2) ^ swz_v16<C>(vrow)) * 16) + (q % 2) * 8);
  asm volatile("" : "+v"(kbase), "+v"(vbase));
  auto read = [&](int m) __attribute__((always_inline)) {
    bf16x8 a;
    if (m < NPV) {
      const int st = m / (D / 16), db = m % (D / 16);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t addr = (vbase ^ (uint32_t)(db * 32)) + (uint32_t)((st * 32 + u * 16) * C::ROW_BYTES);
        const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDS_AS*)(uintptr_t)addr);
        const bf16x4 vb = __builtin_bit_cast(bf16x4, v4);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[u * 4 + e] = vb[e];
      }
    } else {
      const int mq = m - NPV;
      const int ks = mq / (BN / 16), kb = mq % (BN / 16);
      const uint32_t addr = (kbase ^ (uint32_t)(ks * 64)) + (uint32_t)(kb * 16 * C::ROW_BYTES);
      a = *(const bf16x8 LDS_AS*)(uintptr_t)addr;
    }
    return a;
  };
  bf16x8 ring[R + 1];
#pragma unroll
  for (int m = 0; m < R && m < NM; ++m) ring[m] = read(m);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    if (m + R < NM) ring[(m + R) % (R + 1)] = read(m + R);
    const bf16x8 a = ring[m % (R + 1)];
    const f32x4 zero4 = {};
    if (m < NPV) {
      const int st = m / (D / 16), db = m % (D / 16);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        acc[h][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[h][st], acc[h][db], 0, 0, 0);
      if (DO_RS && db == D / 16 - 1) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          lsum[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[h][st], st == 0 ? zero4 : lsum[h], 0, 0, 0);
      }
    } else {
      const int mq = m - NPV;
      const int ks = mq / (BN / 16), kb = mq % (BN / 16);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        s[h][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[h][ks], ks == 0 ? zero4 : s[h][kb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <class VT, bool CAUSAL, bool NEG_SCALE>
__global__ __launch_bounds__(64 * VT::WAVES, (VT::WAVES / 4) * VT::WG_PER_CU)
void attn_fwd_bf16_mf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                               const __bf16* __restrict__ V, __bf16* __restrict__ O,
                               const int32_t* __restrict__ kv_len, float* __restrict__ lse, int H, int N,
                               float c, int n_qtiles) {
  constexpr int D = VT::D, BN = VT::BN, WAVES = VT::WAVES, WG_PER_CU = VT::WG_PER_CU;
  constexpr bool KEYS_SNAKE = VT::KEYS_SNAKE;
  constexpr int R = read_ahead<1>();  // each operand read feeds two 16-cycle MFMAs
  using C = typename VT::C;
  static_assert(VT::PINGPONG && VT::QB == 1 && VT::RS_MFMA && WAVES % 2 == 0, "16x16x32 form: ping-pong, 32 queries per wave");
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int g = lane / 16;  // key (S^T) or d (O^T) group of the lane
  const int n = lane % 16;  // the query of each 16-query block this lane owns

  // ---- work assignment, key order: as in attn_fwd_bf16_kernel ----
  const int G = gridDim.x;
  const int x = blockIdx.x;
  const int xcd = x % 8, idx = x / 8;
  int bh, qt;
  if ((G / n_qtiles) % 8 == 0) {
    bh = xcd + 8 * (idx / n_qtiles);
    qt = idx % n_qtiles;
  } else {
    const int per = G / 8, rem = G % 8;
    const int logical = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    bh = logical / n_qtiles;
    qt = logical % n_qtiles;
  }
  if (CAUSAL) qt = n_qtiles - 1 - qt;
  const int b = bh / H;
  int L = N;
  if (kv_len != nullptr) {
    L = kv_len[b];
    L = L < 0 ? 0 : (L > N ? N : L);
  }
  L = __builtin_amdgcn_readfirstlane(L);
  const int q0 = qt * C::BM;
  int kend = L;
  if (CAUSAL) kend = min(kend, min(N, q0 + C::BM));
  kend = __builtin_amdgcn_readfirstlane(kend);
  const int ntiles = (kend + BN - 1) / BN;
  constexpr int RESIDENT = 32 * WG_PER_CU;
  const bool keys_down = CAUSAL && KEYS_SNAKE && (((n_qtiles - 1 - qt) / RESIDENT) & 1);
  auto ktile = [&](int t) __attribute__((always_inline)) { return keys_down ? ntiles - 1 - t : t; };

  const size_t slice = (size_t)bh * N * D;
  const __bf16* Qs = Q + slice;
  const char* Kg = (const char*)(K + slice);
  const char* Vg = (const char*)(V + slice);
  __bf16* Os = O + slice;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

  // DMA of a K or V tile by NW waves from W0 (as in attn_fwd_bf16_kernel;
  // V rows take this form's swizzle)
  auto issue = [&](auto nw_tag, int w0, const char* gsrc, bool is_v, int t, uint32_t dst)
      __attribute__((always_inline)) {
    constexpr int NW = decltype(nw_tag)::value;
    constexpr int TH = 64 * NW;
    constexpr int NLOADS = C::TILE_BYTES / 16 / TH;
    constexpr int RSTEP = TH * 16 / C::ROW_BYTES;
    static_assert(C::TILE_BYTES % (16 * TH) == 0, "tile must split evenly over the issuing waves");
    static_assert((TH * 16) % C::ROW_BYTES == 0 && RSTEP % 16 == 0, "loads must step by whole swizzle periods");
    const int j0 = ktile(t) * BN;
    const char* gt = gsrc + (size_t)j0 * C::ROW_BYTES;
    int last = kend - 1 - j0;
    const int wl = wave - w0;
    const int pos0 = (wl * 64 + lane) * 16;
    const int row0 = pos0 / C::ROW_BYTES;
    const int lch = ((pos0 % C::ROW_BYTES) / 16) ^ (is_v ? swz_v16<C>(row0) : swz_k<C>(row0));
    const uint32_t l0 = lds_base + dst + (uint32_t)(wl * 64 * 16);
    if (last >= BN - 1) {
      uint32_t o = (uint32_t)(row0 * C::ROW_BYTES + lch * 16);
      asm volatile("" : "+v"(o));
#pragma unroll
      for (int i = 0; i < NLOADS; ++i)
        dma16(gt, o + (uint32_t)(i * TH * 16), __builtin_amdgcn_readfirstlane(l0 + (uint32_t)(i * TH * 16)));
    } else {
      last = __builtin_amdgcn_readfirstlane(last);
      int r0 = row0, c16 = lch * 16;
      asm volatile("" : "+s"(last), "+v"(r0), "+v"(c16));
#pragma unroll
      for (int i = 0; i < NLOADS; ++i) {
        const int lim = last - i * RSTEP;
        const int grow = r0 < lim ? r0 : lim;
        const uint32_t o = (uint32_t)(grow * C::ROW_BYTES + c16) + (uint32_t)(i * TH * 16);
        dma16(gt, o, __builtin_amdgcn_readfirstlane(l0 + (uint32_t)(i * TH * 16)));
      }
    }
  };
  const int qw0 = q0 + wave * 32;  // first query row of this wave; block h: qw0 + 16 h + n
  auto need_mask = [&](int t) __attribute__((always_inline)) {
    const int j0 = ktile(t) * BN;
    return (j0 + BN > L) || (CAUSAL && (j0 + BN - 1 > qw0));
  };

  // ---- Q fragments (B operand of S^T = K Q^T): lane (g, n) holds
  //      Q[qw0 + 16 h + n][32 ks + 8 g .. +7] ----
  bf16x8 qf[2][D / 32];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int qrow = qw0 + 16 * h + n;
    const int qrow_c = qrow < N ? qrow : N - 1;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[h][ks] = __builtin_nontemporal_load((const bf16x8*)(Qs + (size_t)qrow_c * D + ks * 32 + g * 8));
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) asm volatile("" ::"v"(qf[h][ks]));

  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.f;

  constexpr bool RS_STREAM = VT::RS_IN_STREAM;
  f32x4 acc[2][D / 16];
  float m_run[2], l_run[2];
  f32x4 lsum[2];
  bool bad;
  f32x4 s0[2][BN / 16];
  bf16x8 pb[2][BN / 32];

  // row extreme of the raw scores of block h (max, or min for a negative
  // scale) over the lane's values and the three other lanes of its query
  auto row_extreme16 = [&](int h) __attribute__((always_inline)) {
    float m4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) m4[r] = s0[h][0][r];
#pragma unroll
    for (int kb = 1; kb < BN / 16; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) m4[r] = NEG_SCALE ? fminf(m4[r], s0[h][kb][r]) : fmaxf(m4[r], s0[h][kb][r]);
    float mx = NEG_SCALE ? fminf(fminf(m4[0], m4[1]), fminf(m4[2], m4[3]))
                         : fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    const u32x2 p32 = swap_halves(mx);
    mx = NEG_SCALE ? fminf(__uint_as_float(p32[0]), __uint_as_float(p32[1]))
                   : fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
    const u32x2 p16 = swap_rows16(mx);
    return NEG_SCALE ? fminf(__uint_as_float(p16[0]), __uint_as_float(p16[1]))
                     : fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  };
  auto update_shift = [&](int h) __attribute__((always_inline)) {
    const float m_tile = row_extreme16(h) * c;
    if (m_tile > m_run[h] + kTauLog2) {
      const float m_new = fmaxf(m_run[h], m_tile);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[h] - m_new);
      m_run[h] = m_new;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[h][db][r] *= alpha;
      l_run[h] *= alpha;
    }
  };
  auto rowsum_mfma = [&]() __attribute__((always_inline)) {
    const f32x4 zero4 = {};
#pragma unroll
    for (int st = 0; st < BN / 32; ++st)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        lsum[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[h][st], st == 0 ? zero4 : lsum[h], 0, 0, 0);
  };
  // fold the previous tile's row sums (lazy shift and guard as in the 32x32
  // form's fold_sum)
  auto fold_sum = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float rs = lsum[h][0];
      bad = bad || !(rs <= kSafeSumMax);
      l_run[h] += rs;
      if (rs > kLazySumMax && rs <= kSafeSumMax) {
        const float mv = floorf(__builtin_amdgcn_logf(rs));
        const float alpha = __builtin_amdgcn_exp2f(-mv);
        m_run[h] += mv;
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[h][db][r] *= alpha;
        l_run[h] *= alpha;
      }
    }
  };
  auto softmax_tile = [&](int t, auto safe_tag) __attribute__((always_inline)) {
    constexpr bool SAFE = decltype(safe_tag)::value;
    fold_sum();
    const bool msk = need_mask(t);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (msk) {
        // element (kb, r) holds key j0 + 16 kb + 4 g + r: visible iff
        // 16 kb + r <= lim (one per-lane bound per tile, so that no per-element
        // key offset is kept live across the loop)
        const int j0 = ktile(t) * BN, qrow = qw0 + 16 * h + n;
        int lim = L - 1 - j0 - 4 * g;
        if (CAUSAL) lim = min(lim, qrow - j0 - 4 * g);
#pragma unroll
        for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            s0[h][kb][r] = (kb * 16 + r <= lim) ? s0[h][kb][r] : (NEG_SCALE ? INFINITY : -INFINITY);
      }
      if (SAFE || m_run[h] == -INFINITY) update_shift(h);
      const float mu = m_run[h] == -INFINITY ? 0.f : m_run[h];
#pragma unroll
      for (int st = 0; st < BN / 32; ++st) {
        bf16x8 p;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            p[u * 4 + e] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s0[h][2 * st + u][e], c, -mu));
        pb[h][st] = p;
      }
    }
  };

  auto run_pass = [&](auto safe_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[h][db][r] = 0.f;
      m_run[h] = -INFINITY;
      l_run[h] = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) lsum[h][r] = 0.f;
    }
    bad = false;
    // ping-pong schedule, ring hand-over and DMA split exactly as in the
    // 32x32 kernel's ping-pong form
    const int grp = wave / (WAVES / 2);
    auto kd = [&](int t) __attribute__((always_inline)) { return (uint32_t)((t & 1) * C::TILE_BYTES); };
    auto vd = [&](int t) __attribute__((always_inline)) { return (uint32_t)((2 + (t & 1)) * C::TILE_BYTES); };
    std::integral_constant<int, WAVES / 2> half_tag;
    std::integral_constant<int, WAVES> all_tag;
    auto issue_step = [&](int t) __attribute__((always_inline)) {
      if (t + 1 < ntiles) issue(half_tag, WAVES / 2, Kg, false, t + 1, kd(t + 1));
    };
    auto step = [&](int t, auto&& mf) __attribute__((always_inline)) {
      __builtin_amdgcn_s_setprio(2);
      mf();
      __builtin_amdgcn_s_setprio(0);
      if (grp == 1) wait_dma();
      __syncthreads();
      if (!RS_STREAM && t > 0) rowsum_mfma();
      if (kPoison && grp == 1) {
        const int gt = tid - 64 * (WAVES / 2);
        if (t >= 1) poison_lds(lds_base + vd(t + 1), C::TILE_BYTES, 64 * (WAVES / 2), gt);
        if (t + 2 < ntiles) poison_lds(lds_base + kd(t + 2), C::TILE_BYTES, 64 * (WAVES / 2), gt);
      }
      if (grp == 1) issue_step(t + 1);
      else issue(half_tag, 0, Vg, true, t, vd(t));
      softmax_tile(t, safe_tag);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < BN / 32; ++i) asm volatile("" ::"v"(pb[h][i]));
        asm volatile("" ::"v"(l_run[h]));
      }
      if (grp == 0) wait_dma();
      __syncthreads();
    };
    if (ntiles > 0) {
      if constexpr (C::TILE_BYTES % (16 * C::THREADS) == 0) issue(all_tag, 0, Kg, false, 0, kd(0));
      else if (grp == 0) issue(half_tag, 0, Kg, false, 0, kd(0));
      wait_dma();
      __syncthreads();
      if (grp == 1) {
        issue_step(0);
        __syncthreads();
      }
      step(0, [&]() __attribute__((always_inline)) {
        mfma_stream16<C, D, BN, R, false, true, false>(smem, pb, acc, ones, lsum, smem + kd(0), qf, s0, lane);
      });
      for (int t = 1; t < ntiles; ++t)
        step(t, [&]() __attribute__((always_inline)) {
          mfma_stream16<C, D, BN, R, true, true, RS_STREAM>(smem + vd(t - 1), pb, acc, ones, lsum, smem + kd(t), qf,
                                                            s0, lane);
        });
      __builtin_amdgcn_s_setprio(2);
      mfma_stream16<C, D, BN, R, true, false, RS_STREAM>(smem + vd(ntiles - 1), pb, acc, ones, lsum, smem, qf, s0,
                                                         lane);
      __builtin_amdgcn_s_setprio(0);
      if (!RS_STREAM) rowsum_mfma();
      fold_sum();
      if (grp == 0) __syncthreads();  // group 1's last softmax barrier
    }
  };
  int LDS_AS* vote = (int LDS_AS*)(smem + C::LDS_ALLOC);
  if (tid == 0) *vote = 0;
  run_pass(std::false_type{});
  if (bad) *vote = 1;
  __syncthreads();
  if (*vote != 0) run_pass(std::true_type{});

  // ---------------- epilogue: O = O^T / l (as in attn_fwd_bf16_kernel) ----------------
  __syncthreads();
  char LDS_AS* ost = smem + wave * 32 * C::ROW_BYTES;  // this wave's 32 rows: row 16 h + n
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float l_tot = l_run[h];
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int row = 16 * h + n;
    const int qrow = qw0 + row;
    if (lse != nullptr && g == 0 && qrow < N)
      __builtin_nontemporal_store(l_tot > 0.f ? (m_run[h] + log2f(l_tot)) * kLn2 : -INFINITY,
                                  lse + (size_t)bh * N + qrow);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[h][db][e] * inv);
      const int byte = (db * 16 + g * 4) * 2;  // within the row
      const int ch = (byte / 16) ^ (row % C::CHUNKS);
      *(bf16x4 LDS_AS*)(ost + row * C::ROW_BYTES + ch * 16 + byte % 16) = o;
    }
  }
  constexpr int ROWS_PER_STORE = 64 / C::CHUNKS;
#pragma unroll
  for (int i = 0; i < 32 / ROWS_PER_STORE; ++i) {
    const int row = i * ROWS_PER_STORE + lane / C::CHUNKS;
    const int chunk = lane % C::CHUNKS;
    const u32x4 v = *(const u32x4 LDS_AS*)(ost + row * C::ROW_BYTES + ((chunk ^ (row % C::CHUNKS)) * 16));
    if (qw0 + row < N) __builtin_nontemporal_store(v, (u32x4*)(Os + (size_t)(qw0 + row) * D + chunk * 8));
  }
}

template <class VT, bool CAUSAL, bool NEG>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  using C = typename VT::C;
  const int n_qtiles = (a.N + C::BM - 1) / C::BM;
  const long long grid = (long long)a.B * a.H * n_qtiles;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  // exponent multiplier scale * log2(e); an exact zero (scale 0, or a scale so
  // small that the product underflows) becomes the smallest normal float, so
  // masked scores (-inf) still map to exp2(-inf) = 0 while every visible
  // score maps to exp2(0) = 1 exactly: uniform weights, as for c = 0
  float c = a.scale * kLog2e;
  if (c == 0.f) c = FLT_MIN;
  if constexpr (VT::MF16) {
    auto kern = attn_fwd_bf16_mf16_kernel<VT, CAUSAL, NEG>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::THREADS), C::LDS_ALLOC + 16, stream,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o,
                       a.kv_len, a.lse, a.H, a.N, c, n_qtiles);
  } else {
    auto kern = attn_fwd_bf16_kernel<VT, CAUSAL, NEG>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::THREADS), C::LDS_ALLOC + 16, stream,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o,
                       a.kv_len, a.lse, a.H, a.N, c, n_qtiles);
  }
  return hipGetLastError();
}

template <class VT>
hipError_t dispatch_mask(const FwdArgs& a, hipStream_t stream) {
  const bool neg = a.scale < 0.f;
  if (a.causal) return neg ? launch_t<VT, true, true>(a, stream) : launch_t<VT, true, false>(a, stream);
  return neg ? launch_t<VT, false, true>(a, stream) : launch_t<VT, false, false>(a, stream);
}

// The compiled tilings.  Which one a call runs is decided on the host by the
// I/O and issue model of the front end (it evaluates every feasible tiling and
// takes the best compiled one); the set below holds that model's choices for
// the long-sequence workloads plus their nearest neighbours, which the model
// was checked against by measurement.
//   d = 128: ping-pong, 8 waves x 32 queries, 128- or 64-key tiles, one
//            256-row workgroup per CU; and the sequential 4-wave form at two
//            128-row workgroups per CU.
//   d = 64:  ping-pong, 8 waves x 64 queries (two blocks per wave), 64-key
//            tiles, one 512-row workgroup per CU, row sums on the matrix core;
//            16 waves x 32 queries, one 512-row workgroup per CU, VALU row
//            sums; 8 waves x 32 queries at two 256-row workgroups per CU with
//            VALU row sums; and 128-key tiles at one 256-row workgroup per CU.
//                   D    BN  W  QB ST  PP     WPC SNAKE RS_MFMA
using V128_PP128 = Variant<128, 128, 8, 1, 2, true, 1, true, true>;
using V128_PP64 = Variant<128, 64, 8, 1, 2, true, 1, true, true>;
using V128_SEQ64 = Variant<128, 64, 4, 1, 2, false, 2, true, true>;
using V64_PP64_QB2 = Variant<64, 64, 8, 2, 2, true, 1, true, true>;
using V64_PP64 = Variant<64, 64, 8, 1, 2, true, 2, true, false>;
using V64_PP128 = Variant<64, 128, 8, 1, 2, true, 1, true, true>;
using V64_PP64_W16 = Variant<64, 64, 16, 1, 2, true, 1, true, false>;
#ifndef ATTNIO_FWD_SPLIT_D64
#define ATTNIO_FWD_SPLIT_D64 1
#endif
using V64_PP64_QB2_RSS = Variant<64, 64, 8, 2, 2, true, 1, true, true, true, ATTNIO_FWD_SPLIT_D64 != 0>;
using V128_PP128_RSS = Variant<128, 128, 8, 1, 2, true, 1, true, true, true>;
using V128_PP128_RSS_M16 = Variant<128, 128, 8, 1, 2, true, 1, true, true, true, false, true>;

template <class VT>
constexpr Tiling tiling_of() {
  using C = typename VT::C;
  return Tiling{VT::D, C::BM, VT::BN, C::STAGES, VT::WAVES, C::LDS_ALLOC + 16, VT::WG_PER_CU, VT::QB,
                VT::PINGPONG ? 1 : 0, VT::RS_MFMA ? 1 : 0, VT::RS_IN_STREAM ? 1 : 0, VT::MF16 ? 1 : 0};
}

struct Entry {
  Tiling t;
  hipError_t (*launch)(const FwdArgs&, hipStream_t);
};

const Entry kEntries[] = {
    {tiling_of<V128_PP128>(), &dispatch_mask<V128_PP128>},
    {tiling_of<V128_PP64>(), &dispatch_mask<V128_PP64>},
    {tiling_of<V128_SEQ64>(), &dispatch_mask<V128_SEQ64>},
    {tiling_of<V64_PP64_QB2>(), &dispatch_mask<V64_PP64_QB2>},
    {tiling_of<V64_PP64>(), &dispatch_mask<V64_PP64>},
    {tiling_of<V64_PP128>(), &dispatch_mask<V64_PP128>},
    {tiling_of<V64_PP64_W16>(), &dispatch_mask<V64_PP64_W16>},
    {tiling_of<V64_PP64_QB2_RSS>(), &dispatch_mask<V64_PP64_QB2_RSS>},
    {tiling_of<V128_PP128_RSS>(), &dispatch_mask<V128_PP128_RSS>},
    {tiling_of<V128_PP128_RSS_M16>(), &dispatch_mask<V128_PP128_RSS_M16>},
};
constexpr int kNumEntries = (int)(sizeof(kEntries) / sizeof(kEntries[0]));

}  // namespace

int bf16_variant_count() { return kNumEntries; }

bool bf16_variant(int i, Tiling* t) {
  if (i < 0 || i >= kNumEntries) return false;
  *t = kEntries[i].t;
  return true;
}

hipError_t launch_fwd_bf16(int variant, const FwdArgs& a, hipStream_t stream) {
  if (variant < 0 || variant >= kNumEntries || kEntries[variant].t.d != a.d) return hipErrorInvalidValue;
  return kEntries[variant].launch(a, stream);
}

}  // namespace attnio
