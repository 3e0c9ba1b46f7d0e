// Exact attention backward for bf16 on gfx950 (CDNA4).
//
// The backward pass recomputes the probabilities from Q, K, V and the per-row
// log-sum-exp of the forward instead of storing them ("IO-Aware Algorithms",
// How it works: recomputation).  With P = exp(s Q K^T - lse) (masked entries
// 0), the gradients are
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D_i = dO_i . O_i,
//     dQ = s dS K,   dK = s dS^T Q.
// Three kernels, enqueued in this order on the caller's stream:
//   delta: D_i = dO_i . O_i and lse_i * log2(e) per row, into the workspace
//          (padding rows of each head get D = 0, lse = +inf);
//   dk_dv: one workgroup per (batch*head, 128 keys); K and V of those keys stay
//          in registers as MFMA operands while Q, dO and the row statistics of
//          64-row query blocks stream through a three- or four-stage LDS ring;
//          the S and dP MFMAs of block i+1 run under the P / dS arithmetic of
//          block i;
//   dq:    one workgroup per (batch*head, 128 queries); Q and dO stay in
//          registers while 64-key K/V tiles stream through an LDS ring (its own
//          translation unit, attn_bwd_dq_bf16.hip, built with other options).
// Both recompute S and dP; each keeps its accumulators (dK^T, dV^T or dQ^T) in
// registers for its whole loop and writes them once, so no atomics and no
// partial sums reach memory.  Every product is a bf16 MFMA 32x32x16 with fp32
// accumulation; P and dS are rounded to bf16 only as MFMA operands.
//
// Orientation.  dk_dv computes S = Q K^T with the wave's 32 keys across the
// lanes: each lane owns one key, its registers hold 16 queries of a 32-row
// block, and P / dS then sit in the B-operand layout of dV^T += dO^T P and
// dK^T += Q^T dS (the contraction runs over queries); dO^T and Q^T come from
// LDS by transpose reads whose row order matches the registers' query order.
// dq is the forward's orientation: S^T = K Q^T with the wave's 32 queries
// across the lanes (row statistics are lane-local), dS^T in the B-operand
// layout of dQ^T += K^T dS^T, K^T by transpose reads.

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"
#include "tile_ops.h"

namespace attnio {
namespace {

constexpr int kStatPad = 64;  // workspace rows are padded per head to a multiple of this
constexpr int kBwdBQ = 64;  // query rows per dK/dV pipeline step (32 measured slower)

// LDS stages of the dK/dV ring, per head dimension: blocks i and i+1 are read
// during step i and the DMA of block i+STAGES-1 is issued at its start, so a
// block's load has STAGES-2 steps to land
#ifndef ATTNIO_DKDV_STAGES_D64
#define ATTNIO_DKDV_STAGES_D64 4
#endif
#ifndef ATTNIO_DKDV_STAGES_D128
#define ATTNIO_DKDV_STAGES_D128 3
#endif
// 1: the causal compare runs only on the query blocks that meet the key
// block's diagonal and the loop over the later blocks is built without it.
// At d = 128 the second copy of the step pushes the kernel (512 registers)
// into spills inside the loop, whose reloads wait for the DMAs in flight.
#ifndef ATTNIO_DKDV_DIAG_MASK_D64
#define ATTNIO_DKDV_DIAG_MASK_D64 1
#endif
#ifndef ATTNIO_DKDV_DIAG_MASK_D128
#define ATTNIO_DKDV_DIAG_MASK_D128 0
#endif
// 1: the dK/dV stage runs in the two-group ping-pong form
// (attn_bwd_dkdv_pp_bf16.hip) instead of the one-wave form below
#ifndef ATTNIO_DKDV_PINGPONG_D64
#define ATTNIO_DKDV_PINGPONG_D64 1
#endif
#ifndef ATTNIO_DKDV_PINGPONG_D128
#define ATTNIO_DKDV_PINGPONG_D128 1
#endif
constexpr bool dkdv_pingpong(int d) {
  return d == 64 ? ATTNIO_DKDV_PINGPONG_D64 != 0 : ATTNIO_DKDV_PINGPONG_D128 != 0;
}
constexpr int dkdv_stages(int d) { return d == 64 ? ATTNIO_DKDV_STAGES_D64 : ATTNIO_DKDV_STAGES_D128; }
constexpr bool dkdv_diag_mask(int d) {
  return d == 64 ? ATTNIO_DKDV_DIAG_MASK_D64 != 0 : ATTNIO_DKDV_DIAG_MASK_D128 != 0;
}

// ----------------------------------------------------------------------------
// delta: D_i = dO_i . O_i (fp32) and lse_i * log2(e), per row.
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256)
void attn_bwd_delta_kernel(const __bf16* __restrict__ O, const __bf16* __restrict__ dO,
                           const float* __restrict__ lse, float* __restrict__ ws_d,
                           float* __restrict__ ws_l, int N, int NP, long long rows_p) {
  // one row of the padded statistics per LPR lanes; per head the NP values of
  // D are followed by the NP values of lse*log2(e) ([B*H][2][NP]; ws_l =
  // ws_d + NP).  Padding rows (i >= N) get D = 0 and lse = +inf, so a block
  // that reads them computes P = 2^(s c - inf) = 0 and dS = 0 without a select
  constexpr int LPR = D / 8;  // lanes per row, 16 bytes each
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long rp = gid / LPR;
  const int part = (int)(gid % LPR);
  const long long bh = rp / NP;
  const int i = (int)(rp % NP);
  const bool real = rp < rows_p && i < N;
  const long long row = bh * N + i;
  float acc = 0.f;
  if (real) {
    const bf16x8 o = *(const bf16x8*)(O + row * D + part * 8);
    const bf16x8 g = *(const bf16x8*)(dO + row * D + part * 8);
#pragma unroll
    for (int t = 0; t < 8; ++t) acc = __builtin_fmaf((float)o[t], (float)g[t], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off /= 2) acc += __shfl_xor(acc, off, LPR);
  if (rp < rows_p && part == 0) {
    const long long at = bh * 2 * NP + i;
    ws_d[at] = real ? acc : 0.f;
    ws_l[at] = real ? lse[row] * kLog2e : INFINITY;
  }
}

// ----------------------------------------------------------------------------
// dk_dv: 4 waves x 32 keys; 64-row query blocks through a 3- or 4-stage LDS ring.
//
// One wave per SIMD, software-pipelined across query blocks: while the MFMAs of
// S and dP for block i+1 run, the same wave computes P and dS of block i on the
// VALU (one score per MFMA slot, the slots pinned by scheduling barriers);
// then the dV / dK MFMAs of block i.  The loop body is instantiated twice with
// the two S / dP register sets swapping roles, so nothing is copied.
// ----------------------------------------------------------------------------
template <int D, int BQ_>
struct KvCfg {
  static constexpr int WAVES = 4, THREADS = 256, BQ = BQ_, BKV = 32 * WAVES;
  static constexpr int RB = 2 * D;
  static constexpr int QT = BQ * RB;            // one Q or dO block
  static constexpr int STAGE = 2 * QT + 1024;   // Q, dO, row statistics (one 64-lane load)
  static constexpr int STAGES = dkdv_stages(D);
  static_assert(STAGES == 3 || STAGES == 4, "dK/dV ring depth");
  static constexpr int LDS = STAGES * STAGE;
};

template <int D, bool CAUSAL, int BQ_>
__global__ __launch_bounds__(256, 1)
void attn_bwd_dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                          const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                          const float* __restrict__ ws_d,
                          __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                          const int32_t* __restrict__ kv_len, int H, int N, int NP, float c,
                          float scale, int n_kblocks) {
  using C = KvCfg<D, BQ_>;
  constexpr int NB = BQ_ / 32;  // 32-row halves per query block
  constexpr int BQ = C::BQ, BKV = C::BKV, QT = C::QT, STAGE = C::STAGE;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, half = lane / 32, col = lane % 32;
  // XCD-aware assignment: block x runs on XCD x % 8; when B*H is a multiple of
  // 8, head j's key blocks all run on XCD j % 8 (its Q and dO stream through
  // one L2), key block 0 (the longest causal loop) first
  int bh, kblk;
  {
    const int G = gridDim.x, x = blockIdx.x, xcd = x % 8, idx = x / 8;
    if ((G / n_kblocks) % 8 == 0) {
      bh = xcd + 8 * (idx / n_kblocks);
      kblk = idx % n_kblocks;
    } else {
      bh = x / n_kblocks;
      kblk = x % n_kblocks;
    }
  }
  const int b = bh / H;
  int L = N;
  if (kv_len != nullptr) {
    L = kv_len[b];
    L = L < 0 ? 0 : (L > N ? N : L);
  }
  L = __builtin_amdgcn_readfirstlane(L);
  const int k0 = kblk * BKV;
  const int key = k0 + wave * 32 + col;  // the key this lane owns
  const size_t slice = (size_t)bh * N * D;

  // K and V of this lane's key as B operands (K^T and V^T of the products)
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const int kr = key < N ? key : N - 1;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kf[ks] = *(const bf16x8*)(K + slice + (size_t)kr * D + ks * 16 + half * 8);
      vf[ks] = *(const bf16x8*)(V + slice + (size_t)kr * D + ks * 16 + half * 8);
    }
  }
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(kf[ks]), "v"(vf[ks]));

  f32x16 dkt[D / 32], dvt[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dkt[db][r] = 0.f; dvt[db][r] = 0.f; }

  if (k0 < L) {
    const int qb0 = CAUSAL ? k0 / BQ : 0;
    const int nqb = (N + BQ - 1) / BQ - qb0;
    const __bf16* Qs = Q + slice;
    const __bf16* dOs = dO + slice;
    auto stage_of = [&](int i) __attribute__((always_inline)) { return (i % C::STAGES) * STAGE; };
    auto issue = [&](int i) __attribute__((always_inline)) {
      const int q0 = (qb0 + i) * BQ;
      const uint32_t st = lds_base + (uint32_t)stage_of(i);
      dma_rows<D, BQ, C::THREADS>(Qs, q0, N - 1, st, wave, lane);
      dma_rows<D, BQ, C::THREADS>(dOs, q0, N - 1, st + QT, wave, lane);
      if (wave == 0) {
        // lanes 0 .. BQ/4-1: lse*log2e of the BQ rows, the next BQ/4: D, the
        // rest repeat them.  The scalar base is this head's statistics (64-bit
        // address); the lane offset stays below 2 * NP * 4 bytes
        constexpr int NL = BQ / 4;
        const int sub = lane % (2 * NL);
        const uint32_t off = ((sub < NL ? (uint32_t)NP : 0u) + (uint32_t)(q0 + 4 * (sub % NL))) * 4u;
        dma16(ws_d + (size_t)bh * 2 * NP, off, __builtin_amdgcn_readfirstlane(st + 2 * QT));
      }
    };

    // MFMA slot m of S / dP for one block: accumulator m % (2 NB) (S or dP of
    // one of the block's 32-row halves), k step m / (2 NB)
    auto qk_read = [&](const char LDS_AS* st_l, int m) __attribute__((always_inline)) {
      const int acc = m % (2 * NB), ks = m / (2 * NB);
      const char LDS_AS* tile = st_l + ((acc % 2) ? QT : 0);
      return row_operand<D>(tile, (acc / 2) * 32 + col, ks, half);
    };
    auto qk_mfma = [&](f32x16 (&s)[NB], f32x16 (&dp)[NB], const bf16x8& a, int m)
        __attribute__((always_inline)) {
      const int acc = m % (2 * NB), ks = m / (2 * NB), blk = acc / 2;
      const f32x16 zero = {};
      if (acc % 2 == 0)
        s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[ks], ks == 0 ? zero : s[blk], 0, 0, 0);
      else
        dp[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[ks], ks == 0 ? zero : dp[blk], 0, 0, 0);
    };
    constexpr int AHEAD = C::STAGES - 1;    // DMA distance in blocks
    constexpr int NLD = 2 * (BQ * 2 * D / 16 / C::THREADS);  // DMAs per block and wave (+1 on wave 0)
    constexpr int NQK = 2 * NB * (D / 16);  // MFMAs of S and dP per block
    constexpr int NEL = 16 * NB;            // scores per lane per block
    constexpr int R = 4;               // LDS read-ahead (MFMA slots)

    // S / dP of block i alone (prologue)
    auto qk_only = [&](int i, f32x16 (&s)[NB], f32x16 (&dp)[NB]) __attribute__((always_inline)) {
      const char LDS_AS* st_l = smem + stage_of(i);
      bf16x8 ring[R + 1];
#pragma unroll
      for (int m = 0; m < R; ++m) ring[m] = qk_read(st_l, m);
#pragma unroll
      for (int m = 0; m < NQK; ++m) {
        if (m + R < NQK) ring[(m + R) % (R + 1)] = qk_read(st_l, m + R);
        qk_mfma(s, dp, ring[m % (R + 1)], m);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // P and dS of one score (element m of NEL) of block i, into the packed B
    // operands: operand st covers block rows 16 st .. 16 st + 15.
    //
    // Only the causal mask is applied per score.  Query rows at or past N need
    // none: their workspace statistics (lse = +inf, D = 0) give P = 0 and
    // dS = 0.  Keys at or past kv_len need none either: a key's P and dS only
    // reach its own column of dV^T and dK^T, which the store replaces by zero.
    // The causal test key <= q0 + 32 blk + 8 a4 + 4 half + e is one compare of
    // the lane's tq = key - q0 - 4 half against a compile-time constant; the
    // exponent is selected, not the result, so no branch forms around exp2.
    auto pds_elem = [&](const f32x16 (&s)[NB], const f32x16 (&dp)[NB], const float LDS_AS* st_f,
                        int tq, int m, f32x4& l4, f32x4& d4, bf16x8 (&pp)[BQ / 16],
                        bf16x8 (&pds)[BQ / 16], auto mask_tag) __attribute__((always_inline)) {
      const int blk = m / 16, a4 = (m % 16) / 4, e = m % 4, r = a4 * 4 + e;
      const int ql = blk * 32 + a4 * 8 + half * 4;  // first of four consecutive rows
      if (e == 0) {
        l4 = *(const f32x4 LDS_AS*)(st_f + ql);
        d4 = *(const f32x4 LDS_AS*)(st_f + BQ + ql);
      }
      float arg = __builtin_fmaf(s[blk][r], c, -l4[e]);
      if (decltype(mask_tag)::value) arg = (tq <= blk * 32 + a4 * 8 + e) ? arg : -INFINITY;
      const float p = __builtin_amdgcn_exp2f(arg);
      const float ds = p * (dp[blk][r] - d4[e]);  // p = 0 exactly where masked
      const int st = blk * 2 + a4 / 2, t8 = (a4 % 2) * 4 + e;
      pp[st][t8] = (__bf16)p;
      pds[st][t8] = (__bf16)ds;
    };

    // dV^T += dO^T P, dK^T += Q^T dS for block i: slot m -> (st, db, dv|dk)
    auto pv_stream = [&](int i, const bf16x8 (&pp)[BQ / 16], const bf16x8 (&pds)[BQ / 16])
        __attribute__((always_inline)) {
      const char LDS_AS* qt_l = smem + stage_of(i);
      const char LDS_AS* dot_l = qt_l + QT;
      constexpr int NPV = (BQ / 16) * (D / 32) * 2;
      auto rd = [&](int m) __attribute__((always_inline)) {
        const int which = m % 2, db = (m / 2) % (D / 32), st = m / 2 / (D / 32);
        return tr_operand<D>(which ? qt_l : dot_l, db, st, lane);
      };
      bf16x8 ring[R + 1];
#pragma unroll
      for (int m = 0; m < R; ++m) ring[m] = rd(m);
#pragma unroll
      for (int m = 0; m < NPV; ++m) {
        if (m + R < NPV) ring[(m + R) % (R + 1)] = rd(m + R);
        const int which = m % 2, db = (m / 2) % (D / 32), st = m / 2 / (D / 32);
        if (which == 0)
          dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[m % (R + 1)], pp[st], dvt[db], 0, 0, 0);
        else
          dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[m % (R + 1)], pds[st], dkt[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // one step: S / dP of block i+1 (if any) computed under P / dS of block i,
    // then dV / dK of block i
    auto step = [&](int i, f32x16 (&s)[NB], f32x16 (&dp)[NB], f32x16 (&sn)[NB], f32x16 (&dpn)[NB],
                    auto mask_tag) __attribute__((always_inline)) {
      if (i + AHEAD < nqb) issue(i + AHEAD);
      const char LDS_AS* cur = smem + stage_of(i);
      const float LDS_AS* st_f = (const float LDS_AS*)(cur + 2 * QT);
      const int tq = key - (qb0 + i) * BQ - half * 4;  // below 0 on every block past the diagonal
      bf16x8 pp[BQ / 16], pds[BQ / 16];
      f32x4 l4, d4;
      if (i + 1 < nqb) {
        const char LDS_AS* nxt = smem + stage_of(i + 1);
        bf16x8 ring[R + 1];
#pragma unroll
        for (int m = 0; m < R; ++m) ring[m] = qk_read(nxt, m);
#pragma unroll
        for (int m = 0; m < NQK; ++m) {
          if (m + R < NQK) ring[(m + R) % (R + 1)] = qk_read(nxt, m + R);
          qk_mfma(sn, dpn, ring[m % (R + 1)], m);
          // NEL scores over the NQK slots
#pragma unroll
          for (int e = m * NEL / NQK; e < (m + 1) * NEL / NQK; ++e)
            pds_elem(s, dp, st_f, tq, e, l4, d4, pp, pds, mask_tag);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int e = 0; e < NEL; ++e) pds_elem(s, dp, st_f, tq, e, l4, d4, pp, pds, mask_tag);
      }
      pv_stream(i, pp, pds);
      // block i+2 must be in LDS before step i+1; a later block may stay in flight
      if (i + 2 < nqb) {
        if (AHEAD > 2 && i + AHEAD < nqb) {
          if (wave == 0) wait_dma_n<NLD + 1>();
          else wait_dma_n<NLD>();
        } else {
          wait_dma_n<0>();
        }
      }
      __syncthreads();
    };
    issue(0);
#pragma unroll
    for (int j = 1; j < AHEAD; ++j)
      if (j < nqb) issue(j);
    wait_dma_n<0>();
    __syncthreads();
    f32x16 sA[NB], dpA[NB], sB[NB], dpB[NB];
    qk_only(0, sA, dpA);
    // causal: the query blocks 0 .. NDIAG-1 of the loop meet the key block's
    // diagonal; every later block lies wholly below it (all its scores visible)
    using masked_t = std::integral_constant<bool, CAUSAL>;
    using open_t = std::integral_constant<bool, CAUSAL && !dkdv_diag_mask(D)>;
    constexpr int NDIAG = (CAUSAL && dkdv_diag_mask(D)) ? BKV / BQ : 0;
    static_assert(NDIAG % 2 == 0, "diagonal blocks come in loop pairs");
    int i = 0;
    for (; i < NDIAG && i + 1 < nqb; i += 2) {
      step(i, sA, dpA, sB, dpB, masked_t{});
      step(i + 1, sB, dpB, sA, dpA, masked_t{});
    }
    for (; i + 1 < nqb; i += 2) {
      step(i, sA, dpA, sB, dpB, open_t{});
      step(i + 1, sB, dpB, sA, dpA, open_t{});
    }
    if (i < nqb) {
      if (i < NDIAG) step(i, sA, dpA, sB, dpB, masked_t{});
      else step(i, sA, dpA, sB, dpB, open_t{});
    }
  }

  // lane (h, c) holds rows db*32 + (r/4)*8 + 4h + r%4 (head dimension) of its
  // key; a key at or past kv_len gets zero gradients (its accumulators, built
  // without a key mask, are discarded, not multiplied)
  if (key < N) {
    const bool key_ok = key < L;
    __bf16* krow = dK + slice + (size_t)key * D;
    __bf16* vrow = dV + slice + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 ok4, ov4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ok4[e] = (__bf16)(key_ok ? dkt[db][a4 * 4 + e] * scale : 0.f);
          ov4[e] = (__bf16)(key_ok ? dvt[db][a4 * 4 + e] : 0.f);
        }
        *(bf16x4*)(krow + db * 32 + a4 * 8 + half * 4) = ok4;
        *(bf16x4*)(vrow + db * 32 + a4 * 8 + half * 4) = ov4;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const int NP = (a.N + kStatPad - 1) / kStatPad * kStatPad;
  // per head: NP values of D, then NP values of lse*log2(e)
  float* ws_d = a.ws;
  float* ws_l = a.ws + NP;
  const long long rows_p = (long long)a.B * a.H * NP;
  const long long dgrid = (rows_p * (D / 8) + 255) / 256;
  const int n_kblocks = (a.N + 127) / 128;
  const int n_qtiles = (a.N + 127) / 128;
  const long long g_kv = (long long)a.B * a.H * n_kblocks;
  const long long g_q = (long long)a.B * a.H * n_qtiles;
  if (dgrid > 0x7fffffffLL || g_kv > 0x7fffffffLL || g_q > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c = a.scale * kLog2e;
  hipLaunchKernelGGL((attn_bwd_delta_kernel<D>), dim3((unsigned)dgrid), dim3(256), 0, stream,
                     (const __bf16*)a.o, (const __bf16*)a.dout, a.lse, ws_d, ws_l, a.N, NP, rows_p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dkdv_pingpong(D)) {
    e = launch_bwd_dkdv_pp_bf16(a, ws_d, NP, c, stream);
    if (e != hipSuccess) return e;
    return launch_bwd_dq_bf16(a, ws_d, ws_l, NP, c, stream);
  }
  constexpr int kv_lds = KvCfg<D, kBwdBQ>::LDS;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL, kBwdBQ>), dim3((unsigned)g_kv), dim3(256), kv_lds,
                     stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                     (const __bf16*)a.dout, ws_d, (__bf16*)a.dk,
                     (__bf16*)a.dv, a.kv_len, a.H, a.N, NP, c, a.scale, n_kblocks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_bwd_dq_bf16(a, ws_d, ws_l, NP, c, stream);
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N) {
  const size_t NP = (size_t)(N + kStatPad - 1) / kStatPad * kStatPad;
  return 2 * (size_t)B * H * NP * sizeof(float);
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_bwd_t<128, true>(a, stream) : launch_bwd_t<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch_bwd_t<64, true>(a, stream) : launch_bwd_t<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace attnio
