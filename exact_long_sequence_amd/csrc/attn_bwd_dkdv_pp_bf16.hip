// dK/dV kernel of the bf16 attention backward in the ping-pong form (gfx950).
// Launched by launch_bwd_bf16 after the delta kernel has written the row
// statistics; computes the same dV = P^T dO and dK = s dS^T Q as the one-wave
// form in attn_bwd_bf16.hip ("IO-Aware Algorithms", How it works:
// recomputation), with the same orientation (the wave's 32 keys across the
// lanes, P and dS in the B-operand layout of dV^T += dO^T P, dK^T += Q^T dS).
//
// One workgroup per (batch*head, 128 keys), 8 waves in two groups of four;
// waves w and w + 4 share a SIMD and own the same 32 keys.  K and V of the
// workgroup's keys stay in LDS for the whole loop (read as B operands of S and
// dP), and 32-row blocks of Q, dO and their row statistics stream through a
// five-buffer LDS ring.  Group 0 takes the even blocks, group 1 the odd ones,
// half a block apart, so that on every SIMD one wave issues
//   MFMA(j) = dV^T, dK^T += (block j-1 of the group) and S, dP of block j
// while the other computes P and dS of its previous block on the VALU.  Each
// group accumulates dK^T and dV^T of its blocks in registers; at the end the
// two partial sums meet in LDS (fp32) and each group stores one of dK, dV.
//
// Ring hand-over.  Half steps are numbered by workgroup barriers (barrier h
// ends half step h); block X (of the loop) is read in half steps X+1 (S and
// dP by rows), X+2 (its statistics, VALU) and X+3 (dV, dK by transpose
// reads), so it lives in buffer X % 5 and the buffer is free from half step
// X+4.  In half step h the group on the VALU issues the DMA of block h+1 at
// the start of its phase and waits for it at the end of its next (MFMA) half
// step h+1: the buffer's previous block h-4 was last read in half step h-1,
// and block h+1 is first read in half step h+2.

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"
#include "tile_ops.h"

namespace attnio {
namespace {

template <int D>
struct KvPpCfg {
  static constexpr int WAVES = 8, THREADS = 512, BQ = 32, BKV = 128, NBUF = 5;
  static constexpr int RB = 2 * D;
  static constexpr int KVT = BKV * RB;          // the K or the V tile of the workgroup's keys
  static constexpr int QT = BQ * RB;            // one Q or dO block
  static constexpr int STAGE = 2 * QT + 1024;   // Q, dO, row statistics (one 64-lane load)
  static constexpr int RING = 2 * KVT;          // ring offset
  static constexpr int LDS_LOOP = RING + NBUF * STAGE;
  static constexpr int RED = 2 * BKV * D * 4;   // dK^T and dV^T partial sums, fp32
  static constexpr int LDS = LDS_LOOP > RED ? LDS_LOOP : RED;
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 2)
void attn_bwd_dkdv_pp_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                             const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                             const float* __restrict__ ws_d,
                             __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                             const int32_t* __restrict__ kv_len, int H, int N, int NP, float c,
                             float scale, int n_kblocks) {
  using C = KvPpCfg<D>;
  constexpr int BQ = C::BQ, QT = C::QT, KVT = C::KVT;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, half = lane / 32, col = lane % 32;
  const int grp = wave / 4, wl = wave % 4;  // group and wave within it (uniform)
  // XCD-aware assignment (block x runs on XCD x % 8): when B*H is a multiple
  // of 8, head j's key blocks all run on XCD j % 8, key block 0 (the longest
  // causal loop) first
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
  const int k0 = kblk * C::BKV;
  const int key = k0 + wl * 32 + col;  // the key this lane owns
  const size_t slice = (size_t)bh * N * D;

  f32x16 dkt[D / 32], dvt[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dkt[db][r] = 0.f; dvt[db][r] = 0.f; }

  if (k0 < L) {
    const int qb0 = CAUSAL ? k0 / BQ : 0;
    const int nqb = __builtin_amdgcn_readfirstlane((N + BQ - 1) / BQ - qb0);
    const __bf16* Qs = Q + slice;
    const __bf16* dOs = dO + slice;
    const float* stats = ws_d + (size_t)bh * 2 * NP;
    auto stage_off = [&](int X) __attribute__((always_inline)) {
      return (uint32_t)(C::RING + (X % C::NBUF) * C::STAGE);
    };
    // DMA of block X (Q, dO, statistics) by the four waves of one group
    auto issue = [&](int X) __attribute__((always_inline)) {
      const int q0 = (qb0 + X) * BQ;
      const uint32_t st = lds_base + stage_off(X);
      dma_rows<D, BQ, 256>(Qs, q0, N - 1, st, wl, lane);
      dma_rows<D, BQ, 256>(dOs, q0, N - 1, st + QT, wl, lane);
      if (wl == 0) {
        // lanes 0-7: lse*log2e of the 32 rows, lanes 8-15: D, the rest repeat
        // them; the offset stays below 2 * NP * 4 bytes (q0 + 32 <= NP)
        const int sub = lane % 16;
        const uint32_t off = ((sub < 8 ? (uint32_t)NP : 0u) + (uint32_t)(q0 + 4 * (sub % 8))) * 4u;
        dma16(stats, off, __builtin_amdgcn_readfirstlane(st + 2 * QT));
      }
    };

    f32x16 s, dp;
    bf16x8 pp[BQ / 16], pds[BQ / 16];

    // Per-lane LDS byte offsets of the operand reads, relative to a tile's
    // base.  A row read (row_operand) of row `col` at k step ks sits at
    // rl[ks]; the same offset serves the K and V rows of the wave's keys
    // (row wl*32 + col has the swizzle of row col).  The two transpose reads
    // of d block db (tr_operand) sit at trl[db][u] + 16 st * RB (the swizzle
    // does not depend on st).  Only these are kept in registers; the tile
    // base and the constant parts go into the instruction's offset.
    constexpr int RB = C::RB;
    uint32_t rl[D / 16], trl[D / 32][2];
    {
      const int g = lane / 16, jr = (lane % 16) / 4, qq = lane % 4;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        rl[ks] = (uint32_t)(col * RB + (((2 * ks + half) ^ swz<D>(col)) * 16));
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int row = u * 8 + half * 4 + jr;
          const int colb = (db * 32 + (g % 2) * 16 + qq * 4) * 2;
          trl[db][u] = (uint32_t)(row * RB + ((colb / 16) ^ swz<D>(row)) * 16 + (colb % 16));
        }
    }
    auto rd_row = [&](uint32_t base, uint32_t off) __attribute__((always_inline)) {
      return *(const bf16x8 LDS_AS*)(smem + (base + off));
    };
    auto rd_tr = [&](uint32_t base, int db, int st) __attribute__((always_inline)) {
      bf16x8 a;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4 LDS_AS*)(smem + (base + trl[db][u]) + st * 16 * RB));
        const bf16x4 vb = __builtin_bit_cast(bf16x4, v4);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[u * 4 + e] = vb[e];
      }
      return a;
    };

    // MFMA phase of the group's block X as one stream: the dV / dK MFMAs of
    // its previous block X-2 (A = dO^T or Q^T by transpose reads, B = P or dS
    // from registers) alternate with the S / dP MFMAs of block X (A = Q or dO
    // rows, B = K or V rows of the wave's keys), so dependent MFMAs are at
    // least four apart.  Operands are read R MFMAs ahead through register
    // rings; a scheduling barrier after every MFMA pins that distance.
    auto mfma_phase = [&](int X, auto dv_tag, auto sd_tag) __attribute__((always_inline)) {
      constexpr bool DO_DV = decltype(dv_tag)::value, DO_SD = decltype(sd_tag)::value;
      constexpr int NDV = DO_DV ? (BQ / 16) * (D / 32) * 2 : 0;
      constexpr int NSD = DO_SD ? (D / 16) * 2 : 0;
      static_assert(!(DO_DV && DO_SD) || NDV == NSD, "one-to-one interleave");
      constexpr int NM = NDV + NSD, R = 4;
      // opaque copies: the offsets are not expanded into one register per read
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+v"(rl[ks]));
#pragma unroll
      for (int db = 0; db < D / 32; ++db) asm volatile("" : "+v"(trl[db][0]), "+v"(trl[db][1]));
      const uint32_t cur = stage_off(X);
      const uint32_t prv = stage_off(X + 2 * C::NBUF - 2);  // block X - 2
      const uint32_t kvb = (uint32_t)(wl * 32 * RB);
      auto is_sd = [&](int m) __attribute__((always_inline)) {
        return NDV == 0 ? true : (NSD == 0 ? false : m % 2 == 0);
      };
      auto idx = [&](int m) __attribute__((always_inline)) { return (NDV && NSD) ? m / 2 : m; };
      auto read_a = [&](int m) __attribute__((always_inline)) {
        const int n = idx(m);
        if (is_sd(m)) return rd_row(cur + ((n % 2) ? QT : 0), rl[n / 2]);
        const int which = n % 2, db = (n / 2) % (D / 32), st = n / 2 / (D / 32);
        return rd_tr(which ? prv : prv + QT, db, st);
      };
      auto read_b = [&](int m) __attribute__((always_inline)) {
        const int n = idx(m);
        return rd_row(kvb + ((n % 2) ? KVT : 0), rl[n / 2]);
      };
      bf16x8 ra[R + 1], rb[R + 1];
#pragma unroll
      for (int m = 0; m < R && m < NM; ++m) {
        ra[m] = read_a(m);
        if (is_sd(m)) rb[m] = read_b(m);
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (m + R < NM) {
          ra[(m + R) % (R + 1)] = read_a(m + R);
          if (is_sd(m + R)) rb[(m + R) % (R + 1)] = read_b(m + R);
        }
        const int n = idx(m);
        const bf16x8 a = ra[m % (R + 1)];
        if (is_sd(m)) {
          const int ks = n / 2;
          const f32x16 zero = {};
          if (n % 2)
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, rb[m % (R + 1)], ks == 0 ? zero : dp, 0, 0, 0);
          else
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, rb[m % (R + 1)], ks == 0 ? zero : s, 0, 0, 0);
        } else {
          const int which = n % 2, db = (n / 2) % (D / 32), st = n / 2 / (D / 32);
          if (which == 0)
            dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pp[st], dvt[db], 0, 0, 0);
          else
            dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pds[st], dkt[db], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // VALU phase of block X: P = 2^(s c - lse*log2e) and dS = P (dP - D) of
    // the lane's key against the block's 32 rows, packed as the B operands of
    // the dV / dK MFMAs (operand st covers block rows 16 st .. 16 st + 15).
    // Rows at or past N need no mask (their statistics lse = +inf, D = 0 give
    // P = dS = 0); keys at or past kv_len need none (their gradients are
    // stored as zero).  Causal: block X meets or precedes the diagonal of the
    // wave's keys iff X <= wl (a wave-uniform test); only those blocks compare
    // key <= row per score, selecting the exponent so that no branch forms.
    auto valu_phase = [&](int X, auto mask_tag) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(mask_tag)::value;
      const float LDS_AS* st_f = (const float LDS_AS*)(smem + stage_off(X) + 2 * QT);
      const int tq = key - (qb0 + X) * BQ - half * 4;
      f32x4 l4, d4;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int a4 = r / 4, e = r % 4;
        const int ql = a4 * 8 + half * 4;  // first of four consecutive rows
        if (e == 0) {
          l4 = *(const f32x4 LDS_AS*)(st_f + ql);
          d4 = *(const f32x4 LDS_AS*)(st_f + BQ + ql);
        }
        float arg = __builtin_fmaf(s[r], c, -l4[e]);
        if (MASKED) arg = (tq <= a4 * 8 + e) ? arg : -INFINITY;
        const float p = __builtin_amdgcn_exp2f(arg);
        const float ds = p * (dp[r] - d4[e]);
        const int st = a4 / 2, t8 = (a4 % 2) * 4 + e;
        pp[st][t8] = (__bf16)p;
        pds[st][t8] = (__bf16)ds;
      }
    };

    // prologue: K and V of the keys by all waves, block 0 by group 0, block 1
    // by group 1; then group 1 issues block 2 and passes one extra barrier,
    // which puts it half a step behind group 0
    dma_rows<D, C::BKV, C::THREADS>(K + slice, k0, N - 1, lds_base, wave, lane);
    dma_rows<D, C::BKV, C::THREADS>(V + slice, k0, N - 1, lds_base + KVT, wave, lane);
    if (grp < nqb) issue(grp);
    wait_dma();
    __syncthreads();
    if (grp == 1) {
      if (2 < nqb) issue(2);
      __syncthreads();
    }
    // group g owns blocks g, g + 2, ...: n_g of them.  The first two steps
    // are peeled (step 0 has no previous block; only steps 0 and 1 can meet
    // the causal diagonal, X <= wl <= 3), so the loop body is one straight
    // stream whose accumulators stay in place.
    const int ng = grp ? nqb / 2 : (nqb + 1) / 2;
    using yes = std::true_type;
    using no = std::false_type;
    auto step = [&](int j, auto dv_tag, auto diag_tag) __attribute__((always_inline)) {
      const int X = 2 * j + grp;
      __builtin_amdgcn_s_setprio(2);
      mfma_phase(X, dv_tag, yes{});
      __builtin_amdgcn_s_setprio(0);
      wait_dma();
      __syncthreads();
      if (X + 3 < nqb) issue(X + 3);
      if (CAUSAL && decltype(diag_tag)::value && X <= wl) valu_phase(X, yes{});
      else valu_phase(X, no{});
      // keep the VALU work in this half step (its only use is the next MFMAs)
#pragma unroll
      for (int i = 0; i < BQ / 16; ++i) asm volatile("" ::"v"(pp[i]), "v"(pds[i]));
      __syncthreads();
    };
    if (ng > 0) step(0, no{}, yes{});
    if (ng > 1) step(1, yes{}, yes{});
    for (int j = 2; j < ng; ++j) step(j, yes{}, no{});
    // the dV / dK MFMAs of the group's last block, then the barriers that
    // even the counts: 1 + 2 n_0 + e_0 = 2 + 2 n_1 + e_1 with e_0 = 1 when
    // nqb is even (group 1's tail comes half a step after group 0's), e_1 = 1
    // when nqb is odd (group 1 has one block fewer)
    if (ng > 0) {
      __builtin_amdgcn_s_setprio(2);
      mfma_phase(2 * ng + grp, yes{}, no{});
      __builtin_amdgcn_s_setprio(0);
    }
    if ((nqb % 2 == 0) == (grp == 0)) __syncthreads();
    wait_dma();
    __syncthreads();  // every ring read is done: the LDS is free
  }

  // The two groups' partial sums: group 1 hands its dK^T to group 0 and group
  // 0 its dV^T to group 1 through LDS (lane-major, one 16-byte chunk per lane
  // and MFMA row quad), then group 0 stores dK and group 1 stores dV.
  {
    float LDS_AS* red = (float LDS_AS*)smem;
    constexpr int PART = C::BKV * D;  // floats of one partial sum
    auto at = [&](int db, int a4) __attribute__((always_inline)) {
      return (((wl * (D / 32) + db) * 4 + a4) * 64 + lane) * 4;
    };
    auto put = [&](const f32x16 (&acc)[D / 32], float LDS_AS* out) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = acc[db][a4 * 4 + e];
          *(f32x4 LDS_AS*)(out + at(db, a4)) = v4;
        }
    };
    // lane (h, c) holds rows db*32 + (r/4)*8 + 4h + r%4 (head dimension) of
    // its key; a key at or past kv_len gets zero gradients (its sums, built
    // without a key mask, are discarded, not multiplied)
    auto add_store = [&](const f32x16 (&acc)[D / 32], const float LDS_AS* in, __bf16* dst, float mul)
        __attribute__((always_inline)) {
      if (key >= N) return;
      const bool key_ok = key < L;
      __bf16* row = dst + slice + (size_t)key * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 o4 = *(const f32x4 LDS_AS*)(in + at(db, a4));
          bf16x4 w4;
#pragma unroll
          for (int e = 0; e < 4; ++e) w4[e] = (__bf16)(key_ok ? (acc[db][a4 * 4 + e] + o4[e]) * mul : 0.f);
          *(bf16x4*)(row + db * 32 + a4 * 8 + half * 4) = w4;
        }
    };
    if (grp) put(dkt, red);
    else put(dvt, red + PART);
    __syncthreads();
    if (grp) add_store(dvt, red + PART, dV, 1.f);
    else add_store(dkt, red, dK, scale);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_t(const BwdArgs& a, const float* ws_d, int NP, float c, hipStream_t stream) {
  const int n_kblocks = (a.N + KvPpCfg<D>::BKV - 1) / KvPpCfg<D>::BKV;
  const long long g_kv = (long long)a.B * a.H * n_kblocks;
  if (g_kv > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_bwd_dkdv_pp_kernel<D, CAUSAL>), dim3((unsigned)g_kv), dim3(512),
                     KvPpCfg<D>::LDS, stream, (const __bf16*)a.q, (const __bf16*)a.k,
                     (const __bf16*)a.v, (const __bf16*)a.dout, ws_d, (__bf16*)a.dk, (__bf16*)a.dv,
                     a.kv_len, a.H, a.N, NP, c, a.scale, n_kblocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dkdv_pp_bf16(const BwdArgs& a, const float* ws_d, int NP, float c,
                                   hipStream_t stream) {
  if (a.d == 128)
    return a.causal ? launch_t<128, true>(a, ws_d, NP, c, stream) : launch_t<128, false>(a, ws_d, NP, c, stream);
  if (a.d == 64)
    return a.causal ? launch_t<64, true>(a, ws_d, NP, c, stream) : launch_t<64, false>(a, ws_d, NP, c, stream);
  return hipErrorInvalidValue;
}

}  // namespace attnio
