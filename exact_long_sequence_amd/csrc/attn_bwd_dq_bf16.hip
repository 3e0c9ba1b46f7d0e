// dQ kernel of the bf16 attention backward (gfx950).  Launched by
// launch_bwd_bf16 after the delta kernel has written the row statistics.
//
// One workgroup per (batch*head, 128 queries), 4 waves x 32 queries, in the
// forward's orientation: S^T = K Q^T and dP^T = V dO^T with the wave's 32
// queries across the lanes (lse and D are lane-local); 64-key K/V tiles stream
// through a two-stage LDS ring; dQ^T += K^T dS^T with K^T by transpose reads;
// dQ is scaled and written once.  Causal tiles stop at their diagonal and run
// longest first; a head's tiles share one XCD.  This unit is compiled with the VGPR form of MFMA (the
// products' results feed the VALU directly).

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"
#include "tile_ops.h"

namespace attnio {
namespace {

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1)
void attn_bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                        const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                        const float* __restrict__ ws_d, const float* __restrict__ ws_l,
                        __bf16* __restrict__ dQ, const int32_t* __restrict__ kv_len, int H, int N,
                        int NP, float c, float scale, int n_qtiles) {
  constexpr int WAVES = 4, THREADS = 256, BN = 64, BM = 32 * WAVES;
  constexpr int RB = 2 * D;
  constexpr int KT = BN * RB;       // one K or V tile
  constexpr int STAGE = 2 * KT;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, half = lane / 32, col = lane % 32;
  // XCD-aware assignment (block x runs on XCD x % 8): when B*H is a multiple
  // of 8, head j's query tiles all run on XCD j % 8, so its K and V stream
  // through one L2; causal tiles longest first
  int bh, qt;
  {
    const int G = gridDim.x, x = blockIdx.x, xcd = x % 8, idx = x / 8;
    if ((G / n_qtiles) % 8 == 0) {
      bh = xcd + 8 * (idx / n_qtiles);
      qt = idx % n_qtiles;
    } else {
      bh = x / n_qtiles;
      qt = x % n_qtiles;
    }
  }
  if (CAUSAL) qt = n_qtiles - 1 - qt;
  const int b = bh / H;
  int L = N;
  if (kv_len != nullptr) {
    L = kv_len[b];
    L = L < 0 ? 0 : (L > N ? N : L);
  }
  L = __builtin_amdgcn_readfirstlane(L);
  const int q0 = qt * BM;
  int kend = L;
  if (CAUSAL) kend = min(kend, min(N, q0 + BM));
  const int ntiles = (kend + BN - 1) / BN;
  const size_t slice = (size_t)bh * N * D;
  const int qrow = q0 + wave * 32 + col;  // the query this lane owns
  const int last = CAUSAL ? min(L - 1, qrow) : L - 1;  // its last visible key

  bf16x8 qf[D / 16], dof[D / 16];
  float lse2 = 0.f, dlt = 0.f;
  {
    const int qr = qrow < N ? qrow : N - 1;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] = *(const bf16x8*)(Q + slice + (size_t)qr * D + ks * 16 + half * 8);
      dof[ks] = *(const bf16x8*)(dO + slice + (size_t)qr * D + ks * 16 + half * 8);
    }
    lse2 = ws_l[(size_t)bh * 2 * NP + qr];
    dlt = ws_d[(size_t)bh * 2 * NP + qr];
  }
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(qf[ks]), "v"(dof[ks]));
  asm volatile("" ::"v"(lse2), "v"(dlt));

  f32x16 dqt[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqt[db][r] = 0.f;

  if (ntiles > 0) {
    const __bf16* Ks = K + slice;
    const __bf16* Vs = V + slice;
    auto issue = [&](int t) __attribute__((always_inline)) {
      const uint32_t st = lds_base + (uint32_t)((t & 1) * STAGE);
      dma_rows<D, BN, THREADS>(Ks, t * BN, kend - 1, st, wave, lane);
      dma_rows<D, BN, THREADS>(Vs, t * BN, kend - 1, st + KT, wave, lane);
    };
    issue(0);
    wait_dma();
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      if (t + 1 < ntiles) issue(t + 1);
      const char LDS_AS* kt_l = smem + (t & 1) * STAGE;
      const char LDS_AS* vt_l = kt_l + KT;
      const int j0 = t * BN;
      // S^T = K Q^T and dP^T = V dO^T: lane (h, c) holds keys (r/4)*8 + 4h + r%4
      // of each 32-key block for its query c
      f32x16 s[BN / 32], dp[BN / 32];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { s[kb][r] = 0.f; dp[kb][r] = 0.f; }
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 ak = row_operand<D>(kt_l, kb * 32 + col, ks, half);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[ks], s[kb], 0, 0, 0);
          const bf16x8 av = row_operand<D>(vt_l, kb * 32 + col, ks, half);
          dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, dof[ks], dp[kb], 0, 0, 0);
        }
      }
      // dS^T = P^T (dP^T - D), packed as B operands of dQ^T += K^T dS^T.  Key
      // kk = j0 + 32 kb + 8 (r/4) + 4 half + r%4 is visible iff kk <= last
      // (kk < kv_len and, causal, kk <= the query): one compare of a
      // compile-time constant with the lane's tk per score, selecting the
      // exponent (exp2(-inf) = 0, so dS = 0 too) rather than branching
      const int tk = last - j0 - half * 4;
      bf16x8 pds[BN / 16];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp)
#pragma unroll
          for (int t8 = 0; t8 < 8; ++t8) {
            const int r = sp * 8 + t8;
            const float arg = (kb * 32 + (r / 4) * 8 + (r % 4) <= tk)
                                  ? __builtin_fmaf(s[kb][r], c, -lse2) : -INFINITY;
            const float p = __builtin_amdgcn_exp2f(arg);
            pds[kb * 2 + sp][t8] = (__bf16)(p * (dp[kb][r] - dlt));
          }
#pragma unroll
      for (int st = 0; st < BN / 16; ++st)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 a = tr_operand<D>(kt_l, db, st, lane);
          dqt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pds[st], dqt[db], 0, 0, 0);
        }
      wait_dma();
      __syncthreads();
    }
  }

  if (qrow < N) {
    __bf16* orow = dQ + slice + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)(dqt[db][a4 * 4 + e] * scale);
        *(bf16x4*)(orow + db * 32 + a4 * 8 + half * 4) = o;
      }
  }
}

// Ping-pong form of the same computation (the forward's schedule): one
// workgroup per (batch*head, 256 queries), 8 waves in two groups of four,
// waves w and w + 4 on one SIMD, the groups half a tile apart, so that on
// every SIMD one wave issues
//   MFMA(t) = dQ^T += K(t-1)^T dS(t-1)^T (t >= 1), S^T(t), dP^T(t) (t < ntiles)
// while the other computes P and dS of its previous tile on the VALU.  K has
// three LDS buffers (one MFMA phase reads K(t-1) transposed and K(t) by
// rows), V two.  Group 1 issues the DMA of K(t+1) in its VALU(t-1) and waits
// for it at the end of its MFMA(t); group 0 issues V(t+1) in its VALU(t) and
// waits for it at the end of that half step.  Both buffers were last read in
// MFMA(t-1), which both groups have finished by then.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 2)
void attn_bwd_dq_pp_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                           const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                           const float* __restrict__ ws_d, const float* __restrict__ ws_l,
                           __bf16* __restrict__ dQ, const int32_t* __restrict__ kv_len, int H, int N,
                           int NP, float c, float scale, int n_qtiles) {
  constexpr int WAVES = 8, BN = 64, BM = 32 * WAVES;
  constexpr int RB = 2 * D;
  constexpr int KT = BN * RB;  // one K or V tile
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, half = lane / 32, col = lane % 32;
  const int grp = wave / 4, wl = wave % 4;  // group and wave within it (uniform)
  int bh, qt;
  {
    const int G = gridDim.x, x = blockIdx.x, xcd = x % 8, idx = x / 8;
    if ((G / n_qtiles) % 8 == 0) {
      bh = xcd + 8 * (idx / n_qtiles);
      qt = idx % n_qtiles;
    } else {
      bh = x / n_qtiles;
      qt = x % n_qtiles;
    }
  }
  if (CAUSAL) qt = n_qtiles - 1 - qt;
  const int b = bh / H;
  int L = N;
  if (kv_len != nullptr) {
    L = kv_len[b];
    L = L < 0 ? 0 : (L > N ? N : L);
  }
  L = __builtin_amdgcn_readfirstlane(L);
  const int q0 = qt * BM;
  int kend = L;
  if (CAUSAL) kend = min(kend, min(N, q0 + BM));
  kend = __builtin_amdgcn_readfirstlane(kend);
  const int ntiles = (kend + BN - 1) / BN;
  const size_t slice = (size_t)bh * N * D;
  const int qrow = q0 + wave * 32 + col;
  const int last = CAUSAL ? min(L - 1, qrow) : L - 1;

  bf16x8 qf[D / 16], dof[D / 16];
  float lse2 = 0.f, dlt = 0.f;
  {
    const int qr = qrow < N ? qrow : N - 1;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] = *(const bf16x8*)(Q + slice + (size_t)qr * D + ks * 16 + half * 8);
      dof[ks] = *(const bf16x8*)(dO + slice + (size_t)qr * D + ks * 16 + half * 8);
    }
    lse2 = ws_l[(size_t)bh * 2 * NP + qr];
    dlt = ws_d[(size_t)bh * 2 * NP + qr];
  }
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(qf[ks]), "v"(dof[ks]));
  asm volatile("" ::"v"(lse2), "v"(dlt));

  f32x16 dqt[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqt[db][r] = 0.f;

  if (ntiles > 0) {
    const __bf16* Ks = K + slice;
    const __bf16* Vs = V + slice;
    auto kbuf = [&](int t) __attribute__((always_inline)) { return (uint32_t)((t % 3) * KT); };
    auto vbuf = [&](int t) __attribute__((always_inline)) { return (uint32_t)((3 + (t & 1)) * KT); };
    f32x16 s[BN / 32], dp[BN / 32];
    bf16x8 pds[BN / 16];
    // MFMA phase of tile t (see above) as one stream: the dQ MFMAs of tile
    // t - 1 (A = K(t-1)^T by transpose reads), then S^T(t) and dP^T(t)
    // interleaved (ks outer, so dependent MFMAs are four apart).  LDS operands
    // are read R MFMAs ahead through a register ring and a scheduling barrier
    // after every MFMA pins that distance (left to the compiler, the reads
    // trail the MFMAs and the one MFMA wave of the SIMD stalls on them).
    auto mfma_phase = [&](int t, auto dq_tag, auto sdp_tag) __attribute__((always_inline)) {
      constexpr bool DO_DQ = decltype(dq_tag)::value, DO_SDP = decltype(sdp_tag)::value;
      constexpr int NDQ = DO_DQ ? (BN / 16) * (D / 32) : 0;
      constexpr int NSD = DO_SDP ? (D / 16) * (BN / 32) * 2 : 0;
      constexpr int NM = NDQ + NSD, R = 4;
      const char LDS_AS* kp = smem + kbuf(t + 2);  // K(t - 1): (t - 1) % 3 == (t + 2) % 3
      const char LDS_AS* kt_l = smem + kbuf(t);
      const char LDS_AS* vt_l = smem + vbuf(t);
      auto read = [&](int m) __attribute__((always_inline)) {
        if (m < NDQ) return tr_operand<D>(kp, m % (D / 32), m / (D / 32), lane);
        const int mq = m - NDQ, ks = mq / (2 * (BN / 32)), kb = (mq / 2) % (BN / 32);
        return row_operand<D>((mq % 2) ? vt_l : kt_l, kb * 32 + col, ks, half);
      };
      bf16x8 ring[R + 1];
#pragma unroll
      for (int m = 0; m < R && m < NM; ++m) ring[m] = read(m);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (m + R < NM) ring[(m + R) % (R + 1)] = read(m + R);
        const bf16x8 a = ring[m % (R + 1)];
        if (m < NDQ) {
          const int st = m / (D / 32), db = m % (D / 32);
          dqt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pds[st], dqt[db], 0, 0, 0);
        } else {
          const int mq = m - NDQ, ks = mq / (2 * (BN / 32)), kb = (mq / 2) % (BN / 32);
          const f32x16 zero = {};
          if (mq % 2)
            dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dof[ks], ks == 0 ? zero : dp[kb], 0, 0, 0);
          else
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], ks == 0 ? zero : s[kb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // VALU phase of tile t: dS^T = P^T (dP^T - D) as B operands.  Only tiles
    // that reach past some lane's last visible key (the diagonal, the kv_len
    // tail) test each score (one compare of a constant with tk, as in the
    // kernel above); the wave-uniform test per tile drops the compare and the
    // select from the others (two of the 6.5 VALU operations per score).
    const int wave_last = __builtin_amdgcn_readfirstlane(CAUSAL ? min(L - 1, q0 + wave * 32) : L - 1);
    auto valu_phase = [&](int t) __attribute__((always_inline)) {
      const int tk = last - t * BN - half * 4;
      auto body = [&](auto masked_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int sp = 0; sp < 2; ++sp)
#pragma unroll
            for (int t8 = 0; t8 < 8; ++t8) {
              const int r = sp * 8 + t8;
              const float arg = (!MASKED || kb * 32 + (r / 4) * 8 + (r % 4) <= tk)
                                    ? __builtin_fmaf(s[kb][r], c, -lse2) : -INFINITY;
              const float p = __builtin_amdgcn_exp2f(arg);
              pds[kb * 2 + sp][t8] = (__bf16)(p * (dp[kb][r] - dlt));
            }
      };
      if (t * BN + BN - 1 > wave_last) body(std::true_type{});
      else body(std::false_type{});
    };
    // prologue: K(0), V(0) by all waves; group 1 issues K(1) and passes one
    // extra barrier, which puts it half a tile behind group 0
    dma_rows<D, BN, 64 * WAVES>(Ks, 0, kend - 1, lds_base + kbuf(0), wave, lane);
    dma_rows<D, BN, 64 * WAVES>(Vs, 0, kend - 1, lds_base + vbuf(0), wave, lane);
    wait_dma();
    __syncthreads();
    if (grp == 1) {
      if (1 < ntiles) dma_rows<D, BN, 256>(Ks, BN, kend - 1, lds_base + kbuf(1), wl, lane);
      __syncthreads();
    }
    for (int t = 0; t < ntiles; ++t) {
      __builtin_amdgcn_s_setprio(2);
      if (t > 0) mfma_phase(t, std::true_type{}, std::true_type{});
      else mfma_phase(t, std::false_type{}, std::true_type{});
      __builtin_amdgcn_s_setprio(0);
      if (grp == 1) wait_dma();
      __syncthreads();
      if (grp == 1) {
        if (t + 2 < ntiles)
          dma_rows<D, BN, 256>(Ks, (t + 2) * BN, kend - 1, lds_base + kbuf(t + 2), wl, lane);
      } else {
        if (t + 1 < ntiles)
          dma_rows<D, BN, 256>(Vs, (t + 1) * BN, kend - 1, lds_base + vbuf(t + 1), wl, lane);
      }
      valu_phase(t);
      // keep the VALU work in this half step (its only use is the next dQ MFMAs)
#pragma unroll
      for (int i = 0; i < BN / 16; ++i) asm volatile("" ::"v"(pds[i]));
      if (grp == 0) wait_dma();
      __syncthreads();
    }
    __builtin_amdgcn_s_setprio(2);
    mfma_phase(ntiles, std::true_type{}, std::false_type{});
    __builtin_amdgcn_s_setprio(0);
    if (grp == 0) __syncthreads();  // group 1's last VALU barrier
  }

  if (qrow < N) {
    __bf16* orow = dQ + slice + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)(dqt[db][a4 * 4 + e] * scale);
        *(bf16x4*)(orow + db * 32 + a4 * 8 + half * 4) = o;
      }
  }
}

#ifndef ATTNIO_DQ_PINGPONG
#define ATTNIO_DQ_PINGPONG 1
#endif

template <int D, bool CAUSAL>
hipError_t launch_dq_t(const BwdArgs& a, const float* ws_d, const float* ws_l, int NP, float c,
                       hipStream_t stream) {
  // the ping-pong form at d = 128 only: at d = 64 a tile has half the MFMAs
  // for the same VALU work, and the one-group form measured faster there
  if (ATTNIO_DQ_PINGPONG && D == 128) {
    const int n_qtiles = (a.N + 255) / 256;
    const long long g_q = (long long)a.B * a.H * n_qtiles;
    if (g_q > 0x7fffffffLL) return hipErrorInvalidValue;
    constexpr int q_lds = 5 * 64 * 2 * D;  // three K and two V tiles of 64 rows
    hipLaunchKernelGGL((attn_bwd_dq_pp_kernel<D, CAUSAL>), dim3((unsigned)g_q), dim3(512), q_lds, stream,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                       (const __bf16*)a.dout, ws_d, ws_l, (__bf16*)a.dq, a.kv_len, a.H, a.N, NP, c,
                       a.scale, n_qtiles);
    return hipGetLastError();
  }
  const int n_qtiles = (a.N + 127) / 128;
  const long long g_q = (long long)a.B * a.H * n_qtiles;
  if (g_q > 0x7fffffffLL) return hipErrorInvalidValue;
  constexpr int q_lds = 2 * 2 * 64 * 2 * D;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)g_q), dim3(256), q_lds, stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                     (const __bf16*)a.dout, ws_d, ws_l, (__bf16*)a.dq, a.kv_len, a.H, a.N, NP, c,
                     a.scale, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq_bf16(const BwdArgs& a, const float* ws_d, const float* ws_l, int NP,
                              float c, hipStream_t stream) {
  if (a.d == 128)
    return a.causal ? launch_dq_t<128, true>(a, ws_d, ws_l, NP, c, stream)
                    : launch_dq_t<128, false>(a, ws_d, ws_l, NP, c, stream);
  if (a.d == 64)
    return a.causal ? launch_dq_t<64, true>(a, ws_d, ws_l, NP, c, stream)
                    : launch_dq_t<64, false>(a, ws_d, ws_l, NP, c, stream);
  return hipErrorInvalidValue;
}

}  // namespace attnio
