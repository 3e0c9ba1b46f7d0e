// Exact attention backward for bf16 on gfx950 (CDNA4).
//
// The backward pass recomputes the probabilities from Q, K, V and the per-row
// log-sum-exp of the forward instead of storing them ("IO-Aware Algorithms",
// How it works: recomputation).  With P = exp(s Q K^T - lse) (masked entries
// 0), the gradients are
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D_i = dO_i . O_i,
//     dQ = s dS K,   dK = s dS^T Q.
// Three kernels, enqueued in this order on the caller's stream:
//   delta: D_i = dO_i . O_i and lse_i * log2(e) per row, into the workspace;
//   dk_dv: one workgroup per (batch*head, 128 keys); K and V of those keys stay
//          in registers as MFMA operands while Q, dO and the row statistics of
//          64-row query blocks stream through a two-stage LDS ring (DMA of the
//          next block under the current one);
//   dq:    one workgroup per (batch*head, 128 queries); Q and dO stay in
//          registers while 64-key K/V tiles stream through the LDS ring.
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

// ----------------------------------------------------------------------------
// delta: D_i = dO_i . O_i (fp32) and lse_i * log2(e), per row.
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256)
void attn_bwd_delta_kernel(const __bf16* __restrict__ O, const __bf16* __restrict__ dO,
                           const float* __restrict__ lse, float* __restrict__ ws_d,
                           float* __restrict__ ws_l, int N, int NP, long long rows) {
  constexpr int LPR = D / 8;  // lanes per row, 16 bytes each
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid / LPR;
  const int part = (int)(gid % LPR);
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 o = *(const bf16x8*)(O + row * D + part * 8);
    const bf16x8 g = *(const bf16x8*)(dO + row * D + part * 8);
#pragma unroll
    for (int t = 0; t < 8; ++t) acc = __builtin_fmaf((float)o[t], (float)g[t], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off /= 2) acc += __shfl_xor(acc, off, LPR);
  if (row < rows && part == 0) {
    const long long bh = row / N, i = row % N;
    ws_d[bh * NP + i] = acc;
    ws_l[bh * NP + i] = lse[row] * kLog2e;
  }
}

// ----------------------------------------------------------------------------
// dk_dv: 4 waves x 32 keys; 64-row query blocks through a two-stage LDS ring.
// ----------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1)
void attn_bwd_dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                          const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                          const float* __restrict__ ws_d, long long l_off,
                          __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                          const int32_t* __restrict__ kv_len, int H, int N, int NP, float c,
                          float scale, int n_kblocks) {
  constexpr int WAVES = 4, THREADS = 256, BQ = 64, BKV = 32 * WAVES;
  constexpr int RB = 2 * D;
  constexpr int QT = BQ * RB;             // one Q or dO tile
  constexpr int STAGE = 2 * QT + 1024;    // Q, dO, row statistics
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, half = lane / 32, col = lane % 32;
  const int bh = blockIdx.x / n_kblocks, kblk = blockIdx.x % n_kblocks;
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
    auto issue = [&](int i) __attribute__((always_inline)) {
      const int q0 = (qb0 + i) * BQ;
      const uint32_t st = lds_base + (uint32_t)((i & 1) * STAGE);
      dma_rows<D, BQ, THREADS>(Qs, q0, N - 1, st, wave, lane);
      dma_rows<D, BQ, THREADS>(dOs, q0, N - 1, st + QT, wave, lane);
      if (wave == 0) {
        // lanes 0-15: lse*log2e of the 64 rows, 16-31: D, 32-63 repeat 0-31
        // (the two workspace arrays are l_off floats apart)
        const int sub = lane % 32;
        const uint32_t off = (uint32_t)(((sub < 16 ? l_off : 0LL) + (long long)bh * NP + q0 + 4 * (sub % 16)) * 4);
        dma16(ws_d, off, __builtin_amdgcn_readfirstlane(st + 2 * QT));
      }
    };
    issue(0);
    wait_dma();
    __syncthreads();
    for (int i = 0; i < nqb; ++i) {
      if (i + 1 < nqb) issue(i + 1);
      const char LDS_AS* qt_l = smem + (i & 1) * STAGE;
      const char LDS_AS* dot_l = qt_l + QT;
      const float LDS_AS* st_l = (const float LDS_AS*)(qt_l + 2 * QT);
      const int q0 = (qb0 + i) * BQ;

      // S = Q K^T and dP = dO V^T for two 32-row blocks; lane (h, c) holds
      // rows (r/4)*8 + 4h + r%4 of each block, column = its key
      f32x16 s[2], dp[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { s[blk][r] = 0.f; dp[blk][r] = 0.f; }
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 aq = row_operand<D>(qt_l, blk * 32 + col, ks, half);
          s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[ks], s[blk], 0, 0, 0);
          const bf16x8 ad = row_operand<D>(dot_l, blk * 32 + col, ks, half);
          dp[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, vf[ks], dp[blk], 0, 0, 0);
        }
      }
      // P = 2^(S c - lse2), dS = P (dP - D); packed as B operands of the
      // query-contracting products: operand st covers rows 16 st .. 16 st + 15
      bf16x8 pp[BQ / 16], pds[BQ / 16];
      const bool key_ok = key < L;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int ql = blk * 32 + a4 * 8 + half * 4;  // first of four consecutive rows
          const f32x4 l4 = *(const f32x4 LDS_AS*)(st_l + ql);
          const f32x4 d4 = *(const f32x4 LDS_AS*)(st_l + 64 + ql);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = a4 * 4 + e;
            const int q = q0 + ql + e;
            bool ok = key_ok && q < N;
            if (CAUSAL) ok = ok && key <= q;
            const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][r], c, -l4[e])) : 0.f;
            const float ds = ok ? p * (dp[blk][r] - d4[e]) : 0.f;
            const int st = blk * 2 + a4 / 2, t8 = (a4 % 2) * 4 + e;
            pp[st][t8] = (__bf16)p;
            pds[st][t8] = (__bf16)ds;
          }
        }
      // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
      for (int st = 0; st < BQ / 16; ++st)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 a1 = tr_operand<D>(dot_l, db, st, lane);
          dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, pp[st], dvt[db], 0, 0, 0);
          const bf16x8 a2 = tr_operand<D>(qt_l, db, st, lane);
          dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, pds[st], dkt[db], 0, 0, 0);
        }
      wait_dma();
      __syncthreads();
    }
  }

  // lane (h, c) holds rows db*32 + (r/4)*8 + 4h + r%4 (head dimension) of its key
  if (key < N) {
    __bf16* krow = dK + slice + (size_t)key * D;
    __bf16* vrow = dV + slice + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 ok4, ov4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ok4[e] = (__bf16)(dkt[db][a4 * 4 + e] * scale);
          ov4[e] = (__bf16)(dvt[db][a4 * 4 + e]);
        }
        *(bf16x4*)(krow + db * 32 + a4 * 8 + half * 4) = ok4;
        *(bf16x4*)(vrow + db * 32 + a4 * 8 + half * 4) = ov4;
      }
  }
}

// ----------------------------------------------------------------------------
// dq: 4 waves x 32 queries; 64-key K/V tiles through a two-stage LDS ring.
// ----------------------------------------------------------------------------
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
  const int bh = blockIdx.x / n_qtiles;
  int qt = blockIdx.x % n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest first
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

  bf16x8 qf[D / 16], dof[D / 16];
  float lse2 = 0.f, dlt = 0.f;
  {
    const int qr = qrow < N ? qrow : N - 1;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] = *(const bf16x8*)(Q + slice + (size_t)qr * D + ks * 16 + half * 8);
      dof[ks] = *(const bf16x8*)(dO + slice + (size_t)qr * D + ks * 16 + half * 8);
    }
    lse2 = ws_l[(size_t)bh * NP + qr];
    dlt = ws_d[(size_t)bh * NP + qr];
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
      // dS^T = P^T (dP^T - D), packed as B operands of dQ^T += K^T dS^T
      bf16x8 pds[BN / 16];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp)
#pragma unroll
          for (int t8 = 0; t8 < 8; ++t8) {
            const int r = sp * 8 + t8;
            const int kk = j0 + kb * 32 + (r / 4) * 8 + half * 4 + (r % 4);
            bool ok = kk < L;
            if (CAUSAL) ok = ok && kk <= qrow;
            const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -lse2)) : 0.f;
            pds[kb * 2 + sp][t8] = (__bf16)(ok ? p * (dp[kb][r] - dlt) : 0.f);
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

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const int NP = (a.N + kStatPad - 1) / kStatPad * kStatPad;
  float* ws_d = a.ws;
  float* ws_l = a.ws + (size_t)a.B * a.H * NP;
  const long long rows = (long long)a.B * a.H * a.N;
  const long long dgrid = (rows * (D / 8) + 255) / 256;
  const int n_kblocks = (a.N + 127) / 128;
  const int n_qtiles = (a.N + 127) / 128;
  const long long g_kv = (long long)a.B * a.H * n_kblocks;
  const long long g_q = (long long)a.B * a.H * n_qtiles;
  if (dgrid > 0x7fffffffLL || g_kv > 0x7fffffffLL || g_q > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c = a.scale * kLog2e;
  hipLaunchKernelGGL((attn_bwd_delta_kernel<D>), dim3((unsigned)dgrid), dim3(256), 0, stream,
                     (const __bf16*)a.o, (const __bf16*)a.dout, a.lse, ws_d, ws_l, a.N, NP, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int kv_lds = 2 * (2 * 64 * 2 * D + 1024);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)g_kv), dim3(256), kv_lds,
                     stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                     (const __bf16*)a.dout, ws_d, (long long)(ws_l - ws_d), (__bf16*)a.dk,
                     (__bf16*)a.dv, a.kv_len, a.H, a.N, NP, c, a.scale, n_kblocks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int q_lds = 2 * 2 * 64 * 2 * D;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)g_q), dim3(256), q_lds, stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                     (const __bf16*)a.dout, ws_d, ws_l, (__bf16*)a.dq, a.kv_len, a.H, a.N, NP, c,
                     a.scale, n_qtiles);
  return hipGetLastError();
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
