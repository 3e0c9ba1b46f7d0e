// Operator-centric (unfused) attention forward for bf16 on gfx950: the
// baseline the fused kernel is measured against.
//
// "From Attention Graph to FlashAttention - A Memory-Centric Compilation
// Approach in AICF", section 2, describes this execution: every operator of
// the graph is its own kernel and hands its result to the next one through
// memory.  Here that is three kernels per group of heads:
//   scores:  S = scale * Q K^T, the full N x N block of every head, written to
//            HBM in fp32 (the MFMA accumulator type, so the scores keep their
//            precision);
//   softmax: per query row, the mask (causal, key padding) and a two-pass
//            softmax over the row of S (pass 1 online max / sum, pass 2 the
//            normalised probabilities), P written to HBM in bf16;
//   pv:      O = P V, a dense product over all N keys.
// The mask is applied inside the softmax kernel rather than as a kernel of its
// own; every other operator boundary is a round trip through HBM.  Per head
// the intermediates cost 4 N^2 (S write) + 4 N^2 (S read, once per softmax
// pass that misses the caches) + 2 N^2 (P write) + 2 N^2 (P read) bytes, the
// Theta(N^2) traffic that the fused kernel replaces with Theta(N d)
// ("IO-Aware Algorithms", How it works).
//
// Every product is a bf16 MFMA 32x32x16 with fp32 accumulation.

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "kernels.h"
#include "tile_ops.h"

namespace attnio {
namespace {

// ----------------------------------------------------------------------------
// scores: one workgroup per (128 x 128 block of S, head); 4 waves, each a
// 64 x 64 quarter as 2 x 2 MFMA tiles.  Operands come straight from global
// memory: a lane reads 16 contiguous bytes of one row of Q or K per k step.
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256)
void unf_scores_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                       float* __restrict__ S, int N, int nt, float scale) {
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, half = lane / 32, col = lane % 32;
  const int ti = blockIdx.x / nt, tj = blockIdx.x % nt;
  const size_t head = blockIdx.y;  // head within this pass
  const __bf16* Qh = Q + head * (size_t)N * D;
  const __bf16* Kh = K + head * (size_t)N * D;
  const int r0 = ti * 128 + (wave / 2) * 64;
  const int c0 = tj * 128 + (wave % 2) * 64;

  f32x16 acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

  int qr[2], kr[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = r0 + m * 32 + col, j = c0 + m * 32 + col;
    qr[m] = i < N ? i : N - 1;
    kr[m] = j < N ? j : N - 1;
  }
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    bf16x8 a[2], b[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      a[m] = *(const bf16x8*)(Qh + (size_t)qr[m] * D + ks * 16 + half * 8);
      b[m] = *(const bf16x8*)(Kh + (size_t)kr[m] * D + ks * 16 + half * 8);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], b[n], acc[m][n], 0, 0, 0);
  }
  // lane (h, c) holds rows (r/4)*8 + 4h + r%4 of each 32-row tile, column c
  float* Sh = S + head * (size_t)N * N;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int j = c0 + n * 32 + col;
    if (j >= N) continue;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = r0 + m * 32 + (r / 4) * 8 + half * 4 + (r % 4);
        if (i < N) Sh[(size_t)i * N + j] = acc[m][n][r] * scale;
      }
  }
}

// ----------------------------------------------------------------------------
// softmax: one workgroup per (query row, head).  Pass 1 keeps an online
// (max, sum) per thread over the row's visible scores and merges them across
// the workgroup; pass 2 writes exp(s - max) / sum for visible keys and 0 for
// masked ones.  VEC: rows start on 16-byte boundaries (N % 4 == 0).
// ----------------------------------------------------------------------------
template <bool VEC>
__global__ __launch_bounds__(256)
void unf_softmax_kernel(const float* __restrict__ S, __bf16* __restrict__ P,
                        const int32_t* __restrict__ kv_len, int N, int H, int bh0, int causal) {
  const int i = blockIdx.x;
  const size_t head = blockIdx.y;
  const int b = (bh0 + (int)head) / H;
  int L = N;
  if (kv_len != nullptr) {
    L = kv_len[b];
    L = L < 0 ? 0 : (L > N ? N : L);
  }
  const int kend = causal ? (L < i + 1 ? L : i + 1) : L;
  const float* row = S + head * (size_t)N * N + (size_t)i * N;
  __bf16* prow = P + head * (size_t)N * N + (size_t)i * N;
  const int tid = threadIdx.x;

  float m = -INFINITY, l = 0.f;
  auto add = [&](float x) __attribute__((always_inline)) {
    if (x > m) {
      l = l * __builtin_amdgcn_exp2f((m - x) * kLog2e) + 1.f;
      m = x;
    } else {
      l += __builtin_amdgcn_exp2f((x - m) * kLog2e);
    }
  };
  if (VEC) {
    for (int j = tid * 4; j < kend; j += 1024) {
      const f32x4 x = *(const f32x4*)(row + j);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < kend) add(x[e]);
    }
  } else {
    for (int j = tid; j < kend; j += 256) add(row[j]);
  }
  // merge (m, l) over the wave, then over the four waves through LDS
#pragma unroll
  for (int off = 32; off > 0; off /= 2) {
    const float mo = __shfl_xor(m, off), lo = __shfl_xor(l, off);
    const float mn = m > mo ? m : mo;
    const float sc = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mn) * kLog2e);
    const float so = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mo - mn) * kLog2e);
    l = l * sc + lo * so;
    m = mn;
  }
  __shared__ float red[8];
  if (tid % 64 == 0) {
    red[tid / 64] = m;
    red[4 + tid / 64] = l;
  }
  __syncthreads();
  float mt = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) mt = mt > red[w] ? mt : red[w];
  float lt = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (red[w] != -INFINITY) lt += red[4 + w] * __builtin_amdgcn_exp2f((red[w] - mt) * kLog2e);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;

  if (VEC) {
    for (int j = tid * 4; j < N; j += 1024) {
      bf16x4 o;
      if (j < kend) {
        const f32x4 x = *(const f32x4*)(row + j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = (__bf16)(j + e < kend ? __builtin_amdgcn_exp2f((x[e] - mt) * kLog2e) * inv : 0.f);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)0.f;
      }
      *(bf16x4*)(prow + j) = o;
    }
  } else {
    for (int j = tid; j < N; j += 256)
      prow[j] = (__bf16)(j < kend ? __builtin_amdgcn_exp2f((row[j] - mt) * kLog2e) * inv : 0.f);
  }
}

// ----------------------------------------------------------------------------
// pv: one workgroup per (128 query rows, head), 4 waves x 32 rows, computing
// O^T = V^T P^T over all N keys in 64-key steps.  V tiles go to LDS by
// direct-to-LDS loads (two stages) and are read transposed; P^T operands come
// from global memory, two 4-key groups per lane in the row order of the
// transposed V reads.  VEC: P rows start on 8-byte boundaries (N % 4 == 0).
// ----------------------------------------------------------------------------
template <int D, bool VEC>
__global__ __launch_bounds__(256)
void unf_pv_kernel(const __bf16* __restrict__ P, const __bf16* __restrict__ V,
                   __bf16* __restrict__ O, int N, int nqt) {
  constexpr int THREADS = 256, BK = 64, RB = 2 * D;
  constexpr int VT = BK * RB;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, half = lane / 32, col = lane % 32;
  const size_t head = blockIdx.y;
  const int q = blockIdx.x * 128 + wave * 32 + col;
  const int qc = q < N ? q : N - 1;
  const __bf16* prow = P + head * (size_t)N * N + (size_t)qc * N;
  const __bf16* Vh = V + head * (size_t)N * D;
  const int ntiles = (N + BK - 1) / BK;

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  auto issue = [&](int t) __attribute__((always_inline)) {
    dma_rows<D, BK, THREADS>(Vh, t * BK, N - 1, lds_base + (uint32_t)((t & 1) * VT), wave, lane);
  };
  issue(0);
  wait_dma();
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) issue(t + 1);
    const char LDS_AS* vt = smem + (t & 1) * VT;
    const int k0 = t * BK;
#pragma unroll
    for (int st = 0; st < BK / 16; ++st) {
      bf16x8 pb;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int k = k0 + st * 16 + u * 8 + half * 4;  // four consecutive keys
        if (VEC && k + 4 <= N) {
          const bf16x4 p4 = *(const bf16x4*)(prow + k);
#pragma unroll
          for (int e = 0; e < 4; ++e) pb[u * 4 + e] = p4[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) pb[u * 4 + e] = k + e < N ? prow[k + e] : (__bf16)0.f;
        }
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(vt, db, st, lane), pb,
                                                          acc[db], 0, 0, 0);
    }
    wait_dma();
    __syncthreads();
  }
  // lane (h, c) holds O[q][db*32 + (r/4)*8 + 4h + r%4]
  if (q < N) {
    __bf16* orow = O + head * (size_t)N * D + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)acc[db][a4 * 4 + e];
        *(bf16x4*)(orow + db * 32 + a4 * 8 + half * 4) = o;
      }
  }
}

template <int D>
hipError_t launch_unfused_t(const UnfusedArgs& a, hipStream_t stream) {
  const size_t per_head = unfused_head_bytes(a.N);
  const int BH = a.B * a.H;
  const size_t fit = a.ws_bytes / per_head;
  size_t hp_lim = fit < (size_t)BH ? fit : (size_t)BH;
  if (hp_lim > 65535) hp_lim = 65535;  // heads of one pass ride on grid.y
  const int hp_max = (int)hp_lim;
  if (hp_max < 1) return hipErrorInvalidValue;
  const int nt = (a.N + 127) / 128;
  if ((long long)nt * nt > 0x7fffffffLL) return hipErrorInvalidValue;
  const size_t nn = (size_t)a.N * a.N;
  float* S = (float*)a.ws;
  __bf16* P = (__bf16*)((char*)a.ws + (size_t)hp_max * nn * sizeof(float));
  const bool vec = a.N % 4 == 0;
  for (int bh0 = 0; bh0 < BH; bh0 += hp_max) {
    const int hp = BH - bh0 < hp_max ? BH - bh0 : hp_max;
    const size_t off = (size_t)bh0 * a.N * D;
    hipLaunchKernelGGL((unf_scores_kernel<D>), dim3((unsigned)(nt * nt), (unsigned)hp), dim3(256), 0,
                       stream, (const __bf16*)a.q + off, (const __bf16*)a.k + off, S, a.N, nt, a.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (vec)
      hipLaunchKernelGGL((unf_softmax_kernel<true>), dim3((unsigned)a.N, (unsigned)hp), dim3(256), 0,
                         stream, S, P, a.kv_len, a.N, a.H, bh0, a.causal);
    else
      hipLaunchKernelGGL((unf_softmax_kernel<false>), dim3((unsigned)a.N, (unsigned)hp), dim3(256), 0,
                         stream, S, P, a.kv_len, a.N, a.H, bh0, a.causal);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int lds = 2 * 64 * 2 * D;
    const int nqt = (a.N + 127) / 128;
    if (vec)
      hipLaunchKernelGGL((unf_pv_kernel<D, true>), dim3((unsigned)nqt, (unsigned)hp), dim3(256), lds,
                         stream, P, (const __bf16*)a.v + off, (__bf16*)a.o + off, a.N, nqt);
    else
      hipLaunchKernelGGL((unf_pv_kernel<D, false>), dim3((unsigned)nqt, (unsigned)hp), dim3(256), lds,
                         stream, P, (const __bf16*)a.v + off, (__bf16*)a.o + off, a.N, nqt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t unfused_head_bytes(int N) {
  const size_t nn = (size_t)N * N;
  return nn * (sizeof(float) + 2);
}

hipError_t launch_unfused_bf16(const UnfusedArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_unfused_t<128>(a, stream);
  if (a.d == 64) return launch_unfused_t<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace attnio
