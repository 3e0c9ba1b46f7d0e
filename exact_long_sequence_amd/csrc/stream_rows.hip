// Streaming row operators for bf16 on gfx950: row softmax and row LayerNorm
// over the last axis of an [R, N] matrix.
//
// "From Attention Graph to FlashAttention - A Memory-Centric Compilation
// Approach in AICF" names streaming softmax and streaming LayerNorm as the
// next operators for the memory-centric treatment (closing outlook).  Both
// are a row reduction followed by an elementwise map that needs the
// reduction's result, so the naive form reads the row twice (or three times:
// mean, variance, normalise).  The compulsory traffic is one read and one
// write of the row; these kernels reach it whenever the row fits the
// registers of one workgroup (N <= 65536): the row is loaded once into
// registers, reduced, and written from the same registers.  Longer rows are
// streamed: a first pass keeps the running statistics (online max / sum, the
// same update as the attention kernel's online softmax; shifted sums for the
// variance), a second pass re-reads the row and writes it.
//
// One workgroup of 512 threads per row; a thread owns 8 consecutive elements
// per 4096-element sweep (16-byte loads and stores).  LayerNorm rows of 512,
// 1024, 2048, 4096 or 8192 elements go to one wave each instead (eight rows per
// workgroup): the wave's shuffles reduce the row, with no LDS and no workgroup
// barrier, and the many rows in flight per CU keep more loads outstanding.  Rows whose length is not a
// multiple of 8 take a scalar streaming path.  All arithmetic is fp32; the
// output is rounded to bf16 once.

#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"
#include "tile_ops.h"

namespace attnio {
namespace {

constexpr int kRowThreads = 512;
constexpr int kSweep = kRowThreads * 8;  // elements per sweep of the workgroup

// Reductions over the workgroup: wave by shuffles, then the 8 waves through LDS.
__device__ __forceinline__ void block_sum2(float& a, float& b, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off /= 2) {
    a += __shfl_xor(a, off);
    b += __shfl_xor(b, off);
  }
  const int w = threadIdx.x / 64;
  __syncthreads();  // red may still be read by an earlier reduction
  if (threadIdx.x % 64 == 0) {
    red[w] = a;
    red[8 + w] = b;
  }
  __syncthreads();
  a = 0.f;
  b = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a += red[i];
    b += red[8 + i];
  }
}

// (max, sum of 2^(t - max)) pairs, merged exactly; max = -inf means empty.
__device__ __forceinline__ void merge_ml(float& m, float& l, float mo, float lo) {
  const float mn = m > mo ? m : mo;
  const float sa = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
  const float sb = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
  l = l * sa + lo * sb;
  m = mn;
}

__device__ __forceinline__ void block_ml(float& m, float& l, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off /= 2) merge_ml(m, l, __shfl_xor(m, off), __shfl_xor(l, off));
  const int w = threadIdx.x / 64;
  __syncthreads();
  if (threadIdx.x % 64 == 0) {
    red[w] = m;
    red[8 + w] = l;
  }
  __syncthreads();
  m = red[0];
  l = red[8];
#pragma unroll
  for (int i = 1; i < 8; ++i) merge_ml(m, l, red[i], red[8 + i]);
}

// Online update of (max, sum) with one value t (base-2 exponent domain).
__device__ __forceinline__ void online_add(float& m, float& l, float t) {
  if (t > m) {
    l = (m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f(m - t)) + 1.f;
    m = t;
  } else if (t != -INFINITY) {
    l += __builtin_amdgcn_exp2f(t - m);
  }
}

// ----------------------------------------------------------------------------
// softmax: y = 2^(t - max) / sum with t = x * scale * log2(e).
// SW > 0: the row is held in SW sweeps of registers (N <= SW * 4096, N % 8 == 0).
// SW == 0, VEC: two passes of 16-byte accesses; SW == 0, !VEC: scalar.
// ----------------------------------------------------------------------------
template <int SW, bool VEC>
__global__ __launch_bounds__(kRowThreads)
void stream_softmax_kernel(const __bf16* __restrict__ X, __bf16* __restrict__ Y, int N, float c) {
  __shared__ float red[16];
  const int tid = threadIdx.x;
  const __bf16* x = X + (size_t)blockIdx.x * N;
  __bf16* y = Y + (size_t)blockIdx.x * N;
  if (SW > 0) {
    // cached row: max, then the sum of 2^(t - max), then 2^(t - max) again,
    // scaled and stored.  The row stays packed in registers (an empty asm after
    // each pass keeps the compiler from holding its fp32 unpacking, and the
    // exponentials are recomputed rather than kept): 59 instead of 90
    // registers at 8 sweeps, so more rows are in flight per CU.  The row is
    // read and written once, so its accesses are non-temporal.  Bitwise the
    // same result as keeping the exponentials.
    bf16x8 xc[SW > 0 ? SW : 1];
    float xm = -INFINITY;
#pragma unroll
    for (int s = 0; s < SW; ++s) {  // past the row's end: the row's first 16 bytes, unused
      const int j = s * kSweep + tid * 8;
      xc[s] = __builtin_nontemporal_load((const bf16x8*)(x + (j < N ? j : 0)));
    }
#pragma unroll
    for (int s = 0; s < SW; ++s) {
      const int j = s * kSweep + tid * 8;
      if (j < N)
#pragma unroll
        for (int e = 0; e < 8; ++e) xm = fmaxf(xm, (float)xc[s][e]);
    }
#pragma unroll
    for (int s = 0; s < SW; ++s) asm volatile("" : "+v"(xc[s]));
#pragma unroll
    for (int off = 32; off > 0; off /= 2) xm = fmaxf(xm, __shfl_xor(xm, off));
    if (tid % 64 == 0) red[tid / 64] = xm;
    __syncthreads();
    xm = red[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) xm = fmaxf(xm, red[i]);
    const bool empty = xm == -INFINITY;
    const float ms = empty ? 0.f : xm * c;  // c > 0: max of x * c is c * max of x
    float l = 0.f;
#pragma unroll
    for (int s = 0; s < SW; ++s) {
      const int j = s * kSweep + tid * 8;
      if (j < N)
#pragma unroll
        for (int e = 0; e < 8; ++e) l += __builtin_amdgcn_exp2f(__builtin_fmaf((float)xc[s][e], c, -ms));
    }
#pragma unroll
    for (int s = 0; s < SW; ++s) asm volatile("" : "+v"(xc[s]));
    float l2 = 0.f;
    block_sum2(l, l2, red);
    const float inv = empty ? 0.f : 1.f / l;
#pragma unroll
    for (int s = 0; s < SW; ++s) {
      const int j = s * kSweep + tid * 8;
      if (j < N) {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[e] = (__bf16)(__builtin_amdgcn_exp2f(__builtin_fmaf((float)xc[s][e], c, -ms)) * inv);
        __builtin_nontemporal_store(o, (bf16x8*)(y + j));
      }
    }
    return;
  }
  // streamed row: online (max, sum) in one pass, then a second pass
  float m = -INFINITY, l = 0.f;
  if (VEC) {
    for (int j = tid * 8; j < N; j += kSweep) {
      const bf16x8 v = *(const bf16x8*)(x + j);
#pragma unroll
      for (int e = 0; e < 8; ++e) online_add(m, l, (float)v[e] * c);
    }
  } else {
    for (int j = tid; j < N; j += kRowThreads) online_add(m, l, (float)x[j] * c);
  }
  block_ml(m, l, red);
  const bool empty = m == -INFINITY;
  const float inv = empty ? 0.f : 1.f / l;
  const float ms = empty ? 0.f : m;
  if (VEC) {
    for (int j = tid * 8; j < N; j += kSweep) {
      const bf16x8 v = *(const bf16x8*)(x + j);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)(__builtin_amdgcn_exp2f(__builtin_fmaf((float)v[e], c, -ms)) * inv);
      *(bf16x8*)(y + j) = o;
    }
  } else {
    for (int j = tid; j < N; j += kRowThreads)
      y[j] = (__bf16)(__builtin_amdgcn_exp2f(__builtin_fmaf((float)x[j], c, -ms)) * inv);
  }
}

// ----------------------------------------------------------------------------
// LayerNorm: y = (x - mu) * rstd * gamma + beta.  Cached rows take the mean and
// then the mean squared deviation from the registers (the plain two-pass
// definition, no extra memory traffic).  Streamed rows accumulate sums of
// (x - K) and (x - K)^2 with K = x_0 (variance by shifted data), which keeps
// the cancellation small when the row's mean is far from zero.
// ----------------------------------------------------------------------------
template <int SW, bool VEC>
__global__ __launch_bounds__(kRowThreads)
void stream_layernorm_kernel(const __bf16* __restrict__ X, const __bf16* __restrict__ gamma,
                             const __bf16* __restrict__ beta, __bf16* __restrict__ Y, int N,
                             float eps) {
  __shared__ float red[16];
  const int tid = threadIdx.x;
  const __bf16* x = X + (size_t)blockIdx.x * N;
  __bf16* y = Y + (size_t)blockIdx.x * N;
  const float inv_n = 1.f / (float)N;
  float mu, rstd;
  bf16x8 xc[SW > 0 ? SW : 1];
  if (SW > 0) {
    float s1 = 0.f, dummy = 0.f;
#pragma unroll
    for (int s = 0; s < SW; ++s) {
      const int j = s * kSweep + tid * 8;
      if (j < N) {
        xc[s] = *(const bf16x8*)(x + j);
#pragma unroll
        for (int e = 0; e < 8; ++e) s1 += (float)xc[s][e];
      }
    }
    block_sum2(s1, dummy, red);
    mu = s1 * inv_n;
    float s2 = 0.f;
    dummy = 0.f;
#pragma unroll
    for (int s = 0; s < SW; ++s) {
      const int j = s * kSweep + tid * 8;
      if (j < N) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float dv = (float)xc[s][e] - mu;
          s2 = __builtin_fmaf(dv, dv, s2);
        }
      }
    }
    block_sum2(s2, dummy, red);
    rstd = rsqrtf(s2 * inv_n + eps);
  } else {
    const float K = (float)x[0];
    float s1 = 0.f, s2 = 0.f;
    if (VEC) {
      for (int j = tid * 8; j < N; j += kSweep) {
        const bf16x8 v = *(const bf16x8*)(x + j);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float dv = (float)v[e] - K;
          s1 += dv;
          s2 = __builtin_fmaf(dv, dv, s2);
        }
      }
    } else {
      for (int j = tid; j < N; j += kRowThreads) {
        const float dv = (float)x[j] - K;
        s1 += dv;
        s2 = __builtin_fmaf(dv, dv, s2);
      }
    }
    block_sum2(s1, s2, red);
    const float dm = s1 * inv_n;
    float var = s2 * inv_n - dm * dm;
    var = var > 0.f ? var : 0.f;
    mu = K + dm;
    rstd = rsqrtf(var + eps);
  }
  auto val = [&](float xv, int j) __attribute__((always_inline)) {
    float r = (xv - mu) * rstd;
    if (gamma != nullptr) r *= (float)gamma[j];
    if (beta != nullptr) r += (float)beta[j];
    return r;
  };
  auto val8 = [&](const bf16x8& v, int j) __attribute__((always_inline)) {
    bf16x8 g, b, o;
    if (gamma != nullptr) g = *(const bf16x8*)(gamma + j);
    if (beta != nullptr) b = *(const bf16x8*)(beta + j);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = ((float)v[e] - mu) * rstd;
      if (gamma != nullptr) r *= (float)g[e];
      if (beta != nullptr) r += (float)b[e];
      o[e] = (__bf16)r;
    }
    return o;
  };
  if (SW > 0) {
#pragma unroll
    for (int s = 0; s < SW; ++s) {
      const int j = s * kSweep + tid * 8;
      if (j < N) *(bf16x8*)(y + j) = val8(xc[s], j);
    }
  } else if (VEC) {
    for (int j = tid * 8; j < N; j += kSweep) *(bf16x8*)(y + j) = val8(*(const bf16x8*)(x + j), j);
  } else {
    for (int j = tid; j < N; j += kRowThreads) y[j] = (__bf16)val((float)x[j], j);
  }
}

// LayerNorm, one wave per row, kWaveRows rows per workgroup, for N = 512 * PER
// (PER = 1, 2, 4, 8, 16) with gamma and beta both given (AFFINE) or both
// absent: lane l holds elements 512 s + 8 l .. + 7 of sweep s.  Mean, then the
// mean squared deviation from the registers (the cached kernel's definition),
// each reduced over the wave by shuffles.  The row is read and written once,
// so its loads and stores are non-temporal; gamma and beta, shared by every
// row, go through the caches.  Straight-line code with no per-sweep test lets
// the compiler keep all of the row's loads, and the next sweeps' gamma and beta
// loads, in flight.
constexpr int kWaveRows = 8;

template <int PER, bool AFFINE>
__global__ __launch_bounds__(64 * kWaveRows)
void stream_layernorm_wave_kernel(const __bf16* __restrict__ X, const __bf16* __restrict__ gamma,
                                  const __bf16* __restrict__ beta, __bf16* __restrict__ Y, int R, int N,
                                  float eps) {
  const int lane = threadIdx.x % 64;
  const long long row = (long long)blockIdx.x * kWaveRows + threadIdx.x / 64;
  if (row >= R) return;  // whole waves only; the kernel has no barrier
  const __bf16* x = X + row * N;
  __bf16* y = Y + row * N;
  bf16x8 xc[PER];
#pragma unroll
  for (int s = 0; s < PER; ++s) xc[s] = __builtin_nontemporal_load((const bf16x8*)(x + s * 512 + lane * 8));
  float s1 = 0.f;
#pragma unroll
  for (int s = 0; s < PER; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) s1 += (float)xc[s][e];
#pragma unroll
  for (int off = 32; off > 0; off /= 2) s1 += __shfl_xor(s1, off);
  const float inv_n = 1.f / (float)N;
  const float mu = s1 * inv_n;
  float s2 = 0.f;
#pragma unroll
  for (int s = 0; s < PER; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float dv = (float)xc[s][e] - mu;
      s2 = __builtin_fmaf(dv, dv, s2);
    }
#pragma unroll
  for (int off = 32; off > 0; off /= 2) s2 += __shfl_xor(s2, off);
  const float rstd = rsqrtf(s2 * inv_n + eps);
#pragma unroll
  for (int s = 0; s < PER; ++s) {
    const int j = s * 512 + lane * 8;
    bf16x8 o;
    if constexpr (AFFINE) {
      const bf16x8 g = *(const bf16x8*)(gamma + j), b = *(const bf16x8*)(beta + j);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)(((float)xc[s][e] - mu) * rstd * (float)g[e] + (float)b[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)(((float)xc[s][e] - mu) * rstd);
    }
    __builtin_nontemporal_store(o, (bf16x8*)(y + j));
  }
}

template <int PER>
hipError_t launch_layernorm_wave(const RowArgs& a, hipStream_t stream) {
  const unsigned blocks = (unsigned)(((long long)a.R + kWaveRows - 1) / kWaveRows);  // R up to 2^31 - 1
  if (a.gamma != nullptr)
    hipLaunchKernelGGL((stream_layernorm_wave_kernel<PER, true>), dim3(blocks), dim3(64 * kWaveRows), 0, stream,
                       (const __bf16*)a.x, (const __bf16*)a.gamma, (const __bf16*)a.beta, (__bf16*)a.y, a.R,
                       a.N, a.param);
  else
    hipLaunchKernelGGL((stream_layernorm_wave_kernel<PER, false>), dim3(blocks), dim3(64 * kWaveRows), 0, stream,
                       (const __bf16*)a.x, (const __bf16*)a.gamma, (const __bf16*)a.beta, (__bf16*)a.y, a.R,
                       a.N, a.param);
  return hipGetLastError();
}

// Sweeps held in registers for a row of N elements (0: stream the row).
int cached_sweeps(int N) {
  if (N % 8 != 0) return 0;
  const int s = (N + kSweep - 1) / kSweep;
  if (s <= 1) return 1;
  if (s <= 2) return 2;
  if (s <= 4) return 4;
  if (s <= 8) return 8;
  if (s <= 16) return 16;
  return 0;
}

template <int SW, bool VEC>
hipError_t launch_rows(const RowArgs& a, hipStream_t stream) {
  if (a.op == 0)
    hipLaunchKernelGGL((stream_softmax_kernel<SW, VEC>), dim3((unsigned)a.R), dim3(kRowThreads), 0,
                       stream, (const __bf16*)a.x, (__bf16*)a.y, a.N, a.param * kLog2e);
  else
    hipLaunchKernelGGL((stream_layernorm_kernel<SW, VEC>), dim3((unsigned)a.R), dim3(kRowThreads), 0,
                       stream, (const __bf16*)a.x, (const __bf16*)a.gamma, (const __bf16*)a.beta,
                       (__bf16*)a.y, a.N, a.param);
  return hipGetLastError();
}

}  // namespace

int rows_cached_sweeps(int N) { return cached_sweeps(N); }

hipError_t launch_stream_rows(const RowArgs& a, hipStream_t stream) {
  // one wave per row: N = 512 * (1, 2, 4, 8 or 16), gamma and beta both given or both absent
  if (a.op == 1 && a.N % 512 == 0 && a.N <= 8192 && (a.gamma == nullptr) == (a.beta == nullptr)) {
    switch (a.N / 512) {
      case 1: return launch_layernorm_wave<1>(a, stream);
      case 2: return launch_layernorm_wave<2>(a, stream);
      case 4: return launch_layernorm_wave<4>(a, stream);
      case 8: return launch_layernorm_wave<8>(a, stream);
      case 16: return launch_layernorm_wave<16>(a, stream);
      default: break;
    }
  }
  switch (cached_sweeps(a.N)) {
    case 1: return launch_rows<1, true>(a, stream);
    case 2: return launch_rows<2, true>(a, stream);
    case 4: return launch_rows<4, true>(a, stream);
    case 8: return launch_rows<8, true>(a, stream);
    case 16: return launch_rows<16, true>(a, stream);
    default: break;
  }
  return a.N % 8 == 0 ? launch_rows<0, true>(a, stream) : launch_rows<0, false>(a, stream);
}

}  // namespace attnio
