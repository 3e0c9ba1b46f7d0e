// Exact attention forward in fp32 end to end (gfx950, vector ALU).
//
// Same streamed schedule as the bf16 path (load a Q tile, stream K/V tiles,
// partial scores, online softmax update, accumulate: "From Attention Graph to
// FlashAttention - A Memory-Centric Compilation Approach in AICF", section 3),
// but every product, exponential and sum is binary32 with no narrower
// intermediate.  This path serves small fp32 problems, which are bound by
// latency rather than throughput, so it trades MFMA for parallelism over keys:
//
//   workgroup = 8 queries x 32 key lanes (256 threads), two such groups at
//   d = 64 taking the even and the odd key tiles (512 threads)
//   each thread runs its own online softmax over keys j = 32*t + lane of every
//   64-key LDS tile, with its own (m, l, acc[d]) state, rescaled once per
//   tile and only when some lane's running extreme moved;
//   K/V tiles are prefetched into registers one tile ahead of the LDS copy;
//   the 32 partial states of a query (and at d = 64 those of the two groups,
//   through LDS) are merged at the end with the same rescale the online update
//   uses (the streaming reduction merges exactly:
//   "IO-Aware Algorithms", How it works, online softmax).

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "kernels.h"

namespace attnio {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// 8 x 32: measured on MI355X at N = 1024, d = 64 (before the K/V prefetch
// below), 44 us per call against 64 us for 16 x 16 (64 workgroups on 256 CUs)
// and 77 us for 4 x 64; 8 x 64 (two waves per SIMD) ran 91 us: a merge across
// 64 lanes exchanges between the two halves of the wave.  A 1024-row head is
// latency-bound, so the split favours parallelism
constexpr int kQ = 8;         // queries per workgroup
constexpr int kLanes = 32;    // key lanes per query
constexpr int kBN = 64;       // keys per LDS tile
constexpr int kHalf = kQ * kLanes;  // threads that walk one key sequence
// key halves per workgroup: at d = 64 two groups of 256 threads take the even
// and the odd key tiles of the same queries (8 waves, two per SIMD, half the
// keys per thread) and merge their states through LDS at the end; at d = 128
// the fp32 accumulators of two waves per SIMD do not fit the registers
template <int D>
constexpr int halves_of() { return D == 64 ? 2 : 1; }

template <int D, bool CAUSAL, bool NEG>
__global__ __launch_bounds__(kHalf * halves_of<D>())
void attn_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                         const float* __restrict__ V, float* __restrict__ O,
                         const int32_t* __restrict__ kv_len, float* __restrict__ lse, int H,
                         int N, float c, int n_qtiles) {
  constexpr int HALVES = halves_of<D>();
  constexpr int THREADS = kHalf * HALVES;
  constexpr int P = D + 4;  // padded LDS row (floats): keeps 16 rows on distinct banks
  __shared__ __attribute__((aligned(16))) float qs[kQ * P];
  __shared__ __attribute__((aligned(16))) float kvs[HALVES][2][kBN * P];  // per half: K tile, V tile

  const int tid = threadIdx.x;
  const int hf = tid / kHalf;  // key half: tiles hf, hf + HALVES, ...
  const int ht = tid % kHalf;
  const int qi = ht / kLanes;
  const int kl = ht % kLanes;
  float* ks = kvs[hf][0];
  float* vs = kvs[hf][1];

  const int bh = blockIdx.x / n_qtiles;
  int qt = blockIdx.x % n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;
  const int b = bh / H;
  int L = N;
  if (kv_len != nullptr) {
    L = kv_len[b];
    L = L < 0 ? 0 : (L > N ? N : L);
  }
  const int q0 = qt * kQ;
  int kend = L;
  if (CAUSAL) kend = min(kend, min(N, q0 + kQ));

  const size_t slice = (size_t)bh * N * D;
  const float* Qs = Q + slice;
  const float* Ks = K + slice;
  const float* Vs = V + slice;
  float* Os = O + slice;

  for (int e = tid; e < kQ * D / 4; e += THREADS) {
    const int r = e / (D / 4), c4 = e % (D / 4);
    const int gr = min(q0 + r, N - 1);
    *(float4*)&qs[r * P + c4 * 4] = *(const float4*)&Qs[(size_t)gr * D + c4 * 4];
  }

  const int qrow = q0 + qi;
  float m = NEG ? INFINITY : -INFINITY;  // running extreme of the raw scores
  float l = 0.f;
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;

  // K/V tiles go HBM -> registers -> LDS: the loads of a half's next tile are
  // in flight while its current one is computed, and stored to LDS after the
  // barrier.  Half hf takes tiles hf, hf + HALVES, ...; both halves run the
  // same number of steps (a step past the last tile has no valid key, and its
  // loads are clamped to row kend - 1), so every thread meets every barrier.
  constexpr int NL = kBN * D / 4 / kHalf;  // 16-byte loads of K (and of V) per thread
  static_assert(kBN * D / 4 % kHalf == 0, "a tile must split evenly over a half's threads");
  typedef float f32x4 __attribute__((ext_vector_type(4)));  // a native vector: kept in registers
  f32x4 kreg[NL], vreg[NL];
  const int n_tiles = (kend + kBN - 1) / kBN;
  const int n_steps = (n_tiles + HALVES - 1) / HALVES;
  if (kend > 0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = ht + i * kHalf;
      const int r = e / (D / 4), c4 = e % (D / 4);
      const int gr = min(hf * kBN + r, kend - 1);
      kreg[i] = *(const f32x4*)&Ks[(size_t)gr * D + c4 * 4];
      vreg[i] = *(const f32x4*)&Vs[(size_t)gr * D + c4 * 4];
    }
  }
  for (int step = 0; step < n_steps; ++step) {
    const int j0 = (step * HALVES + hf) * kBN;
    __syncthreads();  // every read of the previous tiles is done
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = ht + i * kHalf;
      const int r = e / (D / 4), c4 = e % (D / 4);
      *(f32x4*)&ks[r * P + c4 * 4] = kreg[i];
      *(f32x4*)&vs[r * P + c4 * 4] = vreg[i];
    }
    __syncthreads();
    // the half's next tile (past the last one: rows clamped to kend - 1, unused)
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = ht + i * kHalf;
      const int r = e / (D / 4), c4 = e % (D / 4);
      const int gr = min(j0 + HALVES * kBN + r, kend - 1);
      kreg[i] = *(const f32x4*)&Ks[(size_t)gr * D + c4 * 4];
      vreg[i] = *(const f32x4*)&Vs[(size_t)gr * D + c4 * 4];
    }
    // the lane's keys of this tile: scores first, then one update of the
    // running extreme for all of them, a rescale of the state only when some
    // lane's extreme moved (a wave-uniform test), and one fma per key and
    // element for the accumulation
    constexpr int KPL = kBN / kLanes;  // keys per lane per tile
    float sc[KPL];
    bool okk[KPL];
    float m_new = m;
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      const int jl = t * kLanes + kl;
      const int key = j0 + jl;
      bool ok = key < kend;
      if (CAUSAL) ok = ok && key <= qrow;
      float sv = 0.f;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        const float4 a = *(const float4*)&qs[qi * P + e];
        const float4 k4 = *(const float4*)&ks[jl * P + e];
        sv = __builtin_fmaf(a.x, k4.x, sv);
        sv = __builtin_fmaf(a.y, k4.y, sv);
        sv = __builtin_fmaf(a.z, k4.z, sv);
        sv = __builtin_fmaf(a.w, k4.w, sv);
      }
      sc[t] = sv;
      okk[t] = ok;
      if (ok) m_new = NEG ? fminf(m_new, sv) : fmaxf(m_new, sv);
    }
    if (__builtin_amdgcn_ballot_w64(m_new != m) != 0) {
      // weights exp2((s - m) * c) are relative to the raw-score extreme m
      const float alpha = (m == m_new) ? 1.f : __builtin_amdgcn_exp2f((m - m_new) * c);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] *= alpha;
      m = m_new;
    }
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      const int jl = t * kLanes + kl;
      const float p = okk[t] ? __builtin_amdgcn_exp2f((sc[t] - m) * c) : 0.f;
      l += p;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        const float4 v4 = *(const float4*)&vs[jl * P + e];
        acc[e + 0] = __builtin_fmaf(p, v4.x, acc[e + 0]);
        acc[e + 1] = __builtin_fmaf(p, v4.y, acc[e + 1]);
        acc[e + 2] = __builtin_fmaf(p, v4.z, acc[e + 2]);
        acc[e + 3] = __builtin_fmaf(p, v4.w, acc[e + 3]);
      }
    }
  }

  // merge the 32 key-lane states of each query (lanes 32*q .. 32*q+31 of a wave)
  float m_all = m;
#pragma unroll
  for (int off = kLanes / 2; off > 0; off /= 2) {
    const float o = __shfl_xor(m_all, off, kLanes);
    m_all = NEG ? fminf(m_all, o) : fmaxf(m_all, o);
  }
  const bool empty = NEG ? (m_all == INFINITY) : (m_all == -INFINITY);
  const bool mine_empty = NEG ? (m == INFINITY) : (m == -INFINITY);
  const float w = (empty || mine_empty) ? 0.f : __builtin_amdgcn_exp2f((m - m_all) * c);
  l *= w;
#pragma unroll
  for (int off = kLanes / 2; off > 0; off /= 2) l += __shfl_xor(l, off, kLanes);
#pragma unroll
  for (int e = 0; e < D; ++e) {
    float x = acc[e] * w;
#pragma unroll
    for (int off = kLanes / 2; off > 0; off /= 2) x += __shfl_xor(x, off, kLanes);
    acc[e] = x;
  }
  constexpr int PER = D / kLanes;  // output elements of each lane: kl * PER ..
  if constexpr (HALVES == 2) {
    // half 1 hands its merged (m, l, acc) of each query to half 0 through LDS
    // (the K/V tiles are dead); half 0 merges them with the same rescale
    constexpr int XS = D + 2;  // per query: m, l, acc[D]
    static_assert(kQ * XS <= HALVES * 2 * kBN * P, "exchange fits the tile area");
    float* xch = &kvs[0][0][0];
    __syncthreads();
    if (hf == 1) {
      if (kl == 0) {
        xch[qi * XS] = m_all;
        xch[qi * XS + 1] = l;
      }
#pragma unroll
      for (int e = 0; e < D; ++e)
        if (e / PER == kl) xch[qi * XS + 2 + e] = acc[e];
    }
    __syncthreads();
    if (hf == 1) return;  // no barrier follows
    const float m1 = xch[qi * XS], l1 = xch[qi * XS + 1];
    const float mm = NEG ? fminf(m_all, m1) : fmaxf(m_all, m1);
    const bool e0 = NEG ? (m_all == INFINITY) : (m_all == -INFINITY);
    const bool e1 = NEG ? (m1 == INFINITY) : (m1 == -INFINITY);
    const float w0 = e0 ? 0.f : __builtin_amdgcn_exp2f((m_all - mm) * c);
    const float w1 = e1 ? 0.f : __builtin_amdgcn_exp2f((m1 - mm) * c);
    l = l * w0 + l1 * w1;
#pragma unroll
    for (int e = 0; e < D; ++e)
      if (e / PER == kl) acc[e] = acc[e] * w0 + xch[qi * XS + 2 + e] * w1;
    m_all = mm;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  // log-sum-exp: sum_j 2^(c s_j) = 2^(c m_all) * l (m_all is the raw-score
  // extreme, c * m_all the largest exponent whatever the sign of c)
  if (lse != nullptr && kl == 0 && qrow < N)
    lse[(size_t)bh * N + qrow] = l > 0.f ? (m_all * c + log2f(l)) * kLn2 : -INFINITY;
  if (qrow < N) {
#pragma unroll
    for (int e = 0; e < D; ++e)
      if (e / PER == kl) Os[(size_t)qrow * D + e] = acc[e] * inv;
  }
}

template <int D, bool CAUSAL, bool NEG>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.N + kQ - 1) / kQ;
  const long long grid = (long long)a.B * a.H * n_qtiles;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  // exponent multiplier scale * log2(e); an exact zero becomes the smallest
  // normal float so that (-inf) * c stays -inf (uniform weights, no NaN)
  float c = a.scale * kLog2e;
  if (c == 0.f) c = FLT_MIN;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL, NEG>), dim3((unsigned)grid), dim3(kHalf * halves_of<D>()), 0,
                     stream, (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o,
                     a.kv_len, a.lse, a.H, a.N, c, n_qtiles);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch(const FwdArgs& a, hipStream_t stream) {
  const bool neg = a.scale < 0.f;
  if (a.causal) return neg ? launch_t<D, true, true>(a, stream) : launch_t<D, true, false>(a, stream);
  return neg ? launch_t<D, false, true>(a, stream) : launch_t<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return dispatch<64>(a, stream);
  if (a.d == 128) return dispatch<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace attnio
