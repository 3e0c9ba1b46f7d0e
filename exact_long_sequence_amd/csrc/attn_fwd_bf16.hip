// Fused, streamed exact attention forward for bf16 on gfx950 (CDNA4).
//
// Schedule (the memory-centric pipeline of "From Attention Graph to
// FlashAttention - A Memory-Centric Compilation Approach in AICF", section 3:
// load a Q tile, stream K/V tiles, partial scores, online softmax update,
// accumulate; no score / probability tensor ever leaves the chip):
//
//   one workgroup = one (batch, head, query tile of BM = 32*WAVES rows)
//   Q tile:   HBM -> VGPR once, held as MFMA operands for the whole key loop
//   K/V tile: HBM/L2 -> LDS by direct-to-LDS loads into a double buffer; the
//             loads of tile j+1 are in flight while tile j is computed
//   per wave, per K/V tile of BN keys:
//     S^T = K Q^T            bf16 MFMA 32x32x16, fp32 accumulate
//     online softmax          fp32; one v_exp_f32 per score, per-lane row stats
//     O^T += V^T P^T          bf16 MFMA 32x32x16, V fed by LDS transpose reads
//   epilogue: O = O^T / l, rounded to bf16 once.
//
// Computing the transposed score block S^T (keys down the MFMA rows, the
// wave's 32 queries across the 32 lanes) makes every softmax statistic
// lane-local: each lane owns one query, its 16 values per 32x32 block are that
// query's scores for 16 keys, and the other 16 keys of the block sit in the
// lane 32 apart.  The row max therefore needs one permlane32 swap per tile, the
// row sum none until the epilogue, and the rescale of the output accumulator
// is one multiply by a per-lane scalar.  The accumulator O^T has the same
// lane = query layout, and the probabilities come out of the score MFMA
// already in the B-operand layout of the P x V MFMA.  This is the "parallel
// execution pattern for efficient softmax" of "I/O Analysis is All You Need:
// An I/O Analysis for Long-Sequence Attention" (abstract, optimisation 3)
// mapped onto 64-wide wavefronts.
//
// The rescale of the running output is lazy: the running maximum m only moves
// when some row's maximum exceeds it by more than 2^TAU_LOG2 in the exp2
// domain.  Any shift m >= the true maximum - TAU gives the same softmax (the
// shift cancels between numerator and denominator), so the result is exact up
// to rounding; probabilities are bounded by 2^TAU before normalisation.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace attnio {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTauLog2 = 8.0f;  // lazy-rescale threshold (probabilities <= 2^8)

template <int D, int BN, int WAVES>
struct Cfg {
  static constexpr int BM = 32 * WAVES;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CHUNKS = ROW_BYTES / 16;          // 16-byte chunks per row
  static constexpr int ROWS_PER_256 = 256 / ROW_BYTES;   // rows sharing one 256 B bank line
  static constexpr int TILE_BYTES = BN * ROW_BYTES;      // one K or one V tile
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;     // K + V
  static constexpr int STAGES = 2;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int LOADS = TILE_BYTES / 16 / THREADS;  // 16 B loads per thread per tensor
  static_assert(TILE_BYTES % (16 * THREADS) == 0, "tile must split evenly over threads");
  static_assert(BN % 32 == 0 && D % 32 == 0, "MFMA blocking");
};

// XOR swizzles of the 16-byte chunk index inside an LDS row.  K rows are read
// 16 bytes per lane by 32 consecutive rows; V rows are read 8 bytes per lane by
// the transpose read, 4 rows x 4 chunks per 32 lanes.  Both keep every group of
// lanes that the LDS serves together on distinct banks.
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

template <int D, int BN, int WAVES, bool CAUSAL, bool NEG_SCALE>
__global__ __launch_bounds__(64 * WAVES, 2)
void attn_fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                          const __bf16* __restrict__ V, __bf16* __restrict__ O,
                          const int32_t* __restrict__ kv_len, int H, int N, float c,
                          int n_qtiles) {
  using C = Cfg<D, BN, WAVES>;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int half = lane / 32;   // h
  const int col = lane % 32;    // c: the query this lane owns

  // ---- logical tile id: XCD-aware remap, then (batch*head, query tile) ----
  const int G = gridDim.x;
  const int x = blockIdx.x;
  const int xcd = x % 8, idx = x / 8, per = G / 8, rem = G % 8;
  const int logical = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  const int bh = logical / n_qtiles;
  int qt = logical % n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest query tiles first
  const int b = bh / H;

  int L = N;
  if (kv_len != nullptr) {
    L = kv_len[b];
    L = L < 0 ? 0 : (L > N ? N : L);
  }
  const int q0 = qt * C::BM;
  int kend = L;
  if (CAUSAL) kend = min(kend, min(N, q0 + C::BM));
  const int ntiles = (kend + BN - 1) / BN;

  const size_t slice = (size_t)bh * N * D;
  const __bf16* Qs = Q + slice;
  const char* Kg = (const char*)(K + slice);
  const char* Vg = (const char*)(V + slice);
  __bf16* Os = O + slice;

  // ---- K/V tile loader (direct to LDS) ----
  auto issue_tile = [&](int t, int stage) {
    const int j0 = t * BN;
    char LDS_AS* kl = smem + stage * C::STAGE_BYTES;
    char LDS_AS* vl = kl + C::TILE_BYTES;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int wbase = (i * C::THREADS + wave * 64) * 16;  // wave-uniform LDS offset
      const int pos = wbase + lane * 16;
      const int row = pos / C::ROW_BYTES;
      const int pch = (pos % C::ROW_BYTES) / 16;
      int grow = j0 + row;
      grow = grow < kend ? grow : kend - 1;
      const size_t goffk = (size_t)grow * C::ROW_BYTES + (size_t)((pch ^ swz_k<C>(row)) * 16);
      const size_t goffv = (size_t)grow * C::ROW_BYTES + (size_t)((pch ^ swz_v<C>(row)) * 16);
      __builtin_amdgcn_global_load_lds((const void GLB_AS*)(Kg + goffk), (void LDS_AS*)(kl + wbase), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void GLB_AS*)(Vg + goffv), (void LDS_AS*)(vl + wbase), 16, 0, 0);
    }
  };

  if (ntiles > 0) issue_tile(0, 0);

  // ---- Q fragments (B operand of S^T = K Q^T): lane (h, c) holds
  //      Q[q0 + 32*wave + c][16*ks + 8*h .. +7] for every ks ----
  const int qrow = q0 + wave * 32 + col;
  const int qrow_c = qrow < N ? qrow : N - 1;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = *(const bf16x8*)(Qs + (size_t)qrow_c * D + ks * 16 + half * 8);

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  float m_run = -INFINITY;  // running shift, exp2 domain (scores * c)
  float l_run = 0.f;        // this lane's partial row sum (its 16 keys of each 32)

  // first query row of this wave: blocks entirely above the diagonal are skipped
  const int wq0 = q0 + wave * 32;

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < ntiles) issue_tile(t + 1, stage ^ 1);

    const char LDS_AS* kl = smem + stage * C::STAGE_BYTES;
    const char LDS_AS* vl = kl + C::TILE_BYTES;
    const int j0 = t * BN;

    // ---------------- S^T = K Q^T ----------------
    f32x16 s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const int row = kb * 32 + col;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int ch = (2 * ks + half) ^ swz_k<C>(row);
        const bf16x8 a = *(const bf16x8 LDS_AS*)(kl + row * C::ROW_BYTES + ch * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
    }

    // ---------------- mask (diagonal / padding tiles only) ----------------
    const bool need_mask = (j0 + BN > L) || (CAUSAL && (j0 + BN - 1 > wq0));
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + kb * 32 + (r / 4) * 8 + half * 4 + (r % 4);
          bool ok = key < L;
          if (CAUSAL) ok = ok && (key <= qrow);
          s[kb][r] = ok ? s[kb][r] : (NEG_SCALE ? INFINITY : -INFINITY);
        }
    }

    // ---------------- online softmax (exp2 domain) ----------------
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = NEG_SCALE ? fminf(mx, s[kb][r]) : fmaxf(mx, s[kb][r]);
    {
      const u32x2 pr = swap_halves(mx);
      mx = NEG_SCALE ? fminf(__uint_as_float(pr[0]), __uint_as_float(pr[1]))
                     : fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
    }
    const float m_tile = mx * c;  // row maximum of scores * c (-inf if fully masked)
    const bool grow = m_tile > m_run + kTauLog2;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

    // P = exp2(S*c - m), rounded to bf16, packed as the B operand of O^T += V^T P^T
    bf16x8 pb[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        bf16x8 p;
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8)
          p[t8] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][sp * 8 + t8], c, -m_use));
        pb[kb * 2 + sp] = p;
      }
    {
      const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
      for (int i = 0; i < BN / 16; ++i)
#pragma unroll
        for (int t2 = 0; t2 < 4; ++t2) {
          const bf16x2 pp = {pb[i][2 * t2], pb[i][2 * t2 + 1]};
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
        }
    }

    // ---------------- O^T += V^T P^T ----------------
    // transpose read: lane 16g + 4j + q supplies V row (16*step + 8u + 4h + j),
    // columns 32db + 16(g%2) + 4q .. +3; lane 16g + i receives column
    // 32db + 16(g%2) + i of those four rows.
    const int g = lane / 16;
    const int jr = (lane % 16) / 4;
    const int qq = lane % 4;
#pragma unroll
    for (int st = 0; st < BN / 16; ++st) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        bf16x8 a;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int row = st * 16 + u * 8 + half * 4 + jr;
          const int colb = (db * 32 + (g % 2) * 16 + qq * 4) * 2;  // byte offset in row
          const int ch = (colb / 16) ^ swz_v<C>(row);
          const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (s16x4 LDS_AS*)(vl + row * C::ROW_BYTES + ch * 16 + (colb % 16)));
          const bf16x4 vb = __builtin_bit_cast(bf16x4, v4);
#pragma unroll
          for (int e = 0; e < 4; ++e) a[u * 4 + e] = vb[e];
        }
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], acc[db], 0, 0, 0);
      }
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---------------- epilogue: O = O^T / l ----------------
  const u32x2 lp = swap_halves(l_run);
  const float l_tot = __uint_as_float(lp[0]) + __uint_as_float(lp[1]);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    __bf16* orow = Os + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[db][a4 * 4 + e] * inv);
        *(bf16x4*)(orow + db * 32 + a4 * 8 + half * 4) = o;
      }
  }
}

template <int D, int BN, int WAVES, bool CAUSAL, bool NEG>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  using C = Cfg<D, BN, WAVES>;
  const int n_qtiles = (a.N + C::BM - 1) / C::BM;
  const long long grid = (long long)a.B * a.H * n_qtiles;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c = a.scale * kLog2e;
  auto kern = attn_fwd_bf16_kernel<D, BN, WAVES, CAUSAL, NEG>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::THREADS), C::LDS_BYTES, stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o,
                     a.kv_len, a.H, a.N, c, n_qtiles);
  return hipGetLastError();
}

template <int D, int BN, int WAVES>
hipError_t dispatch_mask(const FwdArgs& a, hipStream_t stream) {
  const bool neg = a.scale < 0.f;
  if (a.causal) return neg ? launch_t<D, BN, WAVES, true, true>(a, stream)
                           : launch_t<D, BN, WAVES, true, false>(a, stream);
  return neg ? launch_t<D, BN, WAVES, false, true>(a, stream)
             : launch_t<D, BN, WAVES, false, false>(a, stream);
}

}  // namespace

bool bf16_tiling(int d, int causal, Tiling* t) {
  (void)causal;
  if (d == 128) {
    using C = Cfg<128, 64, 4>;
    *t = {C::BM, 64, C::STAGES, 4, C::LDS_BYTES};
    return true;
  }
  if (d == 64) {
    using C = Cfg<64, 64, 4>;
    *t = {C::BM, 64, C::STAGES, 4, C::LDS_BYTES};
    return true;
  }
  return false;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return dispatch_mask<128, 64, 4>(a, stream);
  if (a.d == 64) return dispatch_mask<64, 64, 4>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace attnio
