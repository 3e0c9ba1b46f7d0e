// Exact attention forward with fp8 (OCP E4M3) Q, K, V on gfx950's fp8 matrix
// cores; bf16 output.
//
// Same streamed schedule as the bf16 kernel ("From Attention Graph to
// FlashAttention - A Memory-Centric Compilation Approach in AICF", section 3:
// load a Q tile, stream K/V tiles, partial scores, online softmax update,
// accumulate), with the quantisation that the Neural Circuit Diagrams
// abstract lists among the effects its performance model covers:
//   * Q, K, V arrive as E4M3 bytes with one fp32 descale per tensor
//     (x = fp8 * s); S^T = K Q^T runs on v_mfma_scale_f32_32x32x64_f8f6f4 with
//     unit block scales, and the descales fold into the softmax constant;
//   * the probabilities are rounded to E4M3 for O^T += V^T P^T on the same
//     instruction.  The exponent shift is (reference maximum - 8), where the
//     reference follows the running row maximum lazily: it moves to a tile's
//     maximum, and the accumulator is rescaled, only when that maximum exceeds
//     it by more than 0.75 (base 2).  Every probability thus lies in
//     (0, 2^8.75], below E4M3's largest finite value 448, and the row's
//     largest entries sit at the top of the format, where its relative step
//     is 2^-3;
//   * the row sum l is the sum of the same E4M3 probabilities that multiply
//     V, formed on the matrix core (an all-ones operand times P), so O =
//     O^T * v_s / l is an exact convex combination of V's rows up to the
//     fp32 accumulation; O is rounded to bf16 once.
//
// Workgroup: 4 waves x 32 query rows, 128-key K and V tiles through a
// two-stage LDS ring of direct-to-LDS loads.  Each lane owns one query (S^T
// orientation: row statistics are lane-local, the two 16-key halves of a
// 32-key block sit in lanes l and l + 32).  V^T operands come from
// ds_read_b64_tr_b8 transposes whose key order matches the order in which the
// probabilities are packed into the B operand.

#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"
#include "tile_ops.h"

namespace attnio {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kFp8Shift = 8;  // log2 of the probability at the shift's reference maximum (256)
// How far (base 2) a tile's maximum may rise above the reference before the
// shift moves: probabilities then stay below 2^(8 + slack) = 430.5, under
// E4M3's largest finite value 448, and the accumulator is rescaled only when a
// row's maximum has grown by more than the slack since the last move.
#ifndef ATTNIO_FP8_SLACK
#define ATTNIO_FP8_SLACK 0.75f
#endif
constexpr float kFp8Slack = ATTNIO_FP8_SLACK;
static_assert(kFp8Slack >= 0.f && kFp8Slack < 0.8f, "2^(8 + slack) must stay below 448");

// The value of lane l and of lane l ^ 32, in some order, by one
// v_permlane32_swap with x as both operands (lanes 0-31 receive their
// partner's value in the second element, lanes 32-63 in the first).  Every
// lane of the wave must be active.
__device__ __forceinline__ u32x2 pair_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (u32x2){r[0], r[1]};
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // format 0 (E4M3) for both operands, block scales 127 (= 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16-byte chunk swizzle of an LDS row of RB bytes.  Both read patterns must
// spread over distinct banks: 16 consecutive rows at one logical chunk (the K
// operand reads) and, for the V transpose reads of lanes 0-31, rows
// {c..c+3, c+8..c+11} (c a multiple of 4) at two adjacent logical chunks.
// With 128-byte rows two rows share a 256-byte bank line; the line index
// x = row/2 mod 8 maps to x with bits 0 and 1 swapped, which keeps the
// line-pairs {x, x+1, x+4, x+5} of the second pattern in four different chunk
// pairs.  64-byte rows (four per line) need only the line index mod 4.
template <int RB>
__device__ __forceinline__ int swz8(int row) {
  if (RB == 128) {
    const int x = (row / 2) % 8;
    return (x & 4) | ((x & 1) << 1) | ((x >> 1) & 1);
  }
  return (row / 4) % 4;
}

// Direct-to-LDS load of ROWS rows of RB bytes starting at global row r0 (rows
// past last_ok clamped to it), laid out with swz8.
template <int RB, int ROWS, int THREADS>
__device__ __forceinline__ void dma_rows8(const uint8_t* gsrc, int r0, int last_ok, uint32_t lds_tile,
                                          int wave, int lane) {
  constexpr int LOADS = ROWS * RB / 16 / THREADS;
  static_assert(ROWS * RB % (16 * THREADS) == 0, "tile must split evenly");
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pos = (i * THREADS + wave * 64 + lane) * 16;
    const int row = pos / RB;
    const int pch = (pos % RB) / 16;
    const int lch = pch ^ swz8<RB>(row);
    int grow = r0 + row;
    grow = grow < last_ok ? grow : last_ok;
    // unsigned: a head's rows span fewer than 2^32 bytes
    const uint32_t o = (uint32_t)grow * (uint32_t)RB + (uint32_t)(lch * 16);
    const uint32_t l = __builtin_amdgcn_readfirstlane(lds_tile + (uint32_t)((i * THREADS + wave * 64) * 16));
    dma16(gsrc, o, l);
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2)
void attn_fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                         const uint8_t* __restrict__ V, __bf16* __restrict__ O,
                         const int32_t* __restrict__ kv_len, int H, int N, float c, float vs,
                         int n_qtiles) {
  constexpr int THREADS = 256, BN = 128, BM = 128, RB = D;  // RB: bytes per row
  constexpr int KT = BN * RB;
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
  const size_t slice = (size_t)bh * N * RB;
  const int qrow = q0 + wave * 32 + col;

  // Q of this lane's query as B operands: bytes 64 ks + 32 half .. + 31
  i32x8 qf[D / 64];
  {
    const int qr = qrow < N ? qrow : N - 1;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      const i32x4* p = (const i32x4*)(Q + slice + (size_t)qr * RB + ks * 64 + half * 32);
      const i32x4 lo = p[0], hi = p[1];
      qf[ks] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      // wait for Q here: otherwise the compiler's wait for these loads lands
      // inside the loop, where the hardware counter also holds the K/V DMAs
      // just issued for the next tile, and every tile waits for its prefetch
      // (16-byte operands: a 32-byte "v" operand is invalid in the host pass)
      asm volatile("" ::"v"(lo), "v"(hi));
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY;  // running row maximum of s * c (base-2 domain)
  // Row sum on the matrix core: an all-ones A operand (E4M3 1.0 = 0x38 in
  // every byte) times the packed P gives, in every element of the lane's
  // accumulator, the sum of the E4M3 probabilities of its query over the
  // operand's 64 keys -- the same rounded values that multiply V.
  const i32x8 ones8 = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                       0x38383838, 0x38383838, 0x38383838, 0x38383838};
  f32x16 lacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) lacc[r] = 0.f;

  if (ntiles > 0) {
    const uint8_t* Ks = K + slice;
    const uint8_t* Vs = V + slice;
    auto issue = [&](int t) __attribute__((always_inline)) {
      const uint32_t st = lds_base + (uint32_t)((t & 1) * 2 * KT);
      dma_rows8<RB, BN, THREADS>(Ks, t * BN, kend - 1, st, wave, lane);
      dma_rows8<RB, BN, THREADS>(Vs, t * BN, kend - 1, st + KT, wave, lane);
    };
    // Per-lane LDS byte offsets of the operand reads within a tile.  A row's
    // swizzle depends on (row / 2) mod 8 only, so whole 32-row blocks go into
    // the instruction's offset: V^T transpose read u of d block db at
    // tro[db][u % 2] + (2 ps + u / 2) * 32 rows (lane 16g + 2e + q supplies key
    // (2 ps + u/2)*32 + (2 (u%2) + e/4)*8 + 4 (g/2) + e%4, bytes 32 db +
    // 16 (g%2) + 8 q .. + 7; lane 16g + i receives byte i of those 8 keys,
    // i.e. bytes t = 8u + e of its operand); K row read of k step ks (low or
    // high 16 bytes of the lane's 32) at kro[ks][hi] + kb * 32 rows.
    uint32_t tro[D / 32][2], kro[D / 64][2];
    {
      const int g = lane / 16, h = g / 2, e = (lane % 16) / 2, q = lane % 2;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int u2 = 0; u2 < 2; ++u2) {
          const int key = (2 * u2 + e / 4) * 8 + 4 * h + e % 4;
          const int ch = 2 * db + (g % 2);
          tro[db][u2] = (uint32_t)(key * RB + ((ch ^ swz8<RB>(key)) * 16) + q * 8);
        }
#pragma unroll
      for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
          const int ch = ks * 4 + half * 2 + hi;
          kro[ks][hi] = (uint32_t)(col * RB + ((ch ^ swz8<RB>(col)) * 16));
        }
    }
    issue(0);
    wait_dma();
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      // opaque copies: the offsets are not expanded into one register per read
#pragma unroll
      for (int db = 0; db < D / 32; ++db) asm volatile("" : "+v"(tro[db][0]), "+v"(tro[db][1]));
#pragma unroll
      for (int ks = 0; ks < D / 64; ++ks) asm volatile("" : "+v"(kro[ks][0]), "+v"(kro[ks][1]));
      if (t + 1 < ntiles) issue(t + 1);
      const char LDS_AS* kt_l = smem + (t & 1) * 2 * KT;
      const char LDS_AS* vt_l = kt_l + KT;
      const int j0 = t * BN;

      // S^T = K Q^T: lane (h, c) holds keys (r/4)*8 + 4h + r%4 of block kb,
      // query c; each chain starts from the MFMA's zero accumulator input
      f32x16 s[BN / 32];
#pragma unroll
      for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
          const i32x4 lo = *(const i32x4 LDS_AS*)(kt_l + kro[ks][0] + kb * 32 * RB);
          const i32x4 hi = *(const i32x4 LDS_AS*)(kt_l + kro[ks][1] + kb * 32 * RB);
          const i32x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const f32x16 zero = {};
          s[kb] = mfma_fp8(a, qf[ks], ks == 0 ? zero : s[kb]);
        }
      // mask (one uniform test per tile, not per score) only the tiles on the
      // diagonal or past kv_len.  Scores stay unscaled: a masked score becomes
      // the infinity that maps to -inf under the scale c (never 0: the launcher
      // replaces c = 0 by the smallest normal float, which leaves every
      // visible probability exactly 1 relative to the shift), and the tile's
      // largest scaled score is c times the raw maximum (c > 0) or minimum
      // (c < 0), so the scaling costs one fma per score, inside exp2.
      const bool need_mask = (j0 + BN > L) || (CAUSAL && j0 + BN - 1 > q0);
      const bool pos = c > 0.f;
      const float lose = pos ? -INFINITY : INFINITY;
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + kb * 32 + (r / 4) * 8 + half * 4 + (r % 4);
            bool ok = key < L;
            if (CAUSAL) ok = ok & (key <= qrow);  // bitwise: no branch per score
            s[kb][r] = ok ? s[kb][r] : lose;
          }
      }
      float ext = lose;
      if (pos) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) ext = fmaxf(ext, s[kb][r]);
        const u32x2 pr = pair_halves(ext);
        ext = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
      } else {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) ext = fminf(ext, s[kb][r]);
        const u32x2 pr = pair_halves(ext);
        ext = fminf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
      }
      const float tmax = ext * c;  // -inf when every score of the row is masked
      // the shift's reference moves to the tile maximum (and the accumulator is
      // rescaled) only when that maximum exceeds the reference by more than the
      // slack; -inf + slack = -inf, so a row's first visible tile always moves it
      const bool mv = tmax > m_run + kFp8Slack;
      if (__builtin_amdgcn_ballot_w64(mv) != 0) {
        const float m_new = mv ? tmax : m_run;
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        if (mv) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
          for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
          m_run = m_new;
        }
      }
      const float sh = m_run == -INFINITY ? 0.f : m_run - (float)kFp8Shift;
      // P = 2^(s - sh) in (0, 2^(8 + slack)]; packed as E4M3 B operands: operand ps, byte
      // t = 16 b + r holds block 2 ps + b, register r
      i32x8 pb[BN / 64];
#pragma unroll
      for (int ps = 0; ps < BN / 64; ++ps)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int kb = 2 * ps + w / 4, r0 = 4 * (w % 4);
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r0 + e], c, -sh));
          // the low half is written first; the old value passed for the high
          // half is p[0]'s own register (dead after this instruction, so no
          // zeroing move), and the second conversion overwrites that half
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __builtin_bit_cast(int, p[0]), false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
          pb[ps][w] = word;
        }
      // O^T += V^T P^T: V^T by transpose reads.  Read u of operand (ps, db):
      // lane 16g + 2e + q supplies key (2ps + u/2)*32 + (2(u%2) + e/4)*8 + 4h + e%4
      // (h = g/2), bytes 32 db + 16 (g%2) + 8 q .. + 7; lane 16g + i receives
      // byte i of those 8 keys, i.e. bytes t = 8u + e of its operand.
      {
#pragma unroll
        for (int ps = 0; ps < BN / 64; ++ps)
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            i32x8 a;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const char LDS_AS* ap = vt_l + tro[db][u % 2] + (2 * ps + u / 2) * 32 * RB;
              const i32x2 v2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 LDS_AS*)ap);
              a[2 * u] = v2[0];
              a[2 * u + 1] = v2[1];
            }
            oacc[db] = mfma_fp8(a, pb[ps], oacc[db]);
          }
#pragma unroll
        for (int ps = 0; ps < BN / 64; ++ps) lacc = mfma_fp8(ones8, pb[ps], lacc);
      }
      wait_dma();
      __syncthreads();
    }
  }

  // lane (h, c) holds d rows db*32 + (r/4)*8 + 4h + r%4 of O^T for its
  // query, and (in every element of lacc) the query's whole row sum
  const float l_tot = lacc[0];
  const float inv = l_tot > 0.f ? vs / l_tot : 0.f;
  if (qrow < N) {
    __bf16* orow = O + (size_t)bh * N * D + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)(oacc[db][a4 * 4 + e] * inv);
        *(bf16x4*)(orow + db * 32 + a4 * 8 + half * 4) = o;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_fp8_t(const Fp8Args& a, hipStream_t stream) {
  float c = a.scale * a.q_descale * a.k_descale * kLog2e;
  if (c == 0.f) c = FLT_MIN;  // keeps masked scores at -inf (inf * 0 would be NaN)
  const int n_qtiles = (a.N + 127) / 128;
  const long long grid = (long long)a.B * a.H * n_qtiles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  constexpr int lds = 2 * 2 * 128 * D;
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), lds, stream,
                     (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, (__bf16*)a.o,
                     a.kv_len, a.H, a.N, c, a.v_descale, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_fp8_t<128, true>(a, stream) : launch_fp8_t<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch_fp8_t<64, true>(a, stream) : launch_fp8_t<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace attnio
