// Device-side building blocks shared by the bf16 MFMA kernels of the backward
// and of the unfused baseline (gfx950): operand types, the LDS row swizzle,
// direct-to-LDS row loads, and the two ways an MFMA 32x32x16 operand is read
// from an LDS tile of rows (along the row, or transposed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnio {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// 16-byte chunk swizzle of an LDS row of D bf16 values.  A tile is read two
// ways and both must spread over distinct banks:
//   row reads        16 consecutive rows (aligned), one logical chunk each;
//   transpose reads  4 consecutive rows (aligned to 4), 4 adjacent chunks each
//                    (lanes 0-31 of ds_read_b64_tr_b16).
// With x the row's bank-line index (row / rows-per-line, mod chunks-per-row),
// the XOR pattern is a bijection of x (row reads) whose top two bits differ for
// the 4 rows of a transpose read: x with its low bits rotated to the top
// (d = 128: one row per line, x = row mod 16, the two 2-bit halves swapped;
// d = 64: two rows per line, x = (row / 2) mod 8, bit 0 moved to bit 2).
// Writes and every read of a tile use this function, so the layout is
// consistent by construction.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if (D == 128) {
    const int x = row % 16;
    return ((x & 3) << 2) | (x >> 2);
  }
  const int x = (row / 2) % 8;
  return ((x & 1) << 2) | (x >> 1);
}

__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(gbase) : "memory");
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_dma_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// A operand of a 32x32x16 MFMA from an LDS tile of rows of D bf16: lane (h, c)
// gets row `row`, columns 16 ks + 8 h .. + 7 (one 16-byte read).
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const char LDS_AS* tile, int row, int ks, int half) {
  const int ch = (2 * ks + half) ^ swz<D>(row);
  return *(const bf16x8 LDS_AS*)(tile + row * (2 * D) + ch * 16);
}

// A operand of X^T (d down the MFMA rows, the tile's rows along k) for d block
// db and k step st, by two transpose reads: lane 16g + 4j + q supplies tile row
// (16 st + 8u + 4h + j), columns 32 db + 16 (g % 2) + 4 q .. +3, and lane
// 16g + i receives column 32 db + 16 (g % 2) + i of those four rows.  Element
// 4u + e of the result belongs to tile row 16 st + 8u + 4h + e.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char LDS_AS* tile, int db, int st, int lane) {
  const int half = lane / 32, g = lane / 16, jr = (lane % 16) / 4, qq = lane % 4;
  bf16x8 a;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = st * 16 + u * 8 + half * 4 + jr;
    const int colb = (db * 32 + (g % 2) * 16 + qq * 4) * 2;
    const int ch = (colb / 16) ^ swz<D>(row);
    const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 LDS_AS*)(tile + row * (2 * D) + ch * 16 + (colb % 16)));
    const bf16x4 vb = __builtin_bit_cast(bf16x4, v4);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[u * 4 + e] = vb[e];
  }
  return a;
}

// DMA of `rows` rows of D bf16 starting at global row r0 into an LDS tile, by
// the workgroup's THREADS threads; rows >= last_ok + 1 are clamped to last_ok.
template <int D, int ROWS, int THREADS>
__device__ __forceinline__ void dma_rows(const __bf16* gsrc, int r0, int last_ok, uint32_t lds_tile,
                                         int wave, int lane) {
  constexpr int RB = 2 * D;
  constexpr int LOADS = ROWS * RB / 16 / THREADS;
  static_assert(ROWS * RB % (16 * THREADS) == 0, "tile must split evenly");
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pos = (i * THREADS + wave * 64 + lane) * 16;
    const int row = pos / RB;
    const int pch = (pos % RB) / 16;
    const int lch = pch ^ swz<D>(row);
    int grow = r0 + row;
    grow = grow < last_ok ? grow : last_ok;
    // unsigned: a head holds fewer than 2^31 elements, so the byte offset of
    // its last row fits 32 bits unsigned (not signed, at N > 2^23, d = 128)
    const uint32_t o = (uint32_t)grow * (uint32_t)RB + (uint32_t)(lch * 16);
    const uint32_t l = __builtin_amdgcn_readfirstlane(lds_tile + (uint32_t)((i * THREADS + wave * 64) * 16));
    dma16(gsrc, o, l);
  }
}

}  // namespace
}  // namespace attnio
