// Host-side I/O and issue model of the bf16 forward's tilings.
//
// "I/O Analysis is All You Need: An I/O Analysis for Long-Sequence Attention"
// (abstract, optimisation 1) asks for the tiling and schedule to come from an
// I/O analysis of the tall-and-skinny products; "IO-Aware Algorithms" (How it
// works) gives the tiled-product traffic 2MNK -> 2MNK/S and the roofline per
// memory tier; "From Attention Graph to FlashAttention - A Memory-Centric
// Compilation Approach in AICF" (sections 4-5) names the decisions a
// streaming region fixes: tile size, reduction axis, residency, streaming
// order.  Here the decisions are the query-tile height BM = 32 * waves * qb
// (rows resident in registers), the key-tile width BN (rows streamed through
// LDS), the LDS stages, the workgroups per CU and the loop form, and the model
//
//   1. enumerates every combination and keeps those that fit a gfx950 CU:
//      160 KiB of LDS, 512 registers per SIMD lane shared by the waves of the
//      SIMD (at most 256 architectural VGPRs per wave), 8 waves per SIMD,
//      1024 threads per workgroup;
//   2. prices each feasible tiling per (query, key) pair at four levels:
//        matrix-core and VALU issue of the per-tile loop (a phase model of
//        the ping-pong or sequential form, below),
//        LDS reads   4d / (32 qb)   bytes per pair (each wave reads every K
//                                   and V operand once per tile for its
//                                   32 qb queries) at 128 B/clk/CU,
//        L2 -> LDS   4d / BM        bytes per pair (a K/V row is fetched once
//                                   per resident query tile: the 2MNK/S
//                                   traffic of the tiled product) at
//                                   64 B/clk/CU,
//        beyond L2   4d / (32 wpc BM) bytes per pair (the query tiles of one
//                                   head resident on one XCD's 32 CUs share
//                                   one pass over the keys) at 8 TB/s;
//      the predicted cost is the largest of the four (the roofline of the
//      tier that binds);
//   3. ranks, among the tilings predicted within 15% of the cheapest, by the
//      I/O: fewest L2 -> LDS bytes per pair (the tallest resident query tile
//      that fits), then fewest bytes beyond L2 (the most query rows sharing
//      an L2), then the predicted cost, then wider key tiles and fewer
//      stages.  (Measured on MI355X, this order put first the fastest of the
//      compiled tilings at both head sizes; ranking by the predicted cost
//      alone did not at d = 64, where it overstates per-tile overheads.)
//
// The dispatch runs the best-ranked tiling that is compiled into the library.
// The per-pair prices do not depend on the sequence length, so neither does
// the choice; the shape-dependent byte counts of one call (T_min, T_LDS, T_L2)
// come from io_bytes() below.
//
// Phase model (cycles per SIMD; the constants were measured on MI355X with
// per-wave timestamps in instrumented builds of the kernel):
//   MFMA work   M = 32 per 32x32x16 MFMA + 16 per 16x16x32 row-sum MFMA
//                   + 120 waiting for the first LDS operands of the phase;
//   softmax     S = 4 per VALU instruction + DMA bytes / 64 B/clk (the CU's
//                   load path), in solo-rate cycles; VALU instructions per tile =
//                   scores per lane x 2.5 + 26 + 10 (qb - 1), plus, with the
//                   row sum on the VALU, half a dot2 per score weighted by
//                   0.59 / 0.37 (the measured rates of the other VALU work and
//                   of dot2 beside an MFMA stream);
//   overlap     while the SIMD's MFMA pipe is busy a VALU stream beside it runs
//               at rho = 0.45 of its solo rate, so a phase with MFMA work M and
//               softmax work S takes M + max(0, S - rho M);
//   ping-pong   k = waves per SIMD in each phase (waves / 8 per workgroup);
//               one round (every wave advances one tile) = two half steps of
//               k M + max(0, S_k - rho k M), S_k the softmax of k waves plus
//               the DMA of one tile per workgroup (headline tiling: predicted
//               2600 cycles per half step, measured 2545);
//   sequential  n = waves per SIMD, each running both phases: one round =
//               n M + max(0, n S - rho n M) + 250 for the per-tile barrier.
//   MFMA shape  the same products on 16x16x32 instead of 32x32x16 (the d = 128
//               ping-pong form) take the same cycles, but under the chip's
//               power limit a cycle of the smaller shape costs less: a long
//               all-CU stream on random operands delivered 0.834 of the bf16
//               nameplate on 16x16x32 and 0.703 on 32x32x16 (measured).  The
//               issue price of such a tiling is scaled by 0.703 / 0.834.  (The
//               kernel gains less than that ratio: it runs 19% faster clocks
//               but keeps the matrix pipe busy 0.75 instead of 0.86 of them;
//               measured 3.4% faster at the headline shape.)

#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "kernels.h"

namespace attnio {
namespace {

constexpr int kLdsPerCU = 160 * 1024;
constexpr int kRegsPerLane = 512;     // per SIMD lane, shared by the SIMD's waves
constexpr int kMaxArchVgpr = 256;     // architectural VGPRs per wave (no AGPRs used)
constexpr int kMaxWavesPerSimd = 8;
constexpr double kLdsBytesPerClk = 128.0;
constexpr double kL2ToLdsBytesPerClk = 64.0;
constexpr double kHbmBytesPerClkPerCU = 8.0e12 / 2.4e9 / 256.0;
constexpr double kDmaBytesPerClk = 64.0;
constexpr double kBarrierCycles = 250.0;  // the sequential form's per-tile barrier
constexpr double kRho = 0.45;             // VALU rate beside a busy MFMA pipe, relative to solo
constexpr double kDot2Slowdown = 0.59 / 0.37;  // dot2 vs other VALU ops beside an MFMA stream
constexpr double kPhaseStartCycles = 120.0;
constexpr double kMfma16PowerRatio = 0.703 / 0.834;  // 32x32x16 vs 16x16x32 delivered rate, power-limited

int read_ahead(int qb) { return qb == 1 ? 4 : 2; }

}  // namespace

int vgpr_estimate(int d, int BN, int qb, int rowsum_mfma) {
  // per query block: O^T accumulator d/2, Q operands d/4, S^T BN/2, P BN/4;
  // operand read-ahead ring, selection operand and row-sum results, the
  // shift and sum, addresses and loop state (calibrated on the compiled
  // kernels to within 8 registers)
  return qb * (d / 2 + d / 4 + BN / 2 + BN / 4) + 4 * (read_ahead(qb) + 1) +
         (rowsum_mfma ? 4 + 4 * qb : 0) + 2 * qb + 9;
}

bool tiling_fits(const Tiling& t, int* vgpr_est, int* vgpr_budget) {
  const int waves_per_simd = t.waves / 4 * t.wg_per_cu;
  const int budget = std::min(kMaxArchVgpr, kRegsPerLane / std::max(1, waves_per_simd));
  const int est = vgpr_estimate(t.d, t.BN, t.qb, t.rowsum_mfma);
  if (vgpr_est) *vgpr_est = est;
  if (vgpr_budget) *vgpr_budget = budget;
  if (t.waves % 4 != 0 || t.waves * 64 > 1024 || waves_per_simd > kMaxWavesPerSimd) return false;
  if (t.pingpong && (t.waves < 8 || t.stages != 2)) return false;  // two groups, one K and one V per group step
  const int row = t.d * 2;
  const int issuing_waves = t.pingpong ? t.waves / 2 : t.waves;
  if ((t.BN * row) % (16 * 64 * issuing_waves) != 0) return false;     // tile splits over the issuing waves
  if ((64 * issuing_waves * 16) % row != 0) return false;
  if (t.wg_per_cu * t.lds_bytes > kLdsPerCU) return false;
  return est <= budget;
}

void price_tiling(TileEval* e) {
  const Tiling& t = e->t;
  const double d = t.d, BN = t.BN, qb = t.qb, wpc = t.wg_per_cu;
  const double n_pv = (BN / 16) * (d / 32) * qb, n_qk = (d / 16) * (BN / 32) * qb;
  const double n_rs = t.rowsum_mfma ? qb * BN / 16 : 0.0;
  const double scores = qb * 32.0 * BN / 64.0;                        // per lane per tile
  // fma, exp and half a conversion per score, plus the per-tile overhead; a
  // VALU row sum adds half a two-element dot product per score, which beside
  // an MFMA stream runs at 0.37 of its solo rate against 0.59 for the rest
  const double vinst = scores * 2.5 + 26.0 + 10.0 * (qb - 1) +
                       (t.rowsum_mfma ? 0.0 : scores * 0.5 * kDot2Slowdown);
  const double tile_bytes = BN * d * 2.0;                             // one K or one V tile
  // Per phase, the MFMA pipe is busy M_k cycles; the softmax work S_k (in
  // solo-rate cycles) runs at rate rho while the pipe is busy and at full rate
  // after it: phase time = M_k + max(0, S_k - rho M_k).
  double round, pairs;
  if (t.pingpong) {
    const double k = t.waves / 8.0 * wpc;  // waves per SIMD in each phase
    // Row sums issued by the softmax wave use the matrix pipe while the MFMA
    // wave waits for its first LDS operands (about 32 cycles per operand read
    // ahead), at no cost to either wave.  If they do not fit that wait they
    // queue behind the MFMA stream, and the in-order softmax wave cannot
    // start its VALU work until that stream ends: no overlap.  (Measured: at
    // 4 reads ahead the softmax wave's placement is 2% faster than the
    // stream's at d = 128; at 2 reads ahead, QB = 2, 1.8% slower at d = 64.)
    // (In the 16x16x32 form they do not fit, measured: by the softmax wave
    // 6.38 ms against 6.33 ms in the stream at the headline shape.)
    const bool by_softmax = t.rowsum_mfma && !t.rowsum_in_stream;
    const bool fits = !t.mfma16 && 16.0 * n_rs <= 32.0 * read_ahead(t.qb);
    const double M = 32.0 * (n_pv + n_qk) + (by_softmax ? 0.0 : 16.0 * n_rs) + kPhaseStartCycles;
    // per half step each workgroup's softmax group issues one tile's DMA (K or V)
    const double S = k * vinst * 4.0 + wpc * tile_bytes / kDmaBytesPerClk;
    e->mfma_cycles = M;
    e->valu_cycles = S / k;
    const double overlap = (by_softmax && !fits) ? 0.0 : kRho;
    round = 2.0 * (k * M + std::max(0.0, S - overlap * k * M));
    pairs = 2.0 * k * qb * 32.0 * BN;
  } else {
    const double M = 32.0 * (n_pv + n_qk) + 16.0 * n_rs + kPhaseStartCycles;
    const double n = t.waves / 4.0 * wpc;  // waves sharing a SIMD
    // every wave runs both phases; the CU's waves issue both tiles (K and V)
    // of every workgroup, and the tile barrier costs kBarrierCycles
    const double S = n * vinst * 4.0 + 2.0 * wpc * tile_bytes / kDmaBytesPerClk;
    e->mfma_cycles = M;
    e->valu_cycles = S / n;
    round = n * M + std::max(0.0, S - kRho * n * M) + kBarrierCycles;
    pairs = n * qb * 32.0 * BN;
  }
  e->issue_cycles_per_pair = round / pairs / 4.0;                     // per CU (4 SIMDs)
  if (t.mfma16) e->issue_cycles_per_pair *= kMfma16PowerRatio;
  e->lds_read_bytes_per_pair = 4.0 * d / (32.0 * qb);
  e->l2_to_lds_bytes_per_pair = 4.0 * d / t.BM;
  e->beyond_l2_bytes_per_pair = 4.0 * d / (32.0 * wpc * t.BM);
  const double c_lds = e->lds_read_bytes_per_pair / kLdsBytesPerClk;
  const double c_l2 = e->l2_to_lds_bytes_per_pair / kL2ToLdsBytesPerClk;
  const double c_hbm = e->beyond_l2_bytes_per_pair / kHbmBytesPerClkPerCU;
  e->cycles_per_pair = std::max(std::max(e->issue_cycles_per_pair, c_lds), std::max(c_l2, c_hbm));
  e->bound = e->cycles_per_pair == e->issue_cycles_per_pair ? 0 : e->cycles_per_pair == c_lds ? 1
             : e->cycles_per_pair == c_l2 ? 2 : 3;
}

namespace {

// Ranking.  Among the tilings whose predicted cost is within kNearBest of the
// cheapest, the I/O decides, as in the I/O analysis: fewest bytes into LDS per
// pair (the tallest resident query tile), then fewest beyond L2 (the most
// query rows sharing one L2), then the predicted cost, then wider key tiles
// and fewer stages.  Tilings outside that band follow, cheapest first.
constexpr double kNearBest = 1.15;

bool better(const TileEval& a, const TileEval& b, double best) {
  const bool na = a.cycles_per_pair <= kNearBest * best, nb = b.cycles_per_pair <= kNearBest * best;
  if (na != nb) return na;
  if (!na) return a.cycles_per_pair < b.cycles_per_pair;
  if (a.l2_to_lds_bytes_per_pair != b.l2_to_lds_bytes_per_pair)
    return a.l2_to_lds_bytes_per_pair < b.l2_to_lds_bytes_per_pair;
  if (a.beyond_l2_bytes_per_pair != b.beyond_l2_bytes_per_pair)
    return a.beyond_l2_bytes_per_pair < b.beyond_l2_bytes_per_pair;
  if (a.cycles_per_pair != b.cycles_per_pair) return a.cycles_per_pair < b.cycles_per_pair;
  if (a.t.BN != b.t.BN) return a.t.BN > b.t.BN;
  if (a.t.stages != b.t.stages) return a.t.stages < b.t.stages;  // less LDS for the same price
  return a.compiled > b.compiled;  // prefer the built one among equals
}

int compiled_index(const Tiling& t) {
  for (int i = 0; i < bf16_variant_count(); ++i) {
    Tiling c{};
    bf16_variant(i, &c);
    if (c.d == t.d && c.BM == t.BM && c.BN == t.BN && c.stages == t.stages && c.waves == t.waves &&
        c.wg_per_cu == t.wg_per_cu && c.qb == t.qb && c.pingpong == t.pingpong &&
        c.rowsum_mfma == t.rowsum_mfma && c.rowsum_in_stream == t.rowsum_in_stream && c.mfma16 == t.mfma16)
      return i;
  }
  return -1;
}

}  // namespace

int enumerate_tilings(int d, TileEval* out, int max_out) {
  static const int kWaves[] = {4, 8, 16};
  static const int kQB[] = {1, 2};
  static const int kBN[] = {32, 64, 128, 256};
  static const int kStages[] = {2, 3, 4};
  static const int kWPC[] = {1, 2, 3, 4};
  std::vector<TileEval> all(3 * 2 * 4 * 3 * 4 * 2 * 3 * 2);  // every combination (about 440 KB)
  int n = 0;
  for (int w : kWaves)
    for (int qb : kQB)
      for (int bn : kBN)
        for (int st : kStages)
          for (int wpc : kWPC)
            for (int pp = 0; pp < 2; ++pp)
              for (int rs = 0; rs < 3; ++rs)  // VALU; matrix core in the stream; by the softmax wave
                for (int mf = 0; mf < 2; ++mf) {  // MFMA shape: 32x32x16, 16x16x32
                  if (rs == 2 && !pp) continue;
                  // the 16x16x32 form is written for d = 128, ping-pong, 32
                  // queries per wave, row sums on the matrix core
                  if (mf && !(d == 128 && pp && qb == 1 && rs > 0)) continue;
                  TileEval e{};
                  Tiling& t = e.t;
                  t.d = d;
                  t.BM = 32 * w * qb;
                  t.BN = bn;
                  t.stages = st;
                  t.waves = w;
                  t.qb = qb;
                  t.wg_per_cu = wpc;
                  t.pingpong = pp;
                  t.rowsum_mfma = rs > 0;
                  t.rowsum_in_stream = rs == 1;
                  t.mfma16 = mf;
                  const int ring = st * 2 * bn * d * 2, outb = t.BM * d * 2;
                  t.lds_bytes = std::max(ring, outb) + 16;
                  if (!tiling_fits(t, &e.vgpr_estimate, &e.vgpr_budget)) continue;
                  e.compiled = compiled_index(t);
                  price_tiling(&e);
                  all[n++] = e;
                }
  double best = 1e300;
  for (int i = 0; i < n; ++i) best = std::min(best, all[i].cycles_per_pair);
  std::stable_sort(all.begin(), all.begin() + n,
                   [best](const TileEval& a, const TileEval& b) { return better(a, b, best); });
  for (int i = 0; i < n && i < max_out; ++i) out[i] = all[i];
  return n;
}

int chosen_variant(int d) {
  static std::once_flag once[2];
  static int pick[2] = {-1, -1};
  const int slot = d == 128 ? 0 : d == 64 ? 1 : -1;
  if (slot < 0) return -1;
  std::call_once(once[slot], [slot, d] {
    TileEval ev[256];
    const int n = enumerate_tilings(d, ev, 256);
    for (int i = 0; i < n && i < 256; ++i)
      if (ev[i].compiled >= 0) {
        pick[slot] = ev[i].compiled;
        break;
      }
  });
  return pick[slot];
}

void io_bytes(const Tiling& t, int B, int H, int N, int d, int elem, int causal,
              const int32_t* kv_len_host, double* t_min_out, double* t_lds_out, double* t_l2_out,
              double* pairs_out) {
  const double row = (double)d * elem;
  const long long BM = t.BM, BN = t.BN;
  const long long nqt = (N + BM - 1) / BM;
  // query tiles of one head run together on one XCD (32 CUs), `resident` at
  // a time; each such generation streams the keys it needs through L2 once
  const long long resident = 32LL * (t.wg_per_cu > 0 ? t.wg_per_cu : 1);
  // the int32 key-padding lengths are read only when the call has them
  double t_min = kv_len_host ? 4.0 * B : 0.0, t_lds = 0, t_l2 = 0, pairs = 0;
  for (int b = 0; b < B; ++b) {
    long long L = N;
    if (kv_len_host) {
      L = kv_len_host[b];
      L = L < 0 ? 0 : (L > N ? N : L);
    }
    // visible (query, key) pairs of one head: sum_i min(i + 1, L) causal, N L otherwise
    const double p = causal ? (double)L * (double)(L + 1) / 2.0 + (double)(N - L) * (double)L
                            : (double)N * (double)L;
    for (int h = 0; h < H; ++h) {
      pairs += p;
      t_min += row * (2.0 * N + 2.0 * L);
      t_l2 += row * 2.0 * N;  // Q read and O written once
      for (long long qt = 0; qt < nqt; ++qt) {
        long long kend = L;
        if (causal) kend = kend < (qt + 1) * BM ? kend : ((qt + 1) * BM < N ? (qt + 1) * BM : N);
        const long long tiles = (kend + BN - 1) / BN;
        t_lds += row * (double)BM + 2.0 * row * (double)(tiles * BN);
      }
      // one generation = `resident` query tiles running together; K/V of the
      // keys that generation needs come from beyond L2 once per generation,
      // assuming its workgroups walk the keys in step.  Causal generations
      // alternate the key direction, so each one after the first starts on
      // keys the previous one ended on: up to one L2 (4 MiB per XCD) of them
      // is reused.
      const double l2_keys = 4.0 * 1024.0 * 1024.0 / (2.0 * row);
      for (long long g0 = 0; g0 < nqt; g0 += resident) {
        // causal tiles run longest first: generation g covers the highest
        // remaining query tiles, so it needs keys up to its first tile's end
        const long long top = causal ? nqt - g0 : nqt;
        long long kend = L;
        if (causal) kend = kend < top * BM ? kend : (top * BM < N ? top * BM : N);
        double keys = (double)kend;
        if (causal && g0 > 0) keys -= (l2_keys < keys ? l2_keys : keys);
        t_l2 += 2.0 * row * keys;
      }
    }
  }
  if (t_min_out) *t_min_out = t_min;
  if (t_lds_out) *t_lds_out = t_lds;
  if (t_l2_out) *t_l2_out = t_l2;
  if (pairs_out) *pairs_out = pairs;
}

}  // namespace attnio
