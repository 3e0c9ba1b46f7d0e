// C-ABI front end of the attention library: argument checks, device check,
// kernel selection and the host-side I/O model.  See include/attnio.h for the
// contract of every entry point.

#include <hip/hip_runtime.h>
#include <cmath>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "attnio.h"
#include "kernels.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int kMaxDevices = 64;

bool log_enabled() {
  static const bool on = [] {
    const char* e = getenv("ATTNIO_LOG");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

// 1 = gfx950, 0 = other, -1 = not yet probed.
int g_dev_ok[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];

bool current_device_is_gfx950() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t p;
    g_dev_ok[dev] = 0;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess && strncmp(p.gcnArchName, "gfx950", 6) == 0)
      g_dev_ok[dev] = 1;
  });
  return g_dev_ok[dev] == 1;
}

// B, H, N >= 1 and B*H*N*d < 2^31, tested without forming a product that could
// overflow (each partial product stays below 2^31 before the next factor,
// itself below 2^31, multiplies it).
bool shape_ok(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return false;
  const long long lim = 1LL << 31;
  long long p = B;
  for (long long f : {(long long)H, (long long)N, (long long)d}) {
    p *= f;
    if (p >= lim) return false;
  }
  return true;
}

// hipGetLastError() returns and clears the calling thread's last HIP error.
// Called once the arguments are accepted and before anything is enqueued, so
// that the status read after the launches names those launches only, not an
// unrelated earlier HIP call of the caller.
void clear_stale_hip_error() { (void)hipGetLastError(); }

bool overlaps(const void* a, const void* b, size_t bytes) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bytes && y < x + bytes;
}

// [a, a + na) and [b, b + nb) intersect
bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int validate(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
             float scale, int elem) {
  if (!Q || !K || !V || !O) return ATTN_E_NULL;
  if (d != 64 && d != 128) return ATTN_E_HEAD_DIM;
  if (!shape_ok(B, H, N, d)) return ATTN_E_SHAPE;
  const long long total = (long long)B * H * N * d;
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15u) return ATTN_E_ALIGN;
  const size_t bytes = (size_t)total * elem;
  if (overlaps(O, Q, bytes) || overlaps(O, K, bytes) || overlaps(O, V, bytes)) return ATTN_E_ALIAS;
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return ATTN_E_ARG;
  return ATTN_OK;
}

// Under ATTNIO_LOG=1: the model's ranking for head size d, once per process.
void log_tiling_choice(int d) {
  static std::once_flag once[2];
  std::call_once(once[d == 128 ? 0 : 1], [d] {
    attnio::TileEval ev[256];
    const int n = attnio::enumerate_tilings(d, ev, 256);
    const int pick = attnio::chosen_variant(d);
    fprintf(stderr, "[attnio] tiling model, d=%d: %d feasible tilings; best first:\n", d, n);
    for (int i = 0; i < n && i < 6; ++i) {
      const attnio::Tiling& t = ev[i].t;
      fprintf(stderr,
              "[attnio]   BM=%d BN=%d stages=%d waves=%d qb=%d wg/cu=%d %s rowsum=%s mfma=%s vgpr~%d/%d: "
              "%.4f cyc/pair (issue %.4f, LDS %.1f B, L2->LDS %.2f B, beyond L2 %.4f B)%s\n",
              t.BM, t.BN, t.stages, t.waves, t.qb, t.wg_per_cu, t.pingpong ? "ping-pong" : "sequential",
              t.rowsum_mfma ? "mfma" : "valu", t.mfma16 ? "16x16x32" : "32x32x16", ev[i].vgpr_estimate,
              ev[i].vgpr_budget, ev[i].cycles_per_pair,
              ev[i].issue_cycles_per_pair, ev[i].lds_read_bytes_per_pair, ev[i].l2_to_lds_bytes_per_pair,
              ev[i].beyond_l2_bytes_per_pair, ev[i].compiled >= 0 ? " [compiled]" : "");
    }
    attnio::Tiling t{};
    if (attnio::bf16_variant(pick, &t))
      fprintf(stderr, "[attnio]   running compiled tiling %d: BM=%d BN=%d waves=%d qb=%d wg/cu=%d\n", pick,
              t.BM, t.BN, t.waves, t.qb, t.wg_per_cu);
  });
}

int run(bool bf16, const void* Q, const void* K, const void* V, void* O, float* lse, bool want_lse,
        int B, int H, int N, int d, float scale, int causal, const int32_t* kv_len, void* stream,
        int variant = -1) {
  const int rc = validate(Q, K, V, O, B, H, N, d, scale, bf16 ? 2 : 4);
  if (rc != ATTN_OK) return rc;
  if (bf16) {
    if (variant < 0) variant = attnio::chosen_variant(d);
    attnio::Tiling vt{};
    if (!attnio::bf16_variant(variant, &vt) || vt.d != d) return ATTN_E_ARG;
  }
  if (want_lse) {
    if (lse == nullptr) return ATTN_E_NULL;
    if (((uintptr_t)lse) & 3u) return ATTN_E_ALIGN;
    const size_t lb = (size_t)B * H * N * sizeof(float);
    const size_t tb = (size_t)B * H * N * d * (bf16 ? 2 : 4);
    if (ranges_overlap(lse, lb, Q, tb) || ranges_overlap(lse, lb, K, tb) ||
        ranges_overlap(lse, lb, V, tb) || ranges_overlap(lse, lb, O, tb))
      return ATTN_E_ALIAS;
  }
  if (!current_device_is_gfx950()) return ATTN_E_DEVICE;
  clear_stale_hip_error();
  attnio::FwdArgs a{Q, K, V, O, kv_len, B, H, N, d, scale, causal ? 1 : 0, want_lse ? lse : nullptr};
  if (log_enabled()) {
    attnio::Tiling t{};
    if (bf16 && attnio::bf16_variant(variant, &t)) {
      log_tiling_choice(d);
      fprintf(stderr, "[attnio] bf16 B=%d H=%d N=%d d=%d causal=%d kv_len=%s tiling %d: BM=%d BN=%d "
              "stages=%d waves=%d qb=%d wg/cu=%d lds=%d\n", B, H, N, d, causal, kv_len ? "dev" : "none",
              variant, t.BM, t.BN, t.stages, t.waves, t.qb, t.wg_per_cu, t.lds_bytes);
    } else {
      fprintf(stderr, "[attnio] f32 B=%d H=%d N=%d d=%d causal=%d kv_len=%s\n", B, H, N, d, causal,
              kv_len ? "dev" : "none");
    }
  }
  const hipError_t e = bf16 ? attnio::launch_fwd_bf16(variant, a, (hipStream_t)stream)
                            : attnio::launch_fwd_f32(a, (hipStream_t)stream);
  if (e != hipSuccess) {
    if (log_enabled()) fprintf(stderr, "[attnio] launch failed: %s\n", hipGetErrorString(e));
    return ATTN_E_LAUNCH;
  }
  return ATTN_OK;
}


// ---------------------------------------------------------------------------
// Backward scratch without allocation.  attn_bwd_noalloc keeps the backward's
// row statistics in this file-scope device array instead of a caller
// workspace, for callers that cannot allocate.  Each device holds its own copy
// at its own address; in host code `scratch` only names the symbol, so its
// device address is looked up once per device (with that device current) and
// only that address is ever passed to kernels.
constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of this device's scratch array, or nullptr (with the HIP error
// in *err) if it could not be looked up.
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    if (*err == hipSuccess) *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

// Argument checks and launch of the backward.  With check_ws the workspace is
// the caller's (checked for alignment and overlap); otherwise it is this
// device's scratch array.  checks_only: return after the host-side checks.
int run_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
            const float* LSE, void* dQ, void* dK, void* dV, void* workspace, bool check_ws, int B,
            int H, int N, int d, float scale, int causal, const int32_t* kv_len, void* stream,
            bool checks_only = false) {
  if (!dO || !LSE || !dQ || !dK || !dV) return ATTN_E_NULL;
  int rc = validate(Q, K, V, dQ, B, H, N, d, scale, 2);
  if (rc != ATTN_OK) return rc;
  if (!O) return ATTN_E_NULL;
  const size_t tb = (size_t)B * H * N * d * 2;
  const size_t lb = (size_t)B * H * N * sizeof(float);
  const size_t wb = attnio::bwd_workspace_bytes(B, H, N);
  if ((((uintptr_t)O | (uintptr_t)dO | (uintptr_t)dK | (uintptr_t)dV |
        (check_ws ? (uintptr_t)workspace : 0u)) & 15u) ||
      ((uintptr_t)LSE & 3u))
    return ATTN_E_ALIGN;
  // outputs must not overlap any input, each other, or the workspace
  const void* ins[6] = {Q, K, V, O, dO, LSE};
  const size_t in_b[6] = {tb, tb, tb, tb, tb, lb};
  void* outs[4] = {dQ, dK, dV, workspace};
  const size_t out_b[4] = {tb, tb, tb, wb};
  const int n_out = check_ws ? 4 : 3;
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < 6; ++j)
      if (ranges_overlap(outs[i], out_b[i], ins[j], in_b[j])) return ATTN_E_ALIAS;
    for (int j = i + 1; j < n_out; ++j)
      if (ranges_overlap(outs[i], out_b[i], outs[j], out_b[j])) return ATTN_E_ALIAS;
  }
  if (checks_only) return ATTN_OK;
  if (!current_device_is_gfx950()) return ATTN_E_DEVICE;
  if (!check_ws) {
    hipError_t se = hipSuccess;
    workspace = scratch_on_current_device(&se);
    if (workspace == nullptr) {
      if (log_enabled()) fprintf(stderr, "[attnio] scratch lookup failed: %s\n", hipGetErrorString(se));
      return ATTN_E_LAUNCH;
    }
  }
  clear_stale_hip_error();
  attnio::BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, (float*)workspace, kv_len, B, H, N, d, scale,
                    causal ? 1 : 0};
  const hipError_t e = attnio::launch_bwd_bf16(a, (hipStream_t)stream);
  if (e != hipSuccess) {
    if (log_enabled()) fprintf(stderr, "[attnio] backward launch failed: %s\n", hipGetErrorString(e));
    return ATTN_E_LAUNCH;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
             float scale, int causal, const int32_t* kv_len, void* stream) {
  return run(true, Q, K, V, O, nullptr, false, B, H, N, d, scale, causal, kv_len, stream);
}

int attn_fwd_f32(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                 float scale, int causal, const int32_t* kv_len, void* stream) {
  return run(false, Q, K, V, O, nullptr, false, B, H, N, d, scale, causal, kv_len, stream);
}

int attn_fwd_lse(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                 int N, int d, float scale, int causal, const int32_t* kv_len, void* stream) {
  return run(true, Q, K, V, O, LSE, true, B, H, N, d, scale, causal, kv_len, stream);
}

int attn_fwd_f32_lse(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                     int N, int d, float scale, int causal, const int32_t* kv_len, void* stream) {
  return run(false, Q, K, V, O, LSE, true, B, H, N, d, scale, causal, kv_len, stream);
}

size_t attn_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  return attnio::bwd_workspace_bytes(B, H, N);
}

int attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* LSE, void* dQ, void* dK, void* dV, void* workspace, int B, int H, int N,
             int d, float scale, int causal, const int32_t* kv_len, void* stream) {
  if (!workspace) return ATTN_E_NULL;
  return run_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, true, B, H, N, d, scale, causal, kv_len,
                 stream);
}

int attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int N, int d,
                     float scale, int causal, const int32_t* kv_len, void* stream) {
  if (B >= 1 && H >= 1 && N >= 1 && attnio::bwd_workspace_bytes(B, H, N) > kScratchBytes) {
    // run the ordinary checks first so that a bad pointer still reports as such
    const int rc = run_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, nullptr, false, B, H, N, d, scale, causal,
                           kv_len, stream, /*checks_only=*/true);
    return rc != ATTN_OK ? rc : ATTN_E_SCRATCH;
  }
  return run_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, nullptr, false, B, H, N, d, scale, causal, kv_len,
                 stream);
}

size_t attn_fwd_unfused_workspace_bytes(int N) {
  if (N < 1) return 0;
  return attnio::unfused_head_bytes(N);
}

int attn_fwd_unfused(const void* Q, const void* K, const void* V, void* O, void* workspace,
                     size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                     const int32_t* kv_len, void* stream) {
  if (!workspace) return ATTN_E_NULL;
  int rc = validate(Q, K, V, O, B, H, N, d, scale, 2);
  if (rc != ATTN_OK) return rc;
  if ((uintptr_t)workspace & 255u) return ATTN_E_ALIGN;
  if (workspace_bytes < attnio::unfused_head_bytes(N)) return ATTN_E_ARG;
  const size_t tb = (size_t)B * H * N * d * 2;
  const void* ins[4] = {Q, K, V, O};
  for (int j = 0; j < 4; ++j)
    if (ranges_overlap(workspace, workspace_bytes, ins[j], tb)) return ATTN_E_ALIAS;
  if (!current_device_is_gfx950()) return ATTN_E_DEVICE;
  clear_stale_hip_error();
  attnio::UnfusedArgs a{Q, K, V, O, workspace, workspace_bytes, kv_len, B, H, N, d, scale,
                        causal ? 1 : 0};
  const hipError_t e = attnio::launch_unfused_bf16(a, (hipStream_t)stream);
  if (e != hipSuccess) {
    if (log_enabled()) fprintf(stderr, "[attnio] unfused launch failed: %s\n", hipGetErrorString(e));
    return ATTN_E_LAUNCH;
  }
  return ATTN_OK;
}

int attn_fwd_fp8(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                 float scale, float q_descale, float k_descale, float v_descale, int causal,
                 const int32_t* kv_len, void* stream) {
  if (!Q || !K || !V || !O) return ATTN_E_NULL;
  if (d != 64 && d != 128) return ATTN_E_HEAD_DIM;
  if (!shape_ok(B, H, N, d)) return ATTN_E_SHAPE;
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15u) return ATTN_E_ALIGN;
  if (!std::isfinite(scale)) return ATTN_E_ARG;
  for (float s : {q_descale, k_descale, v_descale})
    if (!std::isfinite(s) || !(s > 0.f)) return ATTN_E_ARG;
  // the kernel folds scale, both descales and log2(e) into one fp32 exponent
  // multiplier (same product, same order as its launcher); finite factors
  // whose product overflows would turn every score into +-inf and O into NaN
  if (!std::isfinite(scale * q_descale * k_descale * 1.4426950408889634f)) return ATTN_E_ARG;
  const size_t in_b = (size_t)B * H * N * d, out_b = 2 * in_b;
  if (ranges_overlap(O, out_b, Q, in_b) || ranges_overlap(O, out_b, K, in_b) ||
      ranges_overlap(O, out_b, V, in_b))
    return ATTN_E_ALIAS;
  if (!current_device_is_gfx950()) return ATTN_E_DEVICE;
  clear_stale_hip_error();
  attnio::Fp8Args a{Q, K, V, O, kv_len, B, H, N, d, scale, causal ? 1 : 0,
                    q_descale, k_descale, v_descale};
  const hipError_t e = attnio::launch_fwd_fp8(a, (hipStream_t)stream);
  if (e != hipSuccess) {
    if (log_enabled()) fprintf(stderr, "[attnio] fp8 launch failed: %s\n", hipGetErrorString(e));
    return ATTN_E_LAUNCH;
  }
  return ATTN_OK;
}

namespace {
int run_rows(const void* X, const void* gamma, const void* beta, void* Y, int R, int N, int op,
             float param, void* stream) {
  if (!X || !Y) return ATTN_E_NULL;
  if (R < 1 || N < 1 || (long long)R * N >= (1LL << 40)) return ATTN_E_SHAPE;
  if (((uintptr_t)X | (uintptr_t)Y | (uintptr_t)gamma | (uintptr_t)beta) & 15u) return ATTN_E_ALIGN;
  if (!std::isfinite(param) || !(param > 0.f)) return ATTN_E_ARG;
  const size_t xb = (size_t)R * N * 2, vb = (size_t)N * 2;
  // Y may be X itself (each element is read before it is written, by the same
  // thread); any other overlap is rejected, as is Y overlapping gamma or beta
  if (X != Y && ranges_overlap(X, xb, Y, xb)) return ATTN_E_ALIAS;
  if ((gamma && ranges_overlap(gamma, vb, Y, xb)) || (beta && ranges_overlap(beta, vb, Y, xb)))
    return ATTN_E_ALIAS;
  if (!current_device_is_gfx950()) return ATTN_E_DEVICE;
  clear_stale_hip_error();
  attnio::RowArgs a{X, Y, gamma, beta, R, N, op, param};
  const hipError_t e = attnio::launch_stream_rows(a, (hipStream_t)stream);
  if (e != hipSuccess) {
    if (log_enabled()) fprintf(stderr, "[attnio] row kernel launch failed: %s\n", hipGetErrorString(e));
    return ATTN_E_LAUNCH;
  }
  return ATTN_OK;
}
}  // namespace

int stream_softmax(const void* X, void* Y, int R, int N, float scale, void* stream) {
  return run_rows(X, nullptr, nullptr, Y, R, N, 0, scale, stream);
}

int stream_layernorm(const void* X, const void* gamma, const void* beta, void* Y, int R, int N,
                     float eps, void* stream) {
  return run_rows(X, gamma, beta, Y, R, N, 1, eps, stream);
}

int stream_rows_cached(int N) { return N < 1 ? 0 : attnio::rows_cached_sweeps(N) > 0; }

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "success";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_HEAD_DIM: return "unsupported head size d (supported: 64, 128)";
    case ATTN_E_SHAPE: return "bad shape: B, H, N must be >= 1 and B*H*N*d < 2^31";
    case ATTN_E_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case ATTN_E_LAUNCH: return "kernel launch failed";
    case ATTN_E_DEVICE: return "the current device is not a gfx950 (MI355X) GPU";
    case ATTN_E_ALIAS: return "O overlaps Q, K or V";
    case ATTN_E_ARG: return "argument out of range (scale must be finite)";
    case ATTN_E_SCRATCH:
      return "the backward's statistics need more than the allocation-free entry point's static "
             "scratch (ATTN_NOALLOC_SCRATCH_BYTES); use attn_bwd with a workspace";
    default: return "unknown attnio status code";
  }
}

int attn_version(void) { return kVersion; }

int attn_tiling_count(void) { return attnio::bf16_variant_count(); }

int attn_tiling_get(int index, attn_tiling* out) {
  if (!out) return ATTN_E_NULL;
  if (!attnio::bf16_variant(index, out)) return ATTN_E_ARG;
  return ATTN_OK;
}

int attn_fwd_tiled(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                   float scale, int causal, const int32_t* kv_len, int tiling_index, void* stream) {
  if (tiling_index < 0 || tiling_index >= attnio::bf16_variant_count()) return ATTN_E_ARG;
  return run(true, Q, K, V, O, nullptr, false, B, H, N, d, scale, causal, kv_len, stream, tiling_index);
}

int attn_tiling_enumerate(int d, int dtype, int causal, attn_tiling_eval* out, int max_out) {
  (void)causal;
  if (d != 64 && d != 128) return ATTN_E_HEAD_DIM;
  if (dtype != ATTN_DTYPE_BF16) return ATTN_E_ARG;
  if (!out && max_out > 0) return ATTN_E_NULL;
  attnio::TileEval ev[256];
  const int n = attnio::enumerate_tilings(d, ev, 256);
  for (int i = 0; i < n && i < max_out && i < 256; ++i) out[i] = ev[i];
  return n;
}

namespace {
// The tiling of the path of element type dtype for head size d.
int path_tiling(int d, int dtype, attn_tiling* t) {
  if (d != 64 && d != 128) return ATTN_E_HEAD_DIM;
  *t = attn_tiling{};
  t->d = d;
  switch (dtype) {
    case ATTN_DTYPE_BF16:
      return attnio::bf16_variant(attnio::chosen_variant(d), t) ? ATTN_OK : ATTN_E_HEAD_DIM;
    case ATTN_DTYPE_F32:
      // 8 queries x 32 key lanes per 256-thread workgroup, 64-key tiles in LDS
      t->BM = 8; t->BN = 64; t->stages = 1; t->waves = 4; t->qb = 1; t->wg_per_cu = 1;
      t->lds_bytes = (8 + 2 * 64) * (d + 4) * 4;  // Q, K and V tiles, rows padded by 16 bytes
      return ATTN_OK;
    case ATTN_DTYPE_FP8:
      // 4 waves x 32 queries, 128-key E4M3 tiles, two stages, two workgroups per CU
      t->BM = 128; t->BN = 128; t->stages = 2; t->waves = 4; t->qb = 1; t->wg_per_cu = 2;
      t->lds_bytes = 2 * 2 * 128 * d; t->rowsum_mfma = 1;
      return ATTN_OK;
    default:
      return ATTN_E_ARG;
  }
}
}  // namespace

int attn_query_tiling(int d, int dtype, int causal, int* BM, int* BN, int* stages) {
  (void)causal;
  attn_tiling t{};
  const int rc = path_tiling(d, dtype, &t);
  if (rc != ATTN_OK) return rc;
  if (BM) *BM = t.BM;
  if (BN) *BN = t.BN;
  if (stages) *stages = t.stages;
  return ATTN_OK;
}

int attn_io_bound_bytes(int B, int H, int N, int d, int dtype, int causal, const int32_t* kv_len_host,
                        double* t_min, double* t_lds, double* t_l2) {
  attn_tiling t{};
  const int rc = path_tiling(d, dtype, &t);
  if (rc != ATTN_OK) return rc;
  if (!shape_ok(B, H, N, d)) return ATTN_E_SHAPE;
  const int elem = dtype == ATTN_DTYPE_F32 ? 4 : dtype == ATTN_DTYPE_FP8 ? 1 : 2;
  attnio::io_bytes(t, B, H, N, d, elem, causal != 0, kv_len_host, t_min, t_lds, t_l2, nullptr);
  return ATTN_OK;
}

int attn_io_model(int B, int H, int N, int d, int elem_bytes, int causal,
                  const int32_t* kv_len_host, double out[5]) {
  if (!out) return ATTN_E_NULL;
  if (d != 64 && d != 128) return ATTN_E_HEAD_DIM;
  if (!shape_ok(B, H, N, d)) return ATTN_E_SHAPE;
  if (elem_bytes != 2 && elem_bytes != 4) return ATTN_E_ARG;
  attnio::Tiling t{};
  attnio::bf16_variant(attnio::chosen_variant(d), &t);
  double pairs = 0;
  attnio::io_bytes(t, B, H, N, d, elem_bytes, causal != 0, kv_len_host, &out[0], &out[1], &out[2], &pairs);
  out[3] = 4.0 * d * pairs;
  out[4] = pairs;
  return ATTN_OK;
}

}  // extern "C"
