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

#include "../../include/attnio.h"
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
  if (B < 1 || H < 1 || N < 1) return ATTN_E_SHAPE;
  const long long total = (long long)B * H * N * d;
  if (total >= (1LL << 31)) return ATTN_E_SHAPE;
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15u) return ATTN_E_ALIGN;
  const size_t bytes = (size_t)total * elem;
  if (overlaps(O, Q, bytes) || overlaps(O, K, bytes) || overlaps(O, V, bytes)) return ATTN_E_ALIAS;
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return ATTN_E_ARG;
  return ATTN_OK;
}

int run(bool bf16, const void* Q, const void* K, const void* V, void* O, float* lse, bool want_lse,
        int B, int H, int N, int d, float scale, int causal, const int32_t* kv_len, void* stream) {
  const int rc = validate(Q, K, V, O, B, H, N, d, scale, bf16 ? 2 : 4);
  if (rc != ATTN_OK) return rc;
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
    if (bf16 && attnio::bf16_tiling(d, causal, &t))
      fprintf(stderr, "[attnio] bf16 B=%d H=%d N=%d d=%d causal=%d kv_len=%s BM=%d BN=%d stages=%d waves=%d lds=%d\n",
              B, H, N, d, causal, kv_len ? "dev" : "none", t.BM, t.BN, t.stages, t.waves, t.lds_bytes);
    else
      fprintf(stderr, "[attnio] f32 B=%d H=%d N=%d d=%d causal=%d kv_len=%s\n", B, H, N, d, causal,
              kv_len ? "dev" : "none");
  }
  const hipError_t e = bf16 ? attnio::launch_fwd_bf16(a, (hipStream_t)stream)
                            : attnio::launch_fwd_f32(a, (hipStream_t)stream);
  if (e != hipSuccess) {
    if (log_enabled()) fprintf(stderr, "[attnio] launch failed: %s\n", hipGetErrorString(e));
    return ATTN_E_LAUNCH;
  }
  return ATTN_OK;
}

// number of (query, visible key) pairs of one (b, h) slice
double pair_count(long long N, long long L, bool causal) {
  if (!causal) return (double)N * (double)L;
  // sum_i min(i + 1, L) = L(L+1)/2 + (N - L) L
  return (double)L * (double)(L + 1) / 2.0 + (double)(N - L) * (double)L;
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
  if (B < 1 || H < 1 || N < 1 || (long long)B * H * N * d >= (1LL << 31)) return ATTN_E_SHAPE;
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

int attn_query_tiling(int d, int causal, int* BM, int* BN, int* stages, int* waves) {
  attnio::Tiling t{};
  if (!attnio::bf16_tiling(d, causal, &t)) return ATTN_E_HEAD_DIM;
  if (BM) *BM = t.BM;
  if (BN) *BN = t.BN;
  if (stages) *stages = t.stages;
  if (waves) *waves = t.waves;
  return ATTN_OK;
}

int attn_io_model(int B, int H, int N, int d, int elem_bytes, int causal,
                  const int32_t* kv_len_host, double out[5]) {
  if (!out) return ATTN_E_NULL;
  if (d != 64 && d != 128) return ATTN_E_HEAD_DIM;
  if (B < 1 || H < 1 || N < 1 || (long long)B * H * N * d >= (1LL << 31)) return ATTN_E_SHAPE;
  if (elem_bytes != 2 && elem_bytes != 4) return ATTN_E_ARG;
  attnio::Tiling t{};
  attnio::bf16_tiling(d, causal, &t);
  const double row = (double)d * elem_bytes;
  const long long BM = t.BM, BN = t.BN;
  const long long nqt = (N + BM - 1) / BM;
  // query tiles of one head run together on one XCD (32 CUs), `resident` at
  // a time; each such generation streams the keys it needs through L2 once
  const long long resident = 32LL * (t.wg_per_cu > 0 ? t.wg_per_cu : 1);
  double t_min = 4.0 * B, t_lds = 0, t_l2 = 0, pairs = 0;
  for (int b = 0; b < B; ++b) {
    long long L = N;
    if (kv_len_host) {
      L = kv_len_host[b];
      L = L < 0 ? 0 : (L > N ? N : L);
    }
    const double p = pair_count(N, L, causal != 0);
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
  out[0] = t_min;
  out[1] = t_lds;
  out[2] = t_l2;
  out[3] = 4.0 * d * pairs;
  out[4] = pairs;
  return ATTN_OK;
}

}  // extern "C"
