// Internal launcher declarations shared by the C-ABI front end and the kernel
// translation units.  Not part of the public interface (see include/attnio.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attnio.h"

namespace attnio {

// Launch parameters common to both precisions.  All pointers are device
// pointers already validated by the front end.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* kv_len;  // device int32[B] or nullptr
  int B, H, N, d;
  float scale;
  int causal;
  float* lse;             // device float[B, H, N] or nullptr (log-sum-exp side output)
};

// One tile configuration of the bf16 streaming kernel, and the model's
// evaluation of one (the public structs of include/attnio.h).
using Tiling = attn_tiling;
using TileEval = attn_tiling_eval;

// Host-side tiling model (tile_model.cpp).
int vgpr_estimate(int d, int BN, int qb, int rowsum_mfma);
bool tiling_fits(const Tiling& t, int* vgpr_est, int* vgpr_budget);
void price_tiling(TileEval* e);
// every feasible tiling for head size d, best first; returns the count
int enumerate_tilings(int d, TileEval* out, int max_out);
// compiled variant the forward runs for head size d (the best compiled one)
int chosen_variant(int d);
// T_min, T_LDS, T_L2 and visible pairs of one call with tiling t
void io_bytes(const Tiling& t, int B, int H, int N, int d, int elem, int causal,
              const int32_t* kv_len_host, double* t_min, double* t_lds, double* t_l2, double* pairs);

// Backward launch parameters (device pointers validated by the front end).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* ws;               // bwd_workspace_bytes(B, H, N) bytes
  const int32_t* kv_len;
  int B, H, N, d;
  float scale;
  int causal;
};

// Unfused (operator-centric) forward: S and P of up to ws_bytes / unfused_head_bytes(N)
// heads at a time live in the caller's workspace.
struct UnfusedArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  void* ws;
  size_t ws_bytes;
  const int32_t* kv_len;
  int B, H, N, d;
  float scale;
  int causal;
};

// Streaming row operators on a bf16 [R, N] matrix (op 0: softmax with
// param = scale; op 1: LayerNorm with param = eps, optional gamma / beta).
struct RowArgs {
  const void* x;
  void* y;
  const void* gamma;
  const void* beta;
  int R, N;
  int op;
  float param;
};

// fp8 (E4M3) forward: Q, K, V bytes with per-tensor descales, bf16 O.
struct Fp8Args {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* kv_len;
  int B, H, N, d;
  float scale;
  int causal;
  float q_descale, k_descale, v_descale;
};

// The compiled bf16 forward tilings: count, description of entry i, launch of
// entry i (its head size must be a.d).
int bf16_variant_count();
bool bf16_variant(int i, Tiling* t);
hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream);
int rows_cached_sweeps(int N);
hipError_t launch_stream_rows(const RowArgs& a, hipStream_t stream);
size_t unfused_head_bytes(int N);
hipError_t launch_unfused_bf16(const UnfusedArgs& a, hipStream_t stream);
size_t bwd_workspace_bytes(int B, int H, int N);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
// dQ stage of the backward (ws_d / ws_l: the delta kernel's padded statistics,
// per head NP values of D then NP of lse*log2(e), so head bh's row i is at
// ws_d[bh*2*NP + i] and ws_l[bh*2*NP + i] with ws_l = ws_d + NP;
// c = scale * log2(e)).
hipError_t launch_bwd_dq_bf16(const BwdArgs& a, const float* ws_d, const float* ws_l, int NP,
                              float c, hipStream_t stream);
// dK/dV stage in the two-group (ping-pong) form (attn_bwd_dkdv_pp_bf16.hip);
// same statistics layout and arguments as the dQ stage.
hipError_t launch_bwd_dkdv_pp_bf16(const BwdArgs& a, const float* ws_d, int NP, float c,
                                   hipStream_t stream);
hipError_t launch_fwd_bf16(int variant, const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);

}  // namespace attnio
