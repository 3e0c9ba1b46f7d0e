/*
 * attnio -- exact long-sequence self-attention forward for AMD Instinct MI355X
 * (gfx950), as a plain C ABI.
 *
 * The operation is exact attention, O = softmax(scale * Q K^T + mask) V, the
 * operator graph "Scores = Q x K^T; Mask; Softmax; Output = Scores x V" of
 * "From Attention Graph to FlashAttention - A Memory-Centric Compilation
 * Approach in AICF" (section 1), computed by the streamed schedule of its
 * section 3 (load a Q tile, stream K/V tiles, partial scores, online softmax
 * update, accumulate) so that no N x N intermediate ever reaches memory.  The
 * call plays the role of the special-kernel library entry flash_attention(Q, K,
 * V) of that page's section 4.  Tiling follows the I/O analysis of
 * tall-and-skinny products of "I/O Analysis is All You Need: An I/O Analysis
 * for Long-Sequence Attention" (abstract: I/O-optimal tiling and scheduling,
 * overlap of communication with computation, parallel softmax).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout      Q, K, V, O are contiguous row-major [B, H, N, d] tensors (d is
 *             innermost) in device memory, all of one element type.  O must not
 *             overlap Q, K or V.  Pointers must be 16-byte aligned.
 * d           64 or 128.
 * N           any N >= 1; B, H >= 1; B*H*N*d must be < 2^31.
 * scale       multiplies Q K^T; taken as given (not derived from d).
 * causal      nonzero: query i may attend to key j only if j <= i.
 * kv_len      NULL, or a DEVICE pointer to int32[B]: keys j >= kv_len[b] of
 *             batch b are masked (key padding).  Values are clamped to [0, N]
 *             on the device.  Every query row is still produced; a row with no
 *             visible key (kv_len[b] == 0) is written as zeros.
 * stream      a hipStream_t passed as an opaque pointer (NULL: default stream).
 *             The call only enqueues work: it never synchronises, allocates
 *             nothing and keeps no state between calls; device-side faults
 *             surface at the caller's next synchronisation.
 * Ownership   the caller owns every buffer.
 * Errors      0 on success, a negative ATTN_E* code otherwise.  Arguments are
 *             checked on the host before anything is enqueued; on an error
 *             nothing is enqueued and O is untouched.  attn_strerror() names
 *             each code.  Nothing prints unless ATTNIO_LOG=1 is set.
 */
#ifndef ATTNIO_H
#define ATTNIO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ATTN_OK = 0,
  ATTN_E_NULL = -1,      /* a required pointer is NULL */
  ATTN_E_HEAD_DIM = -2,  /* d is not 64 or 128 */
  ATTN_E_SHAPE = -3,     /* B, H or N < 1, or B*H*N*d >= 2^31 */
  ATTN_E_ALIGN = -4,     /* a tensor pointer is not 16-byte aligned */
  ATTN_E_LAUNCH = -5,    /* the kernel launch was rejected by the HIP runtime */
  ATTN_E_DEVICE = -6,    /* the current device is not a gfx950 GPU */
  ATTN_E_ALIAS = -7,     /* O overlaps Q, K or V */
  ATTN_E_ARG = -8,       /* another argument is out of range */
  ATTN_E_SCRATCH = -9    /* attn_bwd_noalloc: the shape needs more than its static scratch */
};

/* bf16 attention forward: Q, K, V, O hold bfloat16 values.  Products run on
 * bf16 matrix cores with fp32 accumulation; softmax statistics are fp32; the
 * probabilities are rounded to bf16 (round-to-nearest-even) before the P x V
 * product and the row sum is taken over those rounded values; O is rounded to
 * bf16 once, at the end. */
int attn_fwd(const void* Q, const void* K, const void* V, void* O,
             int B, int H, int N, int d, float scale, int causal,
             const int32_t* kv_len, void* stream);

/* fp32 attention forward: Q, K, V, O hold IEEE binary32 values, and every
 * step runs in fp32 with no narrower intermediate. */
int attn_fwd_f32(const void* Q, const void* K, const void* V, void* O,
                 int B, int H, int N, int d, float scale, int causal,
                 const int32_t* kv_len, void* stream);

/* Forward with the log-sum-exp side output ("IO-Aware Algorithms", How it
 * works: the backward pass recomputes the probabilities from Q, K, V and this
 * per-row statistic instead of storing them).  Same contract as attn_fwd /
 * attn_fwd_f32, plus:
 *   LSE   DEVICE float[B, H, N], written for every row: the natural log of
 *         sum_j exp(scale * q_i . k_j) over the visible keys j, or -inf for a
 *         row with no visible key.  It must not overlap Q, K, V or O.
 * Returns ATTN_E_NULL if LSE is NULL, ATTN_E_ALIAS if it overlaps. */
int attn_fwd_lse(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 int B, int H, int N, int d, float scale, int causal,
                 const int32_t* kv_len, void* stream);
int attn_fwd_f32_lse(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     int B, int H, int N, int d, float scale, int causal,
                     const int32_t* kv_len, void* stream);

/* bf16 attention backward ("IO-Aware Algorithms", How it works: the backward
 * pass recomputes the probabilities from Q, K, V and the forward's per-row
 * log-sum-exp instead of reading a stored N x N matrix).  Given the forward's
 * inputs Q, K, V, its output O and LSE (from attn_fwd_lse, same scale, causal
 * and kv_len), and the output gradient dO, it writes
 *   dV = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q,
 * with P_ij = exp(scale q_i.k_j - LSE_i) on visible pairs (0 elsewhere),
 * dS = P * (dO V^T - D) and D_i = dO_i . O_i.
 * Q, K, V, O, dO, dQ, dK, dV are bf16 [B, H, N, d] device tensors laid out as
 * for attn_fwd; LSE is a device float[B, H, N].  Keys past kv_len get zero dK
 * and dV.  workspace: a device buffer of attn_bwd_workspace_bytes(B, H, N)
 * bytes, 16-byte aligned, owned by the caller; its contents on entry do not
 * matter and on return are unspecified.  dQ, dK, dV and the workspace must not
 * overlap each other or any input.  Products run on bf16 matrix cores with
 * fp32 accumulation; P and dS are rounded to bf16 as operands; the gradients
 * are rounded to bf16 once.  Three kernels are enqueued on `stream`; nothing
 * is allocated and nothing synchronises.  Returns 0 or an ATTN_E* code
 * (checks as for attn_fwd, plus NULL and alias checks on every buffer). */
int attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* LSE, void* dQ, void* dK, void* dV, void* workspace,
             int B, int H, int N, int d, float scale, int causal,
             const int32_t* kv_len, void* stream);

/* Bytes of device workspace attn_bwd needs for B x H heads of N rows (host
 * only; 0 for non-positive sizes). */
size_t attn_bwd_workspace_bytes(int B, int H, int N);

/* Size of the static device scratch of attn_bwd_noalloc (32 MiB per GPU). */
#define ATTN_NOALLOC_SCRATCH_BYTES 33554432u

/* attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, kernels, results and errors as
 * attn_bwd, whose workspace is replaced by a static device array of
 * ATTN_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; the call itself allocates nothing (its first call on
 * a device looks up that device's copy of the array, once).  Shapes whose
 * attn_bwd_workspace_bytes(B, H, N) exceeds ATTN_NOALLOC_SCRATCH_BYTES return
 * ATTN_E_SCRATCH (B*H*ceil(N/64)*64 must be at most 4194304 rows).  Every call
 * on one GPU shares that GPU's array and nothing in it needs to start at zero;
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race on it, so such callers must order them. */
int attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* LSE, void* dQ, void* dK, void* dV,
                     int B, int H, int N, int d, float scale, int causal,
                     const int32_t* kv_len, void* stream);

/* fp8 attention forward (quantisation effects, as the Neural Circuit Diagrams
 * abstract lists them among what its performance model covers).  Q, K, V are
 * OCP E4M3 ("e4m3fn") bytes, contiguous [B, H, N, d], all finite; the real
 * inputs are x = fp8(x) * x_descale with one finite, positive fp32 descale per
 * tensor.  O is bf16 [B, H, N, d] (2 bytes per element; must not overlap the
 * inputs).  Q K^T and P V run on gfx950's fp8 matrix cores with fp32
 * accumulation; the probabilities are rounded to E4M3 for the P V product, in
 * (0, 2^8.75 = 430.5] relative to an exponent shift that trails the running
 * row maximum by at most 0.75 (base 2); the row sum is the sum of those same
 * rounded probabilities (formed on the matrix core), and O is rounded to bf16
 * once.  Returns ATTN_E_ARG if a descale is not finite and positive, or if
 * scale * q_descale * k_descale * log2(e) overflows fp32.  Other conventions
 * (d, N, scale, causal, kv_len, stream, errors) as for attn_fwd. */
int attn_fwd_fp8(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                 float scale, float q_descale, float k_descale, float v_descale, int causal,
                 const int32_t* kv_len, void* stream);

/* Operator-centric (unfused) bf16 forward, the baseline the fused kernel is
 * measured against ("From Attention Graph to FlashAttention - A Memory-Centric
 * Compilation Approach in AICF", section 2: one kernel per operator, each
 * result handed to the next operator through memory).  Same inputs, output and
 * conventions as attn_fwd; three kernels per group of heads: scores
 * S = scale Q K^T for all N x N pairs written in fp32, a row softmax that
 * applies the causal / padding mask and writes P in bf16 (normalised in fp32,
 * rounded once), and O = P V over all N keys.  The N x N intermediates live in
 * the caller's workspace: attn_fwd_unfused_workspace_bytes(N) bytes per head
 * (6 N^2), at least one head's worth, 256-byte aligned, not overlapping any
 * tensor; the call processes floor(workspace_bytes / that) heads at a time.
 * Returns ATTN_E_ARG if the workspace holds less than one head. */
int attn_fwd_unfused(const void* Q, const void* K, const void* V, void* O, void* workspace,
                     size_t workspace_bytes, int B, int H, int N, int d, float scale,
                     int causal, const int32_t* kv_len, void* stream);

/* Workspace bytes one head of attn_fwd_unfused needs (host only; 0 for N < 1). */
size_t attn_fwd_unfused_workspace_bytes(int N);

/* Streaming row operators ("From Attention Graph to FlashAttention - A
 * Memory-Centric Compilation Approach in AICF", closing outlook: streaming
 * softmax and streaming LayerNorm as further memory-centric operators).
 * X and Y are contiguous row-major bf16 [R, N] device matrices (16-byte
 * aligned); each row is reduced and mapped on its own, in fp32, and written
 * rounded to bf16 once.  A row that fits one workgroup's registers
 * (stream_rows_cached(N) == 1: N % 8 == 0 and N <= 65536) is read from HBM
 * once; longer rows are read twice.  Y may be X itself (in place); any other
 * overlap is ATTN_E_ALIAS.  R, N >= 1 and R * N < 2^40.  Enqueued on
 * `stream`; nothing allocated, nothing synchronised.
 *
 * stream_softmax:   Y[r, j] = exp(scale X[r, j]) / sum_k exp(scale X[r, k]);
 *                   -inf entries get 0 and a row of all -inf gives zeros.
 *                   scale must be finite and > 0 (else ATTN_E_ARG).
 * stream_layernorm: Y[r, j] = (X[r, j] - mean_r) / sqrt(var_r + eps) * gamma[j]
 *                   + beta[j], with the biased variance; gamma and beta are
 *                   bf16 [N] device vectors (16-byte aligned) or NULL (1 and
 *                   0).  eps must be finite and > 0 (else ATTN_E_ARG). */
int stream_softmax(const void* X, void* Y, int R, int N, float scale, void* stream);
int stream_layernorm(const void* X, const void* gamma, const void* beta, void* Y, int R, int N,
                     float eps, void* stream);

/* 1 if a row of N elements is held in registers (one HBM read), else 0. Host only. */
int stream_rows_cached(int N);

/* Human-readable name of a status code (static storage; never NULL). */
const char* attn_strerror(int code);

/* Library version, as major*10000 + minor*100 + patch. */
int attn_version(void);

/* Element types of the tiling and I/O-model queries. */
enum { ATTN_DTYPE_BF16 = 0, ATTN_DTYPE_F32 = 1, ATTN_DTYPE_FP8 = 2 };

/* One tiling of the bf16 streamed forward ("From Attention Graph to
 * FlashAttention - A Memory-Centric Compilation Approach in AICF", section 5:
 * tile size, reduction axis, residency and streaming order of the streaming
 * region).  A workgroup keeps BM = 32 * waves * qb query rows resident in
 * registers and streams K/V tiles of BN keys through LDS. */
typedef struct attn_tiling {
  int d;            /* head size */
  int BM;           /* query rows resident per workgroup */
  int BN;           /* keys per streamed K/V tile */
  int stages;       /* K/V tile pairs buffered in LDS */
  int waves;        /* wavefronts per workgroup */
  int lds_bytes;    /* LDS per workgroup */
  int wg_per_cu;    /* workgroups resident per CU */
  int qb;           /* 32-row query blocks per wave */
  int pingpong;     /* 1: two wave groups alternate the MFMA and softmax phases */
  int rowsum_mfma;  /* 1: row sums of P formed on the matrix core */
  int rowsum_in_stream; /* 1: those row-sum MFMAs issued in the P x V stream of the
                           MFMA phase; 0 (ping-pong only): by the softmax wave at
                           the start of its half step */
  int mfma16;       /* 1: every product on the 16x16x32 bf16 MFMA (d = 128 ping-pong,
                       32 queries per wave as two blocks of 16); 0: on 32x32x16 */
} attn_tiling;

/* Number of bf16 forward tilings compiled into the library, and the shape of
 * entry `index` (0 <= index < count).  Host only; attn_tiling_get returns 0,
 * ATTN_E_NULL or ATTN_E_ARG. */
int attn_tiling_count(void);
int attn_tiling_get(int index, attn_tiling* out);

/* attn_fwd with an explicit compiled tiling (an index of attn_tiling_get whose
 * d matches) instead of the one the I/O model picks; same contract and
 * results up to rounding order (bitwise equal where the tiling is the picked
 * one).  For measuring the tilings against each other.  ATTN_E_ARG if the
 * index is out of range or its head size differs from d. */
int attn_fwd_tiled(const void* Q, const void* K, const void* V, void* O,
                   int B, int H, int N, int d, float scale, int causal,
                   const int32_t* kv_len, int tiling_index, void* stream);

/* The I/O and issue model's view of one tiling: whether it fits a gfx950 CU
 * (160 KiB of LDS, 512 registers per SIMD lane shared by the SIMD's waves) and
 * what it costs per (query, key) pair at each level of the memory hierarchy
 * ("IO-Aware Algorithms", How it works: the tiled product's traffic
 * 2MNK -> 2MNK/S, and the roofline of each memory tier). */
typedef struct attn_tiling_eval {
  attn_tiling t;
  int compiled;                     /* attn_tiling_get index, or -1 if not built */
  int vgpr_estimate;                /* registers per lane the tiling needs (estimate) */
  int vgpr_budget;                  /* registers per lane its residency leaves */
  double mfma_cycles;               /* MFMA phase per wave per key tile (cycles) */
  double valu_cycles;               /* softmax phase per wave per key tile (cycles) */
  double issue_cycles_per_pair;     /* per CU, from the phase model */
  double lds_read_bytes_per_pair;   /* K/V operand reads from LDS */
  double l2_to_lds_bytes_per_pair;  /* K/V tile fetches into LDS: 4d / BM */
  double beyond_l2_bytes_per_pair;  /* K/V fetched past L2: 4d / (rows resident per XCD) */
  double cycles_per_pair;           /* predicted: the costliest of the four levels */
  int bound;                        /* which: 0 issue, 1 LDS, 2 L2->LDS, 3 beyond L2 */
} attn_tiling_eval;

/* Enumerate every tiling of the bf16 forward for head size d that fits a CU,
 * priced by the model and sorted best first (ties within 1% go to fewer bytes
 * beyond L2, then into LDS, then to wider key tiles); the forward runs the
 * first compiled one.  Writes up to max_out entries, returns how many tilings
 * fit (or a negative code: ATTN_E_HEAD_DIM, ATTN_E_ARG for dtype other than
 * bf16, ATTN_E_NULL).  causal does not change the per-pair prices.  Host only. */
int attn_tiling_enumerate(int d, int dtype, int causal, attn_tiling_eval* out, int max_out);

/* Tile configuration the path of element type `dtype` (ATTN_DTYPE_*) uses for
 * head size d (causal: 1 = causal mask): rows of the resident query tile (BM),
 * keys per streamed K/V tile (BN) and K/V LDS stages.  For bf16 it is the
 * compiled tiling the I/O model picks ("I/O Analysis is All You Need",
 * abstract: I/O-optimal tiling and scheduling); fp32 and fp8 have one tiling
 * each.  Host only.  Returns 0, ATTN_E_HEAD_DIM or ATTN_E_ARG (dtype).  Any
 * output pointer may be NULL. */
int attn_query_tiling(int d, int dtype, int causal, int* BM, int* BN, int* stages);

/* Analytic I/O bounds of one call of the path of element type `dtype`, host
 * only (kv_len_host: a HOST int32[B] or NULL), in bytes:
 *   t_min  the compulsory HBM traffic, Q, K, V read once and O written once
 *          (keys past kv_len never read), plus 4*B bytes of kv_len when
 *          kv_len_host is given: the
 *          Theta(N d) I/O of the fused form ("IO-Aware Algorithms", How it
 *          works), the bound measured traffic is compared with;
 *   t_lds  bytes streamed into LDS by the tiling attn_query_tiling reports
 *          (2MNK -> 2MNK/S with S = BM, same page);
 *   t_l2   predicted bytes fetched beyond L2 (as out[2] of attn_io_model).
 * Any output pointer may be NULL.  Returns 0 or a negative code. */
int attn_io_bound_bytes(int B, int H, int N, int d, int dtype, int causal,
                        const int32_t* kv_len_host, double* t_min, double* t_lds, double* t_l2);

/* I/O model of one call (host only; kv_len_host is a HOST int32[B] or NULL).
 * Fills, in bytes:
 *   out[0] t_min   compulsory HBM traffic: Q, K, V read once, O written once
 *                  (keys past kv_len are never read), plus 4*B bytes of
 *                  kv_len when kv_len_host is given;
 *   out[1] t_lds   bytes streamed into LDS by the chosen tiling (Q once per
 *                  query tile, K/V once per query tile for every key tile the
 *                  tile visits) -- the L2->LDS traffic of the tall-skinny
 *                  products, which shrinks as 1/BM;
 *   out[2] t_l2    predicted traffic beyond L2: the query tiles of one head
 *                  run on one XCD, as many at a time as fit its 32 CUs; each
 *                  such group reads the K/V rows it needs once, and a causal
 *                  group reuses up to one 4 MiB L2 of the keys the previous
 *                  group ended on (groups alternate the key direction).  An
 *                  idealised figure: it assumes a group walks its keys in step;
 *   out[3] flops   algorithmic FLOPs, 4*d per (query, visible key) pair;
 *   out[4] pairs   number of (query, visible key) pairs (one exp each).
 * Returns 0, or a negative code for invalid shapes. */
int attn_io_model(int B, int H, int N, int d, int elem_bytes, int causal,
                  const int32_t* kv_len_host, double out[5]);

#ifdef __cplusplus
}
#endif

#endif /* ATTNIO_H */
