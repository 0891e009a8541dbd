/*
 * w8mp.h -- C ABI of the MI355X (gfx950) quantized-linear library libw8mp.so.
 *
 * Two weight-8-bit / activation-8-bit linear layers, Y = X W^T:
 *
 *  1. LLM.int8 mixed-precision decomposition ("Image21-INT8" model card,
 *     section "Quantization": bitsandbytes LLM.int8 with outlier threshold
 *     6.0, outliers handled in floating point, no calibration). Every input
 *     column that holds some |x| > threshold is taken out to a 16-bit floating
 *     side path; each token row of the rest gets a symmetric absmax int8 code;
 *     the int8 x int8 contraction against rowwise int8 weights accumulates in
 *     int32 and is dequantised by sx[m] * sw[n] / 127^2 (the vector-wise
 *     scheme of LLM.int8(), Dettmers et al. 2022).
 *
 *  2. FP8-E4M3 W8A8 ("Qwen-Image-2.1 Text Encoder: FP8" card, section
 *     "Format": E4M3 weights with one scale per output channel, activations
 *     quantised per token at run time; "Darkstar-Qwen-Image-2.1-Base-ModelOpt-
 *     FP8" card, section "Precision map": static per-tensor input scale).
 *
 *  3. FP8-E4M3 weight-only (W8A16): the same E4M3 weights, widened to bf16
 *     inside the GEMM, with bf16 activations (the same card's weight-only
 *     loader).
 *
 *  4. W4A8: int4 weights with one scale per group of 128 input values and
 *     int8 per-token activations ("Qwen-Image-fni8" card, section "Format").
 *
 * and a block driver that chains one DiT block's int8 linears with the fp16
 * exclusion policy for massive-activation writers.
 *
 * Conventions for every entry point
 *  - Layouts are row-major and dense: X [M,K], W and Wq [N,K] (the [out,in]
 *    order of a linear layer), Y [M,N]. Base pointers must be 16-byte aligned.
 *  - Every array argument is DEVICE memory owned by the caller. The library
 *    keeps no pointer after a call returns and allocates no device memory.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream of
 *    the current device) and is asynchronous: the call returns before the GPU
 *    has finished. Nothing in a call synchronises the host.
 *  - Arguments are validated on the host before any HIP call; a rejected call
 *    touches no memory and enqueues nothing. The status says why, and
 *    w8_last_error() gives a readable detail (thread-local).
 *  - Input values are not inspected: finite inputs are a precondition.
 *  - Results are deterministic: the same inputs give the same bits.
 *
 * Workspaces (every entry point that takes one)
 *  - A workspace is caller-owned device memory, 256-byte aligned, at least as
 *    large as the entry point's size query, which depends on (M, N, K) only.
 *    It must be zero-filled before its first use (e.g. hipMemsetAsync).
 *  - Every workspace starts with the same fixed region: split-K arrival
 *    counters, left zero by every call, and the outlier-column flag words of
 *    the int8 linears, which each call marks with a stamp of its own (a
 *    per-process call counter, never 0) and never clears. One workspace may
 *    therefore serve calls of any shapes and entry points one after another,
 *    without clearing, if it is as large as each call's size query.
 *  - After a call that returns an error before launching anything (a
 *    validation status), the workspace is untouched. After W8_ERR_HIP (a
 *    launch that failed), the workspace still serves later calls: a kernel
 *    that never ran touched no counter, and flags left by the failed call
 *    carry its stamp, which no later call uses (until 2^32 - 1 further int8
 *    calls). A kernel fault leaves the device unusable anyway.
 *  - Sizes are planned for a 256-CU device (MI355X). On a device whose GEMM
 *    plan needs more split-K partials than the workspace holds, the call runs
 *    the same tiles without K-slicing (same results).
 *  - Calls that may overlap (different streams) need distinct workspaces.
 */
#ifndef W8MP_H
#define W8MP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W8_OK = 0,
  W8_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad alignment, bad threshold */
  W8_ERR_UNSUPPORTED = 2,      /* valid request this library does not implement      */
  W8_ERR_WORKSPACE = 3,        /* workspace missing or smaller than the size query   */
  W8_ERR_HIP = 4               /* a HIP launch failed (see w8_last_error)            */
} w8_status;

typedef enum { W8_DT_F16 = 0, W8_DT_BF16 = 1, W8_DT_F32 = 2 } w8_dtype;

typedef enum { W8_Q_INT8 = 0, W8_Q_FP8_E4M3 = 1, W8_Q_INT4_G128 = 2 } w8_qformat;

/* Largest K the int8 contraction accepts: K * 127^2 < 2^31, so the int32
 * accumulator cannot overflow. */
#define W8_INT8_MAX_K 133144

/*
 * quantize_weight_rowwise -- one-off weight quantisation, per output row.
 *
 * The model cards store the quantized weights once and never re-quantise
 * them at load ("Image21-INT8", "Installation and loading"); this call makes
 * that stored form.
 *
 *   W    [N,K] f16 or bf16 (w_dt), device.
 *   fmt  W8_Q_INT8:     sw[n] = max_k |W[n,k]| (fp32),
 *                       Wq[n,k] = clamp(rne(fl32(W[n,k] * fl32(127/sw[n]))), +-127)
 *                       as int8; rows with sw = 0 are all zero.
 *        W8_Q_FP8_E4M3: sw[n] = bf16(fl32(max_k |W[n,k]| / 448)) held in fp32
 *                       (the FP8 card stores one bf16 scale per output channel),
 *                       Wq[n,k] = E4M3FN(fl32(W[n,k] / sw[n])), round to nearest
 *                       even, saturating at +-448, sign of zero kept; rows with
 *                       sw = 0 are all zero.
 *        W8_Q_INT4_G128: int4 codes with one fp32 scale per group of 128 values
 *                       of a row (the per-group int4 weights of the
 *                       "Qwen-Image-fni8" card, section "Format"): for group g
 *                       of row n, sw[g*N + n] = max |W| over the group,
 *                       q = clamp(rne(fl32(W * fl32(7/sw))), +-7), 0 when sw = 0.
 *                       Wq holds the codes packed two per byte, [N, K/2] uint8:
 *                       byte b (0..3) of the 32-bit little-endian word c of a
 *                       row holds k = 8c+b in its low nibble and k = 8c+b+4 in
 *                       its high nibble (4-bit two's complement). Needs
 *                       K % 128 == 0.
 *   Wq   [N,K] int8 / uint8 E4M3 codes, or [N,K/2] packed int4 (output, device).
 *   sw   [N] fp32, or [K/128, N] fp32 for int4 groups (output, device).
 * Requires N >= 1, 16 <= K, K % 16 == 0.
 */
w8_status quantize_weight_rowwise(const void* W, int w_dt, int64_t N, int64_t K, int fmt,
                                  void* Wq, float* sw, void* stream);

/*
 * int8_mixed_linear -- Y = X W^T with the LLM.int8 decomposition.
 *
 *   X          [M,K] f16 or bf16 (x_dt), device.
 *   Wq, sw     the W8_Q_INT8 output of quantize_weight_rowwise ([N,K], [N]).
 *   threshold  outlier threshold t (the model card uses 6.0). A column k is an
 *              outlier column when |X[m,k]| > t for some row m of THIS call.
 *              +inf gives plain vector-wise int8; t < 0 or NaN is rejected.
 *   Y          [M,N] f16 or f32 (y_dt), device, written in full.
 *   workspace  device memory of at least int8_mixed_linear_workspace_size()
 *              bytes (see "Workspaces" above). It holds the codes [M,K], the
 *              scales, the outlier list and the 16-bit outlier operands of up
 *              to 256 outlier columns; a call with more outlier columns reads
 *              them from X and Wq in the GEMM instead (same results, slower).
 *              Do not write to it between calls.
 *
 * What is computed (O = outlier columns, ascending):
 *   sx[m]   = max_{k not in O} |X[m,k]|                     (fp32, exact)
 *   q[m,k]  = 0 for k in O, else clamp(rne(fl32(X * fl32(127/sx[m]))), +-127)
 *   acc     = q Wq^T in int32 (exact)
 *   Y[m,n]  = (sw[n]/127) * ((sx[m]/127) * acc[m,n] + sum_{k in O} X[m,k] Wq[n,k])
 * where the outlier sum runs on 16-bit MFMA in X's own type with fp32
 * accumulation (Wq's integers are exact in both 16-bit types) and the
 * epilogue is fp32, rounded to nearest even into Y.
 * Requires M, N >= 1, 16 <= K <= W8_INT8_MAX_K, K % 16 == 0.
 */
size_t int8_mixed_linear_workspace_size(int64_t M, int64_t N, int64_t K);
w8_status int8_mixed_linear(const void* X, int x_dt, int64_t M, int64_t K,
                            const int8_t* Wq, const float* sw, int64_t N, float threshold,
                            void* Y, int y_dt, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * int8_mixed_linear_noalloc -- int8_mixed_linear without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Arguments,
 * results and errors are those of int8_mixed_linear.
 *
 * The workspace is a static 96 MiB region of the library's own device memory:
 * each device the library runs on holds one copy from the load of the
 * library's code until the process ends. The call allocates nothing (no
 * hipMalloc, no allocating library routine); its first call on a device looks
 * up that device's copy (hipGetSymbolAddress). A shape whose codes, scales and
 * outlier operands do not fit (the int8 workspace without split-K partials;
 * e.g. M x K above about 90 million) is rejected with W8_ERR_UNSUPPORTED
 * before anything runs; split-K partials are used when they fit too, else
 * the same tiles run without K-slicing (same results). Every call on a device
 * shares that device's region, and it keeps the last call's contents: calls
 * that may overlap on one device (different streams, threads) race and give
 * undefined results; serialise them.
 */
w8_status int8_mixed_linear_noalloc(const void* X, int x_dt, int64_t M, int64_t K,
                                    const int8_t* Wq, const float* sw, int64_t N, float threshold,
                                    void* Y, int y_dt, void* stream);

/*
 * The op that produces X, for int8_mixed_linear_fused. X is made from H in the
 * quantisation pass itself and never stored; it is the 16-bit value (H's type)
 * that a separate producer op would store:
 *   W8_PRODUCER_RMSNORM: RMSNorm (Zhang and Sennrich, 2019) with the
 *     x(1+scale)+shift modulation of adaptive layer norm (Peebles and Xie,
 *     2023), a fixed sequence of fp32 operations, each rounded to nearest
 *     even and none fused, then rounded to nearest even in H's type. Per row:
 *       ss   = sum_k H[m,k]^2 in fp64 (each square is exact);
 *       rstd = fl32(1 / fl32(sqrt(fl32(fl32(ss/K) + eps))));
 *       x    = fl32(fl32(H*rstd) * fl32(gamma[k] * fl32(1 + scale[k]))) + shift[k].
 *     gamma (NULL: 1), scale (NULL: 0) and shift (NULL: no addition) are fp32
 *     [K] device vectors, 16-byte aligned.
 *     The kernel adds the float64 squares in its own order, which can differ
 *     from the exactly rounded sum in the last bit of ss; rstd then differs
 *     from the exact reading only when fl32(ss / K) sits at a rounding
 *     boundary (both values are correct readings of the definition).
 *   W8_PRODUCER_GELU_TANH: GELU, tanh form (Hendrycks and Gimpel, 2016):
 *     X = 0.5 H (1 + tanh(sqrt(2/pi)(H + 0.044715 H^3))) correctly rounded
 *     (to nearest, ties to even) in H's type. X is a function of the 16-bit
 *     pattern of H alone; the library reads it from a table of all 65536
 *     results per format, made when the library is built.
 */
typedef enum { W8_PRODUCER_NONE = 0, W8_PRODUCER_RMSNORM = 1, W8_PRODUCER_GELU_TANH = 2 } w8_producer_kind;
typedef struct w8_producer {
  int kind;              /* w8_producer_kind */
  const float* gamma;    /* RMSNorm gain [K], device, or NULL */
  const float* scale;    /* modulation scale [K], device, or NULL */
  const float* shift;    /* modulation shift [K], device, or NULL */
  float eps;             /* RMSNorm epsilon: finite, >= 0 */
} w8_producer;

/*
 * int8_mixed_linear_fused -- Y = producer(H) W^T + bias, with the LLM.int8
 * decomposition of int8_mixed_linear applied to X = producer(H).
 *
 *   H          [M,K] f16 or bf16 (h_dt), device: the producer's input. X has
 *              H's type.
 *   producer   NULL or kind W8_PRODUCER_NONE: X = H (this call is then
 *              int8_mixed_linear plus the bias). A producer needs
 *              K <= 16384 (else W8_ERR_UNSUPPORTED).
 *   bias       NULL or fp32 [N], device: added to the fp32 epilogue result
 *              before the rounding into Y.
 * All other arguments, the workspace (int8_mixed_linear_workspace_size) and
 * the result are as for int8_mixed_linear.
 */
w8_status int8_mixed_linear_fused(const void* H, int h_dt, int64_t M, int64_t K,
                                  const w8_producer* producer, const int8_t* Wq, const float* sw,
                                  const float* bias, int64_t N, float threshold, void* Y, int y_dt,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8_w8a8_linear -- Y = X W^T with E4M3 weights and activations.
 *
 *   X          [M,K] f16 or bf16, device.
 *   Wq8, sw    the W8_Q_FP8_E4M3 output of quantize_weight_rowwise. A
 *              per-tensor weight scale is passed as a constant vector.
 *   act_scale  NULL: dynamic per-token scale sx[m] = fl32(max_k |X[m,k]| / 448).
 *              Otherwise a DEVICE pointer to one fp32 static per-tensor input
 *              scale (must be finite and >= 0; 0 gives zero codes).
 *   Y          [M,N] bf16, f16 or f32, device.
 *   workspace  device memory of at least fp8_w8a8_linear_workspace_size()
 *              bytes (see "Workspaces" above).
 * Codes: xq[m,k] = E4M3FN(fl32(X[m,k] / sx[m])) (saturating), all zero when
 * sx[m] = 0. Y[m,n] = sx[m] * sw[n] * sum_k xq*wq, fp32 accumulation on FP8
 * MFMA, rounded to nearest even into Y. Results are bitwise reproducible for
 * a given device: split-K partial sums are added in a fixed order.
 * Requires M, N >= 1, 16 <= K <= 65536, K % 16 == 0.
 */
size_t fp8_w8a8_linear_workspace_size(int64_t M, int64_t N, int64_t K);
w8_status fp8_w8a8_linear(const void* X, int x_dt, int64_t M, int64_t K,
                          const uint8_t* Wq8, const float* sw, int64_t N,
                          const float* act_scale, void* Y, int y_dt,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8_w8a16_linear -- Y = X W_deq^T with E4M3 weights and bf16 activations
 * (weight-only FP8).
 *
 * The weight-only loader of the FP8 text-encoder card ("Qwen-Image-2.1 Text
 * Encoder: FP8", section "Format"; measured as "weight-only" in section "How
 * it was tested") turns each weight into bf16 as its FP8 value times the bf16
 * scale of its output channel, and computes in bf16:
 *   W_deq[n,k] = rne_bf16(e4m3(Wq8[n,k]) * sw[n])   (the product is exact)
 *   Y[m,n]     = sum_k X[m,k] * W_deq[n,k], fp32 accumulation on bf16 MFMA,
 *                rounded to nearest even into Y.
 * The weights stay E4M3 in memory: they are widened to bf16 on the way from
 * LDS to the matrix cores, never written out.
 *
 *   X          [M,K] bf16, device (other types: W8_ERR_UNSUPPORTED).
 *   Wq8, sw    the W8_Q_FP8_E4M3 output of quantize_weight_rowwise (sw holds
 *              bf16 values); codes 0x7F / 0xFF (NaN) are outside the contract.
 *   Y          [M,N] bf16, f16 or f32, device.
 *   workspace  device memory of at least fp8_w8a16_linear_workspace_size()
 *              bytes (see "Workspaces" above).
 * Results are bitwise reproducible for a given device (split-K partial sums
 * are added in a fixed order).
 * Requires M, N >= 1, 64 <= K <= 65536, K % 64 == 0 (else W8_ERR_UNSUPPORTED).
 */
size_t fp8_w8a16_linear_workspace_size(int64_t M, int64_t N, int64_t K);
w8_status fp8_w8a16_linear(const void* X, int x_dt, int64_t M, int64_t K,
                           const uint8_t* Wq8, const float* sw, int64_t N,
                           void* Y, int y_dt, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * w4a8_linear -- Y = X W^T with int4 per-group weights and int8 per-token
 * activations ("Qwen-Image-fni8" card, section "Format"), on int8 MFMA.
 *
 *   X          [M,K] f16 or bf16, device.
 *   Wq4, sw4   the W8_Q_INT4_G128 output of quantize_weight_rowwise.
 *   Y          [M,N] bf16, f16 or f32, device.
 *   workspace  at least w4a8_linear_workspace_size() bytes (see
 *              "Workspaces" above).
 * Activations are coded per token like int8_mixed_linear with no outlier
 * columns: sx[m] = max_k |X[m,k]|, q = rne(fl32(X * fl32(127/sx))). Each
 * group's int8 x int4 products are summed exactly (int32), the group sum
 * scaled by sw4[g*N + n] / 7 and the total by sx[m] / 127 (fp32), rounded to
 * nearest even into Y. Results are bitwise reproducible for a given device.
 * Requires M, N >= 1, K % 128 == 0, K <= 65536, M*K and N*K/2 below 2^32.
 */
size_t w4a8_linear_workspace_size(int64_t M, int64_t N, int64_t K);
w8_status w4a8_linear(const void* X, int x_dt, int64_t M, int64_t K,
                      const uint8_t* Wq4, const float* sw4, int64_t N,
                      void* Y, int y_dt, void* workspace, size_t workspace_bytes, void* stream);

/*
 * w8_dit_block_forward -- one DiT block's quantized linears, chained on
 * `stream` (a driver over the calls above; fp16 activations throughout):
 *
 *   qkv = LLM.int8 linear of RMSNorm1(X), + b_qkv          [M, 3D]
 *   a   = qkv[:, 2D:3D]                                     attention stub
 *   o   = LLM.int8 linear of a, + b_o                       [M, D]
 *   h   = X + o
 *   u   = LLM.int8 linear of RMSNorm2(h), + b_up            [M, F]
 *   d   = LLM.int8 linear of GELU(u), + b_down              [M, D]
 *   Y   = h + d
 *
 * The "Image21-INT8" card ("Quantization") quantizes the block's linears with
 * LLM.int8; the "Image21-Turbo-OrbitQuant-W4A4" card ("What 4-bit breaks here
 * and what stays in fp16") keeps the MLP output projections that write the
 * near-9000 text-token values in fp16. That is the exclusion policy here:
 * with w_down16 set, d = GELU(u) w_down16^T + b_down is computed in fp16 (fp32
 * sums) from unquantized weights. Attention is outside the quantized path;
 * the stub passes each token's value vector through (as if each token
 * attended only to itself). Every linear's output and each residual sum is
 * rounded once to fp16 (round to nearest even).
 *
 * Weights are the W8_Q_INT8 output of quantize_weight_rowwise; biases are
 * fp32 [N] or NULL; norm1 / norm2 are RMSNorm producers (kind
 * W8_PRODUCER_RMSNORM, or W8_PRODUCER_NONE to skip the norm). Requires
 * M >= 1, D and F multiples of 64 in [64, 16384], 16-byte aligned X, Y,
 * w_down16 and b_down. The workspace (w8_dit_block_workspace_size bytes, see
 * "Workspaces" above) holds one int8 workspace that the four linears share in
 * turn, then the intermediates.
 */
typedef struct w8_dit_block {
  int64_t D;                   /* model width: X, Y [M, D] fp16 */
  int64_t F;                   /* MLP hidden size */
  float threshold;             /* LLM.int8 outlier threshold (6.0 on the card) */
  const int8_t* w_qkv;   const float* s_qkv;  const float* b_qkv;    /* [3D, D], [3D], [3D] */
  const int8_t* w_o;     const float* s_o;    const float* b_o;      /* [D, D], [D], [D] */
  const int8_t* w_up;    const float* s_up;   const float* b_up;     /* [F, D], [F], [F] */
  const int8_t* w_down;  const float* s_down; const float* b_down;   /* [D, F], [D], [D] */
  const uint16_t* w_down16;    /* [D, F] fp16: the excluded writer, or NULL */
  w8_producer norm1, norm2;
} w8_dit_block;

size_t w8_dit_block_workspace_size(int64_t M, int64_t D, int64_t F);
w8_status w8_dit_block_forward(const w8_dit_block* blk, const void* X, int64_t M, void* Y,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Readable name of a status; never NULL. */
const char* w8_status_string(int status);
/* Detail of the last failed call on this host thread ("" if none). */
const char* w8_last_error(void);

/* ------------------------------------------------------------------------
 * Parity exports: the same kernels as above, with their intermediate results
 * written to caller buffers. Used by the test suite.
 * ------------------------------------------------------------------------ */

/* The activation half of int8_mixed_linear_fused (X from H by `producer`, NULL
 * for none; outlier detection, row scales, int8 codes, outlier fix-up).
 * Outputs (device): q [M,K] int8, sx [M] fp32, outlier_idx [K] int32 (first
 * *n_outliers entries valid, ascending), n_outliers [1] int32. Workspace:
 * w8dbg_int8_quantize_activations_workspace_size(M, K) bytes (the common
 * front, then the RMSNorm rstd [M] fp32). */
size_t w8dbg_int8_quantize_activations_workspace_size(int64_t M, int64_t K);
w8_status w8dbg_int8_quantize_activations(const void* X, int x_dt, int64_t M, int64_t K,
                                          const w8_producer* producer, float threshold,
                                          int8_t* q, float* sx, int32_t* outlier_idx,
                                          int32_t* n_outliers, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* X = producer(H) written out [M,K] in H's 16-bit type (the values the fused
 * quantisation pass makes in registers). */
w8_status w8dbg_produce(const void* H, int h_dt, int64_t M, int64_t K, const w8_producer* producer,
                        void* X, void* stream);

/* The int8 MFMA contraction alone: acc [M,N] int32 = q [M,K] . Wq [N,K]^T.
 * tail = 0: the grid int8_mixed_linear would use (split ignored). Otherwise
 * the leftover 256x256 tiles of the last, partial wave of the device (every
 * tile when there are fewer tiles than compute units) run as `split` K-slices
 * of whole tiles (tail = 1; split = 1 runs every tile whole) or of 128x128
 * quarters (tail = 2); tail 1 with split > 1 and tail 2 need K % 64 == 0 and
 * split <= K / 64 (else W8_ERR_UNSUPPORTED). tail = 3 (split must be 1,
 * K % 64 == 0): stream-K, the tiles of the last full wave and the leftover
 * ones (every tile when there are fewer than two waves) shared evenly by one
 * block per compute unit, K step by K step. Workspace:
 * w8dbg_int8_gemm_i32_workspace_size(M, N, K, tail, split) bytes on the
 * current device (may be 0, then workspace may be NULL), zero-filled before
 * first use (left zero by every call). */
size_t w8dbg_int8_gemm_i32_workspace_size(int64_t M, int64_t N, int64_t K, int tail, int split);
w8_status w8dbg_int8_gemm_i32(const int8_t* q, const int8_t* Wq, int64_t M, int64_t N, int64_t K,
                              int tail, int split, int32_t* acc, void* workspace, size_t workspace_bytes,
                              void* stream);

/* The activation half of fp8_w8a8_linear: xq [M,K] E4M3 codes, sx [M] fp32. */
w8_status w8dbg_fp8_quantize_activations(const void* X, int x_dt, int64_t M, int64_t K,
                                         const float* act_scale, uint8_t* xq, float* sx,
                                         void* stream);

/* The GEMM half of fp8_w8a8_linear on given codes and scales: Y [M,N] =
 * sx[m] * sw[n] * sum_k xq[m,k] * Wq8[n,k] (E4M3 codes, fp32 accumulation).
 * split = 0: the output tiling and K-slicing fp8_w8a8_linear would choose
 * (tile ignored). split >= 1: output tiles of tile x tile (128 or 256; 0 means
 * 256) on 64-byte K steps, or, with tile 129 / 192, 128 x 128 / 128 x 192
 * tiles on 128-byte K steps, each with its K range cut into `split` slices;
 * needs K % 64 == 0 and split <= K / 64 (tiles 129 and 192: K % 128 == 0 and
 * split <= K / 128) else W8_ERR_UNSUPPORTED, unless split is 1 (tiles 128
 * and 256). Workspace:
 * w8dbg_fp8_gemm_workspace_size(M, N, K, split, tile) bytes (0 means none,
 * then workspace may be NULL), zero-filled before first use (left zero). */
size_t w8dbg_fp8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int split, int tile);
w8_status w8dbg_fp8_gemm(const uint8_t* xq, const float* sx, const uint8_t* Wq8, const float* sw,
                         int64_t M, int64_t N, int64_t K, int split, int tile, void* Y, int y_dt,
                         void* workspace, size_t workspace_bytes, void* stream);

/* fp8_w8a16_linear with a given output tiling: split = 0 is the linear's own
 * choice (tile ignored); split >= 1 uses tile x tile output blocks (128 or
 * 256; 0 means 256) with each K range cut into `split` slices, split <= K / 64
 * (else W8_ERR_UNSUPPORTED). Same requirements as fp8_w8a16_linear otherwise;
 * workspace: w8dbg_fp8_w8a16_linear_workspace_size(M, N, K, split, tile) bytes
 * (at least 256), zero-filled before first use (left zero). */
/* w4a8_linear with its K range cut into `split` slices of whole groups
 * (split = 0: the linear's own choice; 1 <= split <= K / 128, else
 * W8_ERR_UNSUPPORTED). Workspace: w8dbg_w4a8_linear_workspace_size(M, N, K,
 * split) bytes, zero-filled before first use (left zero). */
/* The plain 16-bit linear of the block driver's exclusion policy:
 * Y [M,N] = X [M,K] . W [N,K]^T, X and W both f16 or both bf16 (x_dt), fp32
 * accumulation on 16-bit MFMA, rounded into Y (bf16/f16/f32). K % 64 == 0,
 * K <= 65536. split = 0: the driver's own tiling (tile ignored); else
 * 1 <= split <= K / 64 and tile = 256: 256x256 blocks, the tiles of the
 * device's full waves whole and the leftover tiles of the last partial wave
 * (every tile when there are fewer tiles than compute units) in `split`
 * K-slices; tile = 128: 128x128 blocks, every one in `split` K-slices (other
 * tiles: W8_ERR_INVALID_ARGUMENT). Workspace:
 * w8dbg_linear16_workspace_size(M, N, K, split, tile) bytes (at least 256) on
 * the current device, zero-filled before first use (left zero). */
size_t w8dbg_linear16_workspace_size(int64_t M, int64_t N, int64_t K, int split, int tile);
w8_status w8dbg_linear16(const void* X, int x_dt, int64_t M, int64_t K, const void* W, int64_t N, int split, int tile,
                         void* Y, int y_dt, void* workspace, size_t workspace_bytes, void* stream);

size_t w8dbg_w4a8_linear_workspace_size(int64_t M, int64_t N, int64_t K, int split);
w8_status w8dbg_w4a8_linear(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq4,
                            const float* sw4, int64_t N, int split, void* Y, int y_dt,
                            void* workspace, size_t workspace_bytes, void* stream);

size_t w8dbg_fp8_w8a16_linear_workspace_size(int64_t M, int64_t N, int64_t K, int split, int tile);
w8_status w8dbg_fp8_w8a16_linear(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq8,
                                 const float* sw, int64_t N, int split, int tile, void* Y, int y_dt,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* int8_mixed_linear that also records a per-block timeline of its GEMM
 * launch: block b writes stamps[8b .. 8b+7] (device memory, int64): [0] its
 * start, [1] the start of its K loop, [2] the end of the K loop, [3] its end,
 * in ticks of the GPU's constant 100 MHz clock (wall_clock64); [4] and [5] the
 * shader-clock counter (clock64) at [1] and [2]. Blocks of the 128x128 tail
 * write [0] and [3] only, a split-K slice that leaves the epilogue to another
 * slice writes no [3]; words a block does not write keep their contents.
 * A stream-K block with several tile pieces keeps [1], [2], [4], [5] of the
 * last piece that wrote them and [3] of the last piece that ran an epilogue.
 * grid (host, 4 ints) receives the launch's block count, the number of blocks
 * that own whole 256x256 tiles (the first ones), 1 if K % 64 == 0 (the
 * kernel that records the timeline) else 0, and what the other blocks are:
 * 0 K-slices of whole tiles, 1 128x128 quarters, 2 stream-K blocks. With
 * stamps NULL only grid is filled and nothing runs. stamps_len < 8 * blocks
 * is an invalid argument. */
w8_status w8dbg_int8_gemm_timeline(const void* X, int x_dt, int64_t M, int64_t K, const int8_t* Wq,
                                   const float* sw, int64_t N, float threshold, void* Y, int y_dt,
                                   void* workspace, size_t workspace_bytes, long long* stamps,
                                   size_t stamps_len, int* grid, void* stream);

/* int8_mixed_linear_fused that also records the caller's HIP events
 * events[0..3] (hipEvent_t, created by the caller; NULL entries are skipped)
 * on `stream`: before the row pass, after it, after the outlier fix-up and
 * after the GEMM. Same arguments, workspace and results otherwise. */
w8_status w8dbg_int8_mixed_linear_events(const void* H, int h_dt, int64_t M, int64_t K, const w8_producer* producer,
                                         const int8_t* Wq, const float* sw, const float* bias, int64_t N,
                                         float threshold, void* Y, int y_dt, void* workspace, size_t workspace_bytes,
                                         void* const* events, void* stream);

/* int8_mixed_linear_fused with the GEMM grid planned for `cus` compute units
 * instead of the device's own (the parity tests' way to run other devices'
 * grids): whole 256x256 tiles in rounds of `cus`, the leftover tiles of a
 * partial round whole, as K-slices or as 128x128 quarters, as that plan
 * chooses. Every output element is the same sequence of operations whichever
 * block computes it, so results equal int8_mixed_linear_fused's bit for bit.
 * Workspace: at least w8dbg_int8_mixed_linear_plan_workspace_size(M, N, K,
 * cus) bytes (0 for an invalid shape or cus), zero-filled before its first
 * use, as for int8_mixed_linear. cus must be in [1, 4096]. */
size_t w8dbg_int8_mixed_linear_plan_workspace_size(int64_t M, int64_t N, int64_t K, int cus);
w8_status w8dbg_int8_mixed_linear_plan(const void* H, int h_dt, int64_t M, int64_t K, const w8_producer* producer,
                                       const int8_t* Wq, const float* sw, const float* bias, int64_t N,
                                       float threshold, void* Y, int y_dt, void* workspace, size_t workspace_bytes,
                                       int cus, void* stream);

/* fp8_w8a8_linear recording events[0..3]: before the activation pass, after
 * it (events 1 and 2), after the GEMM. */
w8_status w8dbg_fp8_w8a8_linear_events(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq8,
                                       const float* sw, int64_t N, const float* act_scale, void* Y, int y_dt,
                                       void* workspace, size_t workspace_bytes, void* const* events, void* stream);

/* Byte offsets in an int8_mixed_linear workspace of shape (M, N, K):
 * offsets[0..10] = split-K counters, flag words (uint32 [K]), nO (int32), the
 * outlier list O (int32 [K]), codes q (int8 [M,K]), sx (fp32 [M]), rstd
 * (fp32 [M]), XO (16-bit [M, P]), WO (16-bit [N, P]), split-K partials, and
 * the outlier columns XO/WO hold (P = nO padded to 32 when it fits). */
w8_status w8dbg_int8_workspace_layout(int64_t M, int64_t N, int64_t K, size_t* offsets);

/* Byte offsets in a w8_dit_block workspace of the block's intermediates after
 * w8_dit_block_forward: offsets[0..6] = qkv, a, o, h, u (fp16), g = GELU(u)
 * (fp16, written only with the 16-bit down-projection), d (fp16; fp32 with
 * the 16-bit down-projection). */
w8_status w8dbg_dit_block_layout(int64_t M, int64_t D, int64_t F, size_t* offsets);

/* Measured MFMA peak (measurement export): `blocks` blocks of 4 waves each
 * issue `iters` rounds of 4 independent back-to-back MFMAs on register
 * operands -- kind 0: v_mfma_i32_32x32x32_i8, 1: v_mfma_scale_f32_32x32x64_f8f6f4
 * (E4M3), 2: v_mfma_f32_32x32x16_bf16; 3 and 4: kinds 0 and 1 with operands
 * that change every round (random bits, as a GEMM's; the matrix cores then
 * draw more power and the chip holds a lower clock) -- and store a checksum
 * per thread in out[blocks * 256] (device). *ops (host) receives the
 * operations launched (2 M N K per instruction); the caller times the
 * launch. */
w8_status w8dbg_mfma_peak(int kind, int blocks, int iters, unsigned* out, double* ops, void* stream);

/* The GEMMs' operand load path measured alone: `blocks` blocks (one per
 * compute unit at a time) each stream 256 rows of a panel (row pitch K bytes,
 * block b reading panel b % panels of buf, which holds at least
 * panels * 256 * K bytes) into LDS with buffer loads, one K step of `seg` (64
 * or 128) bytes of all 256 rows per iteration, `iters` iterations, walking the
 * panel's K steps round robin. *bytes receives the bytes moved; out[blocks]
 * receives a checksum. Invalid sizes (seg not 64/128, K not a multiple of
 * seg, 256 K >= 2^31, buf too small) are W8_ERR_INVALID_ARGUMENT. */
w8_status w8dbg_lds_stream(const void* buf, size_t buf_bytes, int K, int seg, int blocks, int panels, int iters,
                           unsigned* out, double* bytes, void* stream);

/* Checks the packed float32 -> fp16 conversion of the library's epilogues
 * (v_cvt_pk_f16_f32, two values per instruction) against the scalar one
 * (v_cvt_f16_f32, round to nearest even) on every float32 bit pattern x,
 * paired with x ^ 0x5A5A5A5A. out (device, 3 words, out[0..1] zero and out[2]
 * 0xFFFFFFFF on entry) receives the number of mismatching pairs of non-NaN
 * inputs, the number of pairs with a NaN input whose results differ, and the
 * smallest x of a non-NaN mismatch. Asynchronous on `stream`. */
w8_status w8dbg_cvt_f16_pair_check(unsigned* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W8MP_H */
