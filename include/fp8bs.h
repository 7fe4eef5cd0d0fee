/*
 * fp8bs.h -- C ABI of libfp8bs: FP8 (E4M3) block-scaled quantizers and GEMMs
 * for the main linear layers of a decoder, on AMD Instinct MI355X (gfx950).
 *
 * The method: the Puro-2B technical report (lkr-homepage blog, section 2
 * "FP8") runs the matmuls of the main linear layers in FP8 using DeepSeek-V3's
 * fine-grained block quantization, and keeps numerically sensitive operations
 * and training state in BF16 or FP32.  This library implements that path with
 * the following reading of the passage:
 *   - codes are OCP E4M3FN (bias 7, no infinities, largest finite 448);
 *   - activations and gradients are quantized in 1x128 tiles along the
 *     contraction axis, weights in 128x128 blocks, one FP32 scale per tile;
 *   - per tile: a = max(amax, 2^-100); s = a/448 and inv = 448/a, each one
 *     correctly rounded FP32 division; code = E4M3 round-to-nearest-even of
 *     clamp(fl32(x*inv), -448, 448); x is represented by dec(code)*s;
 *   - each GEMM sums, per 128-wide contraction block, the FP8 products in
 *     FP32 and folds that partial sum into an FP32 accumulator multiplied by
 *     the two operands' scales for the block.  Outputs are BF16 or FP32.
 * Beside the quantizers and GEMMs, the BF16 ops that produce linear-layer
 * operands in a decoder (RMSNorm, the MLP's SwiGLU and its backward) are
 * offered with their outputs quantized on produce, and several weights can
 * go through the block quantizer in one launch.
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is a device pointer on the current HIP device,
 *     row-major and contiguous.  BF16 is passed as raw uint16_t bit patterns,
 *     E4M3 codes as uint8_t.
 *   - Ownership: the caller owns every buffer.  The library allocates nothing,
 *     frees nothing and keeps no pointer after a call returns.
 *   - Streams: work is enqueued on `stream` (NULL = the null stream) and the
 *     call returns without waiting.  Outputs are valid once the stream has
 *     reached the call.
 *   - Errors: argument errors are detected before anything is enqueued; the
 *     call then returns the status and leaves every output untouched.  A
 *     failed launch returns FP8BS_ERR_HIP.  Sizes so large that one kernel
 *     launch would need more than 2^32 - 1 work-items along a grid dimension
 *     are refused with FP8BS_ERR_SHAPE before anything is enqueued; with
 *     buffers that fit in device memory only the diagnostics
 *     (fp8_encode_e4m3, fp8bs_hbm_rate, fp8bs_mfma_rate) can reach that.  Faults inside a kernel surface at
 *     the caller's next synchronization of the stream.  Inputs must be finite;
 *     the library does not check this (a non-finite input gives unspecified
 *     codes for its tile).
 *   - Alignment: code and BF16 pointers must be 16-byte aligned, scale and
 *     FP32 pointers 4-byte aligned (FP8BS_ERR_ALIGN otherwise).
 *   - Empty tensors (a zero dimension) are valid; their pointers may be NULL.
 *   - Threads: calls are re-entrant and may be made from several host threads
 *     as long as their output buffers do not overlap.
 *   - Kernel choice: the GEMMs pick a 256x256 or a 128x128 workgroup tile by
 *     shape (and, for wgrad, a split of the contraction); the environment
 *     variable FP8BS_GEMM_KERNEL=small|big, read at each call, forces one of
 *     them, for testing both at any size.  Results agree to the GEMM
 *     tolerance either way.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A hipStream_t, spelled without the HIP headers. */
typedef struct ihipStream_t* fp8bs_stream_t;

typedef enum {
    FP8BS_OK = 0,
    FP8BS_ERR_NULL = 1,        /* a required pointer is NULL */
    FP8BS_ERR_SHAPE = 2,       /* a dimension is negative, or not a multiple of 128 where required */
    FP8BS_ERR_ALIGN = 3,       /* a pointer is not aligned as required */
    FP8BS_ERR_DTYPE = 4,       /* unknown output dtype */
    FP8BS_ERR_WORKSPACE = 5,   /* workspace given but too small */
    FP8BS_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed */
    FP8BS_ERR_UNSUPPORTED = 7, /* the device is not gfx950 */
    FP8BS_ERR_VALUE = 8        /* a scalar argument is out of its range */
} fp8bs_status;

typedef enum {
    FP8BS_OUT_F32 = 0,
    FP8BS_OUT_BF16 = 1         /* round to nearest, ties to even */
} fp8bs_out_dtype;

/*
 * Row-tile quantizer (activations for fprop, gradients for dgrad).
 * Puro-2B report, section 2 "FP8": fine-grained quantization of the FP8
 * matmul operands; 1x128 tiles along the contraction axis.
 *   x  bf16 [M, K]  input
 *   q  u8   [M, K]  E4M3 codes (output)
 *   s  f32  [M, K/128]  s[r][j] is the scale of x[r][128j .. 128j+127] (output)
 * M >= 0 (any value), K >= 0 and a multiple of 128.
 */
fp8bs_status fp8_quantize_rowtile(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s,
                                  fp8bs_stream_t stream);

/*
 * Block quantizer (weights).
 * Puro-2B report, section 2 "FP8": block quantization of the weight operand;
 * 128x128 blocks.
 *   w    bf16 [N, K]  input
 *   q    u8   [N, K]  E4M3 codes (output)
 *   q_t  u8   [K, N]  the same codes transposed, q_t[k][n] == q[n][k]
 *                     (output; may be NULL when dgrad is not needed)
 *   s    f32  [N/128, K/128]  s[i][j] covers rows 128i.. and columns 128j..
 * N, K >= 0 and multiples of 128.
 */
fp8bs_status fp8_quantize_block(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, uint8_t* q_t,
                                float* s, fp8bs_stream_t stream);

/*
 * Several weights through the block quantizer at once, each quantized exactly
 * as fp8_quantize_block quantizes it (same passage): a training step
 * quantizes every weight of a layer (or of the model) after the optimizer
 * step, and one launch over all their 128x128 blocks fills the device where a
 * single weight's 256-1536 blocks do not.
 *   jobs   host array of count descriptions (read before the call returns):
 *          w bf16 [N, K], q u8 [N, K], q_t u8 [K, N] or NULL, s f32 [N/128, K/128]
 * Every job is checked as fp8_quantize_block checks its arguments before
 * anything is launched; the first failing check's status is returned and
 * nothing is written.  Jobs with N or K = 0 are skipped.  One launch per 16
 * jobs.  count >= 0 (jobs may be NULL when it is 0).
 */
typedef struct fp8bs_block_job {
    const uint16_t* w;
    int64_t N, K;
    uint8_t* q;
    uint8_t* q_t;
    float* s;
} fp8bs_block_job;
fp8bs_status fp8_quantize_block_many(const fp8bs_block_job* jobs, int count,
                                     fp8bs_stream_t stream);

/*
 * Token-axis (transposed) quantizer for the weight-gradient operands.
 * The weight gradient contracts over tokens, so its operands are quantized in
 * 1x128 tiles of 128 consecutive tokens of one channel: the row-tile
 * quantizer applied to x transposed (Puro-2B report, section 2 "FP8", read
 * for the weight-gradient matmul).
 *   x   bf16 [M, C]  input (M tokens, C channels)
 *   qt  u8   [C, M]  codes of x transposed (output)
 *   st  f32  [C, M/128]  st[c][b] is the scale of x[128b .. 128b+127][c] (output)
 * M >= 0 and a multiple of 128; C >= 0 and a multiple of 128.
 */
fp8bs_status fp8_quantize_transposed(const uint16_t* x, int64_t M, int64_t C, uint8_t* qt,
                                     float* st, fp8bs_stream_t stream);

/*
 * Both quantizations of one tensor from a single read: the outputs of
 * fp8_quantize_rowtile(x) (for fprop or dgrad) and of
 * fp8_quantize_transposed(x) (for wgrad), bit for bit.  A training step needs
 * both for every activation and output gradient of a main linear layer
 * (Puro-2B report, section 2 "FP8"); one pass reads the BF16 tensor once.
 *   x   bf16 [M, C]
 *   q   u8   [M, C],  s  f32 [M, C/128]      as fp8_quantize_rowtile
 *   qt  u8   [C, M],  st f32 [C, M/128]      as fp8_quantize_transposed
 * M, C >= 0 and multiples of 128.
 */
fp8bs_status fp8_quantize_dual(const uint16_t* x, int64_t M, int64_t C, uint8_t* q, float* s,
                               uint8_t* qt, float* st, fp8bs_stream_t stream);

/*
 * SwiGLU with its output quantized on produce (Puro-2B report, section 2
 * "FP8": only the main linear matmuls run in FP8 and the rest of the step
 * keeps BF16/FP32 precision; in a Qwen3-style decoder, the shapes this
 * library is sized for, the MLP's SwiGLU is such BF16 work).  H = silu(G) * U is formed in FP32 and
 * rounded to BF16, exactly where a separate SwiGLU kernel would round it, and
 * that BF16 H is quantized as fp8_quantize_dual(H) would quantize it: the
 * down projection's two operands (row tiles for its fprop, token-axis tiles
 * for its wgrad) come out of one read of the gate/up output, and H is never
 * written to memory in BF16 unless h is given.
 *   gate_up bf16 [M, 2F]  G = columns 0 .. F-1, U = columns F .. 2F-1
 *   q   u8   [M, F],  s  f32 [M, F/128]      row tiles of H
 *   qt  u8   [F, M],  st f32 [F, M/128]      token-axis tiles of H
 *   h   bf16 [M, F] or NULL                  H itself, when given
 * silu(g) = g / (1 + e^-g), evaluated with the hardware exponential and
 * reciprocal (relative error about 2^-20 at the gate values of real
 * activations; below g = -64, where e^-g overflows or the sigmoid is an FP32
 * denormal, H = g u e^g is formed from logarithms, relative error near
 * 2^-15), so H is within one BF16 unit of the exactly rounded value for any
 * finite inputs and the codes are those of fp8_quantize_dual applied to the
 * H this call forms.  M, F >= 0 and multiples of 128.  Inputs must be finite.
 */
fp8bs_status fp8_swiglu_quantize_dual(const uint16_t* gate_up, int64_t M, int64_t F, uint8_t* q,
                                      float* s, uint8_t* qt, float* st, uint16_t* h,
                                      fp8bs_stream_t stream);

/*
 * RMSNorm with its output quantized on produce (Puro-2B report, section 2
 * "FP8": the FP8 path covers the main linear matmuls and the normalizations
 * stay in BF16/FP32; in a Qwen3-style decoder an RMSNorm produces the input of
 * the attention and MLP input projections, whose fprop and wgrad need its
 * row tiles and token-axis tiles).
 *   x     bf16 [M, C],  gamma bf16 [C],  eps >= 0 and finite
 *   q   u8   [M, C],  s  f32 [M, C/128]      row tiles of Y
 *   qt  u8   [C, M],  st f32 [C, M/128]      token-axis tiles of Y
 *   rstd f32 [M]                             r of every row (the backward needs it)
 *   y   bf16 [M, C] or NULL                  Y itself, when given
 * r[m] = 1 / sqrt(mean_c x[m][c]^2 + eps) (squares summed in FP32, correctly
 * rounded square root and division); Y = x * r * gamma in FP32, rounded to
 * BF16; the codes are those of fp8_quantize_dual applied to that BF16 Y.
 * A row whose sum of squares leaves FP32's range (|x| above about 1e19, or
 * every |x| below about 2^-50 with eps below 2^-60) is summed again scaled by
 * a power of two, so any finite row is in range except those whose r itself
 * exceeds FP32 (every |x| a BF16 subnormal, eps below about 1e-77).
 * Two launches on stream (r, then the quantized tiles).  M, C >= 0 and
 * multiples of 128 (nothing is written when either is 0); FP8BS_ERR_VALUE
 * for a negative or non-finite eps.
 */
fp8bs_status fp8_rmsnorm_quantize_dual(const uint16_t* x, const uint16_t* gamma, float eps,
                                       int64_t M, int64_t C, uint8_t* q, float* s, uint8_t* qt,
                                       float* st, float* rstd, uint16_t* y,
                                       fp8bs_stream_t stream);

/*
 * The SwiGLU's backward with its output quantized on produce (same passage:
 * the elementwise backward stays in BF16/FP32; its result, the gradient of
 * the gate/up projection's output, is the dY of that projection's FP8 dgrad
 * and wgrad, which need both of its quantizations).
 *   dh      bf16 [M, F]   gradient of H = silu(G) * U
 *   gate_up bf16 [M, 2F]  the forward's input (G | U)
 *   q   u8   [M, 2F], s  f32 [M, 2F/128]     row tiles of dGU
 *   qt  u8   [2F, M], st f32 [2F, M/128]     token-axis tiles of dGU
 *   dgate_up bf16 [M, 2F] or NULL            dGU itself, when given
 * dGU[:, f] = dh * u * silu'(g) (gate half), dGU[:, F + f] = dh * silu(g)
 * (up half), silu'(g) = s (1 + g (1 - s)), s = 1 / (1 + e^-g), each formed in
 * FP32 with the hardware exponential and reciprocal and rounded to BF16
 * (below g = -64, dh u (1 + g) e^g and dh g e^g from logarithms, as in
 * fp8_swiglu_quantize_dual); the codes are those of fp8_quantize_dual
 * applied to that BF16 dGU (where dh * u overflows FP32 the gate half is also
 * formed from logarithms, so any finite inputs whose gradient is finite are
 * in range).  M, F >= 0 and multiples of 128.  Inputs must be finite.
 */
fp8bs_status fp8_swiglu_backward_quantize_dual(const uint16_t* dh, const uint16_t* gate_up,
                                               int64_t M, int64_t F, uint8_t* q, float* s,
                                               uint8_t* qt, float* st, uint16_t* dgate_up,
                                               fp8bs_stream_t stream);

/*
 * fprop GEMM: Y = X W^T (Puro-2B report, section 2 "FP8": the forward matmul
 * of a main linear layer in FP8).
 *   xq  u8  [M, K],  xs f32 [M, K/128]          from fp8_quantize_rowtile(X)
 *   wq  u8  [N, K],  ws f32 [N/128, K/128]      from fp8_quantize_block(W)
 *   y   [M, N] of dtype yt (FP32 or BF16)       output
 * y[m][n] = sum_kb xs[m][kb] * ws[n/128][kb] * sum_{k in kb} dec(xq[m][k]) dec(wq[n][k]).
 * M >= 0 (any value); N, K >= 0 and multiples of 128.  K == 0 writes zeros.
 */
fp8bs_status fp8_gemm_fprop(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                            void* y, fp8bs_out_dtype yt, int64_t M, int64_t N, int64_t K,
                            fp8bs_stream_t stream);

/*
 * dgrad GEMM: dX = dY W (Puro-2B report, section 2 "FP8": the input-gradient
 * matmul of a main linear layer in FP8).  W keeps the quantization of the
 * forward pass; its codes are read in the transposed copy.
 *   dyq  u8 [M, N],  dys f32 [M, N/128]         from fp8_quantize_rowtile(dY)
 *   wq_t u8 [K, N],  ws  f32 [N/128, K/128]     q_t and s of fp8_quantize_block(W[N,K])
 *   dx   [M, K] of dtype dxt                    output
 * dx[m][k] = sum_nb dys[m][nb] * ws[nb][k/128] * sum_{n in nb} dec(dyq[m][n]) dec(wq_t[k][n]).
 * M >= 0 (any value); N, K >= 0 and multiples of 128.  N == 0 writes zeros.
 */
fp8bs_status fp8_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wq_t,
                            const float* ws, void* dx, fp8bs_out_dtype dxt, int64_t M, int64_t N,
                            int64_t K, fp8bs_stream_t stream);

/*
 * wgrad GEMM: dW = dY^T X, contracted over M tokens (Puro-2B report, section
 * 2 "FP8": the weight-gradient matmul of a main linear layer in FP8).
 *   dytq u8 [N, M],  dyts f32 [N, M/128]        from fp8_quantize_transposed(dY[M,N])
 *   xtq  u8 [K, M],  xts  f32 [K, M/128]        from fp8_quantize_transposed(X[M,K])
 *   dw   f32 [N, K]                             output
 * dw[n][k] = sum_mb dyts[n][mb] * xts[k][mb] * sum_{m in mb} dec(dytq[n][m]) dec(xtq[k][m]).
 * M, N, K >= 0 and multiples of 128.  M == 0 writes zeros.
 * workspace: optional device scratch for splitting the contraction across
 * workgroups (see fp8_gemm_wgrad_workspace_bytes).  With workspace == NULL or
 * workspace_bytes == 0 the call does not split.  A non-NULL workspace smaller
 * than the query returns FP8BS_ERR_WORKSPACE.  The split result is summed in
 * a fixed order, so it is deterministic run to run.
 */
fp8bs_status fp8_gemm_wgrad(const uint8_t* dytq, const float* dyts, const uint8_t* xtq,
                            const float* xts, float* dw, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, fp8bs_stream_t stream);

/*
 * fp8_gemm_wgrad without any allocation, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The result is that of fp8_gemm_wgrad given a
 * workspace of fp8_gemm_wgrad_workspace_bytes(M, N, K) bytes, bit for bit;
 * the split-K slices live in a static device array of
 * FP8BS_NOALLOC_SCRATCH_BYTES per device, allocated when the library is
 * first used on a device and held until the process ends.
 *   dytq, dyts, xtq, xts, dw, M, N, K: as fp8_gemm_wgrad (caller-owned).
 * Errors as fp8_gemm_wgrad; a shape whose split needs more than
 * FP8BS_NOALLOC_SCRATCH_BYTES returns FP8BS_ERR_WORKSPACE and launches
 * nothing.  All calls on one device share its array and every call writes
 * its slices before reading them: calls that may overlap in time on one
 * device (different streams, different host threads) race on it and must be
 * ordered by the caller.  The call allocates no device memory.
 */
#define FP8BS_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
fp8bs_status fp8_gemm_wgrad_noalloc(const uint8_t* dytq, const float* dyts, const uint8_t* xtq,
                                    const float* xts, float* dw, int64_t M, int64_t N, int64_t K,
                                    fp8bs_stream_t stream);

/* Bytes of workspace fp8_gemm_wgrad uses for this shape on the current
 * device (16-byte aligned); 0 when it would not split.  Negative or invalid
 * shapes give 0. */
size_t fp8_gemm_wgrad_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * wgrad accumulated into an existing FP32 gradient: dw[n][k] += G[n][k],
 * where G is the dW fp8_gemm_wgrad computes for the same operands (Puro-2B
 * report, section 2 "FP8": weight gradients and other training state stay in
 * FP32 beside the FP8 matmuls, so a layer's weight gradient is summed into a
 * held FP32 gradient buffer; this does the sum in the same call instead of a
 * separate pass over dW).
 *   dytq, dyts, xtq, xts, M, N, K: as fp8_gemm_wgrad (caller-owned).
 *   dw f32 [N, K]: read and written (caller-owned, FP32 values on entry).
 * The result is dw + G with G summed first, rounded once per element, so it
 * equals dw + (fp8_gemm_wgrad's result) bit for bit.  M == 0 adds zeros.
 * workspace: optional device scratch (see
 * fp8_gemm_wgrad_accumulate_workspace_bytes: it holds every piece of the
 * split, the first included).  With workspace == NULL, workspace_bytes == 0
 * or a shape that does not split, the call does not split and the GEMM's
 * epilogue adds into dw; a non-NULL workspace smaller than the query returns
 * FP8BS_ERR_WORKSPACE.  The split result is deterministic run to run.
 * Errors and alignment as fp8_gemm_wgrad.
 */
fp8bs_status fp8_gemm_wgrad_accumulate(const uint8_t* dytq, const float* dyts, const uint8_t* xtq,
                                       const float* xts, float* dw, int64_t M, int64_t N,
                                       int64_t K, void* workspace, size_t workspace_bytes,
                                       fp8bs_stream_t stream);

/* Bytes of workspace fp8_gemm_wgrad_accumulate uses for this shape on the
 * current device (16-byte aligned): fp8_gemm_wgrad_workspace_bytes plus one
 * N x K FP32 slice when the shape splits, else 0.  Negative or invalid shapes
 * give 0. */
size_t fp8_gemm_wgrad_accumulate_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * The three GEMMs with each 128-wide block's sum of products formed by the
 * FP8 matrix core (v_mfma_f32_16x16x128_f8f6f4, E4M3 x E4M3) instead of
 * exactly (Puro-2B report, section 2 "FP8": the matmuls run on FP8 tensor
 * cores with DeepSeek-V3's recipe, whose tensor-core accumulation inside each
 * 128-wide interval has limited precision and is promoted to FP32 at every
 * interval).  On gfx950 the matrix core adds each group of eight consecutive
 * products in a fixed-point window about 13-14 bits below the group's largest
 * product, truncating the low bits of smaller ones toward zero: a block sum
 * is off by about 1.5e-5 relative on N(0,1)-like tiles and never by more
 * than 2^-9 times the sum of its products' magnitudes.  The fold into the
 * FP32 accumulator, the outputs, shapes, arguments and errors are those of
 * fp8_gemm_fprop, fp8_gemm_dgrad and fp8_gemm_wgrad; these calls do not meet
 * those calls' FP32 accuracy (relative Frobenius error 1e-5) and run at the
 * FP8 rate, twice the FP16 rate those use.  Always the 256 x 256 tile kernel.
 * fp8_gemm_wgrad_mfma8's workspace: see fp8_gemm_wgrad_mfma8_workspace_bytes
 * (the split rules of fp8_gemm_wgrad).  Results are deterministic.
 */
fp8bs_status fp8_gemm_fprop_mfma8(const uint8_t* xq, const float* xs, const uint8_t* wq,
                                  const float* ws, void* y, fp8bs_out_dtype yt, int64_t M,
                                  int64_t N, int64_t K, fp8bs_stream_t stream);
fp8bs_status fp8_gemm_dgrad_mfma8(const uint8_t* dyq, const float* dys, const uint8_t* wq_t,
                                  const float* ws, void* dx, fp8bs_out_dtype dxt, int64_t M,
                                  int64_t N, int64_t K, fp8bs_stream_t stream);
fp8bs_status fp8_gemm_wgrad_mfma8(const uint8_t* dytq, const float* dyts, const uint8_t* xtq,
                                  const float* xts, float* dw, int64_t M, int64_t N, int64_t K,
                                  void* workspace, size_t workspace_bytes, fp8bs_stream_t stream);
/* Bytes of workspace fp8_gemm_wgrad_mfma8 uses for this shape on the current
 * device; 0 when it would not split or the shape is invalid. */
size_t fp8_gemm_wgrad_mfma8_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * dgrad with its output quantized as it is produced (the row-tile quantizer
 * fused into the GEMM epilogue; Puro-2B technical report, section 2 "FP8":
 * BF16 work next to the FP8 matmuls then needs no separate pass over dX to
 * feed an FP8 GEMM).  dX = dY W exactly as fp8_gemm_dgrad computes it, rounded
 * to BF16 (RNE); the BF16 values are then quantized in 1x128 row tiles along
 * K by the rule of fp8_quantize_rowtile, so the codes and scales equal
 * fp8_quantize_rowtile applied to the BF16 dX bit for bit.
 *   dyq, dys, wq_t, ws as fp8_gemm_dgrad; dx bf16 [M,K] or NULL (then only
 *   the codes are written); dxq e4m3 [M,K]; dxs f32 [M,K/128].
 * Shapes and errors as fp8_gemm_dgrad (dxq, dy/w pointers 16-byte aligned,
 * scales 4-byte aligned).  Always the 256x256 tile kernel, no split.
 */
fp8bs_status fp8_gemm_dgrad_quantized(const uint8_t* dyq, const float* dys, const uint8_t* wq_t,
                                      const float* ws, uint16_t* dx, uint8_t* dxq, float* dxs,
                                      int64_t M, int64_t N, int64_t K, fp8bs_stream_t stream);

/*
 * Unquantized comparator (Puro-2B technical report, section 2 "FP8": FP8
 * training is weighed against BF16 training of the same model):
 *   C[I,J] = A B^T,  A bf16 [I,K], B bf16 [J,K] (contraction contiguous),
 * products accumulated in FP32, C BF16 (RNE) or FP32 [I,J] per ct.
 * Any of the three linear-layer GEMMs is this form once its operands are laid
 * out with the contraction contiguous.  I >= 0; J and K positive multiples of
 * 128 (FP8BS_ERR_SHAPE otherwise; J or K = 0 allowed as empty).  All pointers
 * 16-byte aligned device pointers; caller-owned; asynchronous on stream.
 */
fp8bs_status bf16_gemm_tn(const uint16_t* a, const uint16_t* b, void* c, fp8bs_out_dtype ct,
                          int64_t I, int64_t J, int64_t K, fp8bs_stream_t stream);

/*
 * Diagnostic: the quantizers' FP32 -> E4M3 step on its own, elementwise:
 * q[i] = E4M3 round-to-nearest-even of clamp(x[i], -448, 448).  Lets a test
 * sweep the device conversion over any set of FP32 values.
 *   x f32 [n] (16-byte aligned), q u8 [n] (16-byte aligned); n >= 0.
 */
fp8bs_status fp8_encode_e4m3(const float* x, int64_t n, uint8_t* q, fp8bs_stream_t stream);

/*
 * Diagnostic, outside the FP8 path: the attainable FP16 MFMA rate, against
 * which a GEMM's rate can be priced at the clock the chip actually holds
 * under matrix load (the contraction runs on v_mfma_f32_16x16x32_f16).
 * Runs `blocks` workgroups of 256 threads; every wave issues iters x 128 of
 * those instructions (16384 flop each) on operands whose elements all equal
 * v, with no memory traffic, and each thread stores 16384 * v^2 * iters
 * (exact while that is below 2^24).  Work: blocks * 4 * iters * 128 * 16384
 * flop.
 *   out f32 [blocks * 256], 16-byte aligned device memory, caller-owned.
 *   blocks >= 0 (0 does nothing), iters >= 0; FP8BS_ERR_SHAPE otherwise.
 * Asynchronous on stream: time it with events recorded on the same stream.
 */
fp8bs_status fp8bs_mfma_rate(float* out, int64_t blocks, int iters, float v, fp8bs_stream_t stream);

/*
 * Diagnostic, outside the FP8 path: the HBM streaming rate of the
 * quantizers' access pattern without their arithmetic, against which their
 * bandwidth can be priced.  Reads n BF16 values and writes one byte per
 * value to y0 (its high byte) and, when y1 is not NULL, one more to y1 (its
 * low byte): 2 bytes read and 1 (row-tile or token-axis quantizer) or 2
 * (dual-axis quantizer) bytes written per element, in 16-byte accesses.
 *   x bf16 [n], y0 u8 [n], y1 u8 [n] or NULL; all 16-byte aligned device
 *   memory, caller-owned.  n >= 0 (FP8BS_ERR_SHAPE otherwise).
 * Asynchronous on stream: time it with events recorded on the same stream.
 */
fp8bs_status fp8bs_hbm_rate(const uint16_t* x, int64_t n, uint8_t* y0, uint8_t* y1,
                            fp8bs_stream_t stream);

/* Static string naming a status (never NULL). */
const char* fp8bs_status_string(fp8bs_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
int fp8bs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
